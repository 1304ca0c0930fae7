"""GPU parity of the recurrent decode step (``ttt_decode_step``) against the
fp64 oracle's token-causal recurrence run for one token (L = 1) from the
carried state, and, for a run of consecutive decode steps, against the
oracle over the whole sequence.

Tolerances: fp32 inputs rel-L2 <= 1e-5 on out and state; bf16 inputs
rel-L2 <= 1e-2 on out (rounded to bf16) and <= 1e-5 on the fp32 state
(the state update multiplies exact bf16 values in fp32).  Integer-valued
inputs, whose every product and partial sum is exact in fp32, must match
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def dev(t):
    return None if t is None else t.to(DEV).contiguous()


def run_decode(q, k, v, S, M, eta, eta_scalar, beta):
    """q, k: [B,H,dk]; v: [B,H,dv] (CPU); S, M fp32 [B,H,dk,dv] (CPU) -> (out, S', M') on CPU."""
    Sd, Md = dev(S.clone()), (dev(M.clone()) if M is not None else None)
    out = lac.decode_step(dev(q), dev(k), dev(v), Sd, Md, eta=dev(eta), eta_scalar=eta_scalar, beta=beta)
    torch.cuda.synchronize()
    return out.cpu(), Sd.cpu(), (Md.cpu() if Md is not None else None)


def oracle_step(q, k, v, S, M, eta, eta_scalar, beta):
    """Oracle token-causal recurrence over one token from state (S, M)."""
    eta3 = None if eta is None else eta.reshape(*eta.shape[:2], 1)
    return oracle.token_causal(W.to_f64(q.unsqueeze(2)), W.to_f64(k.unsqueeze(2)), W.to_f64(v.unsqueeze(2)),
                               eta=W.to_f64(eta3), eta_scalar=eta_scalar, beta=beta,
                               S0=W.to_f64(S), M0=W.to_f64(M))


def make(B, H, dk, dv, dtype, beta, seed, per_token=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, dk, generator=g).to(dtype)
    k = (torch.randn(B, H, dk, generator=g) / dk ** 0.5).to(dtype)
    v = torch.randn(B, H, dv, generator=g).to(dtype)
    eta = (0.1 * torch.rand(B, H, generator=g)).float() if per_token else None
    S = 0.02 * torch.randn(B, H, dk, dv, generator=g)
    M = 0.01 * torch.randn(B, H, dk, dv, generator=g) if beta else None
    return q, k, v, eta, S, M


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.0, 0.9])
@pytest.mark.parametrize("B,H,dk,dv", [(2, 3, 40, 72), (1, 2, 128, 128), (3, 1, 1, 4), (1, 1, 1024, 260)])
def test_decode_step_matches_oracle(dtype, beta, B, H, dk, dv):
    """Ragged rows (dk not a multiple of the 16-row groups or 128-row batches),
    ragged columns (dv not a multiple of the 64-column tiles), the smallest
    (dk 1, dv 4) and the largest (dk 1024) head sizes."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    beta = W.f32(beta)
    q, k, v, eta, S, M = make(B, H, dk, dv, tdt, beta, seed=dk * 1000 + dv)
    say(f"decode {dtype} beta {beta} B{B} H{H} dk{dk} dv{dv}")
    out, S1, M1 = run_decode(q, k, v, S, M, eta, 0.0, beta)
    ro, rS, rM = oracle_step(q, k, v, S, M, eta, 0.0, beta)
    eo = oracle.rel_l2(out.float(), ro[:, :, 0])
    eS = oracle.rel_l2(S1, rS)
    say(f"  out rel-L2 {eo:.2e}  S rel-L2 {eS:.2e}")
    assert eo <= (1e-5 if dtype == "f32" else 1e-2), eo
    assert eS <= 1e-5, eS
    if beta:
        eM = oracle.rel_l2(M1, rM)
        assert eM <= 1e-5, eM
    assert out.dtype == tdt


def test_decode_scalar_eta_and_no_state_change_when_eta_zero():
    """eta given as a scalar; eta = 0 leaves S untouched (bit for bit) and
    returns q S."""
    q, k, v, _, S, _ = make(2, 2, 64, 64, torch.float32, 0.0, seed=5)
    out, S1, _ = run_decode(q, k, v, S, None, None, W.f32(0.05), 0.0)
    ro, rS, _ = oracle_step(q, k, v, S, None, None, W.f32(0.05), 0.0)
    assert oracle.rel_l2(out, ro[:, :, 0]) <= 1e-5
    assert oracle.rel_l2(S1, rS) <= 1e-5
    out0, S0, _ = run_decode(q, k, v, S, None, None, 0.0, 0.0)
    assert torch.equal(S0, S)
    assert oracle.rel_l2(out0, torch.einsum("bhi,bhij->bhj", q.double(), S.double()).numpy()) <= 1e-5


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_decode_integer_inputs_bit_exact(beta):
    """Small integers (and beta 0.5): every product and sum is exact in fp32,
    so out, S and M must equal the oracle exactly."""
    g = torch.Generator().manual_seed(17)
    B, H, dk, dv = 2, 2, 48, 68
    q = torch.randint(-2, 3, (B, H, dk), generator=g).float()
    k = torch.randint(-2, 3, (B, H, dk), generator=g).float()
    v = torch.randint(-2, 3, (B, H, dv), generator=g).float()
    S = torch.randint(-3, 4, (B, H, dk, dv), generator=g).float()
    M = torch.randint(-3, 4, (B, H, dk, dv), generator=g).float() if beta else None
    out, S1, M1 = run_decode(q, k, v, S, M, None, 1.0, beta)
    ro, rS, rM = oracle_step(q, k, v, S, M, None, 1.0, beta)
    assert np.array_equal(out.double().numpy(), ro[:, :, 0])
    assert np.array_equal(S1.double().numpy(), rS)
    if beta:
        assert np.array_equal(M1.double().numpy(), rM)


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_decode_steps_follow_the_sequence(beta):
    """L consecutive decode steps from S0 (and M0) give the token-causal
    forward of the whole sequence: every token's output and the final state."""
    g = torch.Generator().manual_seed(99)
    B, H, L, dk, dv = 1, 2, 37, 40, 72
    beta = W.f32(beta)
    q = torch.randn(B, H, L, dk, generator=g)
    k = torch.randn(B, H, L, dk, generator=g) / dk ** 0.5
    v = torch.randn(B, H, L, dv, generator=g)
    eta = (0.1 * torch.rand(B, H, L, generator=g)).float()
    S0 = 0.02 * torch.randn(B, H, dk, dv, generator=g)
    M0 = 0.01 * torch.randn(B, H, dk, dv, generator=g) if beta else None
    Sd, Md = dev(S0.clone()), (dev(M0.clone()) if beta else None)
    outs = []
    for t in range(L):
        outs.append(lac.decode_step(dev(q[:, :, t]), dev(k[:, :, t]), dev(v[:, :, t]), Sd, Md,
                                    eta=dev(eta[:, :, t]), beta=beta))
    out = torch.stack(outs, dim=2).cpu()
    ro, rS, rM = oracle.token_causal(W.to_f64(q), W.to_f64(k), W.to_f64(v), eta=W.to_f64(eta), beta=beta,
                                     S0=W.to_f64(S0), M0=W.to_f64(M0))
    assert oracle.rel_l2(out, ro) <= 1e-5
    assert oracle.rel_l2(Sd.cpu(), rS) <= 1e-5
    if beta:
        assert oracle.rel_l2(Md.cpu(), rM) <= 1e-5


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_decode_full_size(beta):
    """The benchmark's decode workload (B 256, H 16, d 128, bf16, per-sequence
    eta, carried fp32 state), in its launch configuration, checked whole."""
    inp = W.gen_decode(beta=beta)
    say(f"decode full B256 H16 d128 beta {inp.beta}")
    q, k, v = inp.q[:, :, 0], inp.k[:, :, 0], inp.v[:, :, 0]
    eta = inp.eta[:, :, 0]
    out, S1, M1 = run_decode(q, k, v, inp.S0, inp.M0, eta, 0.0, inp.beta)
    ro, rS, rM = oracle_step(q, k, v, inp.S0, inp.M0, eta, 0.0, inp.beta)
    eo, eS = oracle.rel_l2(out.float(), ro[:, :, 0]), oracle.rel_l2(S1, rS)
    say(f"  out rel-L2 {eo:.2e}  S rel-L2 {eS:.2e}")
    assert eo <= 1e-2, eo
    assert eS <= 1e-5, eS
    if inp.beta:
        assert oracle.rel_l2(M1, rM) <= 1e-5


def test_decode_rejects_cpu_and_bad_shapes():
    q = torch.zeros(1, 1, 8, device=DEV)
    S = torch.zeros(1, 1, 8, 8, device=DEV)
    with pytest.raises(ValueError):
        lac.decode_step(q, q, q, S, torch.zeros(1, 1, 8, 4, device=DEV), beta=0.5)
    with pytest.raises(lac.TTTError):
        lac.decode_step(q, q, q, S, None, beta=0.5)   # momentum without M
    with pytest.raises(lac.TTTError):
        lac.decode_step(q, q, torch.zeros(1, 1, 6, device=DEV), torch.zeros(1, 1, 8, 6, device=DEV))
