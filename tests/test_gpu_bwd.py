"""GPU parity of the backward pass (``ttt_bwd_chunked``) against the fp64
oracle's adjoint sweeps (``oracle.token_causal_bwd``), which are themselves
pinned by finite differences and autograd on the CPU.

Tolerances (relative L2 over each compared tensor): fp32 inputs <= 1e-5;
bf16 inputs <= 1e-2 for dq, dk, dv, deta (the intermediate P, R are rounded
to bf16 once before the eta scaling) and <= 1e-4 for dS0 without momentum
(exact bf16 products summed in fp32 over L tokens); with momentum the
states carry bf16-level error too (<= 1e-2).  Integer-valued fp32 inputs with a
dyadic eta are exact and must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "deta", "dS0", "dM0")


def say(msg):
    print(msg, flush=True)


def dev(t):
    return None if t is None else t.to(DEV).contiguous()


def make(B, H, L, dk, dv, dtype, seed, per_token=True, s0=True, dsf=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, L, dk, generator=g).to(dtype)
    k = (torch.randn(B, H, L, dk, generator=g) / dk ** 0.5).to(dtype)
    v = torch.randn(B, H, L, dv, generator=g).to(dtype)
    dout = (torch.randn(B, H, L, dv, generator=g) / L ** 0.5).to(dtype)
    eta = (0.1 * torch.rand(B, H, L, generator=g)).float() if per_token else None
    S0 = 0.02 * torch.randn(B, H, dk, dv, generator=g) if s0 else None
    dSf = 0.05 * torch.randn(B, H, dk, dv, generator=g) if dsf else None
    return q, k, v, dout, eta, S0, dSf


def run_gpu(q, k, v, dout, eta, eta_scalar, S0, dSf, beta=0.0, M0=None, dMf=None):
    res = lac.bwd_chunked(dev(q), dev(k), dev(v), dev(dout), eta=dev(eta), eta_scalar=eta_scalar, beta=beta,
                          S0=dev(S0), M0=dev(M0), dS_final=dev(dSf), dM_final=dev(dMf), need_dM0=beta != 0.0)
    torch.cuda.synchronize()
    return [r.cpu() for r in res if r is not None]


def run_oracle(q, k, v, dout, eta, eta_scalar, S0, dSf, beta=0.0, M0=None, dMf=None):
    dq, dk_, dv_, deta, dS0, dM0 = oracle.token_causal_bwd(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(dout),
                                                            W.to_f64(eta), eta_scalar, beta, W.to_f64(S0),
                                                            W.to_f64(M0), W.to_f64(dSf), W.to_f64(dMf))
    return (dq, dk_, dv_, deta, dS0) + ((dM0,) if beta != 0.0 else ())


def check(got, ref, dtype, what, momentum=False):
    tol = {"dq": 1e-5, "dk": 1e-5, "dv": 1e-5, "deta": 1e-5, "dS0": 1e-5, "dM0": 1e-5} if dtype == "f32" else \
          {"dq": 1e-2, "dk": 1e-2, "dv": 1e-2, "deta": 1e-2, "dS0": 1e-4, "dM0": 1e-4}
    if momentum and dtype == "bf16":
        # the momentum weights w(n) are folded into the bf16 value operand of
        # the state update, one bf16 rounding per product: the states carry
        # bf16-level error like every other output
        tol["dS0"] = tol["dM0"] = 1e-2
    errs = {n: oracle.rel_l2(g.double(), r) for n, g, r in zip(NAMES, got, ref)}
    say(f"{what}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol[n], (n, e)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,dk,dv", [(150, 64, 64), (300, 128, 64), (77, 32, 128), (256, 128, 128)])
def test_bwd_small(dtype, L, dk, dv):
    """Ragged and whole chunks, dk != dv both ways, per-token eta, S0 and
    dS_final given."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    args = make(2, 2, L, dk, dv, tdt, seed=L * 7 + dk + dv)
    q, k, v, dout, eta, S0, dSf = args
    say(f"bwd {dtype} L{L} dk{dk} dv{dv}")
    check(run_gpu(q, k, v, dout, eta, 0.0, S0, dSf), run_oracle(q, k, v, dout, eta, 0.0, S0, dSf), dtype,
          f"bwd {dtype} L{L} dk{dk} dv{dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_scalar_eta_no_states(dtype):
    """Scalar eta, no S0 and no dS_final (both zero)."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v, dout, _, _, _ = make(1, 3, 200, 64, 64, tdt, seed=5, per_token=False, s0=False, dsf=False)
    eta = W.f32(0.05)
    check(run_gpu(q, k, v, dout, None, eta, None, None), run_oracle(q, k, v, dout, None, eta, None, None), dtype,
          f"bwd scalar eta {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.9, 0.5])
def test_bwd_momentum(dtype, beta):
    """Momentum: the adjoint of m_t run as a reversed momentum forward from
    the rescaled boundary states; M0 and dM_final given; dM0 checked too."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    beta = W.f32(beta)
    q, k, v, dout, eta, S0, dSf = make(2, 2, 230, 64, 128, tdt, seed=int(beta * 100))
    g = torch.Generator().manual_seed(9)
    M0 = 0.01 * torch.randn(S0.shape, generator=g)
    dMf = 0.05 * torch.randn(S0.shape, generator=g)
    check(run_gpu(q, k, v, dout, eta, 0.0, S0, dSf, beta, M0, dMf),
          run_oracle(q, k, v, dout, eta, 0.0, S0, dSf, beta, M0, dMf), dtype, f"bwd momentum {dtype} beta {beta}",
          momentum=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.7, 0.1, 0.01, 1e-3, 1e-30])
@pytest.mark.parametrize("with_dmf", [False, True])
@pytest.mark.parametrize("L", [40, 230])
def test_bwd_momentum_small_beta(dtype, beta, with_dmf, L):
    """Small momenta, with and without dM_final (large against the other
    cotangents, so its boundary term dominates the last tokens): the
    boundary is taken without dividing by beta, so the error stays at the
    bf16 (fp32) level for every beta.  L = 40 is shorter than the tail
    correction at beta = 0.7 (it reaches token 0 and dM0)."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    beta = W.f32(beta)
    q, k, v, dout, eta, S0, dSf = make(1, 2, L, 64, 128, tdt, seed=L + 3)
    g = torch.Generator().manual_seed(19)
    M0 = 0.01 * torch.randn(S0.shape, generator=g)
    dMf = torch.randn(S0.shape, generator=g) if with_dmf else None
    check(run_gpu(q, k, v, dout, eta, 0.0, S0, dSf, beta, M0, dMf),
          run_oracle(q, k, v, dout, eta, 0.0, S0, dSf, beta, M0, dMf), dtype,
          f"bwd momentum {dtype} L{L} beta {beta:g} dM_final {with_dmf}", momentum=True)


def test_bwd_momentum_segmented():
    """Momentum on a long sequence of few heads (segmented forward passes
    with the affine look-back, in reverse time)."""
    q, k, v, dout, eta, S0, dSf = make(1, 2, 4500, 128, 128, torch.bfloat16, seed=78)
    beta = W.f32(0.9)
    assert lac.bwd_workspace_size(1, 2, 4500, 128, 128, beta=beta) > 0
    check(run_gpu(q, k, v, dout, eta, 0.0, S0, dSf, beta, None, None),
          run_oracle(q, k, v, dout, eta, 0.0, S0, dSf, beta, None, None), "bf16", "bwd momentum segmented",
          momentum=True)


def test_bwd_integer_exact():
    """Small integers, eta = 1/8: every product and sum is exact in fp32."""
    g = torch.Generator().manual_seed(23)
    B, H, L, d = 1, 2, 70, 32
    q, k, v, dout = (torch.randint(-2, 3, (B, H, L, d), generator=g).float() for _ in range(4))
    S0 = torch.randint(-2, 3, (B, H, d, d), generator=g).float()
    dSf = torch.randint(-2, 3, (B, H, d, d), generator=g).float()
    got = run_gpu(q, k, v, dout, None, 0.125, S0, dSf)
    ref = run_oracle(q, k, v, dout, None, 0.125, S0, dSf)
    for n, a, r in zip(NAMES, got, ref):
        assert np.array_equal(a.double().numpy(), r), n


def test_bwd_segmented_sequence():
    """Few heads on a long sequence: the bf16 forward passes cut the sequence
    into segments joined by the look-back, also when time runs backwards."""
    q, k, v, dout, eta, S0, dSf = make(1, 2, 5000, 128, 128, torch.bfloat16, seed=77)
    assert lac.bwd_workspace_size(1, 2, 5000, 128, 128) > 0
    check(run_gpu(q, k, v, dout, eta, 0.0, S0, dSf), run_oracle(q, k, v, dout, eta, 0.0, S0, dSf), "bf16",
          "bwd segmented L5000")


def test_bwd_lm_scale_sampled_heads():
    """The LM-scale shape (B8 H16 L4096 d128, bf16, per-token eta, S0) with
    seeded cotangents, in the benchmark's launch configuration; sampled
    (b, h) heads recomputed whole by the oracle."""
    inp = W.gen_lm_scale()
    dout, dSf = W.gen_lm_scale_cotangents()
    say("bwd lm-scale: running")
    got = run_gpu(inp.q, inp.k, inp.v, dout, inp.eta, 0.0, inp.S0, dSf)
    for b, h in ((0, 0), (3, 7), (7, 15)):
        sl = lambda t: None if t is None else t[b:b + 1, h:h + 1]
        ref = run_oracle(sl(inp.q), sl(inp.k), sl(inp.v), sl(dout), sl(inp.eta), 0.0, sl(inp.S0), sl(dSf))
        check([g[b:b + 1, h:h + 1] for g in got], ref, "bf16", f"bwd lm-scale head ({b},{h})")


def test_bwd_matches_forward_linearisation():
    """Independent of the oracle's backward: for the fp32 path, <dout, J u>
    from two GPU forward calls (central difference in a direction u of q)
    equals <dq, u> from the GPU backward."""
    q, k, v, dout, eta, S0, _ = make(1, 1, 96, 64, 64, torch.float64, seed=31, dsf=False)
    q, k, v, dout = q.float(), k.float(), v.float(), dout.float()
    u = torch.randn(q.shape, generator=torch.Generator().manual_seed(32))
    h = 1e-2   # the forward is linear in q: the difference is exact up to rounding
    op, _, _ = lac.fwd_chunked(dev(q + h * u), dev(k), dev(v), eta=dev(eta), S0=dev(S0), return_state=True)
    om, _, _ = lac.fwd_chunked(dev(q - h * u), dev(k), dev(v), eta=dev(eta), S0=dev(S0), return_state=True)
    fd = float(((op - om).double().cpu() * dout.double()).sum() / (2 * h))
    dq = run_gpu(q, k, v, dout, eta, 0.0, S0, None)[0]
    an = float((dq.double() * u.double()).sum())
    assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), (fd, an)


# ------------------------------------------------------------------ dL/dbeta
def run_dbeta(q, k, v, dout, eta, eta_scalar, beta, M0, dSf, dMf):
    res = lac.bwd_dbeta(dev(q), dev(k), dev(v), dev(dout), eta=dev(eta), eta_scalar=eta_scalar, beta=beta,
                        M0=dev(M0), dS_final=dev(dSf), dM_final=dev(dMf))
    torch.cuda.synchronize()
    return res.cpu().double().numpy()


def oracle_dbeta(q, k, v, dout, eta, eta_scalar, beta, M0, dSf, dMf):
    return oracle.token_causal_dbeta(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(dout), W.to_f64(eta),
                                     eta_scalar, beta, W.to_f64(M0), W.to_f64(dSf), W.to_f64(dMf))


# rel-L2 over the (b, h) values: fp32 inputs run fp32 MFMA (1e-4: the
# tangent state S' grows like t^2 and its readout sums L tokens); bf16 inputs
# read the three states through bf16 copies, one rounding each (2e-2)
DBETA_TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L,dk,dv,beta", [(150, 64, 64, 0.9), (300, 128, 64, 0.5), (77, 32, 128, 0.9),
                                          (256, 128, 128, 0.0), (33, 64, 32, 0.99), (16, 32, 16, 0.7)])
def test_dbeta_small(dtype, L, dk, dv, beta):
    """Ragged lengths (a partial last block, an empty second block of the
    last 32-token stage, a single block), every supported dk, dv from 16 to
    128, beta from 0 to 0.99; per-token eta, M0, dS_final and dM_final all
    given."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    beta = W.f32(beta)
    q, k, v, dout, eta, S0, dSf = make(2, 3, L, dk, dv, tdt, seed=L + dk + dv)
    g = torch.Generator().manual_seed(L)
    M0 = 0.01 * torch.randn(S0.shape, generator=g)
    dMf = 0.05 * torch.randn(S0.shape, generator=g)
    got = run_dbeta(q, k, v, dout, eta, 0.0, beta, M0, dSf, dMf)
    ref = oracle_dbeta(q, k, v, dout, eta, 0.0, beta, M0, dSf, dMf)
    err = oracle.rel_l2(torch.tensor(got), ref)
    say(f"dbeta {dtype} L{L} dk{dk} dv{dv} beta {beta:g}: rel-L2 {err:.2e}")
    assert err <= DBETA_TOL[dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dbeta_scalar_eta_no_states(dtype):
    """Scalar eta, no M0 and no final-state cotangents (all zero)."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v, dout, _, _, _ = make(1, 2, 200, 64, 64, tdt, seed=9, per_token=False, s0=False, dsf=False)
    got = run_dbeta(q, k, v, dout, None, W.f32(0.05), W.f32(0.8), None, None, None)
    ref = oracle_dbeta(q, k, v, dout, None, W.f32(0.05), W.f32(0.8), None, None, None)
    assert oracle.rel_l2(torch.tensor(got), ref) <= DBETA_TOL[dtype]


def test_dbeta_integer_exact_at_zero():
    """At beta = 0 every weight is 0 or 1, so small integers with eta = 1/8
    keep every product and sum exact in fp32: bit-identical to the oracle."""
    g = torch.Generator().manual_seed(29)
    B, H, L, d = 1, 2, 70, 32
    q, k, v, dout = (torch.randint(-2, 3, (B, H, L, d), generator=g).float() for _ in range(4))
    M0, dSf, dMf = (torch.randint(-2, 3, (B, H, d, d), generator=g).float() for _ in range(3))
    got = run_dbeta(q, k, v, dout, None, 0.125, 0.0, M0, dSf, dMf)
    ref = oracle_dbeta(q, k, v, dout, None, 0.125, 0.0, M0, dSf, dMf)
    assert np.array_equal(got, ref), (got, ref)


def test_dbeta_repeat_bit_identical():
    """The column-tile sums are added in a fixed order: repeated calls agree
    bit for bit."""
    q, k, v, dout, eta, _, dSf = make(2, 2, 500, 128, 128, torch.bfloat16, seed=12)
    a = run_dbeta(q, k, v, dout, eta, 0.0, W.f32(0.9), None, dSf, None)
    b = run_dbeta(q, k, v, dout, eta, 0.0, W.f32(0.9), None, dSf, None)
    assert np.array_equal(a, b)


def test_dbeta_momentum_shape_sampled_heads():
    """The momentum workload's shape (B4 H8 L16384 d128, bf16, eta 0.05,
    beta 0.9) with seeded cotangents; sampled heads recomputed by the oracle."""
    inp = W.gen_momentum()
    dout, dSf = W.gen_lm_scale_cotangents(4, 8, 16384, 128, seed_base=4000)
    say("dbeta momentum shape: running")
    got = run_dbeta(inp.q, inp.k, inp.v, dout, None, inp.eta_scalar, inp.beta, None, dSf, None)
    for b, h in ((0, 0), (3, 7)):
        sl = lambda t: None if t is None else t[b:b + 1, h:h + 1]
        ref = oracle_dbeta(sl(inp.q), sl(inp.k), sl(inp.v), sl(dout), None, inp.eta_scalar, inp.beta, None,
                           sl(dSf), None)
        err = abs(got[b, h] - ref[0, 0]) / abs(ref[0, 0])
        say(f"dbeta momentum head ({b},{h}): {got[b, h]:.6e} vs {ref[0, 0]:.6e} rel {err:.2e}")
        assert err <= DBETA_TOL["bf16"], err
