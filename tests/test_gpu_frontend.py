"""GPU parity of the In-Place front end (gated input Z, LM-aligned target
V-hat, clipped per-token rates) against the fp64 oracle, and of the whole
In-Place layer built from it (front end + chunk-causal forward).

Tolerances: Z and V-hat are rounded to bf16 once (relative L2 <= 1e-2,
expected ~3e-3); clipped rates come from fp32 Gram sums of exact bf16
products (relative 1e-4 per chunk).
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


def bf(*shape, scale=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("T,dm,dff", [(300, 256, 384), (256, 128, 128), (1000, 512, 256)])
def test_gated_input_small(T, dm, dff):
    """Ragged token count, several feature tiles, the smallest shapes."""
    X, Wg, Wu = bf(T, dm, seed=1), bf(dff, dm, scale=dm ** -0.5, seed=2), bf(dff, dm, scale=dm ** -0.5, seed=3)
    Z = lac.inplace_gated_input(X.to(DEV), Wg.to(DEV), Wu.to(DEV)).cpu()
    ref = oracle.inplace_gated_input(W.to_f64(X), W.to_f64(Wg), W.to_f64(Wu))
    e = oracle.rel_l2(Z.double(), ref)
    say(f"gated input T{T} d_model {dm} d_ff {dff}: rel-L2 {e:.2e}")
    assert e <= 1e-2, e


@pytest.mark.parametrize("B,L,dm,taps", [(2, 300, 256, 4), (1, 77, 512, 1), (3, 64, 256, 16)])
def test_lm_target_small(B, L, dm, taps):
    """Look-ahead convolution stays inside each sequence (B > 1), ragged L,
    one tap, sixteen taps."""
    X, Wv = bf(B, L, dm, seed=4), bf(dm, dm, scale=dm ** -0.5, seed=5)
    cw = 0.5 * torch.randn(taps, dm, generator=torch.Generator().manual_seed(6))
    V = lac.inplace_lm_target(X.to(DEV), cw.to(DEV), Wv.to(DEV)).cpu()
    ref = oracle.lm_aligned_target(W.to_f64(X), W.to_f64(cw), W.to_f64(Wv))
    e = oracle.rel_l2(V.double(), ref)
    say(f"lm target B{B} L{L} d{dm} taps {taps}: rel-L2 {e:.2e}")
    assert e <= 1e-2, e


@pytest.mark.parametrize("L,C", [(700, 256), (1024, 1024), (640, 128)])
def test_clip_eta_small(L, C):
    """Per-chunk scales against the oracle's explicitly formed updates; tau
    between two chunk norms so some chunks clip and some do not; ragged last
    chunk."""
    B, dff, dm, eta = 2, 256, 128, 0.01
    Z, V = bf(B, L, dff, seed=7), bf(B, L, dm, seed=8)
    Zd, Vd = W.to_f64(Z), W.to_f64(V)
    norms = sorted(eta * np.linalg.norm(Zd[b, c:c + C].T @ Vd[b, c:c + C]) for b in range(B) for c in range(0, L, C))
    tau = 0.5 * (norms[len(norms) // 2 - 1] + norms[len(norms) // 2])
    got = lac.inplace_clip_eta(Z.to(DEV), V.to(DEV), chunk=C, eta=eta, tau=tau).cpu().double().numpy()
    ref = oracle.clip_scales(Zd, Vd, C, eta, tau)
    err = np.abs(got - ref) / ref
    say(f"clip L{L} C{C}: max rel err {err.max():.2e}, clipped chunks {(ref < eta).sum() // 1}")
    assert err.max() <= 1e-4, err.max()
    assert (ref < eta * (1 - 1e-6)).any() and (ref == eta).any()


def test_inplace_layer_small():
    """Front end + chunk-causal forward (the whole In-Place layer at a small
    size) against the oracle chain in fp64: O_i = Z_i W_{i-1}, W_i =
    W_{i-1} + Z_i^T diag(eta_i) V-hat_i with clipped rates."""
    B, L, dm, dff, taps, C, eta = 1, 1536, 256, 512, 4, 512, 1e-3
    X = bf(B, L, dm, seed=11)
    Wg, Wu = bf(dff, dm, scale=dm ** -0.5, seed=12), bf(dff, dm, scale=dm ** -0.5, seed=13)
    Wv = bf(dm, dm, scale=dm ** -0.5, seed=14)
    cw = 0.5 * torch.randn(taps, dm, generator=torch.Generator().manual_seed(15))
    W0 = 0.02 * torch.randn(dff, dm, generator=torch.Generator().manual_seed(16))
    Zo = oracle.inplace_gated_input(W.to_f64(X), W.to_f64(Wg), W.to_f64(Wu))
    Vo = oracle.lm_aligned_target(W.to_f64(X), W.to_f64(cw), W.to_f64(Wv))
    norms = sorted(eta * np.linalg.norm(Zo[0, c:c + C].T @ Vo[0, c:c + C]) for c in range(0, L, C))
    tau = 0.5 * (norms[0] + norms[1])
    eo = oracle.clip_scales(Zo, Vo, C, eta, tau)
    Oo, Wfo = oracle.chunk_causal(Zo[:, None], Zo[:, None], Vo[:, None], eta=eo[:, None], S0=W0.double().numpy()[None, None],
                                  chunk=C)
    Xd = X.to(DEV)
    Z = lac.inplace_gated_input(Xd, Wg.to(DEV), Wu.to(DEV))
    V = lac.inplace_lm_target(Xd, cw.to(DEV), Wv.to(DEV))
    e = lac.inplace_clip_eta(Z, V, chunk=C, eta=eta, tau=tau)
    O, Wf, _ = lac.fwd_chunked(Z[:, None], Z[:, None], V[:, None], eta=e[:, None].contiguous(),
                               S0=W0.to(DEV)[None, None].contiguous(), chunk=C, mode="chunk_causal",
                               return_state=True)
    torch.cuda.synchronize()
    eO, eW = oracle.rel_l2(O.cpu().double(), Oo), oracle.rel_l2(Wf.cpu().double(), Wfo)
    say(f"In-Place layer: out rel-L2 {eO:.2e}, W_final rel-L2 {eW:.2e}")
    assert eO <= 1e-2 and eW <= 1e-2, (eO, eW)


def test_frontend_full_size_sampled():
    """The benchmark's shapes (T 32768, d_model 2560, d_ff 9728, 4 taps,
    chunks of 1024) in its launch configuration: sampled tokens of Z and
    V-hat, and sampled chunks' clipped rates, recomputed by the oracle."""
    X, Wg, Wu, cw, Wv = W.gen_inplace_frontend(device=DEV)
    say("front end full: running")
    Z = lac.inplace_gated_input(X, Wg, Wu)
    V = lac.inplace_lm_target(X, cw, Wv)
    tau = 50.0
    e = lac.inplace_clip_eta(Z, V, chunk=1024, eta=1e-3, tau=tau)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 1023, 1024, 17000, 32764, 32767])
    Xr = X[0].index_select(0, rows.to(DEV)).cpu()
    Zs = oracle.inplace_gated_input(W.to_f64(Xr), W.to_f64(Wg.cpu()), W.to_f64(Wu.cpu()))
    ez = oracle.rel_l2(Z[0].index_select(0, rows.to(DEV)).cpu().double(), Zs)
    # V-hat rows need the following taps - 1 tokens of X
    Xw = torch.stack([X[0, r:r + 4].cpu() if r + 4 <= X.shape[1] else
                      torch.cat([X[0, r:].cpu(), torch.zeros(r + 4 - X.shape[1], X.shape[2], dtype=X.dtype)])
                      for r in rows.tolist()])
    Yr = np.einsum("rjd,jd->rd", W.to_f64(Xw), W.to_f64(cw.cpu()))
    Vs = Yr @ W.to_f64(Wv.cpu()).T
    ev = oracle.rel_l2(V[0].index_select(0, rows.to(DEV)).cpu().double(), Vs)
    say(f"front end full: Z rows rel-L2 {ez:.2e}, V-hat rows rel-L2 {ev:.2e}")
    assert ez <= 1e-2 and ev <= 1e-2, (ez, ev)
    for ci in (0, 15, 31):
        zc = W.to_f64(Z[0, 1024 * ci:1024 * (ci + 1)].cpu())
        vc = W.to_f64(V[0, 1024 * ci:1024 * (ci + 1)].cpu())
        nrm = 1e-3 * np.linalg.norm(zc.T @ vc)
        ref = 1e-3 * min(1.0, tau / nrm)
        got = float(e[0, 1024 * ci])
        say(f"  chunk {ci}: update norm {nrm:.3f}, rate {got:.4e} (oracle {ref:.4e})")
        assert abs(got - ref) <= 1e-4 * ref
        assert torch.all(e[0, 1024 * ci:1024 * (ci + 1)] == e[0, 1024 * ci])
