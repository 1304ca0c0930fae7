"""The allocation-free forward entry point (``ttt_fwd_chunked_noalloc``)
against the existing one (``ttt_fwd_chunked``), through the C ABI.

Both run the same kernels and launch plan; the look-back walks a fixed
shape, so results do not depend on where the scratch lives or on timing, and
the two entry points must agree bit for bit (stricter than the bf16 bar of
1e-2).  Two calls in a row share the library's static scratch, the second
with a smaller input and another tile form, so it must clear and reuse what
the first left behind.
"""
import pytest
import torch

import workloads as W
import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def rand(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def pair(B, H, L, dk, dv, beta, seed, eta_per_token=True):
    q, k, v = rand((B, H, L, dk), seed), rand((B, H, L, dk), seed + 1, dk ** -0.5), rand((B, H, L, dv), seed + 2)
    eta = torch.sigmoid(rand((B, H, L), seed + 3, dtype=torch.float32)) * 0.1 if eta_per_token else None
    S0 = rand((B, H, dk, dv), seed + 4, 0.02, torch.float32)
    kw = dict(eta=eta, eta_scalar=0.05, beta=W.f32(beta), S0=S0, chunk=64, return_state=True)
    out_n = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=DEV)
    say(f"no-alloc B{B} H{H} L{L} dk{dk} dv{dv} beta {beta}: workspace "
        f"{lac.fwd_workspace_size(B, H, L, dk, dv, beta=W.f32(beta))} bytes")
    ref = lac.fwd_chunked(q, k, v, check_lookback=True, **kw)
    got = lac.fwd_chunked(q, k, v, out=out_n, no_alloc=True, **kw)
    torch.cuda.synchronize()
    for a, b, n in zip(got, ref, ("out", "S_final", "M_final")):
        if b is None:
            assert a is None, n
            continue
        assert torch.equal(a, b), n


def test_noalloc_matches_fwd_two_calls():
    """A segmented momentum call (64-column tiles, 8 segments per tile), then a
    smaller segmented call with 32-column tiles, then one that needs no
    scratch at all."""
    pair(1, 2, 8192, 128, 128, 0.9, seed=100)
    pair(1, 1, 3000, 64, 32, 0.8, seed=200, eta_per_token=False)
    pair(2, 4, 700, 64, 64, 0.0, seed=300)
