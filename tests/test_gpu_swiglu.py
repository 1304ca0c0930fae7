"""GPU parity of the large-chunk SwiGLU fast weight (``ttt_swiglu_fwd_chunked``)
against the fp64 oracle (``oracle.swiglu_fast_weight``), itself pinned by
autograd, per-token SGD loops and finite differences on the CPU.

Tolerances (relative L2): bf16 inputs, so the bf16 bar 1e-2 for the outputs
and for the weight change of the whole call (W_final - W0; its operands are
bf16 activations and bf16 copies of the weights, accumulated in fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


def say(msg):
    print(msg, flush=True)


def run_gpu(inp, eta=True, eta_scalar=0.0):
    W1, W3, W2 = (t.to(DEV).clone() for t in (inp.W1, inp.W3, inp.W2))
    out = lac.swiglu_fwd_chunked(inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV), W1, W3, W2,
                                 eta=inp.eta.to(DEV) if eta else None, eta_scalar=eta_scalar, chunk=inp.chunk,
                                 loss=inp.loss)
    torch.cuda.synchronize()
    return out.cpu(), W1.cpu(), W3.cpu(), W2.cpu()


def run_oracle(inp, eta=True, eta_scalar=0.0, sl=slice(None)):
    f = lambda t: W.to_f64(t[sl].cpu())
    return oracle.swiglu_fast_weight(f(inp.q), f(inp.k), f(inp.v), f(inp.W1), f(inp.W3), f(inp.W2),
                                     eta=f(inp.eta) if eta else None, eta_scalar=eta_scalar, chunk=inp.chunk,
                                     loss=inp.loss)


def check(got, ref, W0, what):
    out, W1, W3, W2 = got
    ro, r1, r3, r2 = ref
    errs = {"out": oracle.rel_l2(out.double(), ro)}
    for nm, g, r, w0 in (("dW1", W1, r1, W0[0]), ("dW3", W3, r3, W0[1]), ("dW2", W2, r2, W0[2])):
        w0 = W.to_f64(w0)
        errs[nm] = oracle.rel_l2(W.to_f64(g) - w0, r - w0)
    say(f"{what}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL, (n, e)


@pytest.mark.parametrize("loss", ["dot", "mse"])
@pytest.mark.parametrize("L,C,dk,dv,m", [(300, 128, 128, 256, 256), (512, 256, 256, 128, 384),
                                          (100, 128, 128, 128, 128), (1000, 384, 128, 128, 256),
                                          (700, 256, 128, 256, 512), (513, 512, 384, 256, 256)])
def test_swiglu_small(loss, L, C, dk, dv, m):
    """Whole and ragged last chunks, a single partial chunk, dk != dv both
    ways, hidden sizes that are not a power of two; per-token eta.  The last
    two shapes (hidden, dv and chunk multiples of 256) take the 256-wide
    tiles of the output, dA and update GEMMs, the others the 128-wide ones;
    the last has a 1-token final chunk.  The step
    size is kept below the stability limit of the MSE step (the top
    eigenvalue of sum_t eta_t a_t a_t^T stays well under 2), so rounding
    differences are not amplified from chunk to chunk."""
    inp = W.gen_swiglu(B=1, H=2, L=L, d=dk, dv=dv, m=m, chunk=C, loss=loss, seed_base=L + dk + m,
                       eta_scale=0.5 / (C ** 0.5 + m ** 0.5) ** 2)
    say(f"swiglu {loss} L{L} C{C} dk{dk} dv{dv} m{m}")
    check(run_gpu(inp), run_oracle(inp), (inp.W1, inp.W3, inp.W2), f"swiglu {loss} L{L} C{C}")


@pytest.mark.parametrize("loss", ["dot", "mse"])
def test_swiglu_scalar_eta_and_long_chunk(loss):
    """Scalar eta; a chunk longer than the sequence is one chunk over all of it."""
    inp = W.gen_swiglu(B=2, H=1, L=200, d=128, m=256, chunk=4096, loss=loss, seed_base=77)
    eta = W.f32(3e-3)
    say(f"swiglu {loss} scalar eta, chunk 4096 > L 200")
    check(run_gpu(inp, eta=False, eta_scalar=eta), run_oracle(inp, eta=False, eta_scalar=eta),
          (inp.W1, inp.W3, inp.W2), f"swiglu {loss} scalar eta")


def test_swiglu_zero_eta_is_pure_readout():
    """eta = 0: the weights stay bit for bit and every chunk reads with W0."""
    inp = W.gen_swiglu(B=1, H=1, L=256, d=128, m=128, chunk=128, seed_base=5)
    out, W1, W3, W2 = run_gpu(inp, eta=False, eta_scalar=0.0)
    assert torch.equal(W1, inp.W1) and torch.equal(W3, inp.W3) and torch.equal(W2, inp.W2)
    ref = oracle.swiglu_apply(W.to_f64(inp.q[0, 0]), W.to_f64(inp.W1[0, 0]), W.to_f64(inp.W3[0, 0]),
                              W.to_f64(inp.W2[0, 0]))
    assert oracle.rel_l2(out[0, 0].double(), ref) <= TOL


def test_swiglu_full_size_sampled_heads():
    """The benchmark's workload (B4 H4 L32768, d 512, hidden 2048, C2048, dot
    loss, per-token eta) in its launch configuration; heads (0, 0) and
    (3, 3) recomputed whole by the oracle (all 16 chunks)."""
    inp = W.gen_swiglu(device=DEV)
    say("swiglu full size: running")
    got = run_gpu(inp)
    for b, h in ((0, 0), (3, 3)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = run_oracle(inp, sl=sl)
        check([g[sl] for g in got], ref, tuple(t[sl].cpu() for t in (inp.W1, inp.W3, inp.W2)),
              f"swiglu full size head ({b},{h})")


def test_swiglu_binding_rejects():
    q = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device=DEV)
    W1 = torch.zeros(1, 1, 128, 128, device=DEV)
    with pytest.raises(ValueError):
        lac.swiglu_fwd_chunked(q, q, q, W1, W1.clone(), W1.clone(), loss="l1")
    with pytest.raises(ValueError):
        lac.swiglu_fwd_chunked(q.float(), q, q, W1, W1.clone(), W1.clone())
    with pytest.raises(lac.TTTError):
        lac.swiglu_fwd_chunked(q, q, q, W1, W1.clone(), W1.clone(), chunk=100)
