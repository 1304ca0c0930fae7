"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (relative L2 over the whole compared tensor, fp64): fp32 inputs
<= 1e-5, bf16 inputs <= 1e-2.  Integer-valued fp32 inputs whose every
partial sum is exact must match bit for bit.  Full-size workloads are run
in the launch configuration the benchmark times and checked on sampled
(batch, head) slices that the oracle recomputes whole.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def to_dev(t):
    return None if t is None else t.to(DEV)


def run_fwd(inp: W.TokenCausalInputs, mode="token_causal", chunk=None):
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    if inp.q is inp.k:
        k = q
    # check_lookback: a segmented call also reports that no look-back wait gave up
    out, Sf, Mf = lac.fwd_chunked(q, k, v, eta=to_dev(inp.eta), eta_scalar=inp.eta_scalar,
                                  beta=inp.beta, S0=to_dev(inp.S0), M0=to_dev(inp.M0),
                                  chunk=chunk or inp.chunk, mode=mode, return_state=True, check_lookback=True)
    torch.cuda.synchronize()
    return out.cpu(), Sf.cpu(), (Mf.cpu() if Mf is not None else None)


def sl(t, b, h):
    return None if t is None else t[b:b + 1, h:h + 1]


def oracle_tc(inp, heads=None, mode="token_causal", chunk=None):
    """Oracle on all heads or on a list of (b, h)."""
    if heads is None:
        heads = [(b, h) for b in range(inp.q.shape[0]) for h in range(inp.q.shape[1])]
    res = []
    for b, h in heads:
        args = (sl(inp.q, b, h), sl(inp.k, b, h), sl(inp.v, b, h))
        if mode == "token_causal":
            o, S, M = oracle.token_causal(*args, eta=sl(inp.eta, b, h), eta_scalar=inp.eta_scalar,
                                          beta=inp.beta, S0=sl(inp.S0, b, h), M0=sl(inp.M0, b, h))
        else:
            o, S = oracle.chunk_causal(*args, eta=sl(inp.eta, b, h), eta_scalar=inp.eta_scalar,
                                       S0=sl(inp.S0, b, h), chunk=chunk or inp.chunk)
            M = None
        res.append((b, h, o, S, M))
    return res


def check(inp, got, ref, tol, what=""):
    out, Sf, Mf = got
    for b, h, o, S, M in ref:
        e = oracle.rel_l2(out[b, h].float(), o[0, 0])
        assert e <= tol, f"{what} out (b={b},h={h}) rel-L2 {e:.3e} > {tol}"
        e = oracle.rel_l2(Sf[b, h], S[0, 0])
        assert e <= tol, f"{what} S_final (b={b},h={h}) rel-L2 {e:.3e} > {tol}"
        if Mf is not None and M is not None:
            e = oracle.rel_l2(Mf[b, h], M[0, 0])
            assert e <= tol, f"{what} M_final (b={b},h={h}) rel-L2 {e:.3e} > {tol}"


def whole_rel(inp, got, ref):
    out = got[0]
    num = den = 0.0
    for b, h, o, _, _ in ref:
        d = out[b, h].double().numpy() - o[0, 0]
        num += float((d * d).sum())
        den += float((o[0, 0] ** 2).sum())
    return (num / den) ** 0.5


# ------------------------------------------------------------- token-causal
def test_small_f32_token_causal():
    inp = W.gen_small_f32()
    say("small fp32 B1 H2 L256 d32 C64")
    got = run_fwd(inp)
    ref = oracle_tc(inp)
    check(inp, got, ref, TOL["f32"], "small fp32")
    # the O(L^2) brute force agrees too
    bf = oracle.bruteforce_token_causal(inp.q, inp.k, inp.v, eta_scalar=inp.eta_scalar)
    assert oracle.rel_l2(got[0], bf) <= TOL["f32"]


@pytest.mark.parametrize("L,d,dv", [(250, 32, 32), (97, 64, 64), (300, 128, 128), (64, 128, 64), (1, 64, 32)])
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_token_causal_fp32_shapes(L, d, dv, beta):
    g = torch.Generator().manual_seed(L * 7 + d + int(beta * 10))
    B, H = 2, 3
    q = torch.randn(B, H, L, d, generator=g) / d ** 0.5
    k = torch.randn(B, H, L, d, generator=g) / d ** 0.5
    v = torch.randn(B, H, L, dv, generator=g)
    eta = 0.1 * torch.sigmoid(torch.randn(B, H, L, generator=g))
    S0 = 0.05 * torch.randn(B, H, d, dv, generator=g)
    M0 = 0.05 * torch.randn(B, H, d, dv, generator=g) if beta else None
    inp = W.TokenCausalInputs(q, k, v, eta, 0.0, W.f32(beta), S0, M0, 32, "f32")
    say(f"fp32 token-causal L{L} d{d} dv{dv} beta{beta}")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["f32"], "fp32")


def test_token_causal_fp32_integer_exact():
    """Integer inputs, eta = 1/8: every fp32 partial sum is exact, so the GPU
    output equals the oracle bit for bit regardless of summation order."""
    g = torch.Generator().manual_seed(99)
    B, H, L, d = 2, 2, 160, 32
    q = torch.randint(-2, 3, (B, H, L, d), generator=g).float()
    k = torch.randint(-2, 3, (B, H, L, d), generator=g).float()
    v = torch.randint(-2, 3, (B, H, L, d), generator=g).float()
    S0 = torch.randint(-2, 3, (B, H, d, d), generator=g).float()
    inp = W.TokenCausalInputs(q, k, v, None, 0.125, 0.0, S0, None, 32, "f32")
    say("fp32 integer exact")
    out, Sf, _ = run_fwd(inp)
    for b, h, o, S, _ in oracle_tc(inp):
        assert np.array_equal(out[b, h].double().numpy(), o[0, 0])
        assert np.array_equal(Sf[b, h].double().numpy(), S[0, 0])


def test_lm_recipe_small_bf16_ragged():
    inp = W.gen_lm_scale(B=2, H=3, L=250, d=128)
    say("LM recipe bf16 B2 H3 L250 d128")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "LM recipe small")


@pytest.mark.parametrize("d,dv", [(64, 64), (32, 32), (128, 64), (64, 128)])
def test_token_causal_bf16_shapes(d, dv):
    inp = W.gen_lm_scale(B=1, H=4, L=200, d=d)
    if dv != d:
        g = torch.Generator().manual_seed(5)
        inp.v = torch.randn(1, 4, 200, dv, generator=g).to(torch.bfloat16)
        inp.S0 = 0.02 * torch.randn(1, 4, d, dv, generator=g)
    say(f"bf16 token-causal d{d} dv{dv}")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "bf16 shapes")


def test_lm_scale_full_sampled_heads():
    """Full LM-scale workload (B8 H16 L4096 d128 C64) in the benchmark's launch
    configuration; sampled heads checked against the oracle."""
    inp = W.gen_lm_scale()
    say("LM-scale full B8 H16 L4096 d128")
    got = run_fwd(inp)
    heads = [(0, 0), (3, 7), (5, 15), (7, 9)]
    ref = oracle_tc(inp, heads)
    check(inp, got, ref, TOL["bf16"], "LM-scale full")
    assert torch.isfinite(got[0].float()).all()


@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_token_causal_bf16_wide_grid(beta):
    """B*H*d_v/64 >= 512 selects the 64-token x 64-column tiling (8 waves)."""
    inp = W.gen_lm_scale(B=16, H=16, L=150, d=128)
    inp.beta = W.f32(beta)
    say(f"bf16 token-causal wide grid B16 H16 L150 beta{beta}")
    got = run_fwd(inp)
    check(inp, got, oracle_tc(inp, [(0, 0), (7, 3), (15, 15)]), TOL["bf16"], "wide grid")


def test_momentum_small():
    inp = W.gen_momentum(B=2, H=2, L=700, d=128)
    say("momentum recipe bf16 B2 H2 L700")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "momentum small")


def test_momentum_full_sampled_heads():
    inp = W.gen_momentum()
    say("momentum full B4 H8 L16384 d128 beta0.9")
    got = run_fwd(inp)
    ref = oracle_tc(inp, [(0, 0), (2, 5), (3, 7)])
    check(inp, got, ref, TOL["bf16"], "momentum full")


# ------------------------------------------------- segmented sequences (look-back)
def _seeded(shape, seed, scale):
    return scale * torch.randn(*shape, generator=torch.Generator().manual_seed(seed))


@pytest.mark.parametrize("beta", [0.0, 0.001, 0.5, 0.9, 0.97])
def test_segmented_sequence_lookback(beta):
    """Two heads of 5000 tokens: too few (head, column tile) pairs to fill the
    chip, so the sequence is cut into segments that run concurrently and
    chain their states through the decoupled look-back (ragged last segment,
    non-zero S0 and, with momentum, M0).  With momentum up to 0.95 the
    segment aggregates come from the plain sum and the momentum aggregate of
    the last chunks (a one-chunk tail at 0.001); 0.97 takes the chunk
    recurrence."""
    inp = W.gen_lm_scale(B=1, H=2, L=5000, d=128)
    inp.beta = W.f32(beta)
    if beta:
        inp.M0 = _seeded((1, 2, 128, 128), 7001, 0.01)
    assert lac.fwd_workspace_size(1, 2, 5000, 128, 128, beta=inp.beta) > 0, "shape is not segmented"
    say(f"segmented look-back bf16 B1 H2 L5000 d128 beta{beta}")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "segmented")


def test_segmented_narrow_columns():
    """d_v = 32 (32 x 32 tile form, two workgroups per CU) with segmentation."""
    g = torch.Generator().manual_seed(7100)
    B, H, L, dk, dv = 1, 1, 3000, 64, 32
    q = torch.randn(B, H, L, dk, generator=g).to(torch.bfloat16)
    k = (torch.randn(B, H, L, dk, generator=g) / 8).to(torch.bfloat16)
    v = torch.randn(B, H, L, dv, generator=g).to(torch.bfloat16)
    S0 = 0.02 * torch.randn(B, H, dk, dv, generator=g)
    inp = W.TokenCausalInputs(q, k, v, None, W.f32(0.05), W.f32(0.8), S0, None, 64, "bf16")
    assert lac.fwd_workspace_size(B, H, L, dk, dv, beta=inp.beta) > 0, "shape is not segmented"
    say("segmented d_v=32 momentum B1 H1 L3000 dk64")
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "segmented dv32")


def test_segmented_chunk_causal():
    """Chunk-causal mode: segment boundaries fall on chunk boundaries."""
    g = torch.Generator().manual_seed(7200)
    B, H, L, d, dv, C = 1, 2, 4500, 64, 64, 192
    z = (torch.randn(B, H, L, d, generator=g) / 8).to(torch.bfloat16)
    vh = torch.randn(B, H, L, dv, generator=g).to(torch.bfloat16)
    eta = 0.05 * torch.rand(B, H, L, generator=g)
    W0 = 0.02 * torch.randn(B, H, d, dv, generator=g)
    inp = W.TokenCausalInputs(z, z, vh, eta, 0.0, 0.0, W0, None, C, "bf16")
    assert lac.fwd_workspace_size(B, H, L, d, dv, chunk=C, mode="chunk_causal") > 0
    say("segmented chunk-causal bf16 B1 H2 L4500 C192")
    got = run_fwd(inp, mode="chunk_causal")
    check(inp, got, oracle_tc(inp, mode="chunk_causal"), TOL["bf16"], "segmented chunk-causal")


@pytest.mark.parametrize("L", [12000, 16384])
def test_segmented_repeat_calls_bit_identical(L):
    """The look-back walks a fixed shape (aggregates back to a fixed
    inclusive state or to the start), so results never depend on which
    segment finished first: 20 back-to-back calls on the same inputs give
    bit-identical outputs and final states.  L = 16384 is the momentum
    workload's shape (B4 H8 d128, 4 segments per column tile); L = 12000 on
    one head cuts 12 segments, so the walk also passes through an inclusive
    state of the chain."""
    inp = W.gen_momentum(L=L) if L == 16384 else W.gen_momentum(B=1, H=1, L=L, d=128)
    B, H = inp.q.shape[:2]
    assert lac.fwd_workspace_size(B, H, L, 128, 128, beta=inp.beta) > 0, "shape is not segmented"
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    say(f"segmented repeat B{B} H{H} L{L} momentum, 20 calls")
    ref = None
    for i in range(20):
        out, Sf, Mf = lac.fwd_chunked(q, k, v, eta_scalar=inp.eta_scalar, beta=inp.beta, chunk=inp.chunk,
                                      return_state=True, check_lookback=True)
        if ref is None:
            ref = (out, Sf, Mf)
            continue
        for a, b, n in zip((out, Sf, Mf), ref, ("out", "S_final", "M_final")):
            assert torch.equal(a, b), (i, n)
    torch.cuda.synchronize()


def test_segmented_lookback_gave_up_is_reported():
    """A look-back wait that gives up is reported, not silent: with a wait
    bound of zero polls (forced from the host) every segment but the first
    gives up at once, the kernel still runs to its end, and the status query
    reports TTT_ERR_TIMEOUT.  A normal call on the same shape afterwards is
    correct and reports nothing."""
    inp = W.gen_momentum(B=1, H=1, L=6000, d=128)
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    say("segmented look-back with a zero wait bound (forced give-up)")
    with pytest.raises(lac.TTTError) as ei:
        lac.fwd_chunked(q, k, v, eta_scalar=inp.eta_scalar, beta=inp.beta, chunk=inp.chunk, check_lookback=True,
                        lookback_polls=-1)
    assert ei.value.status == lac.TTT_ERR_TIMEOUT
    torch.cuda.synchronize()
    check(inp, run_fwd(inp), oracle_tc(inp), TOL["bf16"], "segmented after a forced give-up")


# ------------------------------------------------------------- chunk-causal
@pytest.mark.parametrize("dtype,C", [("bf16", 64), ("bf16", 192), ("f32", 32), ("f32", 96)])
def test_chunk_causal_small(dtype, C):
    g = torch.Generator().manual_seed(C)
    B, H, L, d, dv = 2, 2, 333, 64, 128
    z = torch.randn(B, H, L, d, generator=g) / 8
    vh = torch.randn(B, H, L, dv, generator=g)
    eta = 0.05 * torch.rand(B, H, L, generator=g)
    W0 = 0.02 * torch.randn(B, H, d, dv, generator=g)
    if dtype == "bf16":
        z, vh = z.to(torch.bfloat16), vh.to(torch.bfloat16)
    inp = W.TokenCausalInputs(z, z, vh, eta, 0.0, 0.0, W0, None, C, dtype)
    say(f"chunk-causal {dtype} C{C}")
    got = run_fwd(inp, mode="chunk_causal")
    check(inp, got, oracle_tc(inp, mode="chunk_causal"), TOL[dtype], "chunk-causal")


# ------------------------------------------------------------- state scan
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_state_scan(beta):
    B, H, L, C, dk, dv = 2, 3, 1000, 64, 32, 48
    N = (L + C - 1) // C
    dS, dM = W.gen_state_deltas(B, H, N, dk, dv, seed=6000)
    S0, M0 = W.gen_state_deltas(B, H, 1, dk, dv, seed=6100)
    S0, M0 = S0[:, :, 0].contiguous(), M0[:, :, 0].contiguous()
    say(f"state scan beta{beta}")
    Se, Me, Sf, Mf = lac.chunk_state_scan(dS.to(DEV), dM.to(DEV), beta=W.f32(beta), chunk=C, L=L,
                                          S0=S0.to(DEV), M0=M0.to(DEV))
    torch.cuda.synchronize()
    rSe, rMe, rSf, rMf = oracle.state_scan(dS, dM if beta else None, W.f32(beta), C, L, S0, M0 if beta else None)
    assert oracle.rel_l2(Se.cpu(), rSe) <= 1e-5
    assert oracle.rel_l2(Sf.cpu(), rSf) <= 1e-5
    if beta:
        assert oracle.rel_l2(Me.cpu(), rMe) <= 1e-5
        assert oracle.rel_l2(Mf.cpu(), rMf) <= 1e-5


def test_state_scan_integer_exact():
    B, H, L, C, dk, dv = 1, 2, 640, 64, 16, 16
    dS, _ = W.gen_state_deltas(B, H, L // C, dk, dv, integer=True)
    say("state scan integer exact")
    Se, _, Sf, _ = lac.chunk_state_scan(dS.to(DEV), beta=0.0, chunk=C, L=L)
    torch.cuda.synchronize()
    rSe, _, rSf, _ = oracle.state_scan(dS, None, 0.0, C, L)
    assert np.array_equal(Se.cpu().double().numpy(), rSe)
    assert np.array_equal(Sf.cpu().double().numpy(), rSf)


def test_scan_matches_fused_forward_states():
    """Chunk aggregates scanned on the GPU reproduce the state the fused
    forward kernel carries (momentum, ragged tail)."""
    inp = W.gen_momentum(B=1, H=2, L=300, d=32)
    inp.q, inp.k, inp.v = inp.q.float(), inp.k.float(), inp.v.float()
    dS, dM = oracle.chunk_aggregates(inp.k, inp.v, None, inp.eta_scalar, inp.beta, 32)
    dS, dM = torch.from_numpy(dS).float(), torch.from_numpy(dM).float()
    _, _, Sf, Mf = lac.chunk_state_scan(dS.to(DEV), dM.to(DEV), beta=inp.beta, chunk=32, L=300)
    _, Sg, Mg = run_fwd(inp, chunk=32)
    assert oracle.rel_l2(Sf.cpu(), Sg) <= 1e-5
    assert oracle.rel_l2(Mf.cpu(), Mg) <= 1e-5


# ------------------------------------------------------------- dual form
def run_dual(inp: W.DualInputs, segmented=True):
    out, Wf = lac.dual_form_fwd(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.W0),
                                eta=inp.eta, minibatch=inp.minibatch, return_state=True,
                                segmented=segmented, check_lookback=segmented)
    torch.cuda.synchronize()
    return out.cpu(), Wf.cpu()


def dual_segments(inp: W.DualInputs) -> bool:
    B, H, L, d = inp.q.shape
    return lac.dual_form_workspace_size(B, H, L, d, inp.v.shape[-1], minibatch=inp.minibatch,
                                        dtype=inp.q.dtype) > 0


def check_dual(inp, got, heads, tol, what):
    out, Wf = got
    for b, h in heads:
        o, Wr = oracle.dual_primal(sl(inp.q, b, h), sl(inp.k, b, h), sl(inp.v, b, h), sl(inp.W0, b, h),
                                   inp.eta, inp.minibatch)
        e = oracle.rel_l2(out[b, h].float(), o[0, 0])
        assert e <= tol, f"{what} out (b={b},h={h}) rel-L2 {e:.3e}"
        e = oracle.rel_l2(Wf[b, h], Wr[0, 0])
        assert e <= tol, f"{what} W_final (b={b},h={h}) rel-L2 {e:.3e}"


@pytest.mark.parametrize("segmented", [False, True])
@pytest.mark.parametrize("mb,L", [(16, 300), (64, 1000), (2048, 4096), (1, 70), (48, 200)])
def test_dual_small(mb, L, segmented):
    inp = W.gen_dual(B=1, H=2, L=L, minibatch=mb)
    say(f"dual bf16 b{mb} L{L} segmented={segmented}")
    check_dual(inp, run_dual(inp, segmented), [(0, 0), (0, 1)], TOL["bf16"], "dual")


@pytest.mark.parametrize("segmented", [False, True])
@pytest.mark.parametrize("mb,L", [(256, 1000), (512, 1500), (768, 1536), (4096, 8192), (2048, 2100), (32, 4100)])
def test_dual_large_minibatch(mb, L, segmented):
    """Mini-batches of many 16-token steps with ragged ends: the last
    mini-batch partial (1000, 1500, 2100 tokens), the last 32-token ring
    stage holding one step and a partial tail (4100 tokens, b = 32: one
    stage per mini-batch) and a mini-batch of the whole sequence (8192)."""
    inp = W.gen_dual(B=1, H=3, L=L, minibatch=mb)
    say(f"dual bf16 b{mb} L{L} segmented={segmented}")
    check_dual(inp, run_dual(inp, segmented), [(0, 0), (0, 1), (0, 2)], TOL["bf16"], f"dual b{mb} L{L}")


@pytest.mark.parametrize("mb,L,B,H", [(16, 1000, 1, 2), (16, 4111, 1, 3), (48, 1003, 1, 2), (32, 1500, 2, 1),
                                      (64, 2500, 1, 2), (2048, 8192, 1, 2), (16, 2048, 3, 5),
                                      (16, 2100, 3, 16), (48, 1000, 4, 25), (16, 1000, 2, 64)])
def test_dual_segmented(mb, L, B, H):
    """The segmented form (each segment composes the affine maps of the
    segments before it): several segments per head, ragged last segments
    (L not a multiple of the segment, of 64 or of 16), one-step, per-step
    and stage-end mini-batch ends; against the oracle and against the one-
    chain form, with no look-back wait giving up.  The last two shapes have
    more segments than the slots hold (48 sequences x 6 segments, 100 x 3,
    128 x 3), so segment 0 hands on its end state and its workgroup goes on
    to the last segment; 48 and 128 sequences take the per-XCD ticket
    groups, 100 one counter."""
    inp = W.gen_dual(B=B, H=H, L=L, minibatch=mb)
    assert dual_segments(inp), "this shape should run in segments"
    say(f"dual segmented bf16 B{B} H{H} b{mb} L{L}")
    got = run_dual(inp, True)
    heads = [(b, h) for b in range(B) for h in range(H)][:4]
    check_dual(inp, got, heads, TOL["bf16"], f"dual seg b{mb} L{L}")
    ref = run_dual(inp, False)
    assert oracle.rel_l2(got[0].float(), ref[0].float()) <= 5e-3
    assert oracle.rel_l2(got[1], ref[1]) <= 5e-3


@pytest.mark.parametrize("mb", [16, 64, 48])
def test_dual_many_sequences(mb):
    """Enough sequences to fill the chip without segments (B*H = 512, more
    than one wave per CU covers): one workgroup per sequence."""
    inp = W.gen_dual(B=4, H=128, L=300, minibatch=mb)
    assert not dual_segments(inp)
    say(f"dual bf16 B4 H128 b{mb} L300")
    check_dual(inp, run_dual(inp, True), [(0, 0), (3, 127), (1, 7)], TOL["bf16"], f"dual many b{mb}")


def test_dual_segmented_alternating_inputs():
    """Back-to-back calls with different inputs of one shape reuse the same
    workspace memory: every call must read the maps its own segments
    published, never a previous call's (which would put another sequence's
    maps into the start states)."""
    a = W.gen_dual(B=1, H=4, L=4096, minibatch=16, seed_base=5100)
    b = W.gen_dual(B=1, H=4, L=4096, minibatch=16, seed_base=5200)
    assert dual_segments(a)
    ref = {id(x): run_dual(x, False) for x in (a, b)}
    for x in (a, b, a, b, a):
        got = run_dual(x, True)
        assert oracle.rel_l2(got[0].float(), ref[id(x)][0].float()) <= 5e-3
        assert oracle.rel_l2(got[1], ref[id(x)][1]) <= 5e-3


def test_dual_segmented_long_composition():
    """One sequence of 20000 tokens: 79 segments of 256, so the last one
    composes 78 maps (twenty batches staged through the ring) before its
    tokens; against the oracle and the one-chain form."""
    inp = W.gen_dual(B=1, H=1, L=20000, minibatch=16)
    assert lac.dual_form_workspace_size(1, 1, 20000, 64, 64, minibatch=16) == 512 + 79 * 32768
    say("dual segmented B1 H1 L20000 b16 (79 segments)")
    got = run_dual(inp, True)
    check_dual(inp, got, [(0, 0)], TOL["bf16"], "dual seg 79")
    ref = run_dual(inp, False)
    assert oracle.rel_l2(got[0].float(), ref[0].float()) <= 5e-3


def test_dual_segmented_repeat_bit_identical():
    """Segments compose their predecessors' maps in a fixed order, so
    repeated calls give the same bits whatever the timing."""
    inp = W.gen_dual(B=1, H=4, L=4096, minibatch=16)
    assert dual_segments(inp)
    a = run_dual(inp, True)
    for _ in range(5):
        b = run_dual(inp, True)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("mb", [16, 40])
def test_dual_fp32(mb):
    inp = W.gen_dual(B=1, H=2, L=256, minibatch=mb)
    inp.q, inp.k, inp.v = inp.q.float(), inp.k.float(), inp.v.float()
    say(f"dual fp32 b{mb}")
    check_dual(inp, run_dual(inp), [(0, 0), (0, 1)], TOL["f32"], "dual fp32")


@pytest.mark.parametrize("mb", [16, 2048])
def test_dual_full_sampled_heads(mb):
    inp = W.gen_dual(minibatch=mb)
    say(f"dual full B4 H16 L8192 d64 b{mb}")
    check_dual(inp, run_dual(inp), [(0, 0), (1, 9), (3, 15)], TOL["bf16"], f"dual b{mb}")


def test_dual_fixed_point_exact():
    """v = k W0 makes every gradient zero: out = q W0 exactly (fp32)."""
    inp = W.gen_dual(B=1, H=2, L=200, minibatch=16)
    q, k = inp.q.float(), inp.k.float()
    out, Wf = lac.dual_form_fwd(q.to(DEV), k.to(DEV), (0.5 * k).to(DEV), inp.W0.to(DEV), eta=inp.eta,
                                minibatch=16, return_state=True)
    torch.cuda.synchronize()
    assert oracle.rel_l2(out.cpu(), 0.5 * q) <= 1e-6
    assert oracle.rel_l2(Wf.cpu(), inp.W0) <= 1e-6


@pytest.mark.parametrize("mb", [16, 2048])
def test_dual_fixed_point_exact_bf16(mb):
    """The same fixed point in bf16 (v = k W0 with W0 = I/2 is exact in
    bf16): every corrected value is exactly zero, so out = q/2 and
    W_final = W0 bit for bit, with one-step and with 128-step mini-batches
    (one chain per sequence)."""
    inp = W.gen_dual(B=1, H=2, L=4096, minibatch=mb)
    k = inp.k
    out, Wf = lac.dual_form_fwd(inp.q.to(DEV), k.to(DEV), (0.5 * k.float()).to(torch.bfloat16).to(DEV),
                                inp.W0.to(DEV), eta=inp.eta, minibatch=mb, return_state=True, segmented=False)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), (0.5 * inp.q.float()).to(torch.bfloat16))
    assert torch.equal(Wf.cpu(), inp.W0)


@pytest.mark.parametrize("mb", [16, 2048])
def test_dual_fixed_point_segmented_bf16(mb):
    """The fixed point through segments: a segment's start state is W0
    composed with its predecessors' maps (A - I, B), which agree with W0 =
    A W0 + B only up to the bf16 operand rounding of the maps' chains, so
    out and W_final match q/2 and W0 to that level rather than bit for bit."""
    inp = W.gen_dual(B=1, H=2, L=4096, minibatch=mb)
    assert dual_segments(inp)
    k = inp.k
    out, Wf = lac.dual_form_fwd(inp.q.to(DEV), k.to(DEV), (0.5 * k.float()).to(torch.bfloat16).to(DEV),
                                inp.W0.to(DEV), eta=inp.eta, minibatch=mb, return_state=True, check_lookback=True)
    torch.cuda.synchronize()
    assert oracle.rel_l2(out.cpu().float(), 0.5 * inp.q.float()) <= 2e-3
    assert oracle.rel_l2(Wf.cpu(), inp.W0) <= 2e-3


# ------------------------------------------------------------- properties
def test_head_isolation_and_determinism():
    inp = W.gen_lm_scale(B=2, H=4, L=256, d=64)
    o1 = run_fwd(inp)[0]
    o2 = run_fwd(inp)[0]
    assert torch.equal(o1, o2), "repeated calls must be bit-identical"
    inp.v = inp.v.clone()
    inp.v[1, 2] += 1
    o3 = run_fwd(inp)[0]
    diff = (o3.float() - o1.float()).abs().flatten(2).amax(-1)
    assert diff[1, 2] > 0 and int((diff > 0).sum()) == 1


def test_continuation_equals_one_call():
    """fwd(L1) then fwd(L2, S0 = S_final) equals fwd(L1 + L2) (fixed-size state)."""
    g = torch.Generator().manual_seed(3)
    B, H, L1, L2, d = 1, 2, 96, 160, 64
    q = torch.randn(B, H, L1 + L2, d, generator=g) / 8
    k = torch.randn(B, H, L1 + L2, d, generator=g) / 8
    v = torch.randn(B, H, L1 + L2, d, generator=g)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    full, Sf, Mf = lac.fwd_chunked(qd, kd, vd, eta_scalar=0.1, beta=0.5, return_state=True)
    a, Sa, Ma = lac.fwd_chunked(qd[:, :, :L1], kd[:, :, :L1], vd[:, :, :L1], eta_scalar=0.1, beta=0.5,
                                return_state=True)
    b, Sb, Mb = lac.fwd_chunked(qd[:, :, L1:], kd[:, :, L1:], vd[:, :, L1:], eta_scalar=0.1, beta=0.5,
                                S0=Sa, M0=Ma, return_state=True)
    torch.cuda.synchronize()
    assert oracle.rel_l2(torch.cat([a, b], 2).cpu(), full.cpu()) <= 1e-5
    assert oracle.rel_l2(Sb.cpu(), Sf.cpu()) <= 1e-5


def test_strided_inputs():
    """q, k, v as views of a packed [B, L, H, 3, d] projection give the same result."""
    g = torch.Generator().manual_seed(8)
    B, L, H, d = 2, 130, 3, 64
    qkv = torch.randn(B, L, H, 3, d, generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = (qkv[:, :, :, i].permute(0, 2, 1, 3) for i in range(3))
    o1 = lac.fwd_chunked(q, k, v, eta_scalar=0.05)
    o2 = lac.fwd_chunked(q.contiguous(), k.contiguous(), v.contiguous(), eta_scalar=0.05)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------- In-Place TTT, large fast weight
def run_inplace(Z, V, W0, eta_scalar, C, eta=None):
    Zd, Vd = Z.to(DEV), V.to(DEV)
    out, Wf, _ = lac.fwd_chunked(Zd, Zd, Vd, eta=None if eta is None else eta.to(DEV), eta_scalar=eta_scalar,
                                 S0=W0.to(DEV), chunk=C, mode="chunk_causal", return_state=True)
    torch.cuda.synchronize()
    return out, Wf


@pytest.mark.parametrize("L,C,per_token", [(2048, 256, False), (2000, 512, True), (1024, 1024, False)])
def test_inplace_midsize_vs_oracle(L, C, per_token):
    """dk = 512, dv = 256 (multiples of the 256-wide tiles), ragged and exact L."""
    g = torch.Generator().manual_seed(L + C)
    dk, dv = 512, 256
    a = torch.randn(1, 1, L, dk, generator=g).to(torch.bfloat16).float()
    b = torch.randn(1, 1, L, dk, generator=g).to(torch.bfloat16).float()
    Z = (torch.nn.functional.silu(a) * b).to(torch.bfloat16)
    V = torch.randn(1, 1, L, dv, generator=g).to(torch.bfloat16)
    W0 = 0.02 * torch.randn(1, 1, dk, dv, generator=g)
    eta = (1e-3 * torch.rand(1, 1, L, generator=g)).float() if per_token else None
    say(f"in-place mid-size L{L} C{C} per-token-eta {per_token}")
    out, Wf = run_inplace(Z, V, W0, W.f32(1e-3), C, eta)
    ref, Wr = oracle.chunk_causal(Z, Z, V, eta=eta, eta_scalar=W.f32(1e-3), S0=W0, chunk=C)
    e = oracle.rel_l2(out.cpu().float(), ref)
    ew = oracle.rel_l2(Wf.cpu(), Wr)
    say(f"in-place mid-size: out rel-L2 {e:.2e}, W_final rel-L2 {ew:.2e}")
    assert e <= TOL["bf16"], e
    assert ew <= (TOL["bf16"] if per_token else 1e-5), ew
    # first chunk reads W0 only
    assert oracle.rel_l2(out[0, 0, :C].cpu().float(), (Z[0, 0, :C].double() @ W0[0, 0].double()).numpy()) <= TOL["bf16"]


@pytest.mark.parametrize("C", [512, 256])
def test_inplace_wide_tiles_vs_oracle(C):
    """d_k = 4864 = 16 x 304, d_v = 1280 = 4 x 320 with a scalar eta: the
    update walk runs on the wide 304 x 320 tiles (the In-Place workload's
    path, 64 tiles here); the whole output and the whole final weight against
    the oracle, and the first chunk against its plain GEMM."""
    g = torch.Generator().manual_seed(4864 + C)
    L, dk, dv = 1024, 4864, 1280
    a = torch.randn(1, 1, L, dk, generator=g).to(torch.bfloat16).float()
    b = torch.randn(1, 1, L, dk, generator=g).to(torch.bfloat16).float()
    Z = (torch.nn.functional.silu(a) * b).to(torch.bfloat16)
    V = torch.randn(1, 1, L, dv, generator=g).to(torch.bfloat16)
    W0 = 0.02 * torch.randn(1, 1, dk, dv, generator=g)
    say(f"in-place wide tiles L{L} dk{dk} dv{dv} C{C}")
    out, Wf = run_inplace(Z, V, W0, W.f32(1e-3), C, None)
    ref, Wr = oracle.chunk_causal(Z, Z, V, eta=None, eta_scalar=W.f32(1e-3), S0=W0, chunk=C)
    e = oracle.rel_l2(out.cpu().float(), ref)
    ew = oracle.rel_l2(Wf.cpu(), Wr)
    say(f"in-place wide tiles C{C}: out rel-L2 {e:.2e}, W_final rel-L2 {ew:.2e}")
    assert e <= TOL["bf16"], e
    assert ew <= 1e-5, ew
    assert oracle.rel_l2(out[0, 0, :C].cpu().float(), (Z[0, 0, :C].double() @ W0[0, 0].double()).numpy()) <= TOL["bf16"]


@pytest.mark.parametrize("L", [32768, 131072])
def test_inplace_full_sampled_rows(L):
    """In-Place Wdown update at d_ff 9728, d_model 2560, C 1024 (B = H = 1),
    in the benchmark's launch configuration; sampled rows of O (first, middle
    and last chunks) by the oracle's per-row closed form, plus sampled entries
    of the final weight."""
    say(f"in-place full L{L} d_ff9728 d_model2560 C1024 (generating inputs)")
    Zd = torch.empty((1, 1, L, 9728), dtype=torch.bfloat16, device=DEV)
    Vd = torch.empty((1, 1, L, 2560), dtype=torch.bfloat16, device=DEV)
    Zc = torch.empty((1, 1, L, 9728), dtype=torch.bfloat16)
    Vc = torch.empty((1, 1, L, 2560), dtype=torch.bfloat16)
    inp = W.gen_inplace(L=L, out=(Zc, Vc))
    Zd.copy_(Zc)
    Vd.copy_(Vc)
    say("in-place full: running")
    out, Wf, _ = lac.fwd_chunked(Zd, Zd, Vd, eta_scalar=inp.eta_scalar, S0=inp.S0.to(DEV), chunk=1024,
                                 mode="chunk_causal", return_state=True)
    torch.cuda.synchronize()
    rows = np.array([0, 777, 1023, 1024, 5000, L // 2 + 3, L - 1025, L - 1])
    say("in-place full: oracle rows")
    ref = oracle.chunk_causal_rows(Zc[0, 0], Zc[0, 0], Vc[0, 0], rows, inp.eta_scalar, inp.S0[0, 0], 1024)
    got = out[0, 0, torch.from_numpy(rows).to(DEV)].cpu().float()
    e = oracle.rel_l2(got, ref)
    say(f"in-place full L{L}: sampled-row rel-L2 {e:.2e}")
    assert e <= TOL["bf16"], e
    # final weight W0 + eta Z^T V: three whole rows (2560 entries each) and
    # three whole columns (9728 entries each, through every row tile of the
    # update), fp64 sums over blocks of tokens
    rr = [0, 4321, 9727]
    cc = [0, 1234, 2559]
    say("in-place full: final-weight rows and columns")
    rows_ref = torch.zeros(len(rr), 2560, dtype=torch.float64)
    cols_ref = torch.zeros(9728, len(cc), dtype=torch.float64)
    for t0 in range(0, L, 8192):
        Zb, Vb = Zc[0, 0, t0:t0 + 8192], Vc[0, 0, t0:t0 + 8192]
        rows_ref += Zb[:, rr].double().T @ Vb.double()
        cols_ref += Zb.double().T @ Vb[:, cc].double()
    W0 = inp.S0[0, 0].double()
    rows_ref = W0[rr] + inp.eta_scalar * rows_ref
    cols_ref = W0[:, cc] + inp.eta_scalar * cols_ref
    Wc = Wf[0, 0].cpu().double()
    er, ec = oracle.rel_l2(Wc[rr], rows_ref), oracle.rel_l2(Wc[:, cc], cols_ref)
    say(f"in-place full L{L}: W_final rows rel-L2 {er:.2e}, columns rel-L2 {ec:.2e} "
        f"({len(rr) * 2560 + len(cc) * 9728} entries)")
    # scalar eta: the update sums exact bf16 x bf16 products in fp32
    assert er <= 1e-4 and ec <= 1e-4, (er, ec)
