"""The entry points inside captured HIP graphs.

The segmented token-causal forward and the segmented dual form clear their
flags with a fill kernel (not a memset node), and the backward can fork its dv/deta step onto
a caller's second stream and join it back through events.  Both must capture into a
graph and replay correctly: each test replays the graph several times, with
the inputs changed in place and eager work (an eager call on the same inputs)
in between, and checks every replay against that eager result.
"""
import pytest
import torch

import linear_attention_chunked_amd as lac

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def rel(x, ref):
    x, ref = x.double(), ref.double()
    return float((x - ref).norm() / ref.norm())


def rand(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def test_segmented_forward_in_graph():
    """B1 H2 L4096 d128 bf16: 4 (head, column tile) pairs, so the sequence is
    cut into 4 segments that chain through the look-back flags."""
    B, H, L, d = 1, 2, 4096, 128
    q, k, v = rand((B, H, L, d), 1), rand((B, H, L, d), 2, 1 / d ** 0.5), rand((B, H, L, d), 3)
    eta = torch.sigmoid(rand((B, H, L), 4, dtype=torch.float32)) * 0.1
    S0 = rand((B, H, d, d), 5, 0.02, torch.float32)
    out = torch.empty_like(v)

    def call():
        return lac.fwd_chunked(q, k, v, eta=eta, S0=S0, chunk=64, out=out, return_state=True)

    say("graph: segmented forward, warm-up and capture")
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, S_g, _ = call()
    for rep in range(3):
        q.mul_(0.75)
        v.add_(0.125)
        _, S_e, _ = call()
        o_e = out.clone()
        S_e = S_e.clone()
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        eo, es = rel(out, o_e), rel(S_g, S_e)
        say(f"replay {rep}: out {eo:.2e}  S_final {es:.2e}")
        # the look-back walks a fixed shape: replays equal eager calls bit for bit
        assert torch.equal(out, o_e) and torch.equal(S_g, S_e), (rep, eo, es)


@pytest.mark.parametrize("mb", [16, 2048])
def test_segmented_dual_form_in_graph(mb):
    """B1 H4 L8192 d64 bf16 dual form in segments (flags cleared by a fill
    kernel, maps published and composed in order): replays equal eager calls
    bit for bit."""
    B, H, L, d = 1, 4, 8192, 64
    q, k, v = rand((B, H, L, d), 21, 1 / 8), rand((B, H, L, d), 22, 1 / 8), rand((B, H, L, d), 23, 1 / 8)
    W0 = (0.5 * torch.eye(d, device=DEV)).expand(B, H, d, d).contiguous()
    assert lac.dual_form_workspace_size(B, H, L, d, d, minibatch=mb) > 0
    out = torch.empty_like(v)

    def call():
        return lac.dual_form_fwd(q, k, v, W0, eta=1.0 / d, minibatch=mb, out=out, return_state=True)

    say(f"graph: segmented dual form b{mb}, warm-up and capture")
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, W_g = call()
    for rep in range(3):
        q.mul_(0.75)
        v.add_(0.0625)
        _, W_e = call()
        o_e = out.clone()
        W_e = W_e.clone()
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}: out {rel(out, o_e):.2e}  W_final {rel(W_g, W_e):.2e}")
        assert torch.equal(out, o_e) and torch.equal(W_g, W_e), rep


@pytest.mark.parametrize("side", [False, True])
def test_backward_in_graph(side):
    """B1 H2 L512 d64 bf16 backward (not segmented: results are reproducible),
    on one stream and with the dv/deta step forked onto a second stream."""
    B, H, L, d = 1, 2, 512, 64
    side_stream = torch.cuda.Stream() if side else None
    q, k, v = rand((B, H, L, d), 11), rand((B, H, L, d), 12, 1 / d ** 0.5), rand((B, H, L, d), 13)
    dout = rand((B, H, L, d), 14, 1 / L ** 0.5)
    eta = torch.sigmoid(rand((B, H, L), 15, dtype=torch.float32)) * 0.1
    S0 = rand((B, H, d, d), 16, 0.02, torch.float32)
    dSf = rand((B, H, d, d), 17, 0.02, torch.float32)

    def call():
        return lac.bwd_chunked(q, k, v, dout, eta=eta, S0=S0, dS_final=dSf, side_stream=side_stream)

    say(f"graph: backward (helper stream: {side}), warm-up and capture")
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res_g = call()
    names = ("dq", "dk", "dv", "deta", "dS0")
    for rep in range(3):
        dout.mul_(-1.5)
        q.add_(0.0625)
        res_e = [t.clone() for t in call()[:5]]
        torch.cuda.synchronize()
        for t in res_g[:5]:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        errs = {n: rel(a, b) for n, a, b in zip(names, res_g[:5], res_e)}
        say(f"replay {rep}: " + "  ".join(f"{n} {e:.1e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e == 0.0, (rep, n, e)
