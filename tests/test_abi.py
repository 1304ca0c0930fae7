"""C-ABI checks that need no GPU: the library loads, exports every function
that include/ttt.h declares, the binding's struct matches the C layout, and
invalid arguments are rejected with the documented status before any launch
(validation never touches the HIP runtime, so these run on a CPU host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

import linear_attention_chunked_amd as lac  # noqa: E402

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_ALIAS, ERR_VALUE, ERR_TIMEOUT = range(11)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lac.LIB_PATH):
        from linear_attention_chunked_amd import build
        build.build(verbose=False)
    return lac.load_library()


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ttt_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"ttt_fwd_chunked", "ttt_chunk_state_scan", "ttt_dual_form_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout(lib):
    assert lib.ttt_fwd_args_size() == ctypes.sizeof(lac.FwdArgs)


def test_status_strings(lib):
    for s in range(11):
        assert len(lib.ttt_status_string(s)) > 0
    assert lib.ttt_status_string(123) == b"unknown status"


FAKE = 1 << 32  # aligned fake device addresses; never dereferenced by validation


def fwd_args(**kw):
    a = lac.FwdArgs()
    B, H, L, dk, dv = kw.get("B", 2), kw.get("H", 2), kw.get("L", 128), kw.get("dk", 64), kw.get("dv", 64)
    a.B, a.H, a.L, a.dk, a.dv, a.chunk = B, H, L, dk, dv, kw.get("chunk", 64)
    a.mode, a.dtype = kw.get("mode", 0), kw.get("dtype", 1)
    size_q, size_v = B * H * L * dk * 2, B * H * L * dv * 2
    a.q = kw.get("q", FAKE)
    a.k = kw.get("k", FAKE + size_q + 4096)
    a.v = kw.get("v", FAKE + 2 * (size_q + 4096))
    a.out = kw.get("out", FAKE + 2 * (size_q + 4096) + size_v + 4096)
    a.q_stride = lac._i64x3(H * L * dk, L * dk, dk)
    a.k_stride = lac._i64x3(H * L * dk, L * dk, dk)
    a.v_stride = lac._i64x3(H * L * dv, L * dv, dv)
    a.out_stride = lac._i64x3(H * L * dv, L * dv, dv)
    for name, val in kw.items():
        if name.endswith("_stride"):
            setattr(a, name, lac._i64x3(*val))
    a.eta_scalar = 0.1
    a.beta = kw.get("beta", 0.0)
    return a


def status(lib, a):
    return lib.ttt_fwd_chunked(ctypes.byref(a))


def test_fwd_rejects_before_launch(lib):
    assert status(lib, fwd_args(q=None)) == ERR_NULL
    assert status(lib, fwd_args(out=None)) == ERR_NULL
    assert status(lib, fwd_args(L=0)) == ERR_SHAPE
    assert status(lib, fwd_args(B=-1)) == ERR_SHAPE
    assert status(lib, fwd_args(chunk=0)) == ERR_SHAPE
    assert status(lib, fwd_args(dtype=7)) == ERR_DTYPE
    assert status(lib, fwd_args(mode=5)) == ERR_VALUE
    assert status(lib, fwd_args(beta=1.0)) == ERR_VALUE
    assert status(lib, fwd_args(beta=-0.1)) == ERR_VALUE
    assert status(lib, fwd_args(mode=1, beta=0.5)) == ERR_VALUE
    assert status(lib, fwd_args(q=FAKE + 2)) == ERR_ALIGN
    assert status(lib, fwd_args(q_stride=(2 * 128 * 64, 128 * 64, 68))) == ERR_ALIGN
    assert status(lib, fwd_args(q_stride=(2 * 128 * 64, 128 * 64, 56))) == ERR_SHAPE
    assert status(lib, fwd_args(q_stride=(2 * 128 * 64, 128 * 64, 1 << 23))) == ERR_SHAPE  # L stride bound
    assert status(lib, fwd_args(dk=48)) == ERR_UNSUP
    assert status(lib, fwd_args(dv=256)) == ERR_UNSUP
    assert status(lib, fwd_args(mode=1, chunk=100)) == ERR_UNSUP
    # the In-Place kernels address 256 token rows with 32-bit offsets
    big = dict(mode=1, dk=256, dv=256, chunk=256, L=256, B=1, H=1)
    assert status(lib, fwd_args(q_stride=(256 << 22, 256 << 22, 1 << 22), **big)) == ERR_UNSUP
    assert status(lib, fwd_args(v_stride=(256 << 22, 256 << 22, 1 << 22), **big)) == ERR_UNSUP
    # out overlapping an input
    a = fwd_args()
    a.out = a.v
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args()
    a.out = a.q
    assert status(lib, a) == ERR_ALIAS


def test_fwd_rejects_overlapping_written_buffers(lib):
    """Every written buffer (out, S_final, M_final, the workspace) must miss
    every input and every other written buffer, and out must not overlap
    itself through its strides; inputs may share memory."""
    far = FAKE + (1 << 28)
    st = 2 * 2 * 64 * 64 * 4                       # bytes of one [2,2,64,64] fp32 state
    a = fwd_args()
    a.S0 = a.out                                   # out over S0
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args()
    a.S_final = a.q                                # S_final over q
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args()
    a.S0, a.S0_stride = far + 64 * 64 * 4 * 3, lac._i64x2(0, 0)   # one S0 for all heads ...
    a.S_final = far                                # ... lying inside S_final's head 3
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args(beta=0.5)
    a.S_final, a.M_final = far, far + st - 256     # M_final overlaps S_final
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args()
    a.eta, a.eta_stride = a.out + 64, lac._i64x3(2 * 128, 128, 1)   # eta inside out
    assert status(lib, a) == ERR_ALIAS
    a = fwd_args()
    a.S_final = a.out + 1024                       # S_final inside out
    assert status(lib, a) == ERR_ALIAS
    # out's strides map two heads onto the same rows
    assert status(lib, fwd_args(out_stride=(2 * 128 * 64, 0, 64))) == ERR_ALIAS
    assert status(lib, fwd_args(out_stride=(0, 128 * 64, 64))) == ERR_ALIAS
    assert status(lib, fwd_args(out_stride=(2 * 128 * 64, 64 * 64, 64))) == ERR_ALIAS   # heads interleave rows
    # a workspace (segmented look-back) over q
    a = fwd_args(B=1, H=1, L=4096, dk=128, dv=128)
    need = ctypes.c_size_t(0)
    assert lib.ttt_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)) == OK and need.value > 0
    a.workspace, a.workspace_bytes = a.q, need.value
    assert status(lib, a) == ERR_ALIAS


def test_scan_dual_decode_reject_overlaps(lib):
    f = lib.ttt_chunk_state_scan
    blk = 8 * 8 * 4
    base = lambda **kw: [1, 1, 64, 16, 8, 8, kw.get("dS", FAKE), kw.get("dM", FAKE + 65536), 0.5,
                         kw.get("S0", FAKE + 4 * 65536), None, kw.get("Se", FAKE + 2 * 65536), None,
                         kw.get("Sf", FAKE + 3 * 65536), None, None, 0, None]
    assert f(*base(Se=FAKE)) == ERR_ALIAS                       # in-place scan
    assert f(*base(Sf=FAKE + 4 * 65536 + blk // 2)) == ERR_ALIAS  # S_final over S0
    assert f(*base(Sf=FAKE + 2 * 65536 + blk)) == ERR_ALIAS     # S_final inside S_excl
    d = lib.ttt_dual_form_fwd
    n = 4 * 64 * 64 * 2

    def dargs(**kw):
        return [1, 1, 64, 64, 64, 16, 1, FAKE, FAKE + n, FAKE + 2 * n, kw.get("W0", FAKE + 3 * n), 0, 0.01,
                kw.get("out", FAKE + 4 * n), kw.get("Wf", None), None, 0, None]
    assert d(*dargs(Wf=FAKE + 3 * n)) == ERR_ALIAS               # W_final on W0 (broadcast)
    assert d(*dargs(out=FAKE + 3 * n)) == ERR_ALIAS              # out on W0
    assert d(*dargs(Wf=FAKE + 4 * n + 64)) == ERR_ALIAS          # W_final inside out
    dec = lib.ttt_decode_step
    m = 1 << 20

    def cargs(**kw):
        return [2, 2, 64, 64, 1, FAKE, FAKE + m, FAKE + 2 * m, kw.get("eta", None), 0.1, 0.5,
                kw.get("S", FAKE + 3 * m), FAKE + 4 * m, kw.get("out", FAKE + 5 * m), None]
    assert dec(*cargs(S=FAKE + 256)) == ERR_ALIAS                # S (written) over q
    assert dec(*cargs(eta=FAKE + 5 * m)) == ERR_ALIAS            # eta under out


def test_lookback_status_without_segments(lib):
    """A call that is not segmented never waits: its status query answers 0
    without touching the device; a segmented call without a workspace is
    rejected before any device access."""
    flag = ctypes.c_int32(7)
    a = fwd_args()                                    # B2 H2 L128: one segment per head
    assert lib.ttt_fwd_lookback_status(ctypes.byref(a), ctypes.byref(flag)) == OK and flag.value == 0
    assert lib.ttt_fwd_lookback_status(ctypes.byref(a), None) == ERR_NULL
    a = fwd_args(B=1, H=1, L=4096, dk=128, dv=128)   # segmented
    assert lib.ttt_fwd_lookback_status(ctypes.byref(a), ctypes.byref(flag)) == ERR_WS


def test_noalloc_rejects_oversized_scratch(lib):
    """ttt_fwd_chunked_noalloc: a call whose scratch need exceeds the static
    array (the In-Place fast weight, 9728 x 2560, 32 chunks of snapshots) is
    rejected before any device access; its validation errors are those of
    ttt_fwd_chunked."""
    a = fwd_args(B=1, H=1, L=32768, dk=9728, dv=2560, chunk=1024, mode=1)
    a.k = a.q
    a.v = FAKE + (1 << 36)
    a.out = FAKE + (1 << 37)
    need = ctypes.c_size_t(0)
    assert lib.ttt_fwd_workspace_size(ctypes.byref(a), ctypes.byref(need)) == OK
    assert need.value > (64 << 20)
    assert lib.ttt_fwd_chunked_noalloc(ctypes.byref(a)) == ERR_WS
    assert lib.ttt_fwd_chunked_noalloc(ctypes.byref(fwd_args(q=None))) == ERR_NULL
    assert lib.ttt_fwd_chunked_noalloc(ctypes.byref(fwd_args(dk=48))) == ERR_UNSUP
    b = fwd_args()
    b.out = b.v
    assert lib.ttt_fwd_chunked_noalloc(ctypes.byref(b)) == ERR_ALIAS
    assert lib.ttt_fwd_chunked_noalloc(None) == ERR_NULL


def test_workspace_query(lib):
    a = fwd_args()
    ws = ctypes.c_size_t(123)
    assert lib.ttt_fwd_workspace_size(ctypes.byref(a), ctypes.byref(ws)) == OK
    assert lib.ttt_fwd_workspace_size(ctypes.byref(a), None) == ERR_NULL
    assert lib.ttt_fwd_workspace_size(ctypes.byref(fwd_args(dk=48)), ctypes.byref(ws)) == ERR_UNSUP


def test_scan_rejects_before_launch(lib):
    f = lib.ttt_chunk_state_scan
    args = lambda **kw: [kw.get("B", 1), 1, kw.get("L", 64), kw.get("chunk", 16), kw.get("dk", 8), kw.get("dv", 8),
                         kw.get("dS", FAKE), kw.get("dM", FAKE + 65536), kw.get("beta", 0.5), None, None,
                         FAKE + 2 * 65536, None, None, None, None, 0, None]
    assert f(*args(B=0)) == ERR_SHAPE
    assert f(*args(chunk=0)) == ERR_SHAPE
    assert f(*args(dS=None)) == ERR_NULL
    assert f(*args(dM=None)) == ERR_NULL
    assert f(*args(beta=1.5)) == ERR_VALUE
    assert f(*args(dS=FAKE + 4)) == ERR_ALIGN
    assert f(*args(dk=3, dv=3)) == ERR_UNSUP


def test_dual_rejects_before_launch(lib):
    f = lib.ttt_dual_form_fwd
    n = 4 * 64 * 64 * 2

    def args(**kw):
        return [1, 1, 64, kw.get("d", 64), 64, kw.get("mb", 16), kw.get("dtype", 1),
                kw.get("q", FAKE), FAKE + n, FAKE + 2 * n, kw.get("W0", FAKE + 3 * n), 0, 0.01,
                kw.get("out", FAKE + 4 * n), None, None, 0, None]
    assert f(*args(dtype=3)) == ERR_DTYPE
    assert f(*args(mb=0)) == ERR_SHAPE
    assert f(*args(q=None)) == ERR_NULL
    assert f(*args(W0=None)) == ERR_NULL
    assert f(*args(q=FAKE + 8)) == ERR_ALIGN
    assert f(*args(d=32)) == ERR_UNSUP
    assert f(*args(out=FAKE + n)) == ERR_ALIAS


def test_dual_segment_workspace(lib):
    """The segmented dual form's workspace: asked for by few sequences with
    bf16 mini-batches of a multiple of 16, none otherwise; a short or
    overlapping workspace is rejected before any launch."""
    q = ctypes.c_size_t(0)
    ws = lambda B, H, L, mb, dt=1, d=64: (lib.ttt_dual_form_workspace_size(B, H, L, d, 64, mb, dt, ctypes.byref(q)), q.value)
    st, need = ws(4, 16, 8192, 16)
    # 64 sequences fill the 256 slots with 4 segments, plus a fifth on the CUs
    # segment 0 frees: 1664-token segments, flags (320 + 2 words, in 256-byte
    # units) and a 32 KB block (a map: Delta as bf16 hi and lo, B in fp32; or
    # segment 0's end state) per (b, h, segment)
    assert st == OK and need == 1536 + 64 * 5 * 32768
    assert ws(4, 16, 8192, 2048) == (OK, 1280 + 64 * 4 * 32768)   # whole mini-batches: 4 segments
    assert ws(2, 64, 8192, 16) == (OK, 1792 + 128 * 3 * 32768)   # 128 sequences: 3 segments
    assert ws(4, 64, 8192, 16) == (OK, 0)        # 256 sequences fill the chip unsegmented
    assert ws(1, 3, 1000, 48) == (OK, 256 + 3 * 3 * 32768)    # 3 segments of 384 tokens
    assert ws(4, 16, 8192, 40) == (OK, 0)        # mini-batches not of a multiple of 16
    assert ws(4, 16, 8192, 16, dt=0) == (OK, 0)  # fp32
    assert ws(1, 1, 200, 16) == (OK, 0)          # one segment
    assert ws(4, 16, 8192, 16, d=32)[0] == ERR_UNSUP
    assert lib.ttt_dual_form_workspace_size(4, 16, 8192, 64, 64, 16, 1, None) == ERR_NULL
    f = lib.ttt_dual_form_fwd
    B, H, L = 4, 16, 8192
    n = B * H * L * 64 * 2
    big = 1 << 40

    def args(work, wbytes):
        return [B, H, L, 64, 64, 16, 1, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, 0, 0.01,
                FAKE + 4 * n, None, work, wbytes, None]
    assert f(*args(big, need - 1)) == ERR_WS                    # too small
    assert f(*args(big + 8, need)) == ERR_ALIGN
    assert f(*args(FAKE + 2 * n, need)) == ERR_ALIAS            # on v
    assert f(*args(FAKE + 4 * n + n // 2, need)) == ERR_ALIAS   # inside out
    flag = ctypes.c_int32(7)
    stat = lib.ttt_dual_form_lookback_status
    assert stat(B, H, L, 64, 64, 16, 1, None, 0, None, ctypes.byref(flag)) == OK and flag.value == 0
    assert stat(B, H, L, 64, 64, 16, 1, big, need, None, None) == ERR_NULL
    assert stat(B, H, L, 64, 64, 16, 1, big, need - 1, None, ctypes.byref(flag)) == ERR_WS
    assert stat(16, 16, L, 64, 64, 16, 1, big, 0, None, ctypes.byref(flag)) == OK and flag.value == 0


def test_decode_rejects_before_launch(lib):
    f = lib.ttt_decode_step
    n = 1 << 20

    def args(**kw):
        return [kw.get("B", 2), 2, kw.get("dk", 64), kw.get("dv", 64), kw.get("dtype", 1),
                kw.get("q", FAKE), FAKE + n, FAKE + 2 * n, None, 0.1, kw.get("beta", 0.5),
                kw.get("S", FAKE + 3 * n), kw.get("M", FAKE + 4 * n), kw.get("out", FAKE + 5 * n), None]
    assert f(*args(dtype=2)) == ERR_DTYPE
    assert f(*args(B=0)) == ERR_SHAPE
    assert f(*args(beta=1.0)) == ERR_VALUE
    assert f(*args(q=None)) == ERR_NULL
    assert f(*args(M=None)) == ERR_NULL               # momentum needs M
    assert f(*args(S=FAKE + 3 * n + 4)) == ERR_ALIGN
    assert f(*args(dv=30)) == ERR_UNSUP
    assert f(*args(dk=2048)) == ERR_UNSUP
    assert f(*args(out=FAKE + 3 * n + 256)) == ERR_ALIAS  # out inside S
    assert f(*args(M=FAKE + 3 * n + 512)) == ERR_ALIAS    # M overlapping S


def test_bwd_rejects_before_launch(lib):
    f = lib.ttt_bwd_chunked
    n = 2 * 2 * 64 * 64 * 2       # bytes of one [2,2,64,64] bf16 tensor

    def args(**kw):
        base = [FAKE + i * (n + 4096) for i in range(12)]
        return [2, 2, 64, kw.get("dk", 64), 64, kw.get("dtype", 1),
                kw.get("q", base[0]), base[1], base[2], None, 0.1, kw.get("beta", 0.0), None, None, base[3],
                None, None, kw.get("dq", base[4]), base[5], base[6], None, None, None, None, 0, None, None]
    assert f(*args(dtype=4)) == ERR_DTYPE
    assert f(*args(beta=1.0)) == ERR_VALUE
    assert f(*args(dk=48)) == ERR_UNSUP
    assert f(*args(q=None)) == ERR_NULL
    assert f(*args(q=FAKE + 8)) == ERR_ALIGN
    assert f(*args(dq=FAKE + 256)) == ERR_ALIAS          # gradient buffer inside q
    ws = ctypes.c_size_t(7)
    assert lib.ttt_bwd_workspace_size(2, 2, 64, 64, 64, 1, ctypes.c_float(0.0), ctypes.byref(ws)) == OK
    assert lib.ttt_bwd_workspace_size(2, 2, 64, 64, 64, 1, ctypes.c_float(0.9), ctypes.byref(ws)) == OK
    assert ws.value > 0   # momentum keeps its adjoint start states in the workspace
    assert lib.ttt_bwd_workspace_size(2, 2, 64, 64, 64, 1, ctypes.c_float(0.0), None) == ERR_NULL


def test_dbeta_rejects_before_launch(lib):
    f = lib.ttt_bwd_dbeta
    f.argtypes = None
    n = 2 * 2 * 64 * 64 * 2       # bytes of one [2,2,64,64] bf16 tensor

    def args(**kw):
        base = [FAKE + i * (n + 4096) for i in range(12)]
        return [2, 2, 64, kw.get("dk", 64), kw.get("dv", 64), kw.get("dtype", 1),
                ctypes.c_void_p(kw.get("q", base[0])), ctypes.c_void_p(base[1]), ctypes.c_void_p(base[2]), None,
                ctypes.c_float(0.1), ctypes.c_float(kw.get("beta", 0.9)), None, ctypes.c_void_p(base[3]), None, None,
                ctypes.c_void_p(kw.get("dbeta", base[4])), ctypes.c_void_p(kw.get("ws", base[5])),
                ctypes.c_size_t(kw.get("wsb", 256)), None]
    assert f(*args(dtype=4)) == ERR_DTYPE
    assert f(*args(beta=1.0)) == ERR_VALUE
    assert f(*args(beta=-0.5)) == ERR_VALUE
    assert f(*args(dk=48)) == ERR_UNSUP
    assert f(*args(dv=40)) == ERR_UNSUP
    assert f(*args(q=0)) == ERR_NULL
    assert f(*args(dbeta=0)) == ERR_NULL
    assert f(*args(q=FAKE + 8)) == ERR_ALIGN
    assert f(*args(wsb=4)) == ERR_WS
    assert f(*args(dbeta=FAKE + 256)) == ERR_ALIAS        # output inside q
    assert f(*args(ws=FAKE + 4 * (n + 4096))) == ERR_ALIAS   # workspace on top of dbeta
    ws = ctypes.c_size_t(0)
    # one fp32 partial per (head, 16-column tile, 32-row slice), up to 4 slices
    assert lib.ttt_bwd_dbeta_workspace_size(2, 2, 64, ctypes.byref(ws)) == OK and ws.value == 2 * 2 * 4 * 4 * 4
    assert lib.ttt_bwd_dbeta_workspace_size(2, 2, 64, None) == ERR_NULL


def test_frontend_rejects_before_launch(lib):
    n = 1 << 24
    g = lib.ttt_inplace_gated_input
    assert g(0, 256, 256, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, None) == ERR_SHAPE
    assert g(64, 256, 256, None, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, None) == ERR_NULL
    assert g(64, 256, 256, FAKE + 4, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, None) == ERR_ALIGN
    assert g(64, 200, 256, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, None) == ERR_UNSUP   # d_model % 128
    assert g(64, 256, 256, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 256, None) == ERR_ALIAS     # Z inside X
    t = lib.ttt_inplace_lm_target
    assert t(1, 64, 256, 0, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, n, None) == ERR_VALUE
    assert t(1, 64, 256, 17, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, n, None) == ERR_VALUE
    assert t(1, 64, 384, 4, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, n, None) == ERR_UNSUP
    assert t(1, 64, 256, 4, FAKE, FAKE + n, FAKE + 2 * n, FAKE + 3 * n, FAKE + 4 * n, 16, None) == ERR_WS
    c = lib.ttt_inplace_clip_eta
    assert c(1, 64, 256, 256, 64, FAKE, FAKE + n, ctypes.c_float(0.1), ctypes.c_float(0.0), FAKE + 2 * n,
             FAKE + 3 * n, n, None) == ERR_VALUE                                            # tau must be > 0
    assert c(1, 64, 256, 256, 64, FAKE, FAKE + n, ctypes.c_float(0.1), ctypes.c_float(1.0), FAKE + 2 * n,
             None, 0, None) == ERR_WS


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        lac.fwd_chunked(q, q, q)


def test_workspace_plan_segments_short_grids():
    """Few (head, column tile) pairs on a long sequence get look-back
    workspace (segmented); a grid that fills the chip needs none."""
    import torch
    assert lac.fwd_workspace_size(4, 8, 16384, 128, 128, beta=0.9) > 0
    assert lac.fwd_workspace_size(8, 16, 4096, 128, 128) == 0
    assert lac.fwd_workspace_size(1, 2, 500, 128, 128) == 0          # too short to cut
    assert lac.fwd_workspace_size(1, 1, 3000, 64, 32, beta=0.5) > 0  # 32 x 32 tile form
    assert lac.fwd_workspace_size(1, 2, 4096, 128, 128, dtype=torch.float32) == 0


def test_swiglu_rejects_before_launch(lib):
    B, H, L, dk, dv, m, C = 1, 2, 300, 128, 256, 256, 128
    ws = ctypes.c_size_t(0)
    assert lib.ttt_swiglu_workspace_size(B, H, L, dk, dv, m, C, ctypes.byref(ws)) == OK
    # bf16 weight copies + activations of one 128-token chunk, per head
    per = 2 * m * dk + 2 * dv * m + C * (6 * m + dv)
    assert ws.value >= B * H * per * 2
    assert lib.ttt_swiglu_workspace_size(B, H, L, dk, dv, m, C, None) == ERR_NULL
    assert lib.ttt_swiglu_workspace_size(B, H, 0, dk, dv, m, C, ctypes.byref(ws)) == ERR_SHAPE
    assert lib.ttt_swiglu_workspace_size(B, H, L, 96, dv, m, C, ctypes.byref(ws)) == ERR_UNSUP
    assert lib.ttt_swiglu_workspace_size(B, H, L, dk, dv, 200, C, ctypes.byref(ws)) == ERR_UNSUP
    assert lib.ttt_swiglu_workspace_size(B, H, L, dk, dv, m, 100, ctypes.byref(ws)) == ERR_UNSUP
    big = ctypes.c_size_t(0)
    assert lib.ttt_swiglu_workspace_size(B, H, L, dk, dv, m, 1 << 20, ctypes.byref(big)) == OK
    assert lib.ttt_swiglu_workspace_size(B, H, 384, dk, dv, m, 1 << 20, ctypes.byref(ws)) == OK
    assert big.value == ws.value          # a chunk past the sequence end is the whole sequence
    assert lib.ttt_swiglu_workspace_size(1, 1, 1 << 20, 128, 128, 1 << 14, 1 << 20, ctypes.byref(ws)) == ERR_UNSUP
    n = 1 << 26
    need = ws.value

    def call(**kw):
        a = dict(B=B, H=H, L=L, dk=dk, dv=dv, m=m, C=C, loss=0, q=FAKE, k=FAKE + n, v=FAKE + 2 * n, eta=None,
                 W1=FAKE + 3 * n, W3=FAKE + 4 * n, W2=FAKE + 5 * n, out=FAKE + 6 * n, ws=FAKE + 7 * n, wsb=1 << 30)
        a.update(kw)
        return lib.ttt_swiglu_fwd_chunked(a["B"], a["H"], a["L"], a["dk"], a["dv"], a["m"], a["C"], a["loss"], a["q"],
                                          a["k"], a["v"], a["eta"], ctypes.c_float(0.01), a["W1"], a["W3"], a["W2"],
                                          a["out"], a["ws"], a["wsb"], None)

    assert call(loss=2) == ERR_VALUE
    assert call(q=None) == ERR_NULL
    assert call(W2=None) == ERR_NULL
    assert call(out=FAKE + 6 * n + 8) == ERR_ALIGN
    assert call(ws=None) == ERR_WS
    assert call(wsb=16) == ERR_WS
    assert call(dk=192) == ERR_UNSUP
    assert call(out=FAKE + 2 * n + 512) == ERR_ALIAS     # out inside v
    assert call(W3=FAKE + 3 * n + 1024) == ERR_ALIAS     # W3 overlaps W1
    assert call(ws=FAKE + 5 * n) == ERR_ALIAS            # workspace on W2
    assert call(eta=FAKE + 4 * n) == ERR_ALIAS           # eta inside W3 (written)
