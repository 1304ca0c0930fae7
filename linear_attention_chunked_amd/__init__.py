"""Python binding of the MI355X chunked TTT fast-weight forward library.

Thin ctypes layer over ``liblinear_attention_chunked_amd.so`` (C ABI in
``include/ttt.h``).  It only marshals arguments: PyTorch tensors provide
device memory, strides and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback:
if the library is missing or the device is not a GPU the calls raise.

Entry points (same names as the C ABI):
    fwd_chunked(q, k, v, ...)          token-causal / chunk-causal forward
    chunk_state_scan(dS, dM, ...)      exclusive scan of chunk-state deltas
    dual_form_fwd(q, k, v, W0, ...)    TTT-Linear mini-batch dual form
    decode_step(q, k, v, S, M, ...)    one recurrent token, state updated in place
    bwd_chunked(q, k, v, dout, ...)    backward of the token-causal forward
    inplace_gated_input(X, Wg, Wu)     In-Place front end: Z = silu(X Wg^T) (X Wu^T)
    inplace_lm_target(X, conv_w, Wv)   In-Place front end: V-hat = conv(X) Wv^T
    inplace_clip_eta(Z, Vhat, ...)     In-Place front end: clipped per-token rates
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinear_attention_chunked_amd.so")

TTT_F32, TTT_BF16 = 0, 1
TTT_ERR_TIMEOUT = 10
TOKEN_CAUSAL, CHUNK_CAUSAL = 0, 1
_MODES = {"token_causal": TOKEN_CAUSAL, "chunk_causal": CHUNK_CAUSAL}

_vp = ctypes.c_void_p
_i64x3 = ctypes.c_int64 * 3
_i64x2 = ctypes.c_int64 * 2


class TTTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ttt status {status}: {msg}")
        self.status = status


class FwdArgs(ctypes.Structure):
    """Mirror of ``ttt_fwd_args`` (include/ttt.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("q", _vp), ("k", _vp), ("v", _vp),
        ("q_stride", _i64x3), ("k_stride", _i64x3), ("v_stride", _i64x3),
        ("eta", _vp), ("eta_stride", _i64x3), ("eta_scalar", ctypes.c_float),
        ("beta", ctypes.c_float),
        ("S0", _vp), ("S0_stride", _i64x2),
        ("M0", _vp), ("M0_stride", _i64x2),
        ("out", _vp), ("out_stride", _i64x3),
        ("S_final", _vp), ("M_final", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("stream", _vp),
        ("lookback_polls", ctypes.c_int32),
    ]


_lib = None


def load_library():
    """Load the in-tree HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not built: run `python -m linear_attention_chunked_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ttt_fwd_chunked.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.ttt_fwd_chunked.restype = ctypes.c_int
    lib.ttt_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_fwd_chunked_noalloc.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.ttt_fwd_chunked_noalloc.restype = ctypes.c_int
    lib.ttt_fwd_lookback_status.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(ctypes.c_int32)]
    lib.ttt_fwd_lookback_status.restype = ctypes.c_int
    lib.ttt_fwd_workspace_size.restype = ctypes.c_int
    i32, f32 = ctypes.c_int32, ctypes.c_float
    lib.ttt_chunk_state_scan.argtypes = [i32, i32, i32, i32, i32, i32, _vp, _vp, f32, _vp, _vp,
                                         _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.ttt_chunk_state_scan.restype = ctypes.c_int
    lib.ttt_dual_form_fwd.argtypes = [i32, i32, i32, i32, i32, i32, i32, _vp, _vp, _vp, _vp,
                                      ctypes.c_int64, f32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.ttt_dual_form_fwd.restype = ctypes.c_int
    lib.ttt_dual_form_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_dual_form_workspace_size.restype = ctypes.c_int
    lib.ttt_dual_form_lookback_status.argtypes = [i32, i32, i32, i32, i32, i32, i32, _vp, ctypes.c_size_t, _vp,
                                                  ctypes.POINTER(ctypes.c_int32)]
    lib.ttt_dual_form_lookback_status.restype = ctypes.c_int
    lib.ttt_decode_step.argtypes = [i32, i32, i32, i32, i32, _vp, _vp, _vp, _vp, f32, f32, _vp, _vp,
                                    _vp, _vp]
    lib.ttt_decode_step.restype = ctypes.c_int
    lib.ttt_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, f32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_bwd_workspace_size.restype = ctypes.c_int
    lib.ttt_bwd_chunked.argtypes = [i32, i32, i32, i32, i32, i32, _vp, _vp, _vp, _vp, f32, f32, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp]
    lib.ttt_bwd_chunked.restype = ctypes.c_int
    lib.ttt_bwd_dbeta_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_bwd_dbeta_workspace_size.restype = ctypes.c_int
    lib.ttt_bwd_dbeta.argtypes = [i32, i32, i32, i32, i32, i32, _vp, _vp, _vp, _vp, f32, f32, _vp, _vp, _vp, _vp,
                                  _vp, _vp, ctypes.c_size_t, _vp]
    lib.ttt_bwd_dbeta.restype = ctypes.c_int
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.ttt_inplace_gated_input.argtypes = [i32, i32, i32, _vp, _vp, _vp, _vp, _vp]
    lib.ttt_inplace_gated_input.restype = ctypes.c_int
    lib.ttt_inplace_lm_target_workspace_size.argtypes = [i32, i32, i32, sz]
    lib.ttt_inplace_lm_target_workspace_size.restype = ctypes.c_int
    lib.ttt_inplace_lm_target.argtypes = [i32, i32, i32, i32, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.ttt_inplace_lm_target.restype = ctypes.c_int
    lib.ttt_inplace_clip_eta_workspace_size.argtypes = [i32, i32, i32, sz]
    lib.ttt_inplace_clip_eta_workspace_size.restype = ctypes.c_int
    lib.ttt_inplace_clip_eta.argtypes = [i32, i32, i32, i32, i32, _vp, _vp, f32, f32, _vp, _vp, ctypes.c_size_t,
                                         _vp]
    lib.ttt_inplace_clip_eta.restype = ctypes.c_int
    lib.ttt_swiglu_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, sz]
    lib.ttt_swiglu_workspace_size.restype = ctypes.c_int
    lib.ttt_swiglu_fwd_chunked.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, _vp, _vp, _vp, _vp, f32, _vp, _vp,
                                           _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.ttt_swiglu_fwd_chunked.restype = ctypes.c_int
    lib.ttt_status_string.argtypes = [ctypes.c_int]
    lib.ttt_status_string.restype = ctypes.c_char_p
    lib.ttt_fwd_args_size.argtypes = []
    lib.ttt_fwd_args_size.restype = ctypes.c_size_t
    if lib.ttt_fwd_args_size() != ctypes.sizeof(FwdArgs):
        raise RuntimeError("ttt_fwd_args layout mismatch between library and binding")
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise TTTError(status, load_library().ttt_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TTT_F32
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU path exists)")


def _bhl_strides(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B,H,L,d]")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    return _i64x3(t.stride(0), t.stride(1), t.stride(2))


def _state_strides(t: torch.Tensor | None, name: str):
    if t is None:
        return _i64x2(0, 0)
    if t.dim() != 4 or t.dtype != torch.float32:
        raise ValueError(f"{name} must be fp32 [B,H,dk,dv]")
    if t.stride(-1) != 1 or t.stride(-2) != t.shape[-1]:
        raise ValueError(f"{name}: each [dk,dv] block must be contiguous")
    return _i64x2(t.stride(0), t.stride(1))


def fwd_chunked(q, k, v, *, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None, chunk=64,
                mode="token_causal", out=None, return_state=False, stream=None, check_lookback=False,
                lookback_polls=0, no_alloc=False):
    """Chunked fast-weight forward (``ttt_fwd_chunked``).

    q, k: [B,H,L,dk]; v: [B,H,L,dv] (fp32 or bf16, same dtype; q may be k);
    eta: [B,H,L] fp32 per-token step size or None (eta_scalar for all tokens);
    beta: momentum (token-causal only); S0, M0: fp32 [B,H,dk,dv] or None.
    Returns out [B,H,L,dv] (input dtype), plus (S_final, M_final) when
    return_state (M_final is None unless beta != 0).  check_lookback: wait
    for the call and raise TTTError (TTT_ERR_TIMEOUT) if a look-back wait of
    a segmented call gave up (``ttt_fwd_lookback_status``); lookback_polls:
    the bound of those waits (0: the library default).  no_alloc: call
    ``ttt_fwd_chunked_noalloc`` (no workspace is allocated here; the
    library's static scratch is used, and check_lookback is not available;
    out and the final states must still be given or are allocated as usual)."""
    lib = load_library()
    _require_gpu(q, k, v, eta, S0, M0, out)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    a = FwdArgs()
    a.B, a.H, a.L, a.dk, a.dv, a.chunk = B, H, L, dk, dv, int(chunk)
    a.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    a.dtype = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share one dtype")
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.q_stride, a.k_stride = _bhl_strides(q, "q"), _bhl_strides(k, "k")
    a.v_stride, a.out_stride = _bhl_strides(v, "v"), _bhl_strides(out, "out")
    if eta is not None:
        if eta.dtype != torch.float32 or eta.dim() != 3:
            raise ValueError("eta must be fp32 [B,H,L]")
        a.eta = _ptr(eta)
        a.eta_stride = _i64x3(*eta.stride())
    a.eta_scalar = float(eta_scalar)
    a.beta = float(beta)
    a.S0, a.S0_stride = _ptr(S0), _state_strides(S0, "S0")
    a.M0, a.M0_stride = _ptr(M0), _state_strides(M0, "M0")
    S_final = M_final = None
    if return_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
        if beta != 0.0:
            M_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    a.S_final, a.M_final = _ptr(S_final), _ptr(M_final)
    a.stream = _stream(stream)
    a.lookback_polls = int(lookback_polls)
    if no_alloc:
        if check_lookback:
            raise ValueError("check_lookback needs a caller workspace (not available with no_alloc)")
        _check(lib.ttt_fwd_chunked_noalloc(ctypes.byref(a)))
        return (out, S_final, M_final) if return_state else out
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_fwd_workspace_size(ctypes.byref(a), ctypes.byref(ws)))
    work = None
    if ws.value:
        work = torch.empty(ws.value, dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = _ptr(work), ws.value
    _check(lib.ttt_fwd_chunked(ctypes.byref(a)))
    if check_lookback:
        gave_up = ctypes.c_int32(0)
        _check(lib.ttt_fwd_lookback_status(ctypes.byref(a), ctypes.byref(gave_up)))
        if gave_up.value:
            raise TTTError(TTT_ERR_TIMEOUT, lib.ttt_status_string(TTT_ERR_TIMEOUT).decode())
    if return_state:
        return out, S_final, M_final
    return out


def fwd_workspace_size(B, H, L, dk, dv, *, dtype=torch.bfloat16, beta=0.0, chunk=64,
                       mode="token_causal") -> int:
    """Bytes of device workspace ``ttt_fwd_chunked`` needs for these sizes
    (``ttt_fwd_workspace_size``; no tensors, no GPU needed)."""
    lib = load_library()
    a = FwdArgs()
    a.B, a.H, a.L, a.dk, a.dv, a.chunk = int(B), int(H), int(L), int(dk), int(dv), int(chunk)
    a.mode = _MODES[mode] if isinstance(mode, str) else int(mode)
    a.dtype = TTT_F32 if dtype == torch.float32 else TTT_BF16
    a.beta = float(beta)
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_fwd_workspace_size(ctypes.byref(a), ctypes.byref(ws)))
    return int(ws.value)


def chunk_state_scan(dS, dM=None, *, beta=0.0, chunk, L, S0=None, M0=None, stream=None):
    """Exclusive scan of chunk-state deltas (``ttt_chunk_state_scan``).

    dS, dM: fp32 [B,H,N,dk,dv] contiguous.  Returns (S_excl, M_excl, S_final,
    M_final); the M outputs are None when beta == 0."""
    lib = load_library()
    _require_gpu(dS, dM, S0, M0)
    B, H, N, dk, dv = dS.shape
    for t in (dS, dM, S0, M0):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("scan operands must be contiguous fp32")
    S_excl = torch.empty_like(dS)
    S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dS.device)
    M_excl = M_final = None
    if beta != 0.0:
        M_excl = torch.empty_like(dS)
        M_final = torch.empty_like(S_final)
    _check(lib.ttt_chunk_state_scan(B, H, int(L), int(chunk), dk, dv, _ptr(dS), _ptr(dM), float(beta),
                                    _ptr(S0), _ptr(M0), _ptr(S_excl), _ptr(M_excl), _ptr(S_final),
                                    _ptr(M_final), None, 0, _stream(stream)))
    return S_excl, M_excl, S_final, M_final


def dual_form_fwd(q, k, v, W0, *, eta, minibatch, out=None, return_state=False, stream=None,
                  segmented=True, check_lookback=False):
    """TTT-Linear mini-batch forward, dual form (``ttt_dual_form_fwd``).

    q, k: [B,H,L,d]; v: [B,H,L,dv] contiguous, fp32 or bf16; W0 fp32
    [B,H,d,dv] (or [d,dv] broadcast).  Returns out (and W_final).
    segmented: give the library the workspace it asks for
    (``ttt_dual_form_workspace_size``), so that shapes with few sequences run
    in concurrent segments; False runs every sequence as one chain.
    check_lookback: wait for the call and raise TTTError (TTT_ERR_TIMEOUT) if
    a wait between segments gave up (``ttt_dual_form_lookback_status``)."""
    lib = load_library()
    _require_gpu(q, k, v, W0, out)
    B, H, L, d = q.shape
    dv = v.shape[-1]
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if W0.dtype != torch.float32 or not W0.is_contiguous():
        raise ValueError("W0 must be contiguous fp32")
    w_stride = 0 if W0.dim() == 2 else d * dv
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=q.device)
    W_final = torch.empty((B, H, d, dv), dtype=torch.float32, device=q.device) if return_state else None
    dt = _dtype_code(q)
    ws = ctypes.c_size_t(0)
    if segmented:
        _check(lib.ttt_dual_form_workspace_size(B, H, L, d, dv, int(minibatch), dt, ctypes.byref(ws)))
    work = torch.empty(ws.value, dtype=torch.uint8, device=q.device) if ws.value else None
    _check(lib.ttt_dual_form_fwd(B, H, L, d, dv, int(minibatch), dt, _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(W0), w_stride, float(eta), _ptr(out), _ptr(W_final),
                                 _ptr(work), ws.value, _stream(stream)))
    if check_lookback:
        gave_up = ctypes.c_int32(0)
        _check(lib.ttt_dual_form_lookback_status(B, H, L, d, dv, int(minibatch), dt, _ptr(work), ws.value,
                                                 _stream(stream), ctypes.byref(gave_up)))
        if gave_up.value:
            raise TTTError(TTT_ERR_TIMEOUT, lib.ttt_status_string(TTT_ERR_TIMEOUT).decode())
    if return_state:
        return out, W_final
    return out


def dual_form_workspace_size(B, H, L, d, dv, *, minibatch, dtype=torch.bfloat16) -> int:
    """Bytes of workspace the segmented dual form uses at these sizes
    (``ttt_dual_form_workspace_size``; 0: the shape runs as one chain)."""
    lib = load_library()
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_dual_form_workspace_size(int(B), int(H), int(L), int(d), int(dv), int(minibatch),
                                            TTT_F32 if dtype == torch.float32 else TTT_BF16, ctypes.byref(ws)))
    return int(ws.value)


def decode_step(q, k, v, S, M=None, *, eta=None, eta_scalar=0.0, beta=0.0, out=None, stream=None):
    """One recurrent token per (b, h) (``ttt_decode_step``).

    q, k: [B,H,dk]; v: [B,H,dv] contiguous, fp32 or bf16; eta fp32 [B,H] or
    None (then eta_scalar).  S (and M when beta != 0): fp32 [B,H,dk,dv]
    contiguous, updated in place.  Returns out [B,H,dv] in q's dtype."""
    lib = load_library()
    _require_gpu(q, k, v, S, M, eta, out)
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, H, dv):
        raise ValueError("k must match q and v must be [B,H,dv]")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{nm} must be contiguous and of q's dtype")
    for t, nm in ((S, "S"), (M, "M")):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()
                              or t.shape != (B, H, dk, dv)):
            raise ValueError(f"{nm} must be contiguous fp32 [B,H,dk,dv]")
    if eta is not None and (eta.dtype != torch.float32 or not eta.is_contiguous()
                            or eta.numel() != B * H):
        raise ValueError("eta must be contiguous fp32 [B,H]")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _check(lib.ttt_decode_step(B, H, dk, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                               float(eta_scalar), float(beta), _ptr(S), _ptr(M), _ptr(out),
                               _stream(stream)))
    return out


def bwd_workspace_size(B, H, L, dk, dv, *, dtype=torch.bfloat16, beta=0.0):
    """Workspace bytes ``bwd_chunked`` needs for this shape (0 possible)."""
    lib = load_library()
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_bwd_workspace_size(B, H, L, dk, dv, TTT_BF16 if dtype == torch.bfloat16 else TTT_F32,
                                      float(beta), ctypes.byref(ws)))
    return int(ws.value)


def bwd_chunked(q, k, v, dout, *, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None, dS_final=None,
                dM_final=None, need_deta=True, need_dS0=True, need_dM0=False, stream=None, side_stream=None):
    """Backward of the token-causal forward (``ttt_bwd_chunked``).

    q, k: [B,H,L,dk]; v, dout: [B,H,L,dv], contiguous, fp32 or bf16; eta fp32
    [B,H,L] or None (eta_scalar); S0, M0, dS_final, dM_final fp32
    [B,H,dk,dv] or None.  Returns (dq, dk, dv, deta, dS0, dM0); deta is per
    token; the optional outputs are None unless requested.  side_stream: an
    optional second torch.cuda.Stream on the same device that runs the dv/deta
    step beside the last pass (forked from and joined back to `stream`)."""
    lib = load_library()
    _require_gpu(q, k, v, dout, eta, S0, M0, dS_final, dM_final)
    if q.dim() != 4:
        raise ValueError("q must be [B,H,L,dk]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, H, L, dv) or dout.shape != v.shape:
        raise ValueError("k must match q; v and dout must be [B,H,L,dv]")
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        if not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{nm} must be contiguous and of q's dtype")
    st = (B, H, dk, dv)
    for t, nm, shp in ((eta, "eta", (B, H, L)), (S0, "S0", st), (M0, "M0", st), (dS_final, "dS_final", st),
                       (dM_final, "dM_final", st)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != shp):
            raise ValueError(f"{nm} must be contiguous fp32 {list(shp)}")
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if need_deta else None
    dS0 = torch.empty(st, dtype=torch.float32, device=q.device) if need_dS0 else None
    dM0 = torch.empty(st, dtype=torch.float32, device=q.device) if need_dM0 else None
    wsb = bwd_workspace_size(B, H, L, dk, dv, dtype=q.dtype, beta=beta)
    ws = torch.empty(wsb, dtype=torch.uint8, device=q.device) if wsb else None
    _check(lib.ttt_bwd_chunked(B, H, L, dk, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                               float(eta_scalar), float(beta), _ptr(S0), _ptr(M0), _ptr(dout), _ptr(dS_final),
                               _ptr(dM_final), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(deta), _ptr(dS0), _ptr(dM0),
                               _ptr(ws), wsb, _stream(stream),
                               None if side_stream is None else ctypes.c_void_p(side_stream.cuda_stream)))
    return dq, dk_, dv_, deta, dS0, dM0


def bwd_dbeta(q, k, v, dout, *, eta=None, eta_scalar=0.0, beta=0.0, M0=None, dS_final=None, dM_final=None,
              stream=None):
    """dL/dbeta of the token-causal momentum forward (``ttt_bwd_dbeta``):
    the same inputs and layouts as ``bwd_chunked``; returns fp32 [B,H]."""
    lib = load_library()
    _require_gpu(q, k, v, dout, eta, M0, dS_final, dM_final)
    if q.dim() != 4:
        raise ValueError("q must be [B,H,L,dk]")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, H, L, dv) or dout.shape != v.shape:
        raise ValueError("k must match q; v and dout must be [B,H,L,dv]")
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        if not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{nm} must be contiguous and of q's dtype")
    st = (B, H, dk, dv)
    for t, nm, shp in ((eta, "eta", (B, H, L)), (M0, "M0", st), (dS_final, "dS_final", st),
                       (dM_final, "dM_final", st)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != shp):
            raise ValueError(f"{nm} must be contiguous fp32 {list(shp)}")
    n = ctypes.c_size_t(0)
    _check(lib.ttt_bwd_dbeta_workspace_size(B, H, dv, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check(lib.ttt_bwd_dbeta(B, H, L, dk, dv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                             float(eta_scalar), float(beta), _ptr(M0), _ptr(dout), _ptr(dS_final), _ptr(dM_final),
                             _ptr(out), _ptr(ws), n.value, _stream(stream)))
    return out


def _bf16_contig(*pairs):
    for t, nm in pairs:
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous bf16")


def inplace_gated_input(X, Wg, Wu, *, out=None, stream=None):
    """Z = silu(X Wg^T) * (X Wu^T) (``ttt_inplace_gated_input``).

    X: [..., d_model] bf16; Wg, Wu: [d_ff, d_model] bf16.  Returns Z [..., d_ff]."""
    lib = load_library()
    _require_gpu(X, Wg, Wu, out)
    _bf16_contig((X, "X"), (Wg, "Wg"), (Wu, "Wu"))
    d_ff, d_model = Wg.shape
    if Wu.shape != Wg.shape or X.shape[-1] != d_model:
        raise ValueError("Wg, Wu must be [d_ff, d_model] and X [..., d_model]")
    T = X.numel() // d_model
    if out is None:
        out = torch.empty(X.shape[:-1] + (d_ff,), dtype=torch.bfloat16, device=X.device)
    _check(lib.ttt_inplace_gated_input(T, d_model, d_ff, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(out), _stream(stream)))
    return out


def inplace_lm_target(X, conv_w, Wv, *, out=None, stream=None):
    """V-hat = lookahead_conv(X, conv_w) Wv^T (``ttt_inplace_lm_target``).

    X: [B, L, d_model] bf16; conv_w: [taps, d_model] fp32; Wv: [d_model, d_model] bf16."""
    lib = load_library()
    _require_gpu(X, conv_w, Wv, out)
    _bf16_contig((X, "X"), (Wv, "Wv"))
    if conv_w.dtype != torch.float32 or not conv_w.is_contiguous():
        raise ValueError("conv_w must be contiguous fp32")
    B, L, d = X.shape
    if out is None:
        out = torch.empty_like(X)
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_inplace_lm_target_workspace_size(B, L, d, ctypes.byref(ws)))
    w = torch.empty(ws.value, dtype=torch.uint8, device=X.device)
    _check(lib.ttt_inplace_lm_target(B, L, d, conv_w.shape[0], _ptr(X), _ptr(conv_w), _ptr(Wv), _ptr(out), _ptr(w),
                                     ws.value, _stream(stream)))
    return out


def inplace_clip_eta(Z, Vhat, *, chunk, eta, tau, out=None, stream=None):
    """Per-token rates eta * min(1, tau / ||eta Z_i^T V_i||_F) per chunk
    (``ttt_inplace_clip_eta``).  Z: [B, L, d_ff], Vhat: [B, L, d_model] bf16.
    Returns fp32 [B, L]."""
    lib = load_library()
    _require_gpu(Z, Vhat, out)
    _bf16_contig((Z, "Z"), (Vhat, "Vhat"))
    B, L, d_ff = Z.shape
    d_model = Vhat.shape[-1]
    if out is None:
        out = torch.empty((B, L), dtype=torch.float32, device=Z.device)
    ws = ctypes.c_size_t(0)
    _check(lib.ttt_inplace_clip_eta_workspace_size(B, L, int(chunk), ctypes.byref(ws)))
    w = torch.empty(max(ws.value, 16), dtype=torch.uint8, device=Z.device)
    _check(lib.ttt_inplace_clip_eta(B, L, d_ff, d_model, int(chunk), _ptr(Z), _ptr(Vhat), float(eta), float(tau),
                                    _ptr(out), _ptr(w), ws.value, _stream(stream)))
    return out


_LOSS = {"dot": 0, "mse": 1}


def swiglu_workspace_size(B, H, L, dk, dv, m, chunk):
    """Bytes of workspace ``swiglu_fwd_chunked`` needs (``ttt_swiglu_workspace_size``)."""
    ws = ctypes.c_size_t(0)
    _check(load_library().ttt_swiglu_workspace_size(B, H, L, dk, dv, m, int(chunk), ctypes.byref(ws)))
    return ws.value


def swiglu_fwd_chunked(q, k, v, W1, W3, W2, *, eta=None, eta_scalar=0.0, chunk=2048, loss="dot", out=None,
                       workspace=None, stream=None):
    """Large-chunk SwiGLU fast weight (``ttt_swiglu_fwd_chunked``): per chunk,
    out = W2 (silu(W1 q) * (W3 q)) with the current weights, then one gradient
    step of the weights on sum_t eta_t l_t over the chunk's (k, v) pairs
    (loss "dot": l = -<f(k), v>; "mse": l = 1/2 ||f(k) - v||^2).

    q, k: [B,H,L,dk], v: [B,H,L,dv] contiguous bf16; W1, W3: [B,H,m,dk] and
    W2: [B,H,dv,m] contiguous fp32, UPDATED IN PLACE to the final weights;
    eta: [B,H,L] fp32 or None (eta_scalar).  Returns out [B,H,L,dv] bf16."""
    lib = load_library()
    _require_gpu(q, k, v, W1, W3, W2, eta, out, workspace)
    _bf16_contig((q, "q"), (k, "k"), (v, "v"))
    if loss not in _LOSS:
        raise ValueError("loss must be 'dot' or 'mse'")
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    m = W1.shape[-2]
    if k.shape != q.shape or v.shape[:3] != (B, H, L):
        raise ValueError("q, k must be [B,H,L,dk] and v [B,H,L,dv]")
    for W, shp, nm in ((W1, (B, H, m, dk), "W1"), (W3, (B, H, m, dk), "W3"), (W2, (B, H, dv, m), "W2")):
        if tuple(W.shape) != shp or W.dtype != torch.float32 or not W.is_contiguous():
            raise ValueError(f"{nm} must be contiguous fp32 {list(shp)}")
    if eta is not None and (tuple(eta.shape) != (B, H, L) or eta.dtype != torch.float32 or not eta.is_contiguous()):
        raise ValueError("eta must be contiguous fp32 [B,H,L]")
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=q.device)
    need = swiglu_workspace_size(B, H, L, dk, dv, m, chunk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.ttt_swiglu_fwd_chunked(B, H, L, dk, dv, m, int(chunk), _LOSS[loss], _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(eta), float(eta_scalar), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return out


__all__ = ["swiglu_fwd_chunked", "swiglu_workspace_size", "inplace_gated_input", "inplace_lm_target", "inplace_clip_eta", "fwd_chunked", "chunk_state_scan", "dual_form_fwd", "decode_step", "bwd_chunked", "bwd_workspace_size", "load_library", "TTTError",
           "FwdArgs", "LIB_PATH"]
