"""fp64 CPU oracle for the chunked TTT fast-weight forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with ``linear_attention_chunked_amd`` (the HIP path) and imports nothing from
it; both sides only consume the same seeded inputs from ``workloads``.

Two kinds of routine live here:

* plain definitions (per-token recurrences in C, ``ttt_oracle.c``; the
  per-chunk In-Place update, which is defined per chunk, as NumPy GEMMs);
* second, independent forms used to pin the first ones: the O(L^2) masked
  linear-attention sums, the chunked algorithm in fp64 (aggregates + scan +
  readout + intra-chunk term, in the order the pages give it), the dual-form
  matrix expression, and per-row closed forms for outputs too large to
  compute whole.

Sources (cited by page title and paragraph / section):
  [P1] "KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다" (aitrends.kr/articles/4698)
  [P2] "In-Place 테스트 시점 학습: LLM을 위한 원활한 동적 적응 프레임워크" (aitrends.kr/articles/40879)
  [P4] "RNN의 기억을 작은 모델로 바꾼다면: Test-Time Training 읽기" (ariser.io)
  [P5] "LaCT (Large Chunk Test-Time Training)" wiki (aisparkup.com/wiki/lact)

Parity is pinned for every routine here (see tests/test_oracle_pins.py); no
routine is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libttt_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile ttt_oracle.c with gcc (fp64, OpenMP over independent heads)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i, d = ctypes.c_int, ctypes.c_double
        lib.ttt_oracle_token_causal.argtypes = [i, i, i, i, i, _dp, _dp, _dp, _dp, d, d,
                                                _dp, _dp, _dp, _dp, _dp]
        lib.ttt_oracle_token_causal.restype = None
        lib.ttt_oracle_dual_primal.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp, _dp, d, _dp, _dp]
        lib.ttt_oracle_dual_primal.restype = None
        lib.ttt_oracle_state_scan.argtypes = [i, i, i, i, i, i, _dp, _dp, d, _dp, _dp,
                                              _dp, _dp, _dp, _dp]
        lib.ttt_oracle_state_scan.restype = None
        lib.ttt_oracle_token_causal_bwd.argtypes = [i, i, i, i, i, _dp, _dp, _dp, _dp, d, d, _dp, _dp,
                                                    _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.ttt_oracle_token_causal_bwd.restype = None
        lib.ttt_oracle_token_causal_dbeta.argtypes = [i, i, i, i, i, _dp, _dp, _dp, _dp, d, d, _dp, _dp,
                                                      _dp, _dp, _dp]
        lib.ttt_oracle_token_causal_dbeta.restype = None
        lib.ttt_oracle_threads.argtypes = []
        lib.ttt_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Host threads the C oracle's OpenMP loops use."""
    return int(_load().ttt_oracle_threads())


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_dp) if a is not None else None


# ============================================================== plain definitions
def token_causal(q, k, v, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None):
    """Per-token fast-weight recurrence (C, fp64).  [P1] state-matrix update and
    momentum paragraphs; [P4] "읽는 동안 문제를 하나 더 푼다" update rule.

        g_t = eta_t k_t^T v_t;  m_t = beta m_{t-1} + g_t;  S_t = S_{t-1} + m_t;  o_t = q_t S_t

    q,k: [B,H,L,dk]; v: [B,H,L,dv]; eta: [B,H,L] or None (eta_scalar);
    S0, M0: [B,H,dk,dv] or None (zero).  Returns (out, S_final, M_final)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    eta, S0, M0 = _f64(eta), _f64(S0), _f64(M0)
    out = np.empty((B, H, L, dv))
    Sf = np.empty((B, H, dk, dv))
    Mf = np.empty((B, H, dk, dv))
    _load().ttt_oracle_token_causal(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                    float(eta_scalar), float(beta), _ptr(S0), _ptr(M0),
                                    _ptr(out), _ptr(Sf), _ptr(Mf))
    return out, Sf, Mf


def token_causal_bwd(q, k, v, dout, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None,
                     dS_final=None, dM_final=None):
    """Backward pass of ``token_causal`` (C, fp64): the plain adjoint of the
    per-token recurrence (the pages give the forward rule and train through
    it, [P4] section "가중치가 두 종류라는 점"; the derivative is the chain rule).

    Returns (dq, dk, dv, deta, dS0, dM0); deta is per token [B,H,L] even for a
    scalar eta (whose gradient is its sum over tokens)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    eta, S0, M0, dSf, dMf = _f64(eta), _f64(S0), _f64(M0), _f64(dS_final), _f64(dM_final)
    dq = np.empty((B, H, L, dk))
    dkk = np.empty((B, H, L, dk))
    dvv = np.empty((B, H, L, dv))
    deta = np.empty((B, H, L))
    dS0 = np.empty((B, H, dk, dv))
    dM0 = np.empty((B, H, dk, dv))
    _load().ttt_oracle_token_causal_bwd(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                        float(eta_scalar), float(beta), _ptr(S0), _ptr(M0), _ptr(dout),
                                        _ptr(dSf), _ptr(dMf), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(deta),
                                        _ptr(dS0), _ptr(dM0))
    return dq, dkk, dvv, deta, dS0, dM0


def token_causal_dbeta(q, k, v, dout, eta=None, eta_scalar=0.0, beta=0.0, M0=None, dS_final=None,
                       dM_final=None):
    """dL/dbeta of ``token_causal`` (C, fp64) for L = <dout, out> +
    <dS_final, S_final> + <dM_final, M_final>: the forward-mode derivative of
    the momentum recurrence ([P1] paragraph on momentum; [P4] section
    "가중치가 두 종류라는 점" trains through the updates).  Returns [B,H]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    eta, M0, dSf, dMf = _f64(eta), _f64(M0), _f64(dS_final), _f64(dM_final)
    out = np.empty((B, H))
    _load().ttt_oracle_token_causal_dbeta(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(eta),
                                          float(eta_scalar), float(beta), _ptr(M0), _ptr(dout), _ptr(dSf),
                                          _ptr(dMf), _ptr(out))
    return out


def dual_primal(q, k, v, W0, eta, minibatch):
    """TTT-Linear mini-batch update in primal form (C, fp64).  [P4] section
    "gradient를 효율적인 layer로 만드는 작업".  Returns (out, W_final)."""
    q, k, v, W0 = _f64(q), _f64(k), _f64(v), _f64(W0)
    B, H, L, d = q.shape
    dv = v.shape[-1]
    out = np.empty((B, H, L, dv))
    Wf = np.empty((B, H, d, dv))
    _load().ttt_oracle_dual_primal(B, H, L, d, dv, int(minibatch), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(W0), float(eta), _ptr(out), _ptr(Wf))
    return out, Wf


def state_scan(dS, dM, beta, chunk, L, S0=None, M0=None):
    """Sequential scan of chunk-state aggregates (C, fp64).  [P1] paragraph on
    removing weight normalisation; [P2] paragraph on the associative scan.
    dS, dM: [B,H,N,dk,dv] (dM may be None).  Returns (S_excl, M_excl, S_final, M_final)."""
    dS, dM, S0, M0 = _f64(dS), _f64(dM), _f64(S0), _f64(M0)
    B, H, N, dk, dv = dS.shape
    assert N == (L + chunk - 1) // chunk
    Se = np.empty_like(dS)
    Me = np.empty_like(dS)
    Sf = np.empty((B, H, dk, dv))
    Mf = np.empty((B, H, dk, dv))
    _load().ttt_oracle_state_scan(B, H, int(L), int(chunk), dk, dv, _ptr(dS), _ptr(dM),
                                  float(beta), _ptr(S0), _ptr(M0), _ptr(Se), _ptr(Me),
                                  _ptr(Sf), _ptr(Mf))
    return Se, Me, Sf, Mf


def chunk_causal(q, k, v, eta=None, eta_scalar=0.0, S0=None, chunk=1024):
    """In-Place TTT chunk-causal update, defined per chunk ([P2] paragraphs on
    the Gated-MLP fast weight Wdown and on the chunk-wise update: one gradient
    step per chunk, the updated weight serves the next chunk; delta update on
    top of the existing weight).  For chunk i (NumPy fp64 GEMMs):

        O_i = Q_i W_{i-1};   W_i = W_{i-1} + K_i^T diag(eta_i) V_i,   W_{-1} = S0

    In the In-Place setting Q = K = Z (activations) and V = V-hat (targets).
    q,k: [B,H,L,dk]; v: [B,H,L,dv].  Returns (out, W_final)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    eta = _f64(eta)
    S0 = _f64(S0)
    out = np.empty((B, H, L, dv))
    Wf = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            W = S0[b, h].copy() if S0 is not None else np.zeros((dk, dv))
            for c0 in range(0, L, chunk):
                c1 = min(c0 + chunk, L)
                out[b, h, c0:c1] = q[b, h, c0:c1] @ W
                e = eta[b, h, c0:c1] if eta is not None else np.full(c1 - c0, eta_scalar)
                W = W + k[b, h, c0:c1].T @ (e[:, None] * v[b, h, c0:c1])
            Wf[b, h] = W
    return out, Wf


# ------------------------------------------------------------ In-Place front end
def inplace_gated_input(X, Wg, Wu):
    """Input activation of the fast weight Wdown in the gated MLP ([P2]
    paragraph on the Gated-MLP structure: Wup and Wgate stay fixed slow
    weights, their output Z is what Wdown multiplies).  NumPy fp64:

        Z = silu(X Wg^T) * (X Wu^T),   silu(a) = a / (1 + exp(-a))

    X: [..., d_model]; Wg, Wu: [d_ff, d_model] (rows = output features)."""
    X, Wg, Wu = _f64(X), _f64(Wg), _f64(Wu)
    a = X @ Wg.T
    b = X @ Wu.T
    return a / (1.0 + np.exp(-a)) * b


def lookahead_conv(X, c):
    """The 1D convolution of the LM-aligned target ([P2] paragraph on the
    LM-aligned objective: the target is built from the current and following
    tokens so the update stores next-token information).  Depthwise, K taps
    on tokens t .. t+K-1 of the same sequence, zero past its end:

        Y[b, t] = sum_{j < K, t + j < L} c[j] * X[b, t + j]

    X: [B, L, d]; c: [K, d]."""
    X, c = _f64(X), _f64(c)
    B, L, d = X.shape
    K = c.shape[0]
    Y = np.zeros_like(X)
    for j in range(K):
        Y[:, :L - j] += c[j] * X[:, j:]
    return Y


def lm_aligned_target(X, c, Wv):
    """V-hat = lookahead_conv(X, c) Wv^T ([P2]: 1D convolution, then a
    projection).  Wv: [d_model, d_model] (rows = output features)."""
    return lookahead_conv(X, c) @ _f64(Wv).T


def clip_scales(Z, V, chunk, eta, tau):
    """Per-token learning rates with the update clipped ([P2] paragraph on
    the limitations: a clipping mechanism keeps accumulated updates stable
    over very long contexts).  For chunk i the update is
    dW_i = eta Z_i^T V_i (formed explicitly here); it is scaled to Frobenius
    norm at most tau:

        s_i = min(1, tau / ||dW_i||_F)   (1 when dW_i = 0),  eta_t = eta s_i

    Z: [B, L, d_ff]; V: [B, L, d_model].  Returns eta_t [B, L]."""
    Z, V = _f64(Z), _f64(V)
    B, L, _ = Z.shape
    out = np.empty((B, L))
    for b in range(B):
        for c0 in range(0, L, chunk):
            c1 = min(c0 + chunk, L)
            nrm = float(np.linalg.norm(eta * (Z[b, c0:c1].T @ V[b, c0:c1])))
            s = 1.0 if nrm == 0.0 or nrm <= tau else tau / nrm
            out[b, c0:c1] = eta * s
    return out


# ------------------------------------------------------ nonlinear fast weights
def swiglu_apply(X, W1, W3, W2):
    """The SwiGLU fast-weight MLP applied to token rows ([P5] section on the
    core idea, row "nonlinear fast weights"; [P4] section on the
    hidden state and update rule: the state is the weights of a small model):

        f_W(x) = W2 (silu(W1 x) * (W3 x))

    X: [n, d]; W1, W3: [m, d]; W2: [d, m] (rows = output features)."""
    H1 = X @ W1.T
    H3 = X @ W3.T
    return (H1 / (1.0 + np.exp(-H1)) * H3) @ W2.T


def swiglu_fast_weight(q, k, v, W1, W3, W2, eta=None, eta_scalar=0.0, chunk=2048, loss="dot"):
    """Large-chunk SwiGLU fast weight, chunk-causal ([P5] sections on the
    core idea: the fast weights take one update per large chunk, the chunk's
    tokens acting as one big batch; [P4] section on the update rule:
    W_t = W_{t-1} - eta grad_W l, output from the model; [P2] paragraph on the
    chunk-wise update: chunk i reads the weights left by chunks < i).
    For chunk i, with the weights W = (W1, W3, W2) after chunks < i:

        O_i = f_W(Q_i)
        W  <- W - grad_W  sum_{t in i} eta_t l_t(W)

    l_t is the inner loss of token t on its key / value pair:
        loss="dot": l_t = -<f_W(k_t), v_t>       (key-value binding; for a
                     linear f it is the linear-attention update W += eta k^T v)
        loss="mse": l_t = 1/2 ||f_W(k_t) - v_t||^2  (reconstruction)
    The gradient is taken by the chain rule through the MLP, written out:
        H1 = K W1^T, H3 = K W3^T, S = silu(H1), A = S * H3, Y = A W2^T
        dY = diag(eta) dl/dY        (-V, or Y - V)
        dW2 = dY^T A,  dA = dY W2
        dH3 = dA * S,  dH1 = dA * H3 * silu'(H1),
            silu'(h) = sigma(h) (1 + h (1 - sigma(h)))
        dW1 = dH1^T K, dW3 = dH3^T K
    q, k, v: [B, H, L, d]; W1, W3: [B, H, m, d]; W2: [B, H, d, m]; eta:
    [B, H, L] or None (then eta_scalar).  NumPy fp64.
    Returns (out [B, H, L, d], W1_final, W3_final, W2_final)."""
    if loss not in ("dot", "mse"):
        raise ValueError("loss must be 'dot' or 'mse'")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    eta = _f64(eta)
    W1f, W3f, W2f = _f64(W1).copy(), _f64(W3).copy(), _f64(W2).copy()
    out = np.empty((B, H, L, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            W1c, W3c, W2c = W1f[b, h], W3f[b, h], W2f[b, h]
            for c0 in range(0, L, chunk):
                c1 = min(c0 + chunk, L)
                out[b, h, c0:c1] = swiglu_apply(q[b, h, c0:c1], W1c, W3c, W2c)
                K, V = k[b, h, c0:c1], v[b, h, c0:c1]
                e = eta[b, h, c0:c1] if eta is not None else np.full(c1 - c0, eta_scalar)
                H1 = K @ W1c.T
                H3 = K @ W3c.T
                sg = 1.0 / (1.0 + np.exp(-H1))
                S = H1 * sg
                A = S * H3
                Y = A @ W2c.T
                G = -V if loss == "dot" else Y - V
                dY = e[:, None] * G
                dW2 = dY.T @ A
                dA = dY @ W2c
                dH3 = dA * S
                dH1 = dA * H3 * sg * (1.0 + H1 * (1.0 - sg))
                W1c -= dH1.T @ K
                W3c -= dH3.T @ K
                W2c -= dW2
    return out, W1f, W3f, W2f


# ============================================================ independent forms
def momentum_weights(beta, n):
    """w_n = sum_{i=0..n} beta^i: weight of pair (s, t = s + n) under momentum
    ([P1] momentum paragraph: momentum SGD is a weighted linear attention)."""
    n = np.asarray(n)
    if beta == 0.0:
        return np.ones(n.shape)
    return (1.0 - beta ** (n + 1)) / (1.0 - beta)


def momentum_carry(beta, n):
    """a_n = sum_{i=1..n+1} beta^i: weight of the incoming momentum M0 in S at
    local token n."""
    n = np.asarray(n)
    if beta == 0.0:
        return np.zeros(n.shape)
    return beta * (1.0 - beta ** (n + 1)) / (1.0 - beta)


def bruteforce_token_causal(q, k, v, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None):
    """O(L^2) masked linear attention (NumPy fp64):
        o_t = q_t S0 + a_t q_t M0 + sum_{s<=t} eta_s w_{t-s} (q_t . k_s) v_s
    the parallel form [P1] says the sequential update equals."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    eta = _f64(eta) if eta is not None else np.full((B, H, L), float(eta_scalar))
    t = np.arange(L)
    diff = t[:, None] - t[None, :]
    mask = np.where(diff >= 0, momentum_weights(beta, np.maximum(diff, 0)), 0.0)
    out = np.einsum("bhtd,bhsd->bhts", q, k) * mask[None, None] * eta[:, :, None, :]
    out = out @ v
    if S0 is not None:
        out = out + q @ _f64(S0)
    if M0 is not None:
        out = out + momentum_carry(beta, t)[None, None, :, None] * (q @ _f64(M0))
    return out


def chunk_aggregates(k, v, eta=None, eta_scalar=0.0, beta=0.0, chunk=64):
    """Per-chunk change of (S, m) from a zero start ([P1] associativity
    paragraph, chunk aggregates combined by a scan):
        dS_c = sum_j eta_j w_{n-1-j} k_j^T v_j,  dM_c = sum_j eta_j beta^{n-1-j} k_j^T v_j
    for a chunk of n tokens.  Returns dS, dM [B,H,N,dk,dv]."""
    k, v = _f64(k), _f64(v)
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    eta = _f64(eta) if eta is not None else np.full((B, H, L), float(eta_scalar))
    N = (L + chunk - 1) // chunk
    dS = np.zeros((B, H, N, dk, dv))
    dM = np.zeros((B, H, N, dk, dv))
    for c in range(N):
        c0, c1 = c * chunk, min((c + 1) * chunk, L)
        n = c1 - c0
        j = np.arange(n)
        ws = momentum_weights(beta, n - 1 - j)
        wm = (beta ** (n - 1 - j)) if beta != 0.0 else (j == n - 1).astype(np.float64)
        kc, vc, ec = k[:, :, c0:c1], v[:, :, c0:c1], eta[:, :, c0:c1]
        dS[:, :, c] = np.swapaxes(kc, -1, -2) @ ((ec * ws)[..., None] * vc)
        dM[:, :, c] = np.swapaxes(kc, -1, -2) @ ((ec * wm)[..., None] * vc)
    return dS, dM


def chunked_token_causal(q, k, v, eta=None, eta_scalar=0.0, beta=0.0, S0=None, M0=None, chunk=64):
    """The chunked algorithm in fp64, step by step (NumPy): per chunk, the
    readout of the state at the chunk start, the masked intra-chunk term, then
    the chunk transition by its aggregate.  Token-causal output must not depend
    on `chunk`.  Returns (out, S_final, M_final)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    eta = _f64(eta) if eta is not None else np.full((B, H, L), float(eta_scalar))
    S = _f64(S0).copy() if S0 is not None else np.zeros((B, H, dk, dv))
    M = _f64(M0).copy() if M0 is not None else np.zeros((B, H, dk, dv))
    dS, dM = chunk_aggregates(k, v, eta, 0.0, beta, chunk)
    out = np.empty((B, H, L, dv))
    for c in range((L + chunk - 1) // chunk):
        c0, c1 = c * chunk, min((c + 1) * chunk, L)
        n = c1 - c0
        i = np.arange(n)
        diff = i[:, None] - i[None, :]
        mask = np.where(diff >= 0, momentum_weights(beta, np.maximum(diff, 0)), 0.0)
        qc, kc, vc, ec = q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1], eta[:, :, c0:c1]
        A = (qc @ np.swapaxes(kc, -1, -2)) * mask * ec[:, :, None, :]
        out[:, :, c0:c1] = qc @ S + momentum_carry(beta, i)[:, None] * (qc @ M) + A @ vc
        alpha = float(momentum_carry(beta, n - 1)) if beta != 0.0 else 0.0
        gamma = beta ** n if beta != 0.0 else 0.0
        S = S + alpha * M + dS[:, :, c]
        M = gamma * M + dM[:, :, c]
    return out, S, M


def bruteforce_chunk_causal(q, k, v, eta=None, eta_scalar=0.0, S0=None, chunk=1024):
    """O(L^2) form of the chunk-causal update (NumPy fp64):
        O = Q S0 + (M_blk * (Q K^T)) diag(eta) V,  M_blk[t,s] = 1 iff chunk(s) < chunk(t)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk = q.shape
    eta = _f64(eta) if eta is not None else np.full((B, H, L), float(eta_scalar))
    ch = np.arange(L) // chunk
    mask = (ch[None, :] < ch[:, None]).astype(np.float64)
    out = ((q @ np.swapaxes(k, -1, -2)) * mask * eta[:, :, None, :]) @ v
    if S0 is not None:
        out = out + q @ _f64(S0)
    return out


def chunk_causal_rows(q, k, v, rows, eta_scalar, S0, chunk, block=2048):
    """Selected output rows of the single-state chunk-causal update (B = H = 1),
    by the closed form of `bruteforce_chunk_causal` row by row:
        o_t = q_t S0 + eta * sum_{s < start(chunk(t))} (q_t . k_s) v_s
    q,k [L,dk], v [L,dv] (any float dtype, upcast per block); S0 [dk,dv].
    Used where the whole output is too large for the oracle."""
    rows = np.asarray(rows)
    qr = _f64(q[rows])                                  # [R, dk]
    S0 = _f64(S0)
    acc = np.zeros((len(rows), v.shape[-1]))
    starts = (rows // chunk) * chunk
    limit = int(starts.max())
    for s0 in range(0, limit, block):
        s1 = min(s0 + block, limit)
        kb = _f64(k[s0:s1])                             # [blk, dk]
        g = qr @ kb.T                                   # [R, blk]
        cols = np.arange(s0, s1)
        g = g * (cols[None, :] < starts[:, None])
        acc += g @ _f64(v[s0:s1])
    return qr @ S0 + float(eta_scalar) * acc


def dual_form_matrix(q, k, v, W0, eta, minibatch):
    """Dual form of the mini-batch update as matrix products (NumPy fp64), [P4]
    section "gradient를 효율적인 layer로 만드는 작업".  Per mini-batch n:
        E_n = K_n W_n - V_n
        O_n = Q_n W_n - eta * (tril(Q_n K_n^T)) E_n
        W_{n+1} = W_n - eta * K_n^T E_n
    Returns (out, W_final)."""
    q, k, v, W = _f64(q), _f64(k), _f64(v), _f64(W0).copy()
    B, H, L, d = q.shape
    out = np.empty((B, H, L, v.shape[-1]))
    for n0 in range(0, L, minibatch):
        n1 = min(n0 + minibatch, L)
        qn, kn, vn = q[:, :, n0:n1], k[:, :, n0:n1], v[:, :, n0:n1]
        E = kn @ W - vn
        A = np.tril(qn @ np.swapaxes(kn, -1, -2))
        out[:, :, n0:n1] = qn @ W - eta * (A @ E)
        W = W - eta * (np.swapaxes(kn, -1, -2) @ E)
    return out, W


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64."""
    x, ref = _f64(x), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


if __name__ == "__main__":
    print(build())
    sys.exit(0)
