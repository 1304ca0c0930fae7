"""Seeded synthetic inputs for the chunked TTT fast-weight forward.

This module only draws random tensors and applies the input recipes
(scaling, L2 normalisation of keys, sigmoid of learning-rate logits, the
SiLU-gated MLP activation that produces Z).  It holds none of the fast-weight
arithmetic: the recurrences, chunk aggregates, scans and readouts live in
``oracle/`` (CPU, fp64) and in ``linear_attention_chunked_amd`` (HIP) and
neither of those imports the other.  Both consume the exact bytes produced
here.

Every tensor comes from ``torch.Generator('cpu').manual_seed(seed)``: values
are drawn in fp32, transformed in fp32, then rounded (round-to-nearest-even)
to the workload dtype.  The tensor index ``j`` in ``seed = 1000*cfg + j``
follows the order q, k, v, eta-logits, S0, M0 (for the LM-scale backward,
j = 5, 6 are its cotangents dout and dS_final).  The In-Place (chunk-causal)
workload is drawn chunk by chunk (``seed = 3_000_000 + 4*i + j`` for chunk
``i``; j = 0 a, 1 b, 2 V-hat) so a host never holds fp32 copies of the
long-context tensors.

Workloads (shapes of the pages' settings):
  small-f32   token-causal fp32, B1 H2 L256 d32, C64, eta 0.1, S0 0
  lm-scale    token-causal bf16, B8 H16 L4096 d128, C64, per-token eta, S0 ~ N(0, 0.02^2)
  inplace     In-Place chunk-causal Wdown update, L 32768 / 131072, d_ff 9728, d_model 2560, C1024
  momentum    momentum token-causal bf16, B4 H8 L16384 d128, C128, eta 0.05, beta 0.9
  dual        TTT-Linear mini-batch dual form, B4 H16 L8192 d64, b 16 and 2048, W0 0.5 I
  decode      one recurrent token per sequence, B256 H16 d128, state S0 (and M0) carried in
  bwd         backward of lm-scale: its inputs plus cotangents dout, dS_final
  bwd-momentum backward of momentum: its inputs plus cotangents (seeds 4005, 4006)
  inplace-frontend  gated input, LM-aligned target and clipped rates, T 32768, d_model 2560, d_ff 9728
  swiglu      large-chunk SwiGLU fast weight, B4 H4 L32768, d 512, hidden 2048, C2048,
              per-token eta = sigmoid(N(0,1)) / C, dot inner loss (seeds 10000 + j)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(shape, seed: int) -> torch.Tensor:
    return torch.randn(tuple(shape), generator=_gen(seed), dtype=torch.float32)


def f32(x: float) -> float:
    """Round a Python scalar to the nearest fp32 value (the value the GPU sees)."""
    return float(np.float32(x))


@dataclass
class TokenCausalInputs:
    """Inputs of one token-causal (or chunk-causal) forward call, [B,H,L,d] layout."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    eta: torch.Tensor | None          # [B,H,L] fp32, or None -> eta_scalar
    eta_scalar: float
    beta: float
    S0: torch.Tensor | None           # [B,H,dk,dv] fp32 or None (zero)
    M0: torch.Tensor | None           # [B,H,dk,dv] fp32 or None (zero)
    chunk: int
    dtype: str                        # "f32" | "bf16"
    meta: dict = field(default_factory=dict)


@dataclass
class DualInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    W0: torch.Tensor                  # [B,H,d,dv] fp32
    eta: float
    minibatch: int
    dtype: str
    meta: dict = field(default_factory=dict)


# ------------------------------------------------------------------ small fp32
def gen_small_f32(B=1, H=2, L=256, d=32, chunk=64, seed_base=1000) -> TokenCausalInputs:
    """fp32 q,k,v ~ N(0,1)/sqrt(d); constant eta 0.1; S0 = 0."""
    s = 1.0 / math.sqrt(d)
    q = _randn((B, H, L, d), seed_base + 0) * s
    k = _randn((B, H, L, d), seed_base + 1) * s
    v = _randn((B, H, L, d), seed_base + 2) * s
    return TokenCausalInputs(q, k, v, None, f32(0.1), 0.0, None, None, chunk, "f32",
                             dict(workload="small-f32", B=B, H=H, L=L, dk=d, dv=d))


# ------------------------------------------------------------------ LM-scale
def gen_lm_scale(B=8, H=16, L=4096, d=128, chunk=64, seed_base=2000) -> TokenCausalInputs:
    """bf16 q,v ~ N(0,1); k ~ N(0,1) L2-normalised per token in fp32, then bf16;
    per-token eta = 0.1*sigmoid(N(0,1)) kept in fp32; S0 ~ N(0, 0.02^2) fp32."""
    q = _randn((B, H, L, d), seed_base + 0).to(torch.bfloat16)
    kr = _randn((B, H, L, d), seed_base + 1)
    k = (kr / kr.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    del kr
    v = _randn((B, H, L, d), seed_base + 2).to(torch.bfloat16)
    eta = (0.1 * torch.sigmoid(_randn((B, H, L), seed_base + 3))).float()
    S0 = _randn((B, H, d, d), seed_base + 4) * 0.02
    return TokenCausalInputs(q, k, v, eta, 0.0, 0.0, S0, None, chunk, "bf16",
                             dict(workload="lm-scale", B=B, H=H, L=L, dk=d, dv=d))


def gen_lm_scale_cotangents(B=8, H=16, L=4096, d=128, seed_base=2000):
    """Cotangents for a backward workload (LM-scale by default; the momentum
    workload uses its own seed base): dout ~ N(0,1)/sqrt(L) bf16 [B,H,L,d]
    (j = 5); dS_final ~ N(0, 0.02^2) fp32 [B,H,d,d] (j = 6)."""
    dout = (_randn((B, H, L, d), seed_base + 5) / math.sqrt(L)).to(torch.bfloat16)
    dSf = _randn((B, H, d, d), seed_base + 6) * 0.02
    return dout, dSf


# ------------------------------------------------------------------ In-Place
INPLACE_SEED = 3_000_000


def gen_inplace_chunk(i: int, rows: int, d_ff=9728, d_model=2560):
    """Chunk i of the In-Place workload: Z_i = silu(a)*b (from bf16 a, b, computed
    in fp32, rounded to bf16) and the target V-hat_i ~ N(0,1) bf16."""
    a = _randn((rows, d_ff), INPLACE_SEED + 4 * i + 0).to(torch.bfloat16).float()
    b = _randn((rows, d_ff), INPLACE_SEED + 4 * i + 1).to(torch.bfloat16).float()
    z = (torch.nn.functional.silu(a) * b).to(torch.bfloat16)
    del a, b
    vh = _randn((rows, d_model), INPLACE_SEED + 4 * i + 2).to(torch.bfloat16)
    return z, vh


def gen_inplace_W0(d_ff=9728, d_model=2560, seed=3000):
    return _randn((d_ff, d_model), seed) * 0.02


def gen_inplace(L=32768, d_ff=9728, d_model=2560, chunk=1024, gen_block=1024, out=None):
    """Whole In-Place workload.  Z, V-hat are [1,1,L,d] bf16 (B=H=1); the same
    tensor Z serves as both query and key.  ``out`` may give preallocated
    (Z, V) tensors (on any device) that are filled block by block."""
    if out is None:
        Z = torch.empty((1, 1, L, d_ff), dtype=torch.bfloat16)
        V = torch.empty((1, 1, L, d_model), dtype=torch.bfloat16)
    else:
        Z, V = out
    nblk = (L + gen_block - 1) // gen_block
    for i in range(nblk):
        r0 = i * gen_block
        rows = min(gen_block, L - r0)
        z, vh = gen_inplace_chunk(i, rows, d_ff, d_model)
        Z[0, 0, r0:r0 + rows].copy_(z)
        V[0, 0, r0:r0 + rows].copy_(vh)
    W0 = gen_inplace_W0(d_ff, d_model).reshape(1, 1, d_ff, d_model)
    return TokenCausalInputs(Z, Z, V, None, f32(1e-3), 0.0, W0, None, chunk, "bf16",
                             dict(workload="inplace", B=1, H=1, L=L, dk=d_ff, dv=d_model))


# ------------------------------------------------------------------ momentum
def gen_inplace_frontend(T=32768, d_model=2560, d_ff=9728, taps=4, seed_base=9000, device="cpu"):
    """In-Place front end: X ~ N(0,1) bf16 [1, T, d_model]; Wg, Wu ~ N(0, 1/d_model)
    bf16 [d_ff, d_model] (j = 1, 2); conv_w ~ N(0, 0.5^2) fp32 [taps, d_model]
    (j = 3); Wv ~ N(0, 1/d_model) bf16 [d_model, d_model] (j = 4).  Drawn in
    row blocks so a host never holds an fp32 copy of a whole large tensor;
    ``device`` receives the bf16 tensors."""
    def big(shape, seed, scale):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        g = _gen(seed)
        rows = shape[-2]
        flat = out.view(-1, shape[-1])
        for r0 in range(0, flat.shape[0], 4096):
            r1 = min(r0 + 4096, flat.shape[0])
            flat[r0:r1].copy_((torch.randn((r1 - r0, shape[-1]), generator=g) * scale).to(torch.bfloat16))
        return out
    X = big((1, T, d_model), seed_base + 0, 1.0)
    Wg = big((d_ff, d_model), seed_base + 1, d_model ** -0.5)
    Wu = big((d_ff, d_model), seed_base + 2, d_model ** -0.5)
    conv_w = (_randn((taps, d_model), seed_base + 3) * 0.5).to(device)
    Wv = big((d_model, d_model), seed_base + 4, d_model ** -0.5)
    return X, Wg, Wu, conv_w, Wv


def gen_momentum(B=4, H=8, L=16384, d=128, chunk=128, seed_base=4000) -> TokenCausalInputs:
    """bf16 q,k,v ~ N(0,1)/sqrt(d); eta 0.05; beta 0.9; S0 = M0 = 0."""
    s = 1.0 / math.sqrt(d)
    q = (_randn((B, H, L, d), seed_base + 0) * s).to(torch.bfloat16)
    k = (_randn((B, H, L, d), seed_base + 1) * s).to(torch.bfloat16)
    v = (_randn((B, H, L, d), seed_base + 2) * s).to(torch.bfloat16)
    return TokenCausalInputs(q, k, v, None, f32(0.05), f32(0.9), None, None, chunk, "bf16",
                             dict(workload="momentum", B=B, H=H, L=L, dk=d, dv=d))


# ------------------------------------------------------------------ dual form
def gen_dual(B=4, H=16, L=8192, d=64, minibatch=16, seed_base=5000) -> DualInputs:
    """bf16 q,k,v ~ N(0,1)/sqrt(d); W0 = 0.5*I fp32 per (b,h); eta = 1/d."""
    s = 1.0 / math.sqrt(d)
    q = (_randn((B, H, L, d), seed_base + 0) * s).to(torch.bfloat16)
    k = (_randn((B, H, L, d), seed_base + 1) * s).to(torch.bfloat16)
    v = (_randn((B, H, L, d), seed_base + 2) * s).to(torch.bfloat16)
    W0 = (0.5 * torch.eye(d, dtype=torch.float32)).expand(B, H, d, d).contiguous()
    return DualInputs(q, k, v, W0, f32(1.0 / d), minibatch, "bf16",
                      dict(workload="dual", B=B, H=H, L=L, d=d))


# ------------------------------------------------------------------ decode step
def gen_decode(B=256, H=16, d=128, beta=0.0, seed_base=7000) -> TokenCausalInputs:
    """One decode token per sequence (L = 1) against a carried state, LM-scale
    heads: bf16 q,v ~ N(0,1); k ~ N(0,1) L2-normalised in fp32, then bf16;
    eta = 0.1*sigmoid(N(0,1)) fp32 per (b,h); S0 ~ N(0, 0.02^2) fp32;
    with momentum, M0 ~ N(0, 0.002^2) fp32."""
    q = _randn((B, H, 1, d), seed_base + 0).to(torch.bfloat16)
    kr = _randn((B, H, 1, d), seed_base + 1)
    k = (kr / kr.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    v = _randn((B, H, 1, d), seed_base + 2).to(torch.bfloat16)
    eta = (0.1 * torch.sigmoid(_randn((B, H, 1), seed_base + 3))).float()
    S0 = _randn((B, H, d, d), seed_base + 4) * 0.02
    M0 = _randn((B, H, d, d), seed_base + 5) * 0.002 if beta else None
    return TokenCausalInputs(q, k, v, eta, 0.0, f32(beta), S0, M0, 1, "bf16",
                             dict(workload="decode", B=B, H=H, L=1, dk=d, dv=d))


def gen_state_deltas(B, H, N, dk, dv, seed=6000, scale=1.0, integer=False):
    """Random per-chunk state aggregates dS, dM [B,H,N,dk,dv] fp32 for the
    standalone chunk-state scan (integer-valued when ``integer``)."""
    if integer:
        g = _gen(seed)
        dS = torch.randint(-3, 4, (B, H, N, dk, dv), generator=g).float()
        dM = torch.randint(-3, 4, (B, H, N, dk, dv), generator=g).float()
    else:
        dS = _randn((B, H, N, dk, dv), seed) * scale
        dM = _randn((B, H, N, dk, dv), seed + 1) * scale
    return dS, dM


# --------------------------------------------------- SwiGLU fast weight
@dataclass
class SwigluInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    eta: torch.Tensor
    W1: torch.Tensor
    W3: torch.Tensor
    W2: torch.Tensor
    chunk: int
    loss: str
    config: dict = field(default_factory=dict)


def gen_swiglu(B=4, H=4, L=32768, d=512, m=2048, chunk=2048, loss="dot", seed_base=10000, device="cpu",
               dv=None, eta_scale=None) -> SwigluInputs:
    """Large-chunk SwiGLU fast weight: q, k, v ~ N(0,1) bf16 [B,H,L,d] (j = 0,
    1, 2; v has dv features, default d); eta_t = eta_scale * sigmoid(N(0,1))
    fp32 (j = 3), eta_scale = 1 / chunk by default, which keeps the weights
    bounded over many chunks at the benchmark's sizes; W1, W3 ~
    N(0, 1/d) fp32 [B,H,m,d] (j = 4, 5); W2 ~ N(0, 1/m) fp32 [B,H,dv,m]
    (j = 6).  The token tensors are drawn in row blocks so a host never holds
    an fp32 copy of a whole large tensor; ``device`` receives every tensor."""
    dv = d if dv is None else dv

    def rows(shape, seed, scale, dtype):
        out = torch.empty(shape, dtype=dtype, device=device)
        g = _gen(seed)
        flat = out.view(-1, shape[-1])
        for r0 in range(0, flat.shape[0], 8192):
            r1 = min(r0 + 8192, flat.shape[0])
            flat[r0:r1].copy_((torch.randn((r1 - r0, shape[-1]), generator=g) * scale).to(dtype))
        return out

    q = rows((B, H, L, d), seed_base + 0, 1.0, torch.bfloat16)
    k = rows((B, H, L, d), seed_base + 1, 1.0, torch.bfloat16)
    v = rows((B, H, L, dv), seed_base + 2, 1.0, torch.bfloat16)
    eta_scale = 1.0 / chunk if eta_scale is None else eta_scale
    eta = (torch.sigmoid(_randn((B, H, L), seed_base + 3)) * eta_scale).to(device)
    W1 = rows((B, H, m, d), seed_base + 4, d ** -0.5, torch.float32)
    W3 = rows((B, H, m, d), seed_base + 5, d ** -0.5, torch.float32)
    W2 = rows((B, H, dv, m), seed_base + 6, m ** -0.5, torch.float32)
    return SwigluInputs(q, k, v, eta, W1, W3, W2, chunk, loss,
                        dict(workload="swiglu", B=B, H=H, L=L, dk=d, dv=dv, m=m, chunk=chunk, loss=loss))


def to_f64(t: torch.Tensor | None) -> np.ndarray | None:
    """Exact upcast of a CPU tensor (bf16/fp32) to a contiguous fp64 array."""
    if t is None:
        return None
    return np.ascontiguousarray(t.detach().to("cpu").to(torch.float64).numpy())
