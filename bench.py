"""Benchmark of the chunked TTT fast-weight forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload inplace-128k]

One step = one full pass of the hot path over one batch of synthetic input
(all inputs resident in HBM before timing).  The default workload is the
largest single-GPU configuration: In-Place TTT chunk-causal forward of one
Wdown fast weight (d_ff 9728 x d_model 2560, fp32) over L = 131072 tokens in
chunks of 1024, one ttt_fwd_chunked call (the update walk and the batched
readout).  Prints ONE JSON line.

Warm-up: the W warm-up steps are extended until at least --min-warmup-s
seconds of steps have run (the count actually run is reported), so that the
timed steps see the GPU's steady clocks rather than its ramp.

Timing: every timed step is bracketed by HIP events on the launch stream.
Between steps, outside the events, a 512 MiB scratch buffer is written and
another 512 MiB buffer is read, so that no input is still in the 256 MiB
last-level cache and no dirty line of the scratch write is left in it for the
timed step to write back (--evict selects other modes).  value and
ms_per_step use the mean event time of a step; the median and minimum are
reported beside it, and so is the wall time per step with the eviction
passes (it includes a spin kernel, run once before the timed steps, that
holds the stream until the host is far enough ahead: an event interval must
not time the GPU waiting for the host.  The hold is a few steps' issue time
when a step's GPU time is well above it, as it is with the eviction passes,
and the time to issue every step otherwise; hold_ms reports it).  The GPU
clock is read with rocm-smi during the warm-up (under load, on a host thread,
so the GPU never idles before the timed steps) and after the timed steps
(null when rocm-smi gives none).

Roofline: the dominant kernel's average launch duration is the mean event
time; achieved = algorithmic bytes (or FLOPs) per launch / that duration.
HBM traffic counted by rocprofv3 (FETCH_SIZE / WRITE_SIZE, scaled by a plain
copy's counters) is read from profiles/traffic.json when it was measured on
the current kernel source, else reported as null.

cpu_baseline: the fp64 oracle (C, OpenMP over heads) timed on this host on
the same seeded inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # dense fp32 MFMA / vector

METRIC = "tokens/s + TFLOP/s (MFMA % of peak) for chunked TTT fast-weight forward, 1 GPU"


KERNEL_SOURCES = {
    "tc_fwd_kernel": ("tc_fwd.hip", "common.h"),
    "tcb_fwd_kernel": ("tcb_fwd.hip", "common.h"),
    "ip_update_kernel+ip_readout_kernel": ("inplace.hip", "common.h"),
    "ip_update_wide_kernel+ip_readout_kernel": ("inplace.hip", "common.h"),
    "dual_fwd_kernel": ("dual.hip", "common.h"),
    "dual_ring_kernel": ("dual.hip", "common.h"),
    "dual_seg_kernel": ("dual.hip", "common.h"),
    "decode_kernel": ("decode.hip", "common.h"),
    "fe_gemm_kernel": ("frontend.hip", "gemm.h", "common.h"),
    "tcb_fwd_kernel+bwd_scale_kernels": ("tcb_fwd.hip", "bwd.hip", "common.h"),
    "swiglu_kernels": ("swiglu.hip", "gemm.h", "common.h"),
    "state_scan_kernel": ("scan.hip", "common.h"),
    "dbeta_kernel": ("dbeta.hip", "common.h"),
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the source files a kernel is built from (traffic counters are
    only reported while they match)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_chunked_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- workloads
def setup_workload(name: str, dev: str):
    """Returns (step_fn, info) with inputs already on the device."""
    import torch
    import workloads as W
    import linear_attention_chunked_amd as lac

    if name in ("small-f32", "lm-scale", "momentum"):
        gen = {"small-f32": W.gen_small_f32, "lm-scale": W.gen_lm_scale, "momentum": W.gen_momentum}[name]
        inp = gen()
        B, H, L, dk = inp.q.shape
        dv = inp.v.shape[-1]
        q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
        eta = inp.eta.to(dev) if inp.eta is not None else None
        S0 = inp.S0.to(dev) if inp.S0 is not None else None
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
        es = q.element_size()
        C = inp.chunk
        mom = inp.beta != 0.0

        def step():
            return lac.fwd_chunked(q, k, v, eta=eta, eta_scalar=inp.eta_scalar, beta=inp.beta, S0=S0,
                                   chunk=C, out=out, return_state=True)

        nstate = 2 if mom else 1
        bytes_alg = (B * H * L * (2 * dk + dv) * es                 # q, k, v
                     + (B * H * L * 4 if eta is not None else 0)    # eta
                     + (B * H * dk * dv * 4 if S0 is not None else 0)
                     + B * H * L * dv * es                          # out
                     + nstate * B * H * dk * dv * 4)                # final state(s)
        flop_alg = B * H * L * (4 * nstate * dk * dv + (C + 1) * (dk + dv))
        # the kernel tiles token-causal work in 64-token chunks (32 for fp32)
        # whatever C is: token-causal results do not depend on the chunk
        info = dict(workload=name, B=B, H=H, L=L, dk=dk, dv=dv, chunk=C,
                    kernel_tile_tokens=64 if inp.dtype == "bf16" else 32, mode="token_causal",
                    beta=inp.beta, eta="per-token" if eta is not None else inp.eta_scalar,
                    dtype=inp.dtype, tokens=B * L, bytes_alg=bytes_alg, flop_alg=flop_alg,
                    kernel="tcb_fwd_kernel" if inp.dtype == "bf16" else "tc_fwd_kernel", inputs=inp)
        return step, info
    if name in ("inplace-32k", "inplace-128k"):
        L = 32768 if name == "inplace-32k" else 131072
        d_ff, d_model = 9728, 2560
        Z = torch.empty((1, 1, L, d_ff), dtype=torch.bfloat16, device=dev)
        V = torch.empty((1, 1, L, d_model), dtype=torch.bfloat16, device=dev)
        inp = W.gen_inplace(L=L, out=(Z, V))
        W0 = inp.S0.to(dev)
        out = torch.empty((1, 1, L, d_model), dtype=torch.bfloat16, device=dev)

        def step():
            return lac.fwd_chunked(Z, Z, V, eta_scalar=inp.eta_scalar, S0=W0, chunk=1024,
                                   mode="chunk_causal", out=out, return_state=True)

        bytes_alg = L * (d_ff + 2 * d_model) * 2 + 2 * d_ff * d_model * 4
        flop_alg = 4 * L * d_ff * d_model
        def cpu_sample():
            # the first chunks (all of W), NumPy fp64 GEMMs: two chunks time one
            # chunk, then as many chunks as fit in about 16 s by that estimate
            # run timed (the estimate runs long: ~10 s in practice)
            import oracle
            def run(nc):
                n = nc * 1024
                z, vv = W.to_f64(Z[:, :, :n].cpu()), W.to_f64(V[:, :, :n].cpu())
                t0 = time.perf_counter()
                oracle.chunk_causal(z, z, vv, eta_scalar=inp.eta_scalar, S0=W.to_f64(inp.S0), chunk=1024)
                return time.perf_counter() - t0
            per_chunk = run(2) / 2
            nc = int(min(L // 1024, max(2, 16.0 // per_chunk)))
            dt = run(nc)
            return (nc * 1024, f"the first {nc * 1024} of {L} tokens ({nc} of {L // 1024} chunks, the whole W), "
                    "NumPy fp64 GEMMs", blas_threads(), dt)

        info = dict(workload=name, B=1, H=1, L=L, d_ff=d_ff, d_model=d_model, chunk=1024,
                    mode="chunk_causal", eta=inp.eta_scalar, dtype="bf16", tokens=L,
                    bytes_alg=bytes_alg, flop_alg=flop_alg, kernel="ip_update_wide_kernel+ip_readout_kernel",
                    inputs=None, cpu_sample=cpu_sample)
        return step, info
    if name in ("dual-b16", "dual-b2048"):
        mb = 16 if name == "dual-b16" else 2048
        inp = W.gen_dual(minibatch=mb)
        B, H, L, d = inp.q.shape
        q, k, v, W0 = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.W0.to(dev)
        out = torch.empty_like(v)

        def step():
            return lac.dual_form_fwd(q, k, v, W0, eta=inp.eta, minibatch=mb, out=out, return_state=True)

        bytes_alg = B * H * L * 4 * d * 2 + 2 * B * H * d * d * 4
        flop_alg = B * H * L * (6 * d * d + (mb + 1) * 2 * d)
        info = dict(workload=name, B=B, H=H, L=L, d=d, minibatch=mb, dtype="bf16", tokens=B * L,
                    bytes_alg=bytes_alg, flop_alg=flop_alg, kernel="dual_seg_kernel", inputs=inp)
        return step, info
    if name in ("bwd", "bwd-momentum"):
        mom = name == "bwd-momentum"
        inp = W.gen_momentum() if mom else W.gen_lm_scale()
        B, H, L, dk = inp.q.shape
        dv = inp.v.shape[-1]
        dout, dSf = W.gen_lm_scale_cotangents(B, H, L, dk, seed_base=4000 if mom else 2000)
        q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
        eta = inp.eta.to(dev) if inp.eta is not None else None
        S0 = inp.S0.to(dev) if inp.S0 is not None else None
        do, dS = dout.to(dev), dSf.to(dev)
        side = torch.cuda.Stream()   # the dv/deta step runs beside the last pass

        def step():
            return lac.bwd_chunked(q, k, v, do, eta=eta, eta_scalar=inp.eta_scalar, beta=inp.beta, S0=S0,
                                   dS_final=dS, need_dM0=mom, side_stream=side)

        es = 2
        bytes_alg = (B * H * L * (2 * dk + 2 * dv) * es      # q, k, v, dout
                     + B * H * L * (2 * dk + dv) * es        # dq, dk, dv
                     + B * H * L * 4 * 2                     # eta, deta
                     + 3 * B * H * dk * dv * 4)              # S0, dS_final, dS0
        C = inp.chunk
        nst = 2 if mom else 1
        if mom:
            bytes_alg += B * H * dk * dv * 4          # dM0
        flop_alg = 3 * B * H * L * (4 * nst * dk * dv + (C + 1) * (dk + dv))
        def cpu_sample():
            # 8 (b, h) heads, whole sequences, the C oracle's adjoint sweeps
            import oracle
            sl = lambda t: None if t is None else W.to_f64(t[:1, :8])
            oracle.token_causal_bwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(dout), sl(inp.eta), inp.eta_scalar,
                                    inp.beta, sl(inp.S0), None, sl(dSf), None)
            return (8 * L / H, f"8 of {B * H} (b,h) heads, full L={L}, fp64 adjoint sweeps in C "
                    "(tokens scaled by the head fraction)", oracle.threads())

        info = dict(workload=name, B=B, H=H, L=L, dk=dk, dv=dv, chunk=C, mode="token_causal backward",
                    beta=inp.beta, eta="per-token" if eta is not None else inp.eta_scalar, dtype="bf16",
                    tokens=B * L, bytes_alg=bytes_alg, flop_alg=flop_alg,
                    kernel="tcb_fwd_kernel+bwd_scale_kernels", inputs=None, cpu_sample=cpu_sample)
        return step, info
    if name == "bwd-dbeta":
        # dL/dbeta on the momentum shape (beside the momentum backward)
        inp = W.gen_momentum()
        B, H, L, dk = inp.q.shape
        dv = inp.v.shape[-1]
        dout, dSf = W.gen_lm_scale_cotangents(B, H, L, dk, seed_base=4000)
        q, k, v, do, dS = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), dout.to(dev), dSf.to(dev)

        def step():
            return lac.bwd_dbeta(q, k, v, do, eta_scalar=inp.eta_scalar, beta=inp.beta, dS_final=dS)

        # every column tile reads the full q and k rows (the algorithmic count
        # reads each tensor once): q, k, v, dout, dS_final
        bytes_alg = B * H * L * (2 * dk + 2 * dv) * 2 + B * H * dk * dv * 4
        # per token: 3 state readouts and 3 weighted aggregates (2 dk dv each),
        # the scores q . k and do . v against the 16 tokens of its block
        # (each product counted once; the kernel recomputes the scores per
        # 16-column tile)
        flop_alg = B * H * L * (12 * dk * dv + 2 * 16 * (dk + dv))
        def cpu_sample():
            import oracle
            sl = lambda t: None if t is None else W.to_f64(t[:1, :4])
            oracle.token_causal_dbeta(sl(inp.q), sl(inp.k), sl(inp.v), sl(dout), None, inp.eta_scalar, inp.beta,
                                      None, sl(dSf), None)
            return (4 * L / H, f"4 of {B * H} (b,h) heads, full L={L}, fp64 tangent recurrence in C "
                    "(tokens scaled by the head fraction)", oracle.threads())

        info = dict(workload=name, B=B, H=H, L=L, dk=dk, dv=dv, mode="token_causal dL/dbeta", beta=inp.beta,
                    eta=inp.eta_scalar, dtype="bf16", tokens=B * L, bytes_alg=bytes_alg, flop_alg=flop_alg,
                    kernel="dbeta_kernel", inputs=None, cpu_sample=cpu_sample)
        return step, info
    if name == "inplace-frontend":
        T, dm, dff, taps, C = 32768, 2560, 9728, 4, 1024
        X, Wg, Wu, cw, Wv = W.gen_inplace_frontend(T, dm, dff, taps, device=dev)
        Z = torch.empty((1, T, dff), dtype=torch.bfloat16, device=dev)
        V = torch.empty_like(X)
        E = torch.empty((1, T), dtype=torch.float32, device=dev)

        def step():
            lac.inplace_gated_input(X, Wg, Wu, out=Z)
            lac.inplace_lm_target(X, cw, Wv, out=V)
            return lac.inplace_clip_eta(Z, V, chunk=C, eta=1e-3, tau=50.0, out=E)

        # gated projection and target projection (the clipping norms are extra)
        flop_alg = 2 * 2 * T * dm * dff + 2 * T * dm * dm
        bytes_alg = (T * dm * 2 + 2 * dff * dm * 2 + dm * dm * 2 + taps * dm * 4   # X, weights
                     + T * dff * 2 + T * dm * 2 + T * 4)                           # Z, V-hat, rates
        def cpu_sample():
            # the first chunk of tokens through the whole front end, NumPy fp64
            import oracle
            x = W.to_f64(X[:, :C].cpu())
            z = oracle.inplace_gated_input(x, W.to_f64(Wg.cpu()), W.to_f64(Wu.cpu()))
            vh = oracle.lm_aligned_target(x, W.to_f64(cw.cpu()), W.to_f64(Wv.cpu()))
            oracle.clip_scales(z, vh, C, 1e-3, 50.0)
            return C, f"the first {C} of {T} tokens (one chunk), NumPy fp64"

        info = dict(workload=name, T=T, d_model=dm, d_ff=dff, taps=taps, chunk=C, dtype="bf16", tokens=T,
                    bytes_alg=bytes_alg, flop_alg=flop_alg, kernel="fe_gemm_kernel", inputs=None,
                    cpu_sample=cpu_sample)
        return step, info
    if name in ("swiglu", "swiglu-mse"):
        loss = "mse" if name == "swiglu-mse" else "dot"
        inp = W.gen_swiglu(loss=loss, device=dev)
        B, H, L, dk = inp.q.shape
        dv, m, C = inp.v.shape[-1], inp.W1.shape[-2], inp.chunk
        W1, W3, W2 = inp.W1.clone(), inp.W3.clone(), inp.W2.clone()
        out = torch.empty_like(inp.v)
        ws = torch.empty(lac.swiglu_workspace_size(B, H, L, dk, dv, m, C), dtype=torch.uint8, device=dev)

        def step():
            # every step starts from W0 (the call updates the weights in place)
            W1.copy_(inp.W1)
            W3.copy_(inp.W3)
            W2.copy_(inp.W2)
            return lac.swiglu_fwd_chunked(inp.q, inp.k, inp.v, W1, W3, W2, eta=inp.eta, chunk=C, loss=loss,
                                          out=out, workspace=ws)

        # per token: [q; k] x W13 (2 x 2 m dk x 2), output (dv m x 2, twice for
        # MSE), dA (m dv x 2), dW2 (dv m x 2), dW13 (2 m dk x 2)
        flop_alg = B * H * L * (12 * m * dk + (8 if loss == "mse" else 6) * m * dv)
        bytes_alg = (B * H * L * (2 * dk + 2 * dv) * 2 + B * H * L * 4     # q, k, v, out, eta
                     + 2 * B * H * (2 * m * dk + dv * m) * 4)               # weights in and out
        info = dict(workload=name, B=B, H=H, L=L, dk=dk, dv=dv, m=m, chunk=C, loss=loss, eta="per-token",
                    dtype="bf16", tokens=B * L, bytes_alg=bytes_alg, flop_alg=flop_alg,
                    kernel="swiglu_kernels", inputs=inp)
        return step, info
    if name in ("decode", "decode-momentum"):
        inp = W.gen_decode(beta=0.9 if name == "decode-momentum" else 0.0)
        B, H, _, dk = inp.q.shape
        dv = inp.v.shape[-1]
        q, k, v = inp.q[:, :, 0].to(dev), inp.k[:, :, 0].to(dev), inp.v[:, :, 0].to(dev)
        eta = inp.eta[:, :, 0].contiguous().to(dev)
        S = inp.S0.to(dev)
        M = inp.M0.to(dev) if inp.M0 is not None else None
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)

        def step():
            return lac.decode_step(q, k, v, S, M, eta=eta, beta=inp.beta, out=out)

        nstate = 2 if M is not None else 1
        bytes_alg = B * H * (2 * dk + 2 * dv) * 2 + B * H * 4 + 2 * nstate * B * H * dk * dv * 4
        flop_alg = B * H * dk * dv * (2 * nstate + 2 + 1)
        info = dict(workload=name, B=B, H=H, L=1, dk=dk, dv=dv, beta=inp.beta, eta="per-sequence",
                    dtype="bf16", tokens=B, bytes_alg=bytes_alg, flop_alg=flop_alg, kernel="decode_kernel",
                    inputs=inp)
        return step, info
    if name in ("scan", "scan-momentum"):
        # the standalone chunk-state scan at the LM-scale shape: B8 H16, L 4096
        # in 64-token chunks (N = 64), d_k = d_v = 128, fp32 aggregates
        B, H, L, C, dk, dv = 8, 16, 4096, 64, 128, 128
        N = L // C
        beta = W.f32(0.9) if name == "scan-momentum" else 0.0
        dS_c, dM_c = W.gen_state_deltas(B, H, N, dk, dv, seed=6200)
        S0_c, M0_c = W.gen_state_deltas(B, H, 1, dk, dv, seed=6300)
        S0_c, M0_c = S0_c[:, :, 0].contiguous(), M0_c[:, :, 0].contiguous()
        dS = dS_c.to(dev)
        dM = dM_c.to(dev) if beta else None
        S0 = S0_c.to(dev)
        M0 = M0_c.to(dev) if beta else None

        def step():
            return lac.chunk_state_scan(dS, dM, beta=beta, chunk=C, L=L, S0=S0, M0=M0)

        nstate = 2 if beta else 1
        bytes_alg = nstate * (2 * B * H * N + 2 * B * H) * dk * dv * 4
        flop_alg = nstate * 2 * B * H * N * dk * dv

        def cpu_sample():
            import oracle
            oracle.state_scan(dS_c, dM_c if beta else None, beta, C, L, S0_c, M0_c if beta else None)
            return B * L, f"the whole workload ({B * H} heads, {N} chunks), fp64 sequential scan in C", oracle.threads()

        info = dict(workload=name, B=B, H=H, L=L, N=N, chunk=C, dk=dk, dv=dv, beta=beta, dtype="fp32",
                    tokens=B * L, bytes_alg=bytes_alg, flop_alg=flop_alg, kernel="state_scan_kernel",
                    inputs=None, cpu_sample=cpu_sample)
        return step, info
    raise SystemExit(f"unknown workload {name}")


# --------------------------------------------------------------- CPU baseline
def cpu_baseline(info) -> dict:
    """fp64 oracle on the same seeded inputs (whole workload when it fits
    ~10-30 s of host work, else a head subset scaled to the whole)."""
    import numpy as np
    import oracle
    import workloads as W

    if "cpu_sample" in info:
        t0 = time.perf_counter()
        res = info["cpu_sample"]()
        dt = time.perf_counter() - t0
        tokens, what = res[0], res[1]
        cores = res[2] if len(res) > 2 else blas_threads()   # C oracle (OpenMP) or NumPy's BLAS
        if len(res) > 3:
            dt = res[3]   # the sample timed its own oracle call (after a calibration run)
        return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"{what}; {dt:.2f} s"}
    inp = info["inputs"]
    if inp is None:
        return None
    if info["workload"] in ("swiglu", "swiglu-mse"):
        B, H, L = inp.q.shape[:3]
        f = lambda t: W.to_f64(t[:1, :1].cpu())
        t0 = time.perf_counter()
        oracle.swiglu_fast_weight(f(inp.q), f(inp.k), f(inp.v), f(inp.W1), f(inp.W3), f(inp.W2), eta=f(inp.eta),
                                  chunk=inp.chunk, loss=inp.loss)
        dt = time.perf_counter() - t0
        return {"value": info["tokens"] / (B * H) / dt, "unit": "tokens/s", "cores": blas_threads(),
                "kind": "oracle",
                "sample": f"1 of {B * H} (b,h) heads, full L={L} ({L // inp.chunk} chunks), NumPy fp64 GEMMs; "
                          f"{dt:.2f} s; tokens/s scaled by the head fraction"}
    B, H = inp.q.shape[:2]
    L = inp.q.shape[2]
    heads = B * H   # every workload below runs whole within a few seconds
    bsel = max(1, heads // H)
    hsel = min(H, heads)
    sl = lambda t: None if t is None else W.to_f64(t[:bsel, :hsel])
    args = [sl(inp.q), sl(inp.k), sl(inp.v)]
    # the whole workload takes the C oracle well under a second: it is run
    # again until 3 s have passed and the time per run is reported
    if info["workload"] in ("dual-b16", "dual-b2048"):
        W0 = sl(inp.W0)
        run = lambda: oracle.dual_primal(*args, W0, inp.eta, inp.minibatch)
    else:
        eta, S0, M0 = sl(inp.eta), sl(inp.S0), sl(inp.M0)
        run = lambda: oracle.token_causal(*args, eta=eta, eta_scalar=inp.eta_scalar, beta=inp.beta, S0=S0, M0=M0)
    reps = 0
    t0 = time.perf_counter()
    while True:
        run()
        reps += 1
        if time.perf_counter() - t0 >= 3.0:
            break
    dt = (time.perf_counter() - t0) / reps
    frac = (bsel * hsel) / (B * H)
    tokens_per_s = info["tokens"] * frac / dt
    what = (f"{bsel * hsel} of {B * H} (b,h) heads, full L={L}, fp64 per-token recurrence, run {reps} times, "
            f"{dt:.3f} s each" if L > 1 else f"whole decode step ({B * H} heads) run {reps} times, {dt:.3f} s each")
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": what + "; tokens/s scaled by the head fraction"}


def gpu_sclk_mhz():
    """Current shader clock of GPU 0 in MHz from rocm-smi, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    for ln in r.stdout.splitlines():
        if "sclk" in ln.lower():
            m = re.search(r"\((\d+)\s*Mhz\)", ln, flags=re.I)
            if m:
                return int(m.group(1))
    return None


def blas_threads() -> int:
    """Threads NumPy's BLAS runs the oracle's GEMMs with."""
    from threadpoolctl import threadpool_info
    return max((p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"), default=1)


def load_traffic(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(f"{kernel}:{workload}")
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="inplace-128k",
                    help="inplace-128k (default), lm-scale, small-f32, inplace-32k, momentum, dual-b16, "
                         "dual-b2048, decode, decode-momentum, bwd, bwd-momentum, bwd-dbeta, inplace-frontend, swiglu, swiglu-mse, "
                         "scan, scan-momentum")
    ap.add_argument("--evict", default="write-read", choices=("write-read", "write", "read", "none"),
                    help="what runs between timed steps to clear the last-level cache: write one "
                         "512 MiB buffer and then read another (default), only one of the two, or nothing")
    ap.add_argument("--no-evict", action="store_true", help="same as --evict none")
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="keep warming up until this many seconds of steps have run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X "
              "(multi-GPU sharding is design-only). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return

    step, info = setup_workload(args.workload, dev)
    stream = torch.cuda.current_stream()
    # Before every step (outside the events) 512 MiB, twice the last-level
    # cache, are written and then another 512 MiB are read: the write pushes
    # out the previous step's inputs and outputs, the read then replaces the
    # write's dirty lines with clean ones, so the timed step neither finds its
    # inputs in the cache nor pays for writing back someone else's data
    mode = "none" if args.no_evict else args.evict
    evict_w = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if "write" in mode else None
    evict_r = torch.zeros(128 << 20, dtype=torch.float32, device=dev) if "read" in mode else None
    evict_sink = torch.empty((), dtype=torch.float32, device=dev)

    def evict_pass(i):
        if evict_w is not None:
            evict_w.fill_(i & 0xff)
        if evict_r is not None:
            torch.sum(evict_r, dim=0, out=evict_sink)

    # cycles per ms of torch's spin kernel (for the hold below), measured
    # before the warm-up, away from the timed steps
    ms_per_cycle = None
    if hasattr(torch.cuda, "_sleep"):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        torch.cuda._sleep(1 << 22)
        c1.record(stream)
        torch.cuda.synchronize()
        ms_per_cycle = max(c0.elapsed_time(c1), 1e-3) / (1 << 22)

    # W warm-up steps, continued until the GPU has run the step for at least
    # --min-warmup-s seconds: its clocks take a few hundred ms of load to reach
    # their steady level, and a cold start reads up to 25 % slow.  The warm-up
    # steps are evicted like the timed ones, so that every dispatch of the
    # step's kernels (the ones a kernel trace of this command averages over)
    # starts from the same cache state.
    # The shader clock is read (rocm-smi, about a quarter of a second) on a
    # host thread in the second half of the warm-up, while the GPU is loaded
    # and its clocks have settled.  Read between the warm-up and the timed
    # steps, it left the GPU idle long enough for its clocks to drop, and the
    # timed steps then ran up to 15 % slow
    clk = {}
    clk_thread = threading.Thread(target=lambda: clk.update(mhz=gpu_sclk_mhz()), daemon=True)
    t_w = time.perf_counter()
    n_warm = 0
    for _ in range(args.warmup):
        evict_pass(n_warm)
        step()
        n_warm += 1
    torch.cuda.synchronize()
    while args.min_warmup_s > 0:   # 0: exactly W steps (counter runs), no clock reading
        elapsed = time.perf_counter() - t_w
        if clk_thread.ident is None and elapsed >= 0.5 * args.min_warmup_s:
            clk_thread.start()
        if elapsed >= args.min_warmup_s and clk_thread.ident is not None and not clk_thread.is_alive():
            break
        for _ in range(10):
            evict_pass(n_warm)
            step()
            n_warm += 1
        torch.cuda.synchronize()
    if clk_thread.ident is not None:
        clk_thread.join()
    clk_before = clk.get("mhz")
    warm_s = time.perf_counter() - t_w

    # host time to issue one step (eviction included), after a first pass that
    # loads the eviction kernels, and the step's GPU time (wall time to the
    # synchronisation, which the GPU bounds when it is the slower side)
    evict_pass(0)
    step()
    torch.cuda.synchronize()
    t_h = time.perf_counter()
    for i in range(10):
        evict_pass(i)
        step()
    host_ms = (time.perf_counter() - t_h) * 1000.0 / 10
    torch.cuda.synchronize()
    gpu_ms = (time.perf_counter() - t_h) * 1000.0 / 10
    # The timed steps are queued behind a spin kernel, so that no event
    # interval contains GPU idle time spent waiting for the host.  When a
    # step's GPU time is well above the host's time to issue it (the eviction
    # alone takes ~0.25 ms), a head start of a few steps' issue time keeps the
    # host ahead; otherwise the hold covers issuing every step.  A longer hold
    # than needed costs: after a few ms of a near-idle GPU the timed steps'
    # kernels ran up to 8 % slower than in the warm-up.
    hold_cycles, hold_ms = 0, 0.0
    if ms_per_cycle:
        if host_ms < 0.5 * gpu_ms:
            hold_ms = 3.0 * host_ms + 0.05
        else:
            hold_ms = min(2.0 * args.steps * host_ms + 2.0, 500.0)
        hold_cycles = int(hold_ms / ms_per_cycle)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if hold_cycles:
        torch.cuda._sleep(hold_cycles)
    for i in range(args.steps):
        evict_pass(i)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk_after = gpu_sclk_mhz()
    step_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    launch_ms = sum(step_ms) / args.steps
    ms_per_step = launch_ms
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                            step_ms[len(step_ms) // 2])

    tokens = info["tokens"]
    value = tokens / (ms_per_step / 1000.0)
    gbs = info["bytes_alg"] / (launch_ms / 1000.0) / 1e9
    tflops = info["flop_alg"] / (launch_ms / 1000.0) / 1e12
    peak_f = PEAK_BF16_TFLOPS if info["dtype"] == "bf16" else PEAK_FP32_TFLOPS
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(info["kernel"], info["workload"]),
                "kernel": info["kernel"], "launch_ms": round(launch_ms, 5),
                "bytes_alg_per_launch": info["bytes_alg"]}
    if info["flop_alg"] / peak_f / 1e12 > info["bytes_alg"] / PEAK_HBM_GBS / 1e9:
        roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_f,
                         "unit": "TFLOP/s", "frac": round(tflops / peak_f, 4)})

    cfg = {k: info[k] for k in info if k not in ("inputs", "bytes_alg", "flop_alg", "kernel", "tokens", "cpu_sample")}
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
        "warmup_s": round(warm_s, 3), "ms_per_step": round(ms_per_step, 5),
        "ms_median": round(median_ms, 5), "ms_min": round(step_ms[0], 5),
        "wall_ms_per_step": round(wall * 1000.0 / args.steps, 5), "host_ms_per_step": round(host_ms, 4),
        "hold_ms": round(hold_ms, 3),
        "evict": mode,
        "sclk_mhz": {"before": clk_before, "after": clk_after},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": info["dtype"], "data": "synthetic (seeded Gaussian inputs of the workload's shapes)",
        "config": cfg,
        "tflops": round(tflops, 3), "mfma_frac": round(tflops / peak_f, 5),
        "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(info)
        if cb is not None:
            res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
