// api.cpp -- the extern "C" boundary: argument validation and dispatch.
//
// Validation is complete before the first HIP call, so a rejected call has
// enqueued nothing.  No allocation, no global mutable state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <initializer_list>
#include <utility>

#include "../../include/ttt.h"
#include "internal.h"

namespace {

using ttt::MODE_CC;
using ttt::MODE_MOM;
using ttt::MODE_TC;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == TTT_BF16 ? 2 : 4; }

// [lo, hi) byte range touched by a [B,H,L,d] strided tensor
void span(const void* base, const int64_t* st, int B, int H, int L, int d, size_t es,
          uintptr_t* lo, uintptr_t* hi) {
    const int64_t last = (int64_t)(B - 1) * st[0] + (int64_t)(H - 1) * st[1] + (int64_t)(L - 1) * st[2] + d;
    *lo = reinterpret_cast<uintptr_t>(base);
    *hi = *lo + (uintptr_t)last * es;
}

bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

ttt_status_t check_tensor(const void* p, const int64_t* st, int d, int dtype) {
    if (!p) return TTT_ERR_NULL;
    if (!aligned16(p)) return TTT_ERR_ALIGN;
    const int64_t vec = 16 / (int64_t)esize(dtype);
    for (int i = 0; i < 3; ++i) {
        if (st[i] < 0) return TTT_ERR_SHAPE;
        if (st[i] % vec != 0) return TTT_ERR_ALIGN;
    }
    if (st[2] < d) return TTT_ERR_SHAPE;  // rows must not overlap
    if (st[2] >= (int64_t(1) << 23)) return TTT_ERR_SHAPE;  // in-chunk row offsets use 24-bit products
    return TTT_OK;
}

// the large-fast-weight chunk-causal path (needs a snapshot workspace)
bool use_inplace(const ttt_fwd_args* a, int mode) {
    return mode == MODE_CC && !ttt::tc_fwd_supported(a->dtype, mode, a->dk, a->dv, a->chunk);
}

size_t workspace_bytes_for(const ttt_fwd_args* a, int mode) {
    if (use_inplace(a, mode)) return ttt::inplace_workspace(a->B, a->H, a->L, a->dk, a->dv, a->chunk);
    if (ttt::tcb_supported(a->dtype, a->dk, a->dv))
        return ttt::tcb_workspace(a->B, a->H, a->L, a->dk, a->dv, mode, a->chunk);
    return 0;
}

// sizes, dtype, mode and scalars only (no pointers): also serves the workspace query
ttt_status_t validate_shapes(const ttt_fwd_args* a, int* mode_out) {
    if (!a) return TTT_ERR_NULL;
    if (a->dtype != TTT_F32 && a->dtype != TTT_BF16) return TTT_ERR_DTYPE;
    if (a->B < 1 || a->H < 1 || a->L < 1 || a->dk < 1 || a->dv < 1 || a->chunk < 1)
        return TTT_ERR_SHAPE;
    if (a->mode != TTT_TOKEN_CAUSAL && a->mode != TTT_CHUNK_CAUSAL) return TTT_ERR_VALUE;
    if (!(a->beta >= 0.f && a->beta < 1.f)) return TTT_ERR_VALUE;
    if (a->mode == TTT_CHUNK_CAUSAL && a->beta != 0.f) return TTT_ERR_VALUE;
    const int mode = (a->mode == TTT_CHUNK_CAUSAL) ? MODE_CC : (a->beta != 0.f ? MODE_MOM : MODE_TC);
    if (!ttt::tc_fwd_supported(a->dtype, mode, a->dk, a->dv, a->chunk) &&
        !(mode == MODE_CC && ttt::inplace_supported(a->dtype, a->dk, a->dv, a->chunk)))
        return TTT_ERR_UNSUPPORTED;
    *mode_out = mode;
    return TTT_OK;
}

ttt_status_t validate_fwd(const ttt_fwd_args* a, int* mode_out) {
    ttt_status_t s = validate_shapes(a, mode_out);
    if (s != TTT_OK) return s;
    if ((s = check_tensor(a->q, a->q_stride, a->dk, a->dtype)) != TTT_OK) return s;
    if ((s = check_tensor(a->k, a->k_stride, a->dk, a->dtype)) != TTT_OK) return s;
    if ((s = check_tensor(a->v, a->v_stride, a->dv, a->dtype)) != TTT_OK) return s;
    if ((s = check_tensor(a->out, a->out_stride, a->dv, a->dtype)) != TTT_OK) return s;
    if (a->eta) {
        for (int i = 0; i < 3; ++i)
            if (a->eta_stride[i] < 0) return TTT_ERR_SHAPE;
        if (a->eta_stride[2] >= (int64_t(1) << 23)) return TTT_ERR_SHAPE;
    }
    if (a->S0 && (a->S0_stride[0] < 0 || a->S0_stride[1] < 0)) return TTT_ERR_SHAPE;
    if (a->M0 && (a->M0_stride[0] < 0 || a->M0_stride[1] < 0)) return TTT_ERR_SHAPE;
    // out must not overlap an input
    uintptr_t o0, o1, x0, x1;
    const size_t es = esize(a->dtype);
    span(a->out, a->out_stride, a->B, a->H, a->L, a->dv, es, &o0, &o1);
    span(a->q, a->q_stride, a->B, a->H, a->L, a->dk, es, &x0, &x1);
    if (overlap(o0, o1, x0, x1)) return TTT_ERR_ALIAS;
    span(a->k, a->k_stride, a->B, a->H, a->L, a->dk, es, &x0, &x1);
    if (overlap(o0, o1, x0, x1)) return TTT_ERR_ALIAS;
    span(a->v, a->v_stride, a->B, a->H, a->L, a->dv, es, &x0, &x1);
    if (overlap(o0, o1, x0, x1)) return TTT_ERR_ALIAS;
    const size_t need = workspace_bytes_for(a, *mode_out);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return TTT_ERR_WORKSPACE;
    if (a->workspace && !aligned16(a->workspace)) return TTT_ERR_ALIGN;
    return TTT_OK;
}



ttt_status_t from_hip(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_HIP; }

}  // namespace

extern "C" {

const char* ttt_status_string(ttt_status_t s) {
    switch (s) {
        case TTT_OK: return "ok";
        case TTT_ERR_NULL: return "required pointer is NULL";
        case TTT_ERR_SHAPE: return "size or stride out of range";
        case TTT_ERR_DTYPE: return "unknown dtype";
        case TTT_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case TTT_ERR_UNSUPPORTED: return "no kernel for these dimensions";
        case TTT_ERR_WORKSPACE: return "workspace missing or too small";
        case TTT_ERR_HIP: return "HIP runtime or launch error";
        case TTT_ERR_ALIAS: return "output overlaps an input";
        case TTT_ERR_VALUE: return "scalar argument out of range";
    }
    return "unknown status";
}

size_t ttt_fwd_args_size(void) { return sizeof(ttt_fwd_args); }

ttt_status_t ttt_fwd_workspace_size(const ttt_fwd_args* a, size_t* bytes) {
    if (!a || !bytes) return TTT_ERR_NULL;
    int mode = 0;
    const ttt_status_t s = validate_shapes(a, &mode);
    if (s != TTT_OK) return s;
    *bytes = workspace_bytes_for(a, mode);
    return TTT_OK;
}

ttt_status_t ttt_fwd_chunked(const ttt_fwd_args* a) {
    int mode = 0;
    ttt_status_t s = validate_fwd(a, &mode);
    if (s != TTT_OK) return s;
    ttt::TcParams p{};
    std::memset(&p, 0, sizeof(p));
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.out = a->out;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = a->q_stride[i];
        p.ks[i] = a->k_stride[i];
        p.vs[i] = a->v_stride[i];
        p.os[i] = a->out_stride[i];
        p.es[i] = a->eta ? a->eta_stride[i] : 0;
    }
    p.eta = a->eta;
    p.eta_scalar = a->eta_scalar;
    p.beta = a->beta;
    p.S0 = a->S0;
    p.s0s[0] = a->S0_stride[0];
    p.s0s[1] = a->S0_stride[1];
    p.M0 = a->M0;
    p.m0s[0] = a->M0_stride[0];
    p.m0s[1] = a->M0_stride[1];
    p.S_final = a->S_final;
    p.M_final = (mode == MODE_MOM) ? a->M_final : nullptr;
    p.B = a->B;
    p.H = a->H;
    p.L = a->L;
    p.dk = a->dk;
    p.dv = a->dv;
    p.chunk = a->chunk;
    p.workspace = a->workspace;
    const hipStream_t st = reinterpret_cast<hipStream_t>(a->stream);
    if (use_inplace(a, mode)) return from_hip(ttt::launch_inplace(p, a->workspace, st));
    return from_hip(ttt::launch_tc_fwd(p, a->dtype, mode, st));
}

ttt_status_t ttt_chunk_state_scan(int32_t B, int32_t H, int32_t L, int32_t chunk, int32_t dk,
                                  int32_t dv, const float* dS, const float* dM, float beta,
                                  const float* S0, const float* M0, float* S_excl, float* M_excl,
                                  float* S_final, float* M_final, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (B < 1 || H < 1 || L < 1 || chunk < 1 || dk < 1 || dv < 1) return TTT_ERR_SHAPE;
    if (((int64_t)dk * dv) % 4 != 0) return TTT_ERR_UNSUPPORTED;
    if (!(beta >= 0.f && beta < 1.f)) return TTT_ERR_VALUE;
    if (!dS) return TTT_ERR_NULL;
    if (beta != 0.f && !dM) return TTT_ERR_NULL;
    const void* ptrs[] = {dS, dM, S0, M0, S_excl, M_excl, S_final, M_final};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return TTT_ERR_ALIGN;
    return from_hip(ttt::launch_state_scan(B, H, L, chunk, dk, dv, dS, beta != 0.f ? dM : nullptr, beta,
                                           S0, beta != 0.f ? M0 : nullptr, S_excl, M_excl, S_final,
                                           M_final, reinterpret_cast<hipStream_t>(stream)));
}

ttt_status_t ttt_dual_form_fwd(int32_t B, int32_t H, int32_t L, int32_t d, int32_t dv,
                               int32_t minibatch, int32_t dtype, const void* q, const void* k,
                               const void* v, const float* W0, int64_t W0_stride_bh, float eta,
                               void* out, float* W_final, void* workspace, size_t workspace_bytes,
                               void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_ERR_DTYPE;
    if (B < 1 || H < 1 || L < 1 || d < 1 || dv < 1 || minibatch < 1 || W0_stride_bh < 0)
        return TTT_ERR_SHAPE;
    if (!q || !k || !v || !W0 || !out) return TTT_ERR_NULL;
    const void* ptrs[] = {q, k, v, W0, out, W_final};
    for (const void* x : ptrs)
        if (x && !aligned16(x)) return TTT_ERR_ALIGN;
    if (!ttt::dual_supported(dtype, d, dv, minibatch)) return TTT_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + (size_t)B * H * L * dv * es;
    const struct { const void* p; size_t n; } ins[] = {
        {q, (size_t)B * H * L * d * es}, {k, (size_t)B * H * L * d * es}, {v, (size_t)B * H * L * dv * es}};
    for (const auto& in : ins) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(in.p);
        if (overlap(o0, o1, a0, a0 + in.n)) return TTT_ERR_ALIAS;
    }
    ttt::DualParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.W0 = W0;
    p.W0_stride = W0_stride_bh;
    p.W_final = W_final;
    p.eta = eta;
    p.B = B;
    p.H = H;
    p.L = L;
    p.d = d;
    p.dv = dv;
    p.minibatch = minibatch;
    return from_hip(ttt::launch_dual_fwd(p, dtype, reinterpret_cast<hipStream_t>(stream)));
}

ttt_status_t ttt_bwd_workspace_size(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t dtype,
                                    float beta, size_t* bytes) {
    if (!bytes) return TTT_ERR_NULL;
    if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_ERR_DTYPE;
    if (B < 1 || H < 1 || L < 1 || dk < 1 || dv < 1) return TTT_ERR_SHAPE;
    if (!(beta >= 0.f && beta < 1.f)) return TTT_ERR_VALUE;
    if (!ttt::bwd_supported(dtype, dk, dv)) return TTT_ERR_UNSUPPORTED;
    *bytes = ttt::bwd_workspace(B, H, L, dk, dv, dtype, beta != 0.f);
    return TTT_OK;
}

ttt_status_t ttt_bwd_chunked(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t dtype,
                             const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                             float beta, const float* S0, const float* M0, const void* dout,
                             const float* dS_final, const float* dM_final, void* dq, void* dk_out, void* dv_out,
                             float* deta, float* dS0, float* dM0, void* workspace, size_t workspace_bytes,
                             void* stream) {
    size_t need = 0;
    const ttt_status_t st = ttt_bwd_workspace_size(B, H, L, dk, dv, dtype, beta, &need);
    if (st != TTT_OK) return st;
    if (!q || !k || !v || !dout || !dq || !dk_out || !dv_out) return TTT_ERR_NULL;
    if (need > 0 && (!workspace || workspace_bytes < need)) return TTT_ERR_WORKSPACE;
    const size_t es = esize(dtype);
    const size_t nq = (size_t)B * H * L * dk * es, nv = (size_t)B * H * L * dv * es;
    const size_t ne = (size_t)B * H * L * 4, ns = (size_t)B * H * dk * dv * 4;
    struct Buf { const void* p; size_t n; };
    const Buf ins[] = {{q, nq}, {k, nq}, {v, nv}, {dout, nv}, {eta, ne}, {S0, ns}, {M0, ns}, {dS_final, ns},
                       {dM_final, ns}};
    const Buf outs[] = {{dq, nq}, {dk_out, nq}, {dv_out, nv}, {deta, ne}, {dS0, ns}, {dM0, ns}, {workspace, need}};
    for (const Buf& b : ins)
        if (b.p && !aligned16(b.p)) return TTT_ERR_ALIGN;
    for (const Buf& b : outs)
        if (b.p && !aligned16(b.p)) return TTT_ERR_ALIGN;
    // outputs overlap neither the inputs nor each other
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        if (!outs[i].p || outs[i].n == 0) continue;
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(outs[i].p), a1 = a0 + outs[i].n;
        for (const Buf& b : ins) {
            if (!b.p) continue;
            const uintptr_t b0 = reinterpret_cast<uintptr_t>(b.p);
            if (overlap(a0, a1, b0, b0 + b.n)) return TTT_ERR_ALIAS;
        }
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j) {
            if (!outs[j].p || outs[j].n == 0) continue;
            const uintptr_t b0 = reinterpret_cast<uintptr_t>(outs[j].p);
            if (overlap(a0, a1, b0, b0 + outs[j].n)) return TTT_ERR_ALIAS;
        }
    }
    ttt::BwdParams p;
    std::memset(&p, 0, sizeof(p));
    p.B = B;
    p.H = H;
    p.L = L;
    p.dk_dim = dk;
    p.dv_dim = dv;
    p.dtype = dtype;
    p.q = q;
    p.k = k;
    p.v = v;
    p.eta = eta;
    p.eta_scalar = eta_scalar;
    p.beta = beta;
    p.S0 = S0;
    p.M0 = beta != 0.f ? M0 : nullptr;
    p.dout = dout;
    p.dS_final = dS_final;
    p.dM_final = beta != 0.f ? dM_final : nullptr;
    p.dq = dq;
    p.dk = dk_out;
    p.dv = dv_out;
    p.deta = deta;
    p.dS0 = dS0;
    p.dM0 = dM0;
    p.workspace = workspace;
    return from_hip(ttt::launch_bwd(p, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// the output span [o, o + no) overlaps none of the inputs
bool disjoint(const void* o, size_t no, std::initializer_list<std::pair<const void*, size_t>> ins) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(o), a1 = a0 + no;
    for (const auto& in : ins) {
        if (!in.first) continue;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(in.first);
        if (overlap(a0, a1, b0, b0 + in.second)) return false;
    }
    return true;
}
constexpr int kMaxConvTaps = 16;
}  // namespace

ttt_status_t ttt_inplace_gated_input(int32_t T, int32_t d_model, int32_t d_ff, const void* X, const void* Wg,
                                     const void* Wu, void* Z, void* stream) {
    if (T < 1 || d_model < 1 || d_ff < 1) return TTT_ERR_SHAPE;
    if (!X || !Wg || !Wu || !Z) return TTT_ERR_NULL;
    if (!aligned16(X) || !aligned16(Wg) || !aligned16(Wu) || !aligned16(Z)) return TTT_ERR_ALIGN;
    if (!ttt::fe_gemm_supported(d_model, 2 * d_ff)) return TTT_ERR_UNSUPPORTED;
    const size_t nx = (size_t)T * d_model * 2, nw = (size_t)d_ff * d_model * 2, nz = (size_t)T * d_ff * 2;
    if (!disjoint(Z, nz, {{X, nx}, {Wg, nw}, {Wu, nw}})) return TTT_ERR_ALIAS;
    ttt::FeGemmParams p{};
    p.A0 = Wg;
    p.A1 = Wu;
    p.B = X;
    p.out = Z;
    p.arows = 2 * d_ff;
    p.K = d_model;
    p.T = T;
    p.ldb = d_model;
    p.ldo = d_ff;
    return from_hip(ttt::launch_fe_gemm(p, true, reinterpret_cast<hipStream_t>(stream)));
}

ttt_status_t ttt_inplace_lm_target_workspace_size(int32_t B, int32_t L, int32_t d_model, size_t* bytes) {
    if (!bytes) return TTT_ERR_NULL;
    if (B < 1 || L < 1 || d_model < 1) return TTT_ERR_SHAPE;
    *bytes = (size_t)B * L * d_model * 2;
    return TTT_OK;
}

ttt_status_t ttt_inplace_lm_target(int32_t B, int32_t L, int32_t d_model, int32_t taps, const void* X,
                                   const float* conv_w, const void* Wv, void* Vhat, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (B < 1 || L < 1 || d_model < 1) return TTT_ERR_SHAPE;
    if (taps < 1 || taps > kMaxConvTaps) return TTT_ERR_VALUE;
    if (!X || !conv_w || !Wv || !Vhat) return TTT_ERR_NULL;
    if (!aligned16(X) || !aligned16(conv_w) || !aligned16(Wv) || !aligned16(Vhat)) return TTT_ERR_ALIGN;
    if (!ttt::fe_gemm_supported(d_model, d_model)) return TTT_ERR_UNSUPPORTED;
    const size_t nx = (size_t)B * L * d_model * 2;
    if (!workspace || workspace_bytes < nx) return TTT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TTT_ERR_ALIGN;
    const size_t nw = (size_t)d_model * d_model * 2, nc = (size_t)taps * d_model * 4;
    if (!disjoint(Vhat, nx, {{X, nx}, {conv_w, nc}, {Wv, nw}, {workspace, nx}})) return TTT_ERR_ALIAS;
    if (!disjoint(workspace, nx, {{X, nx}, {conv_w, nc}, {Wv, nw}})) return TTT_ERR_ALIAS;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    ttt::FeConvParams c{};
    c.X = X;
    c.w = conv_w;
    c.Y = workspace;
    c.B = B;
    c.L = L;
    c.d = d_model;
    c.K = taps;
    hipError_t e = ttt::launch_fe_conv(c, st);
    if (e != hipSuccess) return from_hip(e);
    ttt::FeGemmParams p{};
    p.A0 = Wv;
    p.A1 = nullptr;
    p.B = workspace;
    p.out = Vhat;
    p.arows = d_model;
    p.K = d_model;
    p.T = B * L;
    p.ldb = d_model;
    p.ldo = d_model;
    return from_hip(ttt::launch_fe_gemm(p, false, st));
}

ttt_status_t ttt_inplace_clip_eta_workspace_size(int32_t B, int32_t L, int32_t chunk, size_t* bytes) {
    if (!bytes) return TTT_ERR_NULL;
    if (B < 1 || L < 1 || chunk < 1) return TTT_ERR_SHAPE;
    *bytes = (size_t)B * ((L + chunk - 1) / chunk) * ttt::fe_gram_pairs(chunk) * sizeof(float);
    return TTT_OK;
}

ttt_status_t ttt_inplace_clip_eta(int32_t B, int32_t L, int32_t d_ff, int32_t d_model, int32_t chunk, const void* Z,
                                  const void* Vhat, float eta, float tau, float* eta_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    size_t need = 0;
    ttt_status_t s = ttt_inplace_clip_eta_workspace_size(B, L, chunk, &need);
    if (s != TTT_OK) return s;
    if (d_ff < 1 || d_model < 1) return TTT_ERR_SHAPE;
    if (!(tau > 0.f) || !(eta == eta)) return TTT_ERR_VALUE;
    if (!Z || !Vhat || !eta_out) return TTT_ERR_NULL;
    if (!aligned16(Z) || !aligned16(Vhat) || !aligned16(eta_out)) return TTT_ERR_ALIGN;
    if (d_ff % 128 != 0 || d_model % 128 != 0) return TTT_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < need) return TTT_ERR_WORKSPACE;
    const size_t nz = (size_t)B * L * d_ff * 2, nv = (size_t)B * L * d_model * 2, ne = (size_t)B * L * 4;
    if (!disjoint(eta_out, ne, {{Z, nz}, {Vhat, nv}, {workspace, need}})) return TTT_ERR_ALIAS;
    if (!disjoint(workspace, need, {{Z, nz}, {Vhat, nv}})) return TTT_ERR_ALIAS;
    ttt::FeGramParams p{};
    p.Z = Z;
    p.V = Vhat;
    p.B = B;
    p.L = L;
    p.chunk = chunk;
    p.dz = d_ff;
    p.dv = d_model;
    p.eta = eta;
    p.tau = tau;
    p.partial = reinterpret_cast<float*>(workspace);
    p.eta_out = eta_out;
    return from_hip(ttt::launch_fe_clip(p, reinterpret_cast<hipStream_t>(stream)));
}

ttt_status_t ttt_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q,
                             const void* k, const void* v, const float* eta, float eta_scalar, float beta,
                             float* S, float* M, void* out, void* stream) {
    if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_ERR_DTYPE;
    if (B < 1 || H < 1 || dk < 1 || dv < 1) return TTT_ERR_SHAPE;
    if (!(beta >= 0.f && beta < 1.f)) return TTT_ERR_VALUE;
    if (!q || !k || !v || !S || !out) return TTT_ERR_NULL;
    if (beta != 0.f && !M) return TTT_ERR_NULL;
    const void* ptrs[] = {q, k, v, S, out, eta, beta != 0.f ? M : nullptr};
    for (const void* x : ptrs)
        if (x && !aligned16(x)) return TTT_ERR_ALIGN;
    if (!ttt::decode_supported(dtype, dk, dv)) return TTT_ERR_UNSUPPORTED;
    const size_t es = esize(dtype);
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + (size_t)B * H * dv * es;
    const struct { const void* p; size_t n; } ins[] = {
        {q, (size_t)B * H * dk * es}, {k, (size_t)B * H * dk * es}, {v, (size_t)B * H * dv * es},
        {S, (size_t)B * H * dk * dv * 4}, {beta != 0.f ? M : nullptr, (size_t)B * H * dk * dv * 4}};
    for (const auto& in : ins) {
        if (!in.p) continue;
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(in.p);
        if (overlap(o0, o1, a0, a0 + in.n)) return TTT_ERR_ALIAS;
    }
    if (beta != 0.f) {   // S and M are both written: they must not overlap either
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(S), m0 = reinterpret_cast<uintptr_t>(M);
        const size_t n = (size_t)B * H * dk * dv * 4;
        if (overlap(s0, s0 + n, m0, m0 + n)) return TTT_ERR_ALIAS;
    }
    ttt::DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.eta = eta;
    p.eta_scalar = eta_scalar;
    p.beta = beta;
    p.S = S;
    p.M = beta != 0.f ? M : nullptr;
    p.B = B;
    p.H = H;
    p.dk = dk;
    p.dv = dv;
    return from_hip(ttt::launch_decode(p, dtype, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// chunk length the kernels run with: a chunk longer than the sequence is
// the whole sequence (rounded up to the 128-token tiles)
int64_t swiglu_chunk(int32_t L, int32_t chunk) { return std::min<int64_t>(chunk, ((int64_t)L + 127) / 128 * 128); }
}  // namespace

ttt_status_t ttt_swiglu_workspace_size(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t m,
                                       int32_t chunk, size_t* bytes) {
    if (!bytes) return TTT_ERR_NULL;
    if (B < 1 || H < 1 || L < 1 || dk < 1 || dv < 1 || m < 1 || chunk < 1) return TTT_ERR_SHAPE;
    const int64_t C = swiglu_chunk(L, chunk);
    if (!ttt::swiglu_supported(dk, dv, m, (int)C)) return TTT_ERR_UNSUPPORTED;
    const int64_t span = std::max({(int64_t)2 * m * dk, (int64_t)dv * m, C * std::max({(int64_t)dk, (int64_t)dv,
                                                                                         (int64_t)2 * m})});
    if (span >= ((int64_t)1 << 31)) return TTT_ERR_UNSUPPORTED;
    *bytes = ttt::swiglu_workspace((int)((int64_t)B * H), dk, dv, m, (int)C);
    return TTT_OK;
}

ttt_status_t ttt_swiglu_fwd_chunked(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t m,
                                    int32_t chunk, int32_t loss, const void* q, const void* k, const void* v,
                                    const float* eta, float eta_scalar, float* W1, float* W3, float* W2,
                                    void* out, void* workspace, size_t workspace_bytes, void* stream) {
    size_t need = 0;
    const ttt_status_t st = ttt_swiglu_workspace_size(B, H, L, dk, dv, m, chunk, &need);
    if (st != TTT_OK) return st;
    if (loss != TTT_LOSS_DOT && loss != TTT_LOSS_MSE) return TTT_ERR_VALUE;
    if (!q || !k || !v || !W1 || !W3 || !W2 || !out) return TTT_ERR_NULL;
    const void* ptrs[] = {q, k, v, eta, W1, W3, W2, out};
    for (const void* x : ptrs)
        if (x && !aligned16(x)) return TTT_ERR_ALIGN;
    if (!workspace || workspace_bytes < need) return TTT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return TTT_ERR_ALIGN;
    const size_t BH = (size_t)B * H;
    const size_t nq = BH * L * dk * 2, nv = BH * L * dv * 2, ne = BH * L * 4;
    const size_t n13 = BH * m * dk * 4, n2 = BH * dv * m * 4;
    if (!disjoint(out, nv, {{q, nq}, {k, nq}, {v, nv}, {eta, ne}, {W1, n13}, {W3, n13}, {W2, n2}, {workspace, need}}))
        return TTT_ERR_ALIAS;
    if (!disjoint(W1, n13, {{q, nq}, {k, nq}, {v, nv}, {eta, ne}, {W3, n13}, {W2, n2}, {workspace, need}}))
        return TTT_ERR_ALIAS;
    if (!disjoint(W3, n13, {{q, nq}, {k, nq}, {v, nv}, {eta, ne}, {W2, n2}, {workspace, need}})) return TTT_ERR_ALIAS;
    if (!disjoint(W2, n2, {{q, nq}, {k, nq}, {v, nv}, {eta, ne}, {workspace, need}})) return TTT_ERR_ALIAS;
    if (!disjoint(workspace, need, {{q, nq}, {k, nq}, {v, nv}, {eta, ne}})) return TTT_ERR_ALIAS;
    ttt::SwParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.eta = eta;
    p.eta_scalar = eta_scalar;
    p.W1 = W1;
    p.W3 = W3;
    p.W2 = W2;
    p.out = out;
    p.workspace = workspace;
    p.BH = (int)BH;
    p.L = L;
    p.dk = dk;
    p.dv = dv;
    p.m = m;
    p.chunk = (int)swiglu_chunk(L, chunk);
    p.loss = loss;
    return from_hip(ttt::launch_swiglu(p, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
