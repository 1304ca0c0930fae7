// bwd.hip -- backward pass of the token-causal fast-weight forward (beta = 0).
//
// [P1] ("KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다",
// aitrends.kr/articles/4698), paragraphs on the state-matrix update and the
// one-step output identity, give the forward rule S_t = S_{t-1} + eta_t k_t^T v_t,
// o_t = q_t S_t; [P4] ("RNN의 기억을 작은 모델로 바꾼다면: Test-Time Training
// 읽기", ariser.io), section on the two kinds of weights, trains the outer
// model through these updates.  The backward pass is the chain rule of that
// recurrence.  With D_t = dS_final + sum_{u >= t} q_u^T do_u (the adjoint of
// the state, accumulated from the end of the sequence):
//
//     dq_t   = do_t S_t^T          = do_t S0^T + sum_{s <= t} eta_s (do_t . v_s) k_s
//     P_t    = k_t D_t             = k_t dS_final + sum_{u >= t} (k_t . q_u) do_u
//     R_t    = v_t D_t^T           = v_t dS_final^T + sum_{u >= t} (v_t . do_u) q_u
//     dv_t   = eta_t P_t,  dk_t = eta_t R_t,  deta_t = P_t . v_t,  dS0 = D_0.
//
// Each of dq, P and R is a token-causal linear-attention forward of its own:
//     dq : queries do,  keys v,  values k,  rate eta, initial state S0^T
//     P  : queries k,   keys q,  values do, rate 1,   initial state dS_final,
//          with time reversed (u >= t is causal from the end)
//     R  : queries v,   keys do, values q,  rate 1,   initial state dS_final^T,
//          time reversed
// so the backward runs the forward kernels three times (time reversal is a
// negative L stride with the base at the last token; the transposed states
// are read in place; the R pass scales its output rows by eta on the way
// out) and one elementwise pass over 16-byte vectors that scales P by eta
// and forms deta.  The final state of the P pass is D_0 = dS0.
#include "common.h"
#include "internal.h"

namespace ttt {

namespace {

// 16-byte vectors of a row of T
template <typename T> struct Vec;
template <> struct Vec<float> {
    static constexpr int N = 4;
    typedef f32x4 raw;
    static TTT_DEV void unpack(const raw& r, float* x) { for (int i = 0; i < 4; ++i) x[i] = r[i]; }
    static TTT_DEV raw pack(const float* x) { return raw{x[0], x[1], x[2], x[3]}; }
};
template <> struct Vec<bf16_t> {
    static constexpr int N = 8;
    typedef u32x4 raw;
    static TTT_DEV void unpack(const raw& r, float* x) {
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r[i] << 16);
            x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
        }
    }
    static TTT_DEV raw pack(const float* x) {
        return raw{pack2bf(x[0], x[1]), pack2bf(x[2], x[3]), pack2bf(x[4], x[5]), pack2bf(x[6], x[7])};
    }
};

// dv = eta P in place and deta = P . v: one thread per 16-byte vector of P;
// the GV threads of a row (GV = dv / vector length, a power of two that
// divides 64) sit in one wave and sum their partial dot products by shuffles
template <typename T, int GV>
__global__ __launch_bounds__(256) void bwd_scale_dv_kernel(BwdParams p) {
    typedef Vec<T> VT;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nvec = (int64_t)p.B * p.H * p.L * GV;
    float dot = 0.f;
    const int64_t row = i / GV;
    if (i < nvec) {
        typename VT::raw* P = reinterpret_cast<typename VT::raw*>(p.dv) + i;
        const typename VT::raw vr = reinterpret_cast<const typename VT::raw*>(p.v)[i];
        const float eta = p.eta ? p.eta[row] : p.eta_scalar;
        float x[VT::N], y[VT::N];
        VT::unpack(*P, x);
        VT::unpack(vr, y);
#pragma unroll
        for (int e = 0; e < VT::N; ++e) {
            dot += x[e] * y[e];
            x[e] *= eta;
        }
        *P = VT::pack(x);
    }
#pragma unroll
    for (int o = GV / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    if (p.deta && i < nvec && (i % GV) == 0) p.deta[row] = dot;
}

template <typename T>
hipError_t launch_epilogue(const BwdParams& b, hipStream_t s) {
    constexpr int N = Vec<T>::N;
    const int64_t rows = (int64_t)b.B * b.H * b.L;
    const int gv = b.dv_dim / N;
    const dim3 block(256), gridv((unsigned)((rows * gv + 255) / 256));
    switch (gv) {
        case 4: hipLaunchKernelGGL((bwd_scale_dv_kernel<T, 4>), gridv, block, 0, s, b); break;
        case 8: hipLaunchKernelGGL((bwd_scale_dv_kernel<T, 8>), gridv, block, 0, s, b); break;
        case 16: hipLaunchKernelGGL((bwd_scale_dv_kernel<T, 16>), gridv, block, 0, s, b); break;
        case 32: hipLaunchKernelGGL((bwd_scale_dv_kernel<T, 32>), gridv, block, 0, s, b); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// contiguous [B, H, L, d] tensor, optionally walked from its last token
void set_seq(int64_t* st, const void** ptr, const void* base, int H, int L, int d, size_t es, bool rev) {
    st[0] = (int64_t)H * L * d;
    st[1] = (int64_t)L * d;
    st[2] = rev ? -(int64_t)d : (int64_t)d;
    *ptr = rev ? static_cast<const char*>(base) + (size_t)(L - 1) * d * es : base;
}

TcParams pass_params(const BwdParams& b) {
    TcParams p{};
    p.B = b.B;
    p.H = b.H;
    p.L = b.L;
    p.chunk = 64;
    p.beta = 0.f;
    p.workspace = b.workspace;
    return p;
}

}  // namespace

bool bwd_supported(int dtype, int dk, int dv) {
    return tc_fwd_supported(dtype, MODE_TC, dk, dv, 64) && tc_fwd_supported(dtype, MODE_TC, dv, dk, 64);
}

size_t bwd_workspace(int B, int H, int L, int dk, int dv, int dtype) {
    if (dtype != 1) return 0;
    size_t w = 0;
    if (tcb_supported(dtype, dv, dk)) w = tcb_workspace(B, H, L, dv, dk, MODE_TC, 64);   // dq and R
    if (tcb_supported(dtype, dk, dv)) {
        const size_t wp = tcb_workspace(B, H, L, dk, dv, MODE_TC, 64);                  // P
        if (wp > w) w = wp;
    }
    return w;
}

hipError_t launch_bwd(const BwdParams& b, hipStream_t s) {
    if (!bwd_supported(b.dtype, b.dk_dim, b.dv_dim)) return hipErrorInvalidValue;
    const size_t es = b.dtype == 1 ? 2 : 4;
    const int H = b.H, L = b.L, dk = b.dk_dim, dv = b.dv_dim;
    hipError_t e;

    // dq: queries do, keys v, values k (rate eta), state S0^T
    {
        TcParams p = pass_params(b);
        p.dk = dv;
        p.dv = dk;
        set_seq(p.qs, &p.q, b.dout, H, L, dv, es, false);
        set_seq(p.ks, &p.k, b.v, H, L, dv, es, false);
        set_seq(p.vs, &p.v, b.k, H, L, dk, es, false);
        const void* o;
        set_seq(p.os, &o, b.dq, H, L, dk, es, false);
        p.out = const_cast<void*>(o);
        p.eta = b.eta;
        p.es[0] = (int64_t)H * L;
        p.es[1] = L;
        p.es[2] = 1;
        p.eta_scalar = b.eta_scalar;
        p.S0 = b.S0;
        p.s0s[0] = (int64_t)H * dk * dv;
        p.s0s[1] = (int64_t)dk * dv;
        p.s0_trans = 1;
        if ((e = launch_tc_fwd(p, b.dtype, MODE_TC, s)) != hipSuccess) return e;
    }
    // P (into dv): queries k, keys q, values do, time reversed, state dS_final;
    // its final state is D_0 = dS0
    {
        TcParams p = pass_params(b);
        p.dk = dk;
        p.dv = dv;
        set_seq(p.qs, &p.q, b.k, H, L, dk, es, true);
        set_seq(p.ks, &p.k, b.q, H, L, dk, es, true);
        set_seq(p.vs, &p.v, b.dout, H, L, dv, es, true);
        const void* o;
        set_seq(p.os, &o, b.dv, H, L, dv, es, true);
        p.out = const_cast<void*>(o);
        p.eta_scalar = 1.f;
        p.S0 = b.dS_final;
        p.s0s[0] = (int64_t)H * dk * dv;
        p.s0s[1] = (int64_t)dk * dv;
        p.S_final = b.dS0;
        if ((e = launch_tc_fwd(p, b.dtype, MODE_TC, s)) != hipSuccess) return e;
    }
    // R (into dk): queries v, keys do, values q, time reversed, state dS_final^T
    {
        TcParams p = pass_params(b);
        p.dk = dv;
        p.dv = dk;
        set_seq(p.qs, &p.q, b.v, H, L, dv, es, true);
        set_seq(p.ks, &p.k, b.dout, H, L, dv, es, true);
        set_seq(p.vs, &p.v, b.q, H, L, dk, es, true);
        const void* o;
        set_seq(p.os, &o, b.dk, H, L, dk, es, true);
        p.out = const_cast<void*>(o);
        p.eta_scalar = 1.f;
        p.S0 = b.dS_final;
        p.s0s[0] = (int64_t)H * dk * dv;
        p.s0s[1] = (int64_t)dk * dv;
        p.s0_trans = 1;
        // dk = eta R: the rows are scaled by eta on the way out (time reversed too)
        p.use_oscale = 1;
        p.oscale = b.eta ? b.eta + (L - 1) : nullptr;
        p.ocs[0] = (int64_t)H * L;
        p.ocs[1] = L;
        p.ocs[2] = -1;
        p.oscale_scalar = b.eta_scalar;
        if ((e = launch_tc_fwd(p, b.dtype, MODE_TC, s)) != hipSuccess) return e;
    }
    // dv = eta P, deta = P . v
    return b.dtype == 1 ? launch_epilogue<bf16_t>(b, s) : launch_epilogue<float>(b, s);
}

}  // namespace ttt
