// bwd.hip -- backward pass of the token-causal fast-weight forward.
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
//
// With momentum (m_t = beta m_{t-1} + g_t, S_t = S_{t-1} + m_t) the gradients
// of g_t are read from the adjoint of m_t,
//     A_t = sum_{u >= t} w(u - t) q_u^T do_u + c_t dS_final + beta^{L-1-t} dM_final,
//     w(n) = 1 + beta + ... + beta^n,  c_t = w(L - 1 - t),
// which, in reversed time tau = L-1-t, is the state S' of the momentum
// forward itself run on the increments q_u^T do_u.  Its start states decide
// the boundary part.  The forward reaches only the shapes const and
// beta^{tau+1} from a start state, while the boundary is
// c_t dS_final + beta^tau dM_final = dS_final / (1 - beta) + beta^tau E,
// E = dM_final - beta dS_final / (1 - beta).  Two ways in:
//   beta >= kDirectBeta: S0' = dM_final / beta and
//     M0' = (beta dS_final - (1 - beta) dM_final) / beta^2 give the whole
//     boundary (their O(1/beta) parts cancel; above the threshold the
//     cancellation costs at most a factor 1/beta^2 < 2 in the bf16 readout
//     of the first reversed chunk);
//   beta <  kDirectBeta: S0' = dS_final / (1 - beta), M0' = 0 give the
//     constant, and the decaying beta^tau E is added exactly in fp32 to the
//     rows of P and R of the last tokens where beta^tau is not negligible
//     (bwd_tail_kernel; at most ~75 tokens per sequence).  No division by
//     beta, so any beta in (0, 1) is well conditioned.
// So dq, P = k A and R = v A^T are three momentum forwards, dv = eta P,
// dk = eta R, deta = P . v as before, and with S'_f, M'_f the P pass's final
// states:
//     dS0 = (1 - beta) S'_f + beta M'_f   (the adjoint of S0: A_0 - beta A_1;
//                                          the tail term cancels in it)
//     dM0 = beta S'_f (+ beta^L E in the tail form)   (m_0 = beta M0 + g_0).
// (The gradient with respect to beta itself is not computed.)
#include "common.h"
#include <cmath>

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

// momentum above which the reversed passes take the whole boundary from
// their start states (below it: the tail correction)
constexpr float kDirectBeta = 0.75f;

// start states of the reversed passes, elementwise (NULL inputs are zero):
//   direct: S0' = dM_final / beta, M0' = (beta dS_final - (1 - beta) dM_final) / beta^2
//   tail:   S0' = dS_final / (1 - beta), M0' = 0
__global__ __launch_bounds__(256) void bwd_init_kernel(const float* dSf, const float* dMf, float beta, int direct,
                                                       float* S0p, float* M0p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float a = dSf ? dSf[i] : 0.f, c = dMf ? dMf[i] : 0.f;
    if (direct) {
        S0p[i] = c / beta;
        M0p[i] = (beta * a - (1.f - beta) * c) / (beta * beta);
    } else {
        S0p[i] = a / (1.f - beta);
        M0p[i] = 0.f;
    }
}

// The decaying boundary term of the momentum adjoint, added to the last
// `tail` tokens of every sequence (tau = L-1-t < tail):
//   which = 0:  P_t  += beta^tau k_t E          (in the dv buffer, before the epilogue)
//   which = 1:  dk_t += eta_t beta^tau v_t E^T  (after the R pass)
// with E = dM_final - beta / (1 - beta) dS_final (NULL inputs are zero).
// One workgroup per (b, h): E is staged once in LDS (row stride dv + 1, so
// the column walk of which = 1 is conflict free), then the tail tokens are
// walked in order; thread j < n_out owns output column j of every token.
constexpr int kTailMaxD = 128;   // dk, dv <= 128 (the backward's supported head sizes)
template <typename T>
__global__ __launch_bounds__(256) void bwd_tail_kernel(BwdParams p, int tail, int which) {
    __shared__ float E[kTailMaxD * (kTailMaxD + 1)];   // [dk][dv + 1]
    __shared__ float x[kTailMaxD];                     // the token's k (which 0) or v (which 1)
    const int dk = p.dk_dim, dv = p.dv_dim, ld = dv + 1;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int64_t sbase = (int64_t)bh * dk * dv;
    const float c = p.beta / (1.f - p.beta);
    for (int e = tid; e < dk * dv; e += 256) {
        const float a = p.dS_final ? p.dS_final[sbase + e] : 0.f;
        const float m = p.dM_final ? p.dM_final[sbase + e] : 0.f;
        E[(e / dv) * ld + (e % dv)] = m - c * a;
    }
    const int n_in = which == 0 ? dk : dv, n_out = which == 0 ? dv : dk;
    const T* in = static_cast<const T*>(which == 0 ? p.k : p.v);
    T* io = static_cast<T*>(which == 0 ? p.dv : p.dk);
    float bt = 1.f;   // beta^tau
    for (int tau = 0; tau < tail; ++tau, bt *= p.beta) {
        const int64_t row = (int64_t)bh * p.L + (p.L - 1 - tau);
        __syncthreads();   // E written / the previous token's x read
        for (int i = tid; i < n_in; i += 256) x[i] = (float)in[row * n_in + i];
        __syncthreads();
        if (tid < n_out) {
            float acc = 0.f;
            if (which == 0) {
                for (int i = 0; i < dk; ++i) acc += x[i] * E[i * ld + tid];
            } else {
                for (int j = 0; j < dv; ++j) acc += x[j] * E[tid * ld + j];
                acc *= p.eta ? p.eta[row] : p.eta_scalar;
            }
            const int64_t o = row * n_out + tid;
            io[o] = (T)((float)io[o] + bt * acc);
        }
    }
}

// tokens whose boundary weight beta^tau is above 2^-30 (beta in (0, 1))
int tail_tokens(float beta, int L) {
    int n = 1;
    for (double w = beta; n < L && w >= 0x1p-30; w *= beta) ++n;
    return n;
}

// dS0 = (1 - beta) S'_f + beta M'_f,  dM0 = beta S'_f + bL E, where bL =
// beta^L in the tail form when its boundary term reaches token 0 (else 0)
__global__ __launch_bounds__(256) void bwd_state_kernel(const float* Sf, const float* Mf, float beta, float bL,
                                                        const float* dSf, const float* dMf, float* dS0, float* dM0,
                                                        int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float sv = Sf[i];
    if (dS0) dS0[i] = (1.f - beta) * sv + beta * Mf[i];
    if (dM0) {
        float d = beta * sv;
        if (bL != 0.f) {
            const float a = dSf ? dSf[i] : 0.f, m = dMf ? dMf[i] : 0.f;
            d += bL * (m - beta / (1.f - beta) * a);
        }
        dM0[i] = d;
    }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = 0.f;
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
    p.beta = b.beta;
    p.workspace = b.workspace;
    return p;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// workspace: [forward passes' look-back][S0'][M0'][S'_f][M'_f] (the last
// four with momentum only)
size_t fwd_ws(int B, int H, int L, int dk, int dv, int dtype, int mode) {
    if (dtype != 1) return 0;
    size_t w = 0;
    if (tcb_supported(dtype, dv, dk)) w = tcb_workspace(B, H, L, dv, dk, mode, 64);   // dq and R
    if (tcb_supported(dtype, dk, dv)) {
        const size_t wp = tcb_workspace(B, H, L, dk, dv, mode, 64);                  // P
        if (wp > w) w = wp;
    }
    return align256(w);
}

}  // namespace

bool bwd_supported(int dtype, int dk, int dv) {
    return tc_fwd_supported(dtype, MODE_TC, dk, dv, 64) && tc_fwd_supported(dtype, MODE_TC, dv, dk, 64);
}

size_t bwd_workspace(int B, int H, int L, int dk, int dv, int dtype, bool momentum) {
    const int mode = momentum ? MODE_MOM : MODE_TC;
    size_t w = fwd_ws(B, H, L, dk, dv, dtype, mode);
    if (momentum) w += 4 * align256((size_t)B * H * dk * dv * sizeof(float));
    return w;
}

hipError_t launch_tail(const BwdParams& b, int tail, int which, hipStream_t s) {
    if (b.dk_dim > kTailMaxD || b.dv_dim > kTailMaxD) return hipErrorInvalidValue;
    if (b.dtype == 1)
        hipLaunchKernelGGL((bwd_tail_kernel<bf16_t>), dim3(b.B * b.H), dim3(256), 0, s, b, tail, which);
    else
        hipLaunchKernelGGL((bwd_tail_kernel<float>), dim3(b.B * b.H), dim3(256), 0, s, b, tail, which);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& b, hipStream_t s, hipStream_t s2) {
    if (!bwd_supported(b.dtype, b.dk_dim, b.dv_dim)) return hipErrorInvalidValue;
    const size_t es = b.dtype == 1 ? 2 : 4;
    const int H = b.H, L = b.L, dk = b.dk_dim, dv = b.dv_dim;
    const bool mom = b.beta != 0.f;
    const int mode = mom ? MODE_MOM : MODE_TC;
    const int64_t nst = (int64_t)b.B * H * dk * dv;
    const dim3 sgrid((unsigned)((nst + 255) / 256)), sblock(256);
    float *S0p = nullptr, *M0p = nullptr, *Sfp = nullptr, *Mfp = nullptr;
    // tail form: tokens that get the decaying boundary term (0: none)
    const bool direct = b.beta >= kDirectBeta;
    const int tail = (mom && !direct && (b.dS_final || b.dM_final)) ? tail_tokens(b.beta, L) : 0;
    if (mom) {
        char* w = static_cast<char*>(b.workspace) + fwd_ws(b.B, H, L, dk, dv, b.dtype, mode);
        const size_t sb = align256((size_t)nst * sizeof(float));
        S0p = reinterpret_cast<float*>(w);
        M0p = reinterpret_cast<float*>(w + sb);
        Sfp = reinterpret_cast<float*>(w + 2 * sb);
        Mfp = reinterpret_cast<float*>(w + 3 * sb);
        hipLaunchKernelGGL(bwd_init_kernel, sgrid, sblock, 0, s, b.dS_final, b.dM_final, b.beta, direct ? 1 : 0,
                           S0p, M0p, nst);
    }
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
        p.M0 = b.M0;
        p.m0s[0] = p.s0s[0];
        p.m0s[1] = p.s0s[1];
        p.s0_trans = 1;
        if ((e = launch_tc_fwd(p, b.dtype, mode, s)) != hipSuccess) return e;
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
        p.S0 = mom ? S0p : b.dS_final;
        p.s0s[0] = (int64_t)H * dk * dv;
        p.s0s[1] = (int64_t)dk * dv;
        p.M0 = M0p;
        p.m0s[0] = p.s0s[0];
        p.m0s[1] = p.s0s[1];
        p.S_final = mom ? Sfp : b.dS0;
        p.M_final = Mfp;
        if ((e = launch_tc_fwd(p, b.dtype, mode, s)) != hipSuccess) return e;
    }
    if (tail > 0 && (e = launch_tail(b, tail, 0, s)) != hipSuccess) return e;
    // dv = eta P, deta = P . v: needs only P.  With a caller's helper stream
    // it runs there beside the R pass (which writes only dk), forked from
    // `s` by an event and joined back before the call's last kernel: the R
    // pass is bound by latency and leaves wave slots free on every CU.
    // Without one it runs on `s` before the R pass.
    struct Events {   // destroyed on every return; the runtime defers it until they complete
        hipEvent_t p = nullptr, epi = nullptr;
        ~Events() {
            if (p) (void)hipEventDestroy(p);
            if (epi) (void)hipEventDestroy(epi);
        }
    } ev;
    const bool fork = s2 != nullptr && s2 != s;
    if (fork) {
        if ((e = hipEventCreateWithFlags(&ev.p, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&ev.epi, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventRecord(ev.p, s)) != hipSuccess || (e = hipStreamWaitEvent(s2, ev.p, 0)) != hipSuccess)
            return e;   // nothing is enqueued on s2 before its wait succeeded
        // from here on s2 has forked off s: every return joins it back first
        if ((e = b.dtype == 1 ? launch_epilogue<bf16_t>(b, s2) : launch_epilogue<float>(b, s2)) != hipSuccess) {
            if (hipEventRecord(ev.epi, s2) == hipSuccess) (void)hipStreamWaitEvent(s, ev.epi, 0);
            return e;
        }
        if ((e = hipEventRecord(ev.epi, s2)) != hipSuccess) return e;
    } else if ((e = b.dtype == 1 ? launch_epilogue<bf16_t>(b, s) : launch_epilogue<float>(b, s)) != hipSuccess) {
        return e;
    }
    // the join of the fork (if any), also on the error paths below
    auto join = [&](hipError_t err) {
        if (fork) {
            const hipError_t j = hipStreamWaitEvent(s, ev.epi, 0);
            if (err == hipSuccess) err = j;
        }
        return err;
    };
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
        p.S0 = mom ? S0p : b.dS_final;
        p.s0s[0] = (int64_t)H * dk * dv;
        p.s0s[1] = (int64_t)dk * dv;
        p.M0 = M0p;
        p.m0s[0] = p.s0s[0];
        p.m0s[1] = p.s0s[1];
        p.s0_trans = 1;
        // dk = eta R: the rows are scaled by eta on the way out (time reversed too)
        p.use_oscale = 1;
        p.oscale = b.eta ? b.eta + (L - 1) : nullptr;
        p.ocs[0] = (int64_t)H * L;
        p.ocs[1] = L;
        p.ocs[2] = -1;
        p.oscale_scalar = b.eta_scalar;
        if ((e = launch_tc_fwd(p, b.dtype, mode, s)) != hipSuccess) return join(e);
    }
    if (tail > 0 && (e = launch_tail(b, tail, 1, s)) != hipSuccess) return join(e);
    // beta^L E reaches dM0 when the tail covers token 0
    const float bL = (tail > 0 && tail >= L) ? (float)std::pow((double)b.beta, (double)L) : 0.f;
    if (mom && (b.dS0 || b.dM0))
        hipLaunchKernelGGL(bwd_state_kernel, sgrid, sblock, 0, s, Sfp, Mfp, b.beta, bL, b.dS_final, b.dM_final,
                           b.dS0, b.dM0, nst);
    else if (b.dM0)   // no momentum: m_0 does not depend on M0
        hipLaunchKernelGGL(bwd_zero_kernel, sgrid, sblock, 0, s, b.dM0, nst);
    return join(hipGetLastError());
}

}  // namespace ttt
