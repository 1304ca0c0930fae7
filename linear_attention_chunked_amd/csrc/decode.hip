// decode.hip -- one recurrent token per (batch, head) with the state in HBM.
//
// [P1] ("KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다",
// aitrends.kr/articles/4698), paragraphs on the state-matrix update and on the
// one-step output identity; [P4] ("RNN의 기억을 작은 모델로 바꾼다면: Test-Time
// Training 읽기", ariser.io), sections on the inner update rule and on the
// fixed-size state.  One step of the token-causal recurrence, in place:
//     m <- beta m + eta k^T v,   S <- S + m,   o = q S   (after the update).
//
// The step is memory-bound on the state (dk x dv fp32, plus m with momentum):
// every state byte is read once and written once with 16-byte accesses.  A
// workgroup owns COLS state columns of one (b, h) (whole 512-byte rows when
// dv >= 128); q and k are staged in LDS as fp32 first.  Thread (row group rg,
// column quad cq) walks rows rg, rg + RG, ... in batches of 16: all loads of a
// batch are issued before its first update (row indexes clamped to the last
// row, so the loads carry no branch that would make the compiler wait on each
// one), then each row is updated and stored if it exists.  With momentum the
// two state streams are loaded and stored non-temporally.  The readout
// o = q S is reduced over the row groups through LDS.
#include "common.h"
#include "internal.h"

namespace ttt {

namespace {

TTT_DEV float ld1(const float* p) { return *p; }
TTT_DEV float ld1(const bf16_t* p) { return bf2f(__builtin_bit_cast(uint16_t, *p)); }
TTT_DEV f32x4 ldv4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
TTT_DEV f32x4 ldv4(const bf16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}

template <bool NT>
TTT_DEV f32x4 ld_state(const float* p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
TTT_DEV void st_state(float* p, const f32x4& v) {
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = v;
}

constexpr int DC_DKMAX = 1024;   // longest key dimension (LDS staging of q, k)
constexpr int DC_NB = 16;        // rows per thread per load batch

}  // namespace

template <typename T, bool MOM, int COLS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    constexpr int CQ = COLS / 4, RG = 256 / CQ;
    __shared__ float sq[DC_DKMAX], sk[DC_DKMAX];
    __shared__ f32x4 sRed[RG][CQ];
    const int tid = threadIdx.x, cq = tid % CQ, rg = tid / CQ;
    const int bh = blockIdx.x;
    const int col = blockIdx.y * COLS + 4 * cq;
    const int dk = p.dk, dv = p.dv;
    const bool active = col < dv;
    {
        const T* q = reinterpret_cast<const T*>(p.q) + (int64_t)bh * dk;
        const T* k = reinterpret_cast<const T*>(p.k) + (int64_t)bh * dk;
        for (int i = tid; i < dk; i += 256) {
            sq[i] = ld1(q + i);
            sk[i] = ld1(k + i);
        }
    }
    float* S = p.S + (int64_t)bh * dk * dv + col;
    float* M = MOM ? p.M + (int64_t)bh * dk * dv + col : nullptr;
    const float eta = p.eta ? p.eta[bh] : p.eta_scalar;
    __syncthreads();

    f32x4 acc = zero4();
    if (active) {
        const f32x4 v4 = ldv4(reinterpret_cast<const T*>(p.v) + (int64_t)bh * dv + col);
        for (int r0 = rg; r0 < dk; r0 += RG * DC_NB) {
            f32x4 s4[DC_NB], m4[MOM ? DC_NB : 1];
#pragma unroll
            for (int u = 0; u < DC_NB; ++u) {
                const int i = min(r0 + RG * u, dk - 1);
                s4[u] = ld_state<MOM>(S + (int64_t)i * dv);
                if (MOM) m4[u] = ld_state<MOM>(M + (int64_t)i * dv);
            }
#pragma unroll
            for (int u = 0; u < DC_NB; ++u) {
                const int i = r0 + RG * u;
                if (i < dk) {
                    const f32x4 g = (eta * sk[i]) * v4;
                    if (MOM) {
                        m4[u] = p.beta * m4[u] + g;
                        s4[u] += m4[u];
                        st_state<MOM>(M + (int64_t)i * dv, m4[u]);
                    } else {
                        s4[u] += g;
                    }
                    st_state<MOM>(S + (int64_t)i * dv, s4[u]);
                    acc += sq[i] * s4[u];
                }
            }
        }
    }
    sRed[rg][cq] = acc;
    __syncthreads();
    if (rg == 0 && active) {
        f32x4 o = zero4();
#pragma unroll
        for (int r = 0; r < RG; ++r) o += sRed[r][cq];
        st4(reinterpret_cast<T*>(p.out) + (int64_t)bh * dv + col, o);
    }
}

bool decode_supported(int dtype, int dk, int dv) {
    return (dtype == 0 || dtype == 1) && dk >= 1 && dk <= DC_DKMAX && dv >= 4 && dv % 4 == 0;
}

template <typename T, int COLS>
static void launch_cols(const DecodeParams& p, hipStream_t s) {
    const dim3 grid(p.B * p.H, (p.dv + COLS - 1) / COLS), block(256);
    if (p.beta != 0.f) hipLaunchKernelGGL((decode_kernel<T, true, COLS>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((decode_kernel<T, false, COLS>), grid, block, 0, s, p);
}

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s) {
    if (!decode_supported(dtype, p.dk, p.dv)) return hipErrorInvalidValue;
    const bool wide = p.dv >= 128;   // whole 512-byte rows per workgroup
    if (dtype == 1) wide ? launch_cols<bf16_t, 128>(p, s) : launch_cols<bf16_t, 64>(p, s);
    else wide ? launch_cols<float, 128>(p, s) : launch_cols<float, 64>(p, s);
    return hipGetLastError();
}

}  // namespace ttt
