// scan.hip -- exclusive scan of per-chunk fast-weight state deltas.
//
// [P1] ("KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다",
// aitrends.kr/articles/4698), paragraph on dropping weight normalisation:
// the state updates then compose associatively and a prefix scan applies.
// [P2] ("In-Place 테스트 시점 학습", aitrends.kr/articles/40879), paragraph
// on the associative scan: chunk updates computed independently, combined by
// a prefix sum, equal to the sequential update.
//
// The chunk transition of a chunk of n tokens acts on the pair (S, m):
//     S' = S + alpha_n m + dS_c,   m' = beta^n m + dM_c,
// alpha_n = beta + ... + beta^n (derived from m_t = beta m_{t-1} + g_t,
// S_t = S_{t-1} + m_t).  It is element-wise in the dk x dv entries, so the
// state entries are independent scans: each thread owns 4 consecutive
// entries of one (b, h) and walks the chunks in order, fp32 in registers.
// Threads of a wave cover 1 KB of contiguous state per chunk, so every load
// and store is a full 16-byte coalesced access and each byte moves once.
#include "common.h"
#include "internal.h"

#include <cmath>

namespace ttt {

__global__ __launch_bounds__(256) void state_scan_kernel(
    int64_t n4, int64_t per4, int N, const f32x4* __restrict__ dS, const f32x4* __restrict__ dM,
    float alpha_full, float gamma_full, float alpha_last, float gamma_last,
    const f32x4* __restrict__ S0, const f32x4* __restrict__ M0,
    f32x4* __restrict__ S_excl, f32x4* __restrict__ M_excl,
    f32x4* __restrict__ S_final, f32x4* __restrict__ M_final, int use_m) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n4) return;
    const int64_t bh = e / per4, o = e % per4;
    f32x4 S = S0 ? S0[e] : zero4();
    f32x4 M = (use_m && M0) ? M0[e] : zero4();
    const int64_t base = bh * (int64_t)N * per4 + o;
    f32x4 d_s = dS[base];
    f32x4 d_m = use_m ? dM[base] : zero4();
    for (int c = 0; c < N; ++c) {
        const int64_t off = base + (int64_t)c * per4;
        f32x4 nd_s = zero4(), nd_m = zero4();
        if (c + 1 < N) {  // issue the next chunk's loads before this chunk's math
            nd_s = dS[off + per4];
            if (use_m) nd_m = dM[off + per4];
        }
        if (S_excl) S_excl[off] = S;
        if (use_m && M_excl) M_excl[off] = M;
        const float a = (c == N - 1) ? alpha_last : alpha_full;
        const float gm = (c == N - 1) ? gamma_last : gamma_full;
        if (use_m) {
            S = S + a * M + d_s;
            M = gm * M + d_m;
        } else {
            S = S + d_s;
        }
        d_s = nd_s;
        d_m = nd_m;
    }
    if (S_final) S_final[e] = S;
    if (use_m && M_final) M_final[e] = M;
}

// alpha_n = beta + ... + beta^n = beta (1 - beta^n) / (1 - beta), gamma_n = beta^n
// (closed forms in fp64; beta in [0, 1))
static void affine_coeffs(double beta, int n, float* alpha, float* gamma) {
    const double bn = std::pow(beta, (double)n);
    *alpha = (float)(beta * (1.0 - bn) / (1.0 - beta));
    *gamma = (float)bn;
}

hipError_t launch_state_scan(int B, int H, int L, int chunk, int dk, int dv,
                             const float* dS, const float* dM, float beta,
                             const float* S0, const float* M0,
                             float* S_excl, float* M_excl, float* S_final, float* M_final,
                             hipStream_t stream) {
    const int N = (L + chunk - 1) / chunk;
    const int64_t per4 = (int64_t)dk * dv / 4;
    const int64_t n4 = (int64_t)B * H * per4;
    const int use_m = (beta != 0.f) ? 1 : 0;
    float af, gf, al, gl;
    affine_coeffs(beta, chunk, &af, &gf);
    affine_coeffs(beta, L - (N - 1) * chunk, &al, &gl);
    const int blocks = (int)((n4 + 255) / 256);
    hipLaunchKernelGGL(state_scan_kernel, dim3(blocks), dim3(256), 0, stream, n4, per4, N,
                       (const f32x4*)dS, (const f32x4*)dM, af, gf, al, gl, (const f32x4*)S0,
                       (const f32x4*)M0, (f32x4*)S_excl, (f32x4*)M_excl, (f32x4*)S_final,
                       (f32x4*)M_final, use_m);
    return hipGetLastError();
}

}  // namespace ttt
