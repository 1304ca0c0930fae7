// frontend.hip -- the In-Place TTT front end around the chunk-causal update.
//
// [P2] ("In-Place 테스트 시점 학습: LLM을 위한 원활한 동적 적응 프레임워크",
// aitrends.kr/articles/40879):
//   * paragraph on the Gated-MLP structure: Wup and Wgate are fixed slow
//     weights; the activation Z = silu(X Wgate^T) * (X Wup^T) is what the fast
//     weight Wdown multiplies;
//   * paragraph on the LM-aligned objective: the target V-hat is built by a
//     1D convolution over the current and following tokens and a projection;
//   * paragraph on the limitations: a clipping mechanism keeps the
//     accumulated updates stable over very long contexts.
//
// Kernels:
//   fe_gemm_kernel<GATED>  C = epilogue(A B^T) with both operands K-contiguous
//                          (weights in row = output feature layout, tokens in
//                          row = token layout).  GATED: A interleaves the rows
//                          of Wgate and Wup (row 2f = gate f, 2f+1 = up f), so
//                          the two values of one output sit in consecutive
//                          accumulator registers of one lane and the epilogue
//                          silu(g) * u needs no exchange.
//   fe_conv_kernel         the depthwise look-ahead convolution (memory-bound).
//   fe_gram_kernel         per chunk and pair of 128-token tiles, the Gram
//                          products (Z Z^T) and (V V^T) on MFMA and the sum of
//                          their elementwise product: ||Z_i^T V_i||_F^2 without
//                          forming the d_ff x d_model update.
//   fe_clip_kernel         per chunk: eta_t = eta * min(1, tau / ||eta Z_i^T V_i||_F).
//
// GEMM main loops: gemm.h's DLoop (4 waves as 2 x 2, each wave 32 TI x 32 TJ
// outputs of v_mfma_f32_32x32x16_bf16, K-steps of 32 streamed with direct
// global-to-LDS loads into a ring of three swizzled [rows][32] LDS tiles).
#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace ttt {

namespace {

using namespace gemm;

constexpr int FE_NT = GM_NT;   // threads per workgroup

// Tile order: groups of 8 token tiles walk all feature tiles, so the 32 or
// so workgroups resident on one XCD share a few token and feature tiles
// through its L2.
TTT_DEV void tile_of(int lid, int n_tok, int n_feat, int* tt, int* ft) {
    constexpr int G = 8;
    const int group = lid / (G * n_feat), first = group * G;
    const int gsz = min(G, n_tok - first);
    const int r = lid % (G * n_feat);
    *tt = first + r % gsz;
    *ft = r / gsz;
}

}  // namespace

// ------------------------------------------------------------------ projections
// C[t][f] = epilogue over A (features) x B (tokens).  A: rows of K elements
// (Linear-layout weights), B: token rows (row stride ldb), out: token rows
// (row stride ldo).  GATED: features f of the output come from A rows 2f
// (Wgate row f) and 2f + 1 (Wup row f).
template <bool GATED>
__global__ __launch_bounds__(FE_NT) void fe_gemm_kernel(FeGemmParams p) {
    constexpr int TI = 4, TJ = 4;
    using LP = DLoop<false, false, TI, TJ>;
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int n_feat = p.arows / BM, n_tok = (p.T + BN - 1) / BN;
    int tt, ft;
    tile_of(xcd_logical(blockIdx.x, gridDim.x), n_tok, n_feat, &tt, &ft);
    const int a0 = ft * BM, t0 = tt * BN;

    const bf16_t* A0 = reinterpret_cast<const bf16_t*>(p.A0);
    const bf16_t* A1 = reinterpret_cast<const bf16_t*>(p.A1);
    const bf16_t* Bm = reinterpret_cast<const bf16_t*>(p.B);
    typename LP::OA a;
    typename LP::OB b;
    a.init_rows([&](int r) {
        const int row = a0 + r;
        return GATED ? ((row & 1) ? A1 : A0) + (int64_t)(row >> 1) * p.K : A0 + (int64_t)row * p.K;
    }, tid);
    b.init_rows([&](int r) { return Bm + (int64_t)min(t0 + r, p.T - 1) * p.ldb; }, tid);
    Acc<TI, TJ> acc;
    zero(acc);
    LP::run(acc, p.K / GM_BK, a, b, smem, tid);

    // acc[i][j][r]: A row 32 TI wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
    // token 32 TJ wn + 32 j + lane % 32
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int t = t0 + 32 * TJ * wn + 32 * j + (lane & 31);
        if (t >= p.T) continue;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.out) + (int64_t)t * p.ldo;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int arow = a0 + 32 * TI * wm + 32 * i + 8 * q + 4 * (lane >> 5);
                const f32x16& a = acc[i][j];
                if (GATED) {
                    // rows 2f, 2f+1 -> (gate, up) of feature f
                    const float g0 = a[4 * q], u0 = a[4 * q + 1], g1 = a[4 * q + 2], u1 = a[4 * q + 3];
                    // silu with the hardware reciprocal (v_rcp_f32, 1 ulp), not an
                    // IEEE division sequence
                    const float z0 = g0 * __builtin_amdgcn_rcpf(1.f + __expf(-g0)) * u0;
                    const float z1 = g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * u1;
                    *reinterpret_cast<uint32_t*>(orow + (arow >> 1)) = pack2bf(z0, z1);
                } else {
                    st4(orow + arow, f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]});
                }
            }
    }
}

// ---------------------------------------------------------------- convolution
// Y[b, t, c] = sum_{j < K, t + j < L} w[j][c] X[b, t + j, c]; one thread per 8 channels
__global__ __launch_bounds__(256) void fe_conv_kernel(FeConvParams p) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nv = p.d / 8;
    const int64_t nvec = (int64_t)p.B * p.L * nv;
    if (i >= nvec) return;
    const int cv = (int)(i % nv);
    const int64_t row = i / nv;
    const int t = (int)(row % p.L);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.K && t + j < p.L; ++j) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.X) + (row + j) * p.d + 8 * cv);
        const float* w = p.w + (int64_t)j * p.d + 8 * cv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w[2 * e] * __uint_as_float(x[e] << 16);
            acc[2 * e + 1] += w[2 * e + 1] * __uint_as_float(x[e] & 0xffff0000u);
        }
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(p.Y) + row * p.d + 8 * cv) =
        u32x4{pack2bf(acc[0], acc[1]), pack2bf(acc[2], acc[3]), pack2bf(acc[4], acc[5]), pack2bf(acc[6], acc[7])};
}

// --------------------------------------------------------------------- Gram
// Block (pair, chunk, b): token tiles (si, ti) of the chunk with si <= ti;
// partial = w * sum_{s in si, t in ti} (z_s . z_t)(v_s . v_t), w = 2 off the diagonal.
__global__ __launch_bounds__(FE_NT) void fe_gram_kernel(FeGramParams p) {
    constexpr int TI = 2, TJ = 2;
    // register-staged loads: measured 10 % faster here than the direct-load ring
    using LP = Loop<false, false, TI, TJ>;
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS];
    __shared__ float sRed[FE_NT / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int pair = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    // pair -> (si, ti), si <= ti, row-major over the upper triangle
    int si = 0, rem = pair;
    while (rem >= p.ntiles - si) {
        rem -= p.ntiles - si;
        ++si;
    }
    const int ti = si + rem;
    const int c0 = chunk * p.chunk;
    const int cend = min(c0 + p.chunk, p.L);
    const int s0 = c0 + si * BM, u0 = c0 + ti * BN;
    float part = 0.f;
    if (s0 < cend && u0 < cend) {   // uniform
        const int64_t rowb = (int64_t)b * p.L;
        Acc<TI, TJ> az, av;
        zero(az);
        zero(av);
        auto gram = [&](Acc<TI, TJ>& acc, const bf16_t* base, int ld) {
            typename LP::OA oa;
            typename LP::OB ob;
            const bf16_t* seq = base + rowb * ld;   // this sequence's rows (offsets below 2^31)
            oa.init(seq, ld, s0, cend, tid);
            ob.init(seq, ld, u0, cend, tid);
            LP::run(acc, ld / GM_BK, oa, ob, smem, tid);
        };
        gram(az, reinterpret_cast<const bf16_t*>(p.Z), p.dz);
        gram(av, reinterpret_cast<const bf16_t*>(p.V), p.dv);
        // rows (tokens s) past the chunk end were clamped: mask them out
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int u = u0 + 32 * TJ * wn + 32 * j + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int s = s0 + 32 * TI * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (s < cend && u < cend) part += az[i][j][r] * av[i][j][r];
                }
            }
        if (si != ti) part *= 2.f;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) sRed[wave] = part;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < FE_NT / 64; ++w) t += sRed[w];
        p.partial[((int64_t)b * gridDim.y + chunk) * gridDim.x + pair] = t;
    }
}

// eta_t = eta * min(1, tau / (eta * sqrt(sum of the chunk's partials))); one block per (chunk, b)
__global__ __launch_bounds__(256) void fe_clip_kernel(FeGramParams p, int npairs) {
    const int chunk = blockIdx.x, b = blockIdx.y;
    __shared__ float sScale;
    if (threadIdx.x == 0) {
        const float* part = p.partial + ((int64_t)b * gridDim.x + chunk) * npairs;
        double sum = 0.0;
        for (int i = 0; i < npairs; ++i) sum += part[i];
        const double nrm = (double)p.eta * sqrt(sum > 0.0 ? sum : 0.0);
        sScale = (nrm > (double)p.tau) ? (float)((double)p.tau / nrm) : 1.f;
    }
    __syncthreads();
    const int c0 = chunk * p.chunk, c1 = min(c0 + p.chunk, p.L);
    for (int t = c0 + threadIdx.x; t < c1; t += 256) p.eta_out[(int64_t)b * p.L + t] = p.eta * sScale;
}

// ------------------------------------------------------------------ launchers
bool fe_gemm_supported(int K, int nfeat_rows) { return K % 128 == 0 && nfeat_rows % 256 == 0; }

hipError_t launch_fe_gemm(const FeGemmParams& p, bool gated, hipStream_t s) {
    if (!fe_gemm_supported(p.K, p.arows)) return hipErrorInvalidValue;
    const int n_tok = (p.T + 255) / 256, n_feat = p.arows / 256;
    const dim3 grid((unsigned)(n_tok * n_feat)), block(FE_NT);
    if (gated) hipLaunchKernelGGL((fe_gemm_kernel<true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fe_gemm_kernel<false>), grid, block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fe_conv(const FeConvParams& p, hipStream_t s) {
    if (p.d % 8 != 0) return hipErrorInvalidValue;
    const int64_t nvec = (int64_t)p.B * p.L * (p.d / 8);
    hipLaunchKernelGGL(fe_conv_kernel, dim3((unsigned)((nvec + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

int fe_gram_pairs(int chunk) {
    const int nt = (chunk + 127) / 128;
    return nt * (nt + 1) / 2;
}

hipError_t launch_fe_clip(const FeGramParams& pin, hipStream_t s) {
    FeGramParams p = pin;
    if (p.dz % 128 != 0 || p.dv % 128 != 0) return hipErrorInvalidValue;
    p.ntiles = (p.chunk + 127) / 128;
    const int npairs = fe_gram_pairs(p.chunk);
    const int nchunks = (p.L + p.chunk - 1) / p.chunk;
    hipLaunchKernelGGL(fe_gram_kernel, dim3(npairs, nchunks, p.B), dim3(FE_NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fe_clip_kernel, dim3(nchunks, p.B), dim3(256), 0, s, p, npairs);
    return hipGetLastError();
}

}  // namespace ttt
