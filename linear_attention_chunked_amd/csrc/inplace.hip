// inplace.hip -- chunk-causal forward for large fast weights (In-Place TTT).
//
// [P2] ("In-Place 테스트 시점 학습: LLM을 위한 원활한 동적 적응 프레임워크",
// aitrends.kr/articles/40879): the down projection Wdown of a gated MLP is the
// fast weight; the sequence is cut in chunks, chunk i reads the weight left
// by chunks < i and then applies one delta update; the chunk updates combine
// by a prefix sum (paragraphs on Wdown as the fast weight, on the chunk-wise
// update and on the associative scan).  Per (b, h):
//     O_i = Z_i W_{i-1},   W_i = W_{i-1} + Z_i^T diag(eta_i) V_i,   W_{-1} = W0.
//
// The state (dk x dv, e.g. 9728 x 2560 fp32 = 99.6 MB) cannot stay on chip, so
// the forward runs in two MFMA-bound passes:
//   1. update walk: every workgroup owns a 256 x 256 tile of W in fp32
//      accumulators and walks the chunks in order (the prefix sum of the
//      chunk deltas happens in registers); before chunk i it writes the bf16
//      snapshot W_{i-1}^T of its tile to the workspace.  K = chunk tokens.
//   2. readout: O_i^T = W_{i-1}^T Z_i^T for all chunks at once, a batched GEMM
//      over (chunk, token tile, dv tile), K = dk.
// Both use v_mfma_f32_32x32x16_bf16 with fp32 accumulation, 256 x 256 block
// tiles (4 waves of 128 x 128), K-steps of 32 double-buffered in LDS.  The
// update pass reads Z and V token-major, so its operands come out of LDS with
// the gfx950 transposing read ds_read_b64_tr_b16 instead of a transposed copy.
#include "common.h"
#include "internal.h"

#include <type_traits>

namespace ttt {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int IP_BM = 256, IP_BN = 256, IP_BK = 32;
constexpr int IPU_BN = 128;           // update pass: 256 x 128 tiles (waves 128 x 64)
constexpr int IP_NT = 256;             // threads per workgroup
constexpr int IP_PADN = 8;             // [row][k] tiles: 16-byte row pad
constexpr int IP_PADT = 32;            // [k][row] tiles: 64-byte row pad

TTT_DEV void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane a loads 4 consecutive 16-bit values (8 bytes at its address);
// lane i of the group then receives slot j = the value lane 4j + i/4 loaded
// in its slot i%4.  So if lane a points at X[k(a/4)][c0 + 4(a%4)] of a
// row-major tile, lane i gets column c0 + i of rows k(0..3): an MFMA operand
// fragment read across the rows of a [k][col] tile.
TTT_DEV u32x2 ds_read_tr(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Operand fragment (32 rows x 16 k) of a 32x32x16 MFMA from a [k][row] LDS
// tile with row stride ld (elements).  Lane l gets row r0 + l%32 and
// k = k0 + 8*(l/32) + 0..7 (the same k assignment as frag_rows below).
TTT_DEV bf16x8 frag_tr(const bf16_t* s, int ld, int r0, int k0, int lane) {
    const int G = lane >> 4, a = lane & 15;
    const int h = G >> 1;                       // which 8-k half
    const int rbase = r0 + 16 * (G & 1) + 4 * (a & 3);
    const int kk = k0 + 8 * h + (a >> 2);
    const u32x2 lo = ds_read_tr(s + (kk + 0) * ld + rbase);
    const u32x2 hi = ds_read_tr(s + (kk + 4) * ld + rbase);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// Operand fragment from a [row][k] LDS tile (k contiguous).
TTT_DEV bf16x8 frag_rows(const bf16_t* s, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(s + (r0 + (lane & 31)) * ld + k0 + 8 * (lane >> 5));
}

// ------------------------------------------------------------------ pass 1
// grid.x = (dk/256) * (dv/128) tiles,
// grid.y = B*H.  snap: [B*H][N][dv][dk] bf16 (transposed snapshots).
struct IpUpdateParams {
    const bf16_t* k;          // Z   [B,H,L,dk] (strides ks)
    const bf16_t* v;          // V   [B,H,L,dv]
    int64_t ks[3], vs[3];
    const float* eta;
    int64_t es[3];
    float eta_scalar;
    const float* S0;
    int64_t s0s[2];
    float* S_final;
    bf16_t* snap;
    int H, L, dk, dv, chunk, nchunks;
};

// PT = per-token step sizes: V fragments are scaled by eta_t (and rounded to
// bf16) before the MFMA.  With one scalar eta != 0 the accumulator instead
// holds W / eta, the exact bf16 x bf16 products are summed in fp32 and eta is
// applied when W leaves the registers (snapshots, final weight).
template <bool PT>
__global__ __launch_bounds__(IP_NT) void ip_update_kernel(IpUpdateParams p) {
    constexpr int LDA = IP_BM + IP_PADT, LDB = IPU_BN + IP_PADT;
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][IP_BK * LDA];   // Z slice  [k=token][m=dk]
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][IP_BK * LDB];   // V slice  [k=token][n=dv]
    __shared__ float sE[2][IP_BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;   // 2 x 2 waves, 128 x 64 each
    const int tiles_n = p.dv / IPU_BN;
    // logical order (bh, dk tile, dv tile): the workgroups one XCD runs at a
    // time share a few Z column slices and stream them through one L2
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    const int tile = lid % gridDim.x;
    const int m0 = (tile / tiles_n) * IP_BM, n0 = (tile % tiles_n) * IPU_BN;
    const int bh = lid / gridDim.x, b = bh / p.H, h = bh % p.H;
    const bf16_t* Zg = p.k + b * p.ks[0] + h * p.ks[1] + m0;
    const bf16_t* Vg = p.v + b * p.vs[0] + h * p.vs[1] + n0;
    const float* Eg = p.eta ? p.eta + b * p.es[0] + h * p.es[1] : nullptr;
    const int L = p.L;

    // accumulators: 4 x 2 tiles of 32 x 32, W[m][n] with lane = column
    f32x16 acc[4][2];
    {
        const float* W0 = p.S0 ? p.S0 + b * p.s0s[0] + h * p.s0s[1] : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int col = n0 + 64 * wn + 32 * j + (lane & 31);
                    const float w0 = W0 ? W0[(int64_t)row * p.dv + col] : 0.f;
                    acc[i][j][r] = PT ? w0 : w0 / p.eta_scalar;
                }
    }

    // staging: per K-step 32 tokens x 256 of Z (4 x 16 B per thread) and
    // 32 tokens x 128 of V (2 x 16 B per thread).  NS register sets are in
    // flight: the loads of step s+NS are issued at the top of step s and
    // written to LDS at the end of step s+NS-1.  Every lane issues the same
    // loads each step (token rows past L re-read row L-1 and are zeroed when
    // written to LDS), so the compiler's waits only drain the oldest set.
    constexpr int NS = 4;
    u32x4 ra[NS][4], rb[NS][2];
    float re[NS];
    uint32_t zoff[4], voff[2];
    int zrow[4], vrow[2];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int u = tid + x * IP_NT;              // 0..1023
        zrow[x] = u >> 5;
        zoff[x] = (uint32_t)((u & 31) * 8);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int u = tid + x * IP_NT;              // 0..511
        vrow[x] = u >> 4;
        voff[x] = (uint32_t)((u & 15) * 8);
    }
    const int kpc = p.chunk / IP_BK;                // K-steps per chunk
    const int total_steps = p.nchunks * kpc;
    auto step_t0 = [&](int st) { return (st / kpc) * p.chunk + (st % kpc) * IP_BK; };
    auto load = [&](int st, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
        const int t0 = step_t0(min(st, total_steps - 1));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int t = min(t0 + zrow[x], L - 1);
            ra[k][x] = *reinterpret_cast<const u32x4*>(Zg + (int64_t)t * p.ks[2] + zoff[x]);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int t = min(t0 + vrow[x], L - 1);
            rb[k][x] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)t * p.vs[2] + voff[x]);
        }
        if (PT) re[k] = Eg ? Eg[(int64_t)min(t0 + (tid & (IP_BK - 1)), L - 1) * p.es[2]] : p.eta_scalar;
    };
    auto stage = [&](int st, int buf, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
        const int t0 = step_t0(st);
        const u32x4 z4 = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int u = tid + x * IP_NT;
            *reinterpret_cast<u32x4*>(&sA[buf][zrow[x] * LDA + (u & 31) * 8]) = (t0 + zrow[x] < L) ? ra[k][x] : z4;
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int u = tid + x * IP_NT;
            *reinterpret_cast<u32x4*>(&sB[buf][vrow[x] * LDB + (u & 15) * 8]) = (t0 + vrow[x] < L) ? rb[k][x] : z4;
        }
        if (PT && tid < IP_BK) sE[buf][tid] = (t0 + tid < L) ? re[k] : 0.f;
    };
    const float out_scale = PT ? 1.f : p.eta_scalar;   // acc -> W
    bf16_t* snap = p.snap + (int64_t)bh * p.nchunks * p.dk * p.dv;

    // snapshot W_{chunk-1}^T (bf16) of this tile: [n][m] layout
    auto snapshot = [&](int chunk) __attribute__((always_inline)) {
        bf16_t* sp = snap + (int64_t)chunk * p.dk * p.dv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = n0 + 64 * wn + 32 * j + (lane & 31);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = m0 + 128 * wm + 32 * i + 8 * q + 4 * (lane >> 5);
                    const f32x4 v4 = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    st4(sp + (int64_t)col * p.dk + row, v4 * out_scale);
                }
            }
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const bf16_t* A = sA[buf];
        const bf16_t* Bt = sB[buf];
#pragma unroll
        for (int kk = 0; kk < IP_BK; kk += 16) {
            bf16x8 af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = frag_tr(A, LDA, 128 * wm + 32 * i, kk, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) bfr[j] = frag_tr(Bt, LDB, 64 * wn + 32 * j, kk, lane);
            if (PT) {
                // eta of the 8 tokens this lane's fragments cover
                const int kb = kk + 8 * (lane >> 5);
                float e[8];
                for (int x = 0; x < 8; ++x) e[x] = sE[buf][kb + x];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const u32x4 w = __builtin_bit_cast(u32x4, bfr[j]);
                    u32x4 o;
                    for (int x = 0; x < 4; ++x) {
                        const float lo = __uint_as_float(w[x] << 16) * e[2 * x];
                        const float hi = __uint_as_float(w[x] & 0xffff0000u) * e[2 * x + 1];
                        o[x] = pack2bf(lo, hi);
                    }
                    bfr[j] = __builtin_bit_cast(bf16x8, o);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma32(acc[i][j], af[i], bfr[j]);
        }
    };

    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    static_assert(NS == 4, "the step sequence below is written for four register sets");
    load(0, K0{});
    load(1, K1{});
    load(2, K2{});
    load(3, K3{});
    stage(0, 0, K0{});
    __syncthreads();
    // step st: refill the set step st just freed, compute from LDS, write step
    // st+1 to the other LDS buffer
    auto step = [&](int st, auto CUR, auto NXT) __attribute__((always_inline)) {
        if (st >= total_steps) return;               // (uniform)
        if (st % kpc == 0) snapshot(st / kpc);
        load(st + NS, CUR);
        compute(st & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (st + 1 < total_steps) stage(st + 1, (st + 1) & 1, NXT);
        __syncthreads();
    };
    for (int st = 0; st < total_steps; st += NS) {
        step(st, K0{}, K1{});
        step(st + 1, K1{}, K2{});
        step(st + 2, K2{}, K3{});
        step(st + 3, K3{}, K0{});
    }

    if (p.S_final) {
        float* Wf = p.S_final + (int64_t)bh * p.dk * p.dv;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int col = n0 + 64 * wn + 32 * j + (lane & 31);
                    Wf[(int64_t)row * p.dv + col] = acc[i][j][r] * out_scale;
                }
    }
}

// ------------------------------------------------------------------ pass 2
// O_c^T tile [256 dv][256 tokens] = snap_c^T [dv][dk] x Z_c^T; grid.x =
// nchunks * (chunk/256) * (dv/256), grid.y = B*H.
struct IpReadoutParams {
    const bf16_t* q;          // Z [B,H,L,dk]
    int64_t qs[3];
    bf16_t* out;              // O [B,H,L,dv]
    int64_t os[3];
    const bf16_t* snap;
    int H, L, dk, dv, chunk, nchunks;
};

__global__ __launch_bounds__(IP_NT) void ip_readout_kernel(IpReadoutParams p) {
    constexpr int LD = IP_BK + IP_PADN;
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][IP_BM * LD];    // snap^T [n][k]
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][IP_BN * LD];    // Z      [t][k]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = p.dv / IP_BM;                 // dv tiles
    const int tiles_t = p.chunk / IP_BN;              // token tiles per chunk
    // logical order (bh, chunk, token tile, dv tile): one XCD runs the tiles
    // of one chunk together, so they share the chunk's Z rows and snapshot
    // columns through its L2
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    int x = lid % gridDim.x;
    const int nt = x % tiles_n;
    x /= tiles_n;
    const int tt = x % tiles_t;
    const int chunk = x / tiles_t;
    const int n0 = nt * IP_BM;                        // dv offset
    const int t0 = chunk * p.chunk + tt * IP_BN;      // token offset
    const int bh = lid / gridDim.x, b = bh / p.H, h = bh % p.H;
    if (t0 >= p.L) return;                            // whole tile past the end (uniform)
    const bf16_t* S = p.snap + ((int64_t)bh * p.nchunks + chunk) * p.dk * p.dv + (int64_t)n0 * p.dk;
    const bf16_t* Zg = p.q + b * p.qs[0] + h * p.qs[1];
    bf16_t* Og = p.out + b * p.os[0] + h * p.os[1];
    const int L = p.L;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    u32x4 ra[4], rb[4];
    auto load = [&](int k0) {
        for (int y = 0; y < 4; ++y) {
            const int u = tid + y * IP_NT;            // 0..1023: 256 rows x 4 x 16 B
            const int row = u >> 2, c = (u & 3) * 8;
            ra[y] = *reinterpret_cast<const u32x4*>(S + (int64_t)row * p.dk + k0 + c);
            const int t = t0 + row;
            rb[y] = (t < L) ? *reinterpret_cast<const u32x4*>(Zg + t * p.qs[2] + k0 + c) : u32x4{0, 0, 0, 0};
        }
    };
    auto stage = [&](int buf) {
        for (int y = 0; y < 4; ++y) {
            const int u = tid + y * IP_NT;
            const int row = u >> 2, c = (u & 3) * 8;
            *reinterpret_cast<u32x4*>(&sA[buf][row * LD + c]) = ra[y];
            *reinterpret_cast<u32x4*>(&sB[buf][row * LD + c]) = rb[y];
        }
    };

    const int steps = p.dk / IP_BK;
    load(0);
    stage(0);
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        if (s + 1 < steps) load((s + 1) * IP_BK);
#pragma unroll
        for (int kk = 0; kk < IP_BK; kk += 16) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = frag_rows(sA[buf], LD, 128 * wm + 32 * i, kk, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = frag_rows(sB[buf], LD, 128 * wn + 32 * j, kk, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma32(acc[i][j], af[i], bfr[j]);
        }
        if (s + 1 < steps) stage(buf ^ 1);
        __syncthreads();
    }

    // acc[i][j]: O^T[n][t], lane = token column, 4 consecutive n per group
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + 128 * wn + 32 * j + (lane & 31);
            if (t >= L) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + 128 * wm + 32 * i + 8 * q + 4 * (lane >> 5);
                const f32x4 v4 = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                       acc[i][j][4 * q + 3]};
                st4(Og + t * p.os[2] + n, v4);
            }
        }
}

bool inplace_supported(int dtype, int dk, int dv, int chunk) {
    return dtype == 1 && dk % IP_BM == 0 && dv % IP_BN == 0 && chunk % IP_BN == 0 && dk >= IP_BM &&
           dv >= IP_BN;  // IP_BN is a multiple of the update tile IPU_BN
}

size_t inplace_workspace(int B, int H, int L, int dk, int dv, int chunk) {
    const int64_t N = (L + chunk - 1) / chunk;
    return (size_t)B * H * N * dk * dv * sizeof(bf16_t);
}

hipError_t launch_inplace(const TcParams& p, void* workspace, hipStream_t s) {
    const int N = (p.L + p.chunk - 1) / p.chunk;
    IpUpdateParams u;
    u.k = reinterpret_cast<const bf16_t*>(p.k);
    u.v = reinterpret_cast<const bf16_t*>(p.v);
    for (int i = 0; i < 3; ++i) {
        u.ks[i] = p.ks[i];
        u.vs[i] = p.vs[i];
        u.es[i] = p.es[i];
    }
    u.eta = p.eta;
    u.eta_scalar = p.eta_scalar;
    u.S0 = p.S0;
    u.s0s[0] = p.s0s[0];
    u.s0s[1] = p.s0s[1];
    u.S_final = p.S_final;
    u.snap = reinterpret_cast<bf16_t*>(workspace);
    u.H = p.H;
    u.L = p.L;
    u.dk = p.dk;
    u.dv = p.dv;
    u.chunk = p.chunk;
    u.nchunks = N;
    const dim3 g1((p.dk / IP_BM) * (p.dv / IPU_BN), p.B * p.H);
    if (p.eta || p.eta_scalar == 0.f) {
        hipLaunchKernelGGL(ip_update_kernel<true>, g1, dim3(IP_NT), 0, s, u);
    } else {
        hipLaunchKernelGGL(ip_update_kernel<false>, g1, dim3(IP_NT), 0, s, u);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    IpReadoutParams r;
    r.q = reinterpret_cast<const bf16_t*>(p.q);
    r.out = reinterpret_cast<bf16_t*>(p.out);
    for (int i = 0; i < 3; ++i) {
        r.qs[i] = p.qs[i];
        r.os[i] = p.os[i];
    }
    r.snap = u.snap;
    r.H = p.H;
    r.L = p.L;
    r.dk = p.dk;
    r.dv = p.dv;
    r.chunk = p.chunk;
    r.nchunks = N;
    const dim3 g2(N * (p.chunk / IP_BN) * (p.dv / IP_BM), p.B * p.H);
    hipLaunchKernelGGL(ip_readout_kernel, g2, dim3(IP_NT), 0, s, r);
    return hipGetLastError();
}

}  // namespace ttt
