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
//   1. update walk: every workgroup owns a tile of W in fp32 accumulators
//      and walks the chunks in order (the prefix sum of the chunk deltas
//      happens in registers); before chunk i it writes the bf16 snapshot
//      W_{i-1}^T of its tile to the workspace.  K = chunk tokens.
//      Snapshots are stored blocked by 16 rows of W: element (n, m) of
//      W_{i-1}^T at ((m / 16) dv + n) 16 + m % 16, i.e. [dk/16][dv][16].  The
//      update's accumulators hold 4 consecutive m of one n per lane, so a
//      lane group writes whole 32-byte blocks and a store instruction 512
//      contiguous bytes; the readout still streams both operands along dk
//      (a 32-wide k step of a row n is two 32-byte blocks).
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
constexpr int IP_PADT = 32;            // [k][row] tiles: 64-byte row pad
constexpr int IP_SNR = IP_BM + 8;      // snapshot staging row: 256 m values + pad

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
// k = k0 + 8*(l/32) + 0..7 (the k assignment the readout's row fragments use).
TTT_DEV bf16x8 frag_tr(const bf16_t* s, int ld, int r0, int k0, int lane) {
    const int G = lane >> 4, a = lane & 15;
    const int h = G >> 1;                       // which 8-k half
    const int rbase = r0 + 16 * (G & 1) + 4 * (a & 3);
    const int kk = k0 + 8 * h + (a >> 2);
    const u32x2 lo = ds_read_tr(s + (kk + 0) * ld + rbase);
    const u32x2 hi = ds_read_tr(s + (kk + 4) * ld + rbase);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
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
    __shared__ __attribute__((aligned(16))) bf16_t sS[IPU_BN * IP_SNR];   // snapshot staging [n][m]

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
    // 32 tokens x 128 of V (2 x 16 B per thread); K-step st covers tokens
    // [32 st, 32 st + 32) (a chunk is a whole number of K-steps).  NS register
    // sets are in flight: the loads of step st+NS are issued at the top of
    // step st and written to LDS at the end of step st+NS-1.  Every lane issues
    // the same loads each step (token rows past L re-read row L-1 and are
    // zeroed when written to LDS), and the per-lane offsets are fixed.
    constexpr int NS = 4;
    u32x4 ra[NS][4], rb[NS][2];
    float re[NS];
    uint32_t zoff[4], voff[2];
    int zrow[4], vrow[2], zlds[4], vlds[2];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int u = tid + x * IP_NT;              // 0..1023: 32 rows x 32 chunks
        zrow[x] = u >> 5;
        zoff[x] = (uint32_t)(zrow[x] * (int)p.ks[2] + (u & 31) * 8);
        zlds[x] = zrow[x] * LDA + (u & 31) * 8;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int u = tid + x * IP_NT;              // 0..511: 32 rows x 16 chunks
        vrow[x] = u >> 4;
        voff[x] = (uint32_t)(vrow[x] * (int)p.vs[2] + (u & 15) * 8);
        vlds[x] = vrow[x] * LDB + (u & 15) * 8;
    }
    const int kpc = p.chunk / IP_BK;                // K-steps per chunk
    const int total_steps = p.nchunks * kpc;
    const int full_steps = L / IP_BK;               // steps with all 32 tokens in range
    auto load = [&](int st, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
        const int t0 = min(st, full_steps - 1) * IP_BK;  // whole steps only; see the tail below
        const bf16_t* Zs = Zg + (int64_t)t0 * p.ks[2];
        const bf16_t* Vs = Vg + (int64_t)t0 * p.vs[2];
#pragma unroll
        for (int x = 0; x < 4; ++x) ra[k][x] = *reinterpret_cast<const u32x4*>(Zs + zoff[x]);
#pragma unroll
        for (int x = 0; x < 2; ++x) rb[k][x] = *reinterpret_cast<const u32x4*>(Vs + voff[x]);
        if (PT) re[k] = Eg ? Eg[(int64_t)(t0 + (tid & (IP_BK - 1))) * p.es[2]] : p.eta_scalar;
    };
    auto stage = [&](int buf, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
#pragma unroll
        for (int x = 0; x < 4; ++x) *reinterpret_cast<u32x4*>(&sA[buf][zlds[x]]) = ra[k][x];
#pragma unroll
        for (int x = 0; x < 2; ++x) *reinterpret_cast<u32x4*>(&sB[buf][vlds[x]]) = rb[k][x];
        if (PT && tid < IP_BK) sE[buf][tid] = re[k];
    };
    const float out_scale = PT ? 1.f : p.eta_scalar;   // acc -> W
    bf16_t* snap = p.snap + (int64_t)bh * p.nchunks * p.dk * p.dv;

    // snapshot W_{chunk-1}^T (bf16) of this tile in the blocked layout.  A
    // lane holds 4 consecutive m of one n, so the tile goes through LDS ([n][m]
    // rows of 512 bytes) and leaves as 16-byte halves of the (m / 16, n)
    // blocks, consecutive lanes on consecutive addresses; the next snapshot is
    // a chunk of K-steps (and their barriers) later, so one barrier suffices.
    auto snapshot = [&](int chunk) __attribute__((always_inline)) {
        const int nl = 64 * wn + (lane & 31), ml = 128 * wm + 4 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v4 = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    st4(&sS[(nl + 32 * j) * IP_SNR + ml + 32 * i + 8 * q], v4 * out_scale);
                }
        __syncthreads();
        bf16_t* sp = snap + (int64_t)chunk * p.dk * p.dv + ((int64_t)(m0 >> 4) * p.dv + n0) * 16;
        // x -> (16-row block cb, column r, half hf): consecutive x, consecutive 16 bytes
        for (int x = tid; x < IPU_BN * (IP_BM / 8); x += IP_NT) {
            const int hf = x & 1, r = (x >> 1) % IPU_BN, cb = (x >> 1) / IPU_BN;
            *reinterpret_cast<u32x4*>(sp + ((int64_t)cb * p.dv + r) * 16 + 8 * hf) =
                *reinterpret_cast<const u32x4*>(&sS[r * IP_SNR + 16 * cb + 8 * hf]);
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
    if (full_steps > 0) {
        load(0, K0{});
        load(1, K1{});
        load(2, K2{});
        load(3, K3{});
        stage(0, K0{});
    }
    __syncthreads();
    // whole steps: refill the set this step just freed, compute from LDS,
    // write step st+1 to the other LDS buffer
    auto step = [&](int st, auto CUR, auto NXT) __attribute__((always_inline)) {
        load(st + NS, CUR);
        compute(st & 1);
        __builtin_amdgcn_sched_barrier(0);
        // unconditional: after the last whole step it writes clamped, unused
        // data to the idle buffer (the tail below rewrites buffer 0 after a
        // barrier), and no path skips the wait for this set's loads
        stage((st + 1) & 1, NXT);
        __syncthreads();
    };
    // chunk boundaries fall on multiples of kpc (a multiple of 8), so they
    // only ever meet the first step of a group of four
    int next_snap = 0, snap_idx = 0;
    auto boundary = [&](int at) __attribute__((always_inline)) {
        if (at == next_snap) {
            snapshot(snap_idx);
            ++snap_idx;
            next_snap += kpc;
        }
    };
    int st = 0;
    for (; st + NS <= full_steps; st += NS) {
        boundary(st);
        step(st, K0{}, K1{});
        step(st + 1, K1{}, K2{});
        step(st + 2, K2{}, K3{});
        step(st + 3, K3{}, K0{});
    }
    // up to three whole steps left: their data sit in sets 0, 1, 2
    if (st < full_steps) {
        boundary(st);
        step(st, K0{}, K1{});
        if (st + 1 < full_steps) step(st + 1, K1{}, K2{});
        if (st + 2 < full_steps) step(st + 2, K2{}, K3{});
    }
    // a last step with fewer than 32 tokens: rows past L are zeroed
    if (full_steps * IP_BK < L) {
        const int t0 = full_steps * IP_BK;
        boundary(full_steps);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int t = min(t0 + zrow[x], L - 1);
            const u32x4 v = *reinterpret_cast<const u32x4*>(Zg + (int64_t)(t - zrow[x]) * p.ks[2] + zoff[x]);
            *reinterpret_cast<u32x4*>(&sA[0][zlds[x]]) = (t0 + zrow[x] < L) ? v : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int t = min(t0 + vrow[x], L - 1);
            const u32x4 v = *reinterpret_cast<const u32x4*>(Vg + (int64_t)(t - vrow[x]) * p.vs[2] + voff[x]);
            *reinterpret_cast<u32x4*>(&sB[0][vlds[x]]) = (t0 + vrow[x] < L) ? v : u32x4{0, 0, 0, 0};
        }
        if (PT && tid < IP_BK) {
            const int t = t0 + tid;
            sE[0][tid] = (t < L) ? (Eg ? Eg[(int64_t)t * p.es[2]] : p.eta_scalar) : 0.f;
        }
        __syncthreads();
        compute(0);
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

// ------------------------------------------------- pass 1, wide tiles
// The update walk with one workgroup per CU: a 304 x 320 tile of W
// (d_ff 9728 = 32 x 304, d_model 2560 = 8 x 320 give exactly 256 tiles, one
// wave of workgroups on 256 CUs).  Every token of the walk brings
// (304 + 320) x 2 bytes from L2 for 304 x 320 x 2 FLOP: 156 FLOP per byte,
// against 85 for the 256 x 128 tiles of ip_update_kernel, whose 760 tiles
// fill the chip in three waves.
//   - 8 waves, two per SIMD.  Wave w owns column tiles 5 (w % 4) .. +4
//     (16 columns each) and row tiles 0..9 (w < 4) or 10..18 (w >= 4) of 16
//     rows: waves w and w + 4 share a SIMD and together run its 95
//     v_mfma_f32_16x16x32_bf16 per K-step of 32 tokens, with at most 50
//     16 x 16 accumulators (200 registers) per wave.
//   - Operands stream straight from global memory into LDS with gfx950's
//     16-byte buffer loads to LDS, a ring of four K-step buffers (156 KB;
//     loads three steps ahead), one barrier per step.  A wave-load instruction writes 64
//     consecutive 16-byte LDS slots; which global piece each lane fetches
//     sets the layout.
//   - LDS A (Z): [32 k][304 m], 608-byte rows (38 pieces), logical token k
//     in row k with bits 2 and 3 swapped: a half-wave's transposing fragment
//     read then touches 8 consecutive rows, whose bank octets (3 row mod 8)
//     are all distinct.  LDS B (V-hat): [32 k][320 n], 640-byte rows (40
//     pieces); the four waves' blocks of 5 column tiles are rotated per row,
//     block g of row k at block (g + rotB(k)) mod 4, so that the 8 rows of a
//     half-wave read fall on distinct bank octets while a wave's 5 tiles stay
//     contiguous (fragment addresses are one base plus constant offsets).
//     Both layouts were checked conflict-free by a model of the 64 banks.
//   - Scalar eta only (the accumulators hold W / eta, as in ip_update_kernel);
//     L and the chunk a multiple of 32.  Other cases use ip_update_kernel.
constexpr int IW_MT = 19;                  // 16-row tiles per workgroup tile
constexpr int IW_MH = 10;                  // row tiles of the first half (waves 0..3)
constexpr int IW_NTW = 5;                  // 16-column tiles per wave
constexpr int IW_BM = 16 * IW_MT;          // 304
constexpr int IW_BN = 4 * 16 * IW_NTW;     // 320
constexpr int IW_BK = 32;
constexpr int IW_NB = 4;                   // LDS ring stages (three K-steps of loads in flight)
constexpr int IW_NT = 512;                 // threads per workgroup
constexpr int IW_PA = IW_BM / 8;           // 38 pieces per A row
constexpr int IW_PB = IW_BN / 8;           // 40 pieces per B row
constexpr int IW_LA = IW_BK * IW_PA / 64;  // 19 wave-loads per step (A)
constexpr int IW_LB = IW_BK * IW_PB / 64;  // 20 wave-loads per step (B)
constexpr int IW_LW = 5;                   // wave-loads per wave and step (39 + 1 repeat)
constexpr int IW_SA = IW_BK * IW_BM;       // elements per A stage
constexpr int IW_SB = IW_BK * IW_BN;       // elements per B stage
static_assert(IW_LA * 64 == IW_BK * IW_PA && IW_LB * 64 == IW_BK * IW_PB, "whole wave-loads");
static_assert(8 * IW_LW == IW_LA + IW_LB + 1, "five wave-loads per wave");

TTT_DEV int iw_rowA(int k) { return (k & ~12) | ((k >> 1) & 4) | ((k << 1) & 8); }   // an involution
TTT_DEV int iw_rotB(int k) { return ((k >> 1) & 1) + 2 * ((k >> 3) & 1); }
// physical piece of logical piece q (of 40) in B row k
TTT_DEV int iw_pieceB(int k, int q) {
    const int t = q >> 1, g = t / IW_NTW, j = t % IW_NTW;
    return 2 * (IW_NTW * ((g + iw_rotB(k)) & 3) + j) + (q & 1);
}

typedef __attribute__((address_space(3))) void iw_lds_t;

TTT_DEV void mma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

bool ip_wide_supported(const IpUpdateParams& p, bool per_token) {
    return !per_token && p.dk % IW_BM == 0 && p.dv % IW_BN == 0 && p.chunk % IW_BK == 0 && p.L % IW_BK == 0 &&
           (int64_t)IW_BK * p.ks[2] * 2 < (int64_t(1) << 31) && (int64_t)IW_BK * p.vs[2] * 2 < (int64_t(1) << 31);
}

// One body for both halves of the row tiles: wave w runs row tiles
// mbase .. mbase + mt - 1 (mt = 10 or 9, wave-uniform); the tenth
// accumulator row of the second half stays unused (a uniform branch skips
// its reads, products and stores), which keeps one register allocation.
TTT_DEV void ip_wide_body(const IpUpdateParams& p, bf16_t* sA, bf16_t* sB, int wave, int lane, int m0, int n0,
                          int bh, const bf16_t* Zg, const bf16_t* Vg) {
    constexpr int MT = IW_MH;
    const int mbase = wave < 4 ? 0 : IW_MH, mt = wave < 4 ? IW_MH : IW_MT - IW_MH;
    const int G = lane >> 4, a16 = lane & 15, g = wave & 3;
    const int ldz = (int)p.ks[2], ldv = (int)p.vs[2];
    const int b = bh / p.H, h = bh % p.H;
    const int ncol = n0 + 80 * g + a16;   // this lane's column in tile j: ncol + 16 j

    // accumulators: acc[i][j] = W[m0 + 16 (mbase + i) + 4 G + r][ncol + 16 j] / eta
    f32x4 acc[MT][IW_NTW];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < IW_NTW; ++j) acc[i][j] = zero4();
    if (p.S0) {
        const float inv_eta = 1.f / p.eta_scalar;
        const float* W0 = p.S0 + b * p.s0s[0] + h * p.s0s[1] + (int64_t)(m0 + 16 * mbase + 4 * G) * p.dv + ncol;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < mt) {
#pragma unroll
                for (int j = 0; j < IW_NTW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = W0[(int64_t)(16 * i + r) * p.dv + 16 * j] * inv_eta;
            }
        }
    }

    // this lane's five 16-byte pieces per K-step: wave-load y = 5 wave + x of
    // the step's 39 (A: 0..18, B: 19..38; y = 39 repeats y = 38), each at a
    // fixed byte offset from the step's first token row
    uint32_t voff[IW_LW];
#pragma unroll
    for (int x = 0; x < IW_LW; ++x) {
        const int y = min(IW_LW * wave + x, IW_LA + IW_LB - 1);
        if (y < IW_LA) {
            const int P = 64 * y + lane, R = P / IW_PA, piece = P % IW_PA;
            voff[x] = (uint32_t)((iw_rowA(R) * ldz + 8 * piece) * 2);
        } else {
            // physical slot P holds the logical piece whose block rotates onto it
            const int P = 64 * (y - IW_LA) + lane, R = P / IW_PB, piece = P % IW_PB;
            const int t = piece >> 1, q = 2 * (IW_NTW * (((t / IW_NTW) - iw_rotB(R)) & 3) + t % IW_NTW) + (piece & 1);
            voff[x] = (uint32_t)((R * ldv + 8 * q) * 2);
        }
    }
    const int total_steps = p.L / IW_BK, kpc = p.chunk / IW_BK;
    // loads of K-step st into the stage buffers a, b
    auto issue = [&](int st, bf16_t* a, bf16_t* b) __attribute__((always_inline)) {
        const int s = min(st, total_steps - 1);
        const int64_t t0 = (int64_t)s * IW_BK;
        const __amdgpu_buffer_rsrc_t rz =
            __builtin_amdgcn_make_buffer_rsrc((void*)(Zg + t0 * ldz), 0, IW_BK * ldz * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + t0 * ldv), 0, IW_BK * ldv * 2, 0x00020000);
#pragma unroll
        for (int x = 0; x < IW_LW; ++x) {
            const int y = min(IW_LW * wave + x, IW_LA + IW_LB - 1);   // wave-uniform
            if (y < IW_LA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (iw_lds_t*)(a + 512 * y), 16, voff[x], 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (iw_lds_t*)(b + 512 * (y - IW_LA)), 16, voff[x], 0, 0,
                                                         0);
        }
    };

    // fragment addresses (elements within a stage) for the k-half hk of a
    // 16 x 32 operand: lane (G, a16) reads logical k = 8 G + 4 hk + a16 / 4
    // (tile i of A and tile j of B at constant offsets 16 i, 16 j from them)
    int aoff[2], boff[2];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
        const int k = 8 * G + 4 * hk + (a16 >> 2);
        aoff[hk] = iw_rowA(k) * IW_BM + 16 * mbase + 4 * (a16 & 3);
        boff[hk] = k * IW_BN + 8 * iw_pieceB(k, 2 * IW_NTW * g + ((a16 & 3) >> 1)) + 4 * (a16 & 1);
    }
    auto frag = [&](const bf16_t* base, int o0, int o1) __attribute__((always_inline)) {
        const u32x2 lo = ds_read_tr(base + o0);
        const u32x2 hi = ds_read_tr(base + o1);
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    auto compute = [&](const bf16_t* A, const bf16_t* Bs) __attribute__((always_inline)) {
        bf16x8 bf[IW_NTW];
#pragma unroll
        for (int j = 0; j < IW_NTW; ++j) bf[j] = frag(Bs, boff[0] + 16 * j, boff[1] + 16 * j);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < mt) {
                const bf16x8 af = frag(A, aoff[0] + 16 * i, aoff[1] + 16 * i);
#pragma unroll
                for (int j = 0; j < IW_NTW; ++j) mma16(acc[i][j], af, bf[j]);
            }
        }
    };

    bf16_t* snap = p.snap + (int64_t)bh * p.nchunks * p.dk * p.dv;
    // W_{c-1}^T of this tile in the blocked layout: a lane's 4 values (4
    // consecutive m of one n) leave as one 8-byte store, the 4 lane groups
    // fill the 32-byte block of (m / 16, n), and the 16 columns of a tile
    // are consecutive blocks: 512 contiguous bytes per store instruction
    auto snapshot = [&](int c) __attribute__((always_inline)) {
        bf16_t* sp = snap + (int64_t)c * p.dk * p.dv + ((int64_t)((m0 >> 4) + mbase) * p.dv + ncol) * 16 + 4 * G;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < mt) {
#pragma unroll
                for (int j = 0; j < IW_NTW; ++j) {
                    const f32x4 v = acc[i][j] * p.eta_scalar;
                    *reinterpret_cast<u32x2*>(sp + (int64_t)i * p.dv * 16 + 256 * j) =
                        u32x2{pack2bf(v[0], v[1]), pack2bf(v[2], v[3])};
                }
            }
        }
    };

    // vmcnt field of s_waitcnt (gfx9: bits 3..0 and 15..14); lgkmcnt and
    // expcnt at their maxima
    constexpr int AHEAD = IW_NB - 1;   // K-steps of loads in flight
    constexpr int NW = IW_LW * (AHEAD - 1);
    constexpr int WAIT_ONE_STEP = (NW & 15) | ((NW >> 4) << 14) | (0x7 << 4) | (0xf << 8);
#pragma unroll
    for (int x = 0; x < AHEAD; ++x) issue(x, sA + x * IW_SA, sB + x * IW_SB);
    for (int st = 0; st < total_steps; ++st) {
        if (st % kpc == 0) snapshot(st / kpc);
        // this wave's loads of step st are done once only the later steps' are
        // left; the barrier makes every wave's done, and ends every wave's
        // reads of the buffer that step st + AHEAD refills
        __builtin_amdgcn_s_waitcnt(WAIT_ONE_STEP);
        __builtin_amdgcn_s_barrier();
        const int rd = st % IW_NB, wr = (st + AHEAD) % IW_NB;
        ring_step(sA + wr * IW_SA, sB + wr * IW_SB, sA + rd * IW_SA, sB + rd * IW_SB,
                  [&](bf16_t* a, bf16_t* b) __attribute__((always_inline)) { issue(st + AHEAD, a, b); }, compute);
    }
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));   // the clamped loads still in flight
    __builtin_amdgcn_s_barrier();

    if (p.S_final) {
        float* Wf = p.S_final + (int64_t)bh * p.dk * p.dv + (int64_t)(m0 + 16 * mbase + 4 * G) * p.dv + ncol;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i < mt) {
#pragma unroll
                for (int j = 0; j < IW_NTW; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Wf[(int64_t)(16 * i + r) * p.dv + 16 * j] = acc[i][j][r] * p.eta_scalar;
            }
        }
    }
}

__global__ __launch_bounds__(IW_NT) void ip_update_wide_kernel(IpUpdateParams p) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[IW_NB * IW_SA];
    __shared__ __attribute__((aligned(16))) bf16_t sB[IW_NB * IW_SB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles_n = p.dv / IW_BN;
    // logical order (bh, row tile, column tile): an XCD runs a contiguous
    // range, i.e. a few row tiles with all their column tiles, which share
    // the row tiles' Z columns through its L2
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    const int tile = lid % gridDim.x;
    const int m0 = (tile / tiles_n) * IW_BM, n0 = (tile % tiles_n) * IW_BN;
    const int bh = lid / gridDim.x, b = bh / p.H, h = bh % p.H;
    const bf16_t* Zg = p.k + b * p.ks[0] + h * p.ks[1] + m0;
    const bf16_t* Vg = p.v + b * p.vs[0] + h * p.vs[1] + n0;
    ip_wide_body(p, sA, sB, wave, lane, m0, n0, bh, Zg, Vg);
}

// ------------------------------------------------------------------ pass 2
// O_c^T tile [256 dv][256 tokens] = snap_c^T [dv][dk] x Z_c^T (snapshots in
// the blocked [dk/16][dv][16] layout); grid.x =
// nchunks * (chunk/256) * (dv/256), grid.y = B*H.
struct IpReadoutParams {
    const bf16_t* q;          // Z [B,H,L,dk]
    int64_t qs[3];
    bf16_t* out;              // O [B,H,L,dv]
    int64_t os[3];
    const bf16_t* snap;
    int H, L, dk, dv, chunk, nchunks;
};

// Readout LDS tiles: [256 rows][32 k] bf16 with 64-byte rows (4 chunks of
// 16 bytes), chunk c of row r stored at c ^ ((r >> 2) & 3): conflict-free for
// the row-order staging writes and for the fragment reads (16 rows per pass).
TTT_DEV int ro_swz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(IP_NT) void ip_readout_kernel(IpReadoutParams p) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][IP_BM * IP_BK];    // snap^T [n][k]
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][IP_BN * IP_BK];    // Z      [t][k]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = p.dv / IP_BM;                 // dv tiles
    const int tiles_t = p.chunk / IP_BN;              // token tiles per chunk
    // logical order (bh, chunk, dv tile, token tile): one XCD runs the tiles
    // of one chunk together, so they share the chunk's Z rows and snapshot
    // columns through its L2; with the token tiles innermost, the tiles that
    // read one snapshot column block run at the same time (read once from
    // memory; the Z rows, a third of the snapshot's bytes, are the operand
    // read again when a chunk's tiles straddle two rounds of the XCD's CUs)
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    int x = lid % gridDim.x;
    const int tt = x % tiles_t;
    x /= tiles_t;
    const int nt = x % tiles_n;
    const int chunk = x / tiles_n;
    const int n0 = nt * IP_BM;                        // dv offset
    const int t0 = chunk * p.chunk + tt * IP_BN;      // token offset
    const int bh = lid / gridDim.x, b = bh / p.H, h = bh % p.H;
    if (t0 >= p.L) return;                            // whole tile past the end (uniform)
    const bf16_t* S = p.snap + ((int64_t)bh * p.nchunks + chunk) * p.dk * p.dv + (int64_t)n0 * 16;
    const bf16_t* Zt = p.q + b * p.qs[0] + h * p.qs[1] + (int64_t)t0 * p.qs[2];
    bf16_t* Og = p.out + b * p.os[0] + h * p.os[1];
    const int L = p.L;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // staging: 256 rows x 4 chunks per operand, thread -> 4 (row, chunk) pairs;
    // per-lane offsets are the same for every K-step, which moves them by 32
    // elements (Z) or two 16-row blocks of the snapshot (token rows past L
    // read row L-1: their outputs are never stored)
    constexpr int NS = 4;                             // K-steps of loads in flight
    u32x4 ra[NS][4], rb[NS][4];
    uint32_t aoff[4], boff[4];
    int loff[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) {
        const int u = tid + y * IP_NT, row = u >> 2, c = u & 3;
        aoff[y] = (uint32_t)((c >> 1) * 16 * p.dv + row * 16 + 8 * (c & 1));
        boff[y] = (uint32_t)(min(row, L - 1 - t0) * (int)p.qs[2] + 8 * c);
        loff[y] = row * IP_BK + 8 * (c ^ ro_swz(row));
    }
    const int steps = p.dk / IP_BK;
    auto load = [&](int st, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
        const int s = min(st, steps - 1), k0 = s * IP_BK;
        const uint32_t a0 = (uint32_t)s * (uint32_t)(IP_BK * p.dv);   // two 16-row blocks per step
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            ra[k][y] = *reinterpret_cast<const u32x4*>(S + (aoff[y] + a0));
            rb[k][y] = *reinterpret_cast<const u32x4*>(Zt + boff[y] + k0);
        }
    };
    auto stage = [&](int buf, auto SET) __attribute__((always_inline)) {
        constexpr int k = decltype(SET)::value;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            *reinterpret_cast<u32x4*>(&sA[buf][loff[y]]) = ra[k][y];
            *reinterpret_cast<u32x4*>(&sB[buf][loff[y]]) = rb[k][y];
        }
    };
    // fragment reads: lane -> row r0 + lane%32 (r0 a multiple of 32), k half lane/32
    const int lrow = lane & 31;
    const int fb0 = lrow * IP_BK + 8 * ((lane >> 5) ^ ro_swz(lrow));        // kk = 0
    const int fb1 = lrow * IP_BK + 8 * ((2 | (lane >> 5)) ^ ro_swz(lrow));  // kk = 16
    // The k = 0 fragments of a step are read right after the barrier that
    // publishes its buffer, while the last row of the previous step's k = 16
    // products is still to be issued: those products cover the LDS latency
    // that would otherwise stall the matrix core after every barrier.
    bf16x8 a0[4], b0[4], a1[4], b1[4];
    auto read_k0 = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[i] = *reinterpret_cast<const bf16x8*>(sA[buf] + (128 * wm + 32 * i) * IP_BK + fb0);
#pragma unroll
        for (int j = 0; j < 4; ++j) b0[j] = *reinterpret_cast<const bf16x8*>(sB[buf] + (128 * wn + 32 * j) * IP_BK + fb0);
    };
    auto compute_head = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a1[i] = *reinterpret_cast<const bf16x8*>(sA[buf] + (128 * wm + 32 * i) * IP_BK + fb1);
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[j] = *reinterpret_cast<const bf16x8*>(sB[buf] + (128 * wn + 32 * j) * IP_BK + fb1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma32(acc[i][j], a0[i], b0[j]);
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma32(acc[i][j], a1[i], b1[j]);
    };
    auto compute_tail = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) mma32(acc[3][j], a1[3], b1[j]);
    };

    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    using K2 = std::integral_constant<int, 2>;
    using K3 = std::integral_constant<int, 3>;
    load(0, K0{});
    load(1, K1{});
    load(2, K2{});
    load(3, K3{});
    stage(0, K0{});
    __syncthreads();
    read_k0(0);
    auto step = [&](int st, auto CUR, auto NXT) __attribute__((always_inline)) {
        load(st + NS, CUR);
        compute_head(st & 1);
        __builtin_amdgcn_sched_barrier(0);
        // unconditional (clamped, unused data after the last step): no path
        // skips the wait for this set's loads
        stage((st + 1) & 1, NXT);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        read_k0((st + 1) & 1);     // after the last step: unused
        compute_tail();
        __builtin_amdgcn_sched_barrier(0);
    };
    // steps is a multiple of 8 (dk a multiple of 256)
    for (int st = 0; st < steps; st += NS) {
        step(st, K0{}, K1{});
        step(st + 1, K1{}, K2{});
        step(st + 2, K2{}, K3{});
        step(st + 3, K3{}, K0{});
    }

    // acc[i][j]: O^T[n][t], lane = token column, 4 consecutive n per group.
    // The output rows leave through LDS ([token][n], 512-byte rows) as whole
    // 16-byte pieces, 32 tokens (one j of one wave column) per pass, in the
    // K-loop's A buffers (free now).
    constexpr int ORW = IP_BM + 8;   // staged row: 256 n values + pad
    bf16_t* sO = &sA[0][0];
    static_assert(32 * ORW <= 2 * IP_BM * IP_BK, "staging fits the A buffers");
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
        const int j = pass % 4;
        __syncthreads();
        if (wn == pass / 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v4 = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                           acc[i][j][4 * q + 3]};
                    st4(&sO[(lane & 31) * ORW + 128 * wm + 32 * i + 8 * q + 4 * (lane >> 5)], v4);
                }
        }
        __syncthreads();
        constexpr int PR = IP_BM / 8;   // 16-byte pieces per row
        for (int x = tid; x < 32 * PR; x += IP_NT) {
            const int r = x / PR, c = x % PR, t = t0 + 32 * pass + r;
            if (t < L)
                *reinterpret_cast<u32x4*>(Og + t * p.os[2] + n0 + 8 * c) =
                    *reinterpret_cast<const u32x4*>(&sO[r * ORW + 8 * c]);
        }
    }
}

bool inplace_supported(int dtype, int dk, int dv, int chunk) {
    // IP_BN is a multiple of the update tile IPU_BN; snapshot offsets are 32-bit
    return dtype == 1 && dk % IP_BM == 0 && dv % IP_BN == 0 && chunk % IP_BN == 0 && dk >= IP_BM &&
           dv >= IP_BN && (int64_t)dk * dv < (int64_t(1) << 31);
}

// 256 token rows of any operand stay below 2^31 bytes from a tile's first row
bool inplace_strides_ok(int64_t q_row, int64_t k_row, int64_t v_row) {
    const int64_t lim = (int64_t(1) << 31) / (2 * IP_BN);
    return q_row < lim && k_row < lim && v_row < lim;
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
    if (ip_wide_supported(u, p.eta || p.eta_scalar == 0.f)) {
        const dim3 gw((p.dk / IW_BM) * (p.dv / IW_BN), p.B * p.H);
        hipLaunchKernelGGL(ip_update_wide_kernel, gw, dim3(IW_NT), 0, s, u);
    } else {
    const dim3 g1((p.dk / IP_BM) * (p.dv / IPU_BN), p.B * p.H);
    if (p.eta || p.eta_scalar == 0.f) {
        hipLaunchKernelGGL(ip_update_kernel<true>, g1, dim3(IP_NT), 0, s, u);
    } else {
        hipLaunchKernelGGL(ip_update_kernel<false>, g1, dim3(IP_NT), 0, s, u);
    }
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
