// gemm.h -- bf16 MFMA GEMM main loops for gfx950, shared by the kernels
// whose work is a plain dense contraction with a fused epilogue (the
// SwiGLU fast weight, the In-Place front end).
//
// C[BM x BN] += A[BM x K] B[BN x K]^T per workgroup: 256 threads as 2 x 2
// waves, each wave TI x TJ tiles of v_mfma_f32_32x32x16_bf16 (block tile
// 64 TI x 64 TJ), K-steps of 32.  Accumulator (i, j, r) of a lane holds row
// 32 TI wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4 and column
// 32 TJ wn + 32 j + lane % 32 of the block tile (acc_row / acc_col).
//
// Two operand layouts, one fragment order (lane l: row r0 + l % 32,
// k = k0 + 8 (l / 32) + 0..7):
//   KROW = false  row-major, K contiguous (weights [out][in], token rows
//                 contracted over features); LDS [row][32] with a 16-byte
//                 XOR swizzle.
//   KROW = true   token-major data contracted over tokens; fragments through
//                 the transposing LDS read ds_read_b64_tr_b16.
// Two loops:
//   Loop   global loads staged through registers (2-4 K-steps in flight),
//          two LDS buffers.
//   DLoop  gfx950 16-byte direct global-to-LDS loads into a ring of three
//          LDS buffers; one plain s_barrier per K-step, with explicit
//          s_waitcnt vmcnt accounting of the wave's own loads.
#pragma once
#include "common.h"

#include <type_traits>

namespace ttt {
namespace gemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int GM_BK = 32;      // k per step
constexpr int GM_NT = 256;     // threads per workgroup (2 x 2 waves)
constexpr int GM_NS = 4;       // k-steps of loads in flight
constexpr int GM_PAD = 32;     // [k][row] LDS tiles: 64-byte row pad

TTT_DEV void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
TTT_DEV int swz(int r) { return (r >> 2) & 3; }

// gfx950 transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane a loads 4 consecutive 16-bit values; lane i then holds the
// values lanes 4j + i/4 loaded in slot i%4 (j = 0..3).
TTT_DEV u32x2 ds_read_tr(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// One operand of C = A B^T: R = 64 T rows of the block tile, K elements each.
//   KROW = false: row-major, K contiguous ([row][k] in memory); LDS tile
//                 [row][32] with a 16-byte XOR swizzle.
//   KROW = true : token-major data contracted over tokens ([k][row] in
//                 memory); LDS tile [32][row + pad], fragments by the
//                 transposing read.
// Both give lane l the fragment of row r0 + l % 32, k = k0 + 8 (l / 32) + 0..7.
template <bool KROW, int T>
struct Opnd {
    static constexpr int R = 64 * T;
    static constexpr int LD = KROW ? R + GM_PAD : GM_BK;
    static constexpr int BUF = KROW ? GM_BK * LD : R * GM_BK;   // elements per LDS buffer
    const bf16_t* base;   // wave-uniform
    uint32_t off[T];      // element offsets of this thread's 16-byte pieces
    int kr[T];
    int lo[T];
    uint32_t ld;
    int lim;

    // KROW = false: rows off0 .. off0 + R - 1 of a [rows][ld] matrix at b,
    // rows >= rowlim clamped.  KROW = true: columns off0 .. off0 + R - 1 of
    // a [k][ld] matrix at b, k rows >= rowlim clamped.  Offsets from b stay
    // below 2^31 elements (checked by the launcher).
    TTT_DEV void init(const bf16_t* b, int ld_, int off0, int rowlim, int tid) {
        base = b;
        ld = (uint32_t)ld_;
        lim = rowlim;
#pragma unroll
        for (int y = 0; y < T; ++y) {
            const int u = tid + y * GM_NT;
            if (!KROW) {
                const int r = u >> 2, c = u & 3;
                off[y] = (uint32_t)min(off0 + r, rowlim - 1) * ld + 8 * c;
                lo[y] = r * GM_BK + 8 * (c ^ swz(r));
                kr[y] = 0;
            } else {
                const int kk = u / (8 * T), c = u % (8 * T);
                off[y] = (uint32_t)(off0 + 8 * c);
                kr[y] = kk;
                lo[y] = kk * LD + 8 * c;
            }
        }
    }
    TTT_DEV u32x4 load(int y, int st) const {
        if (!KROW) return *reinterpret_cast<const u32x4*>(base + (off[y] + (uint32_t)(st * GM_BK)));
        const uint32_t t = (uint32_t)min(st * GM_BK + kr[y], lim - 1);
        return *reinterpret_cast<const u32x4*>(base + (off[y] + t * ld));
    }
    TTT_DEV bf16x8 frag(const bf16_t* s, int r0, int k0, int lane) const {
        if (!KROW) {
            const int row = r0 + (lane & 31);
            const int c = (k0 >> 3) + (lane >> 5);
            return *reinterpret_cast<const bf16x8*>(s + row * GM_BK + 8 * (c ^ swz(row)));
        }
        const int G = lane >> 4, a = lane & 15;
        const int rb = r0 + 16 * (G & 1) + 4 * (a & 3);
        const int kk = k0 + 8 * (G >> 1) + (a >> 2);
        const u32x2 lo2 = ds_read_tr(s + (kk + 0) * LD + rb);
        const u32x2 hi2 = ds_read_tr(s + (kk + 4) * LD + rb);
        return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    }
};

// TI x TJ accumulator tiles of 32 x 32 per wave: block tile (64 TI) x (64 TJ)
template <int TI, int TJ>
using Acc = f32x16[TI][TJ];

template <int TI, int TJ>
TTT_DEV void zero(Acc<TI, TJ>& acc) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// acc += A B^T over `steps` k-steps of 32 (steps a multiple of 4): NS
// k-steps of global loads in flight in registers, two LDS buffers.
template <int K>
using IC = std::integral_constant<int, K>;

template <bool AK, bool BKR, int TI, int TJ, int NS = GM_NS>
struct Loop {
    using OA = Opnd<AK, TI>;
    using OB = Opnd<BKR, TJ>;
    static constexpr int LDS = 2 * (OA::BUF + OB::BUF);
    static_assert(NS >= 2 && NS <= 4, "2 to 4 register sets");

    TTT_DEV static void run(Acc<TI, TJ>& acc, int steps, const OA& a, const OB& b, bf16_t* smem, int tid) {
        bf16_t* sA = smem;
        bf16_t* sB = smem + 2 * OA::BUF;
        const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
        u32x4 ra[NS][TI], rb[NS][TJ];
        auto load = [&](int st, auto SET) __attribute__((always_inline)) {
            constexpr int k = decltype(SET)::value;
            const int s = min(st, steps - 1);
#pragma unroll
            for (int y = 0; y < TI; ++y) ra[k][y] = a.load(y, s);
#pragma unroll
            for (int y = 0; y < TJ; ++y) rb[k][y] = b.load(y, s);
        };
        auto stage = [&](int buf, auto SET) __attribute__((always_inline)) {
            constexpr int k = decltype(SET)::value;
#pragma unroll
            for (int y = 0; y < TI; ++y) *reinterpret_cast<u32x4*>(&sA[buf * OA::BUF + a.lo[y]]) = ra[k][y];
#pragma unroll
            for (int y = 0; y < TJ; ++y) *reinterpret_cast<u32x4*>(&sB[buf * OB::BUF + b.lo[y]]) = rb[k][y];
        };
        auto compute = [&](int buf) __attribute__((always_inline)) {
            const bf16_t* A = sA + buf * OA::BUF;
            const bf16_t* B = sB + buf * OB::BUF;
#pragma unroll
            for (int kk = 0; kk < GM_BK; kk += 16) {
                bf16x8 af[TI], bfr[TJ];
#pragma unroll
                for (int i = 0; i < TI; ++i) af[i] = a.frag(A, 32 * TI * wm + 32 * i, kk, lane);
#pragma unroll
                for (int j = 0; j < TJ; ++j) bfr[j] = b.frag(B, 32 * TJ * wn + 32 * j, kk, lane);
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) mma32(acc[i][j], af[i], bfr[j]);
            }
        };
        load(0, IC<0>{});
        load(1, IC<1>{});
        if constexpr (NS > 2) load(2, IC<2>{});
        if constexpr (NS > 3) load(3, IC<3>{});
        stage(0, IC<0>{});
        __syncthreads();
        // refill the set this step frees, compute from LDS, write step st+1
        // to the other LDS buffer.  The write is unconditional (after the last
        // step it stores clamped, unused data into the idle buffer): a
        // conditional write leaves a path on which the set's load was never
        // waited for, and the wait the compiler then puts before the next
        // reuse of those registers stalls every step.
        auto step = [&](int st, auto CUR, auto NXT) __attribute__((always_inline)) {
            load(st + NS, CUR);
            compute(st & 1);
            __builtin_amdgcn_sched_barrier(0);
            stage((st + 1) & 1, NXT);
            __syncthreads();
        };
        if constexpr (NS == 2 || NS == 4) {
            // steps is a multiple of 4: whole groups, no branch inside
            for (int st = 0; st < steps; st += NS) {
                step(st, IC<0>{}, IC<1 % NS>{});
                step(st + 1, IC<1 % NS>{}, IC<2 % NS>{});
                if constexpr (NS > 3) {
                    step(st + 2, IC<2>{}, IC<3>{});
                    step(st + 3, IC<3>{}, IC<0>{});
                }
            }
        } else {
            for (int st = 0; st < steps; st += NS) {
                step(st, IC<0>{}, IC<1>{});
                if (st + 1 < steps) step(st + 1, IC<1>{}, IC<2>{});
                if (st + 2 < steps) step(st + 2, IC<2>{}, IC<0>{});
            }
        }
    }
};

// ------------------------------------------------ direct global -> LDS loads
// The same GEMM loop with gfx950's 16-byte global_load_lds: each load
// instruction writes the wave's 64 x 16 bytes to consecutive LDS addresses,
// so the data never pass through VGPRs.  Three LDS buffers form a ring: at
// step st the loads of step st + 2 are issued right after the barrier that
// ends everyone's reads of step st - 1, and step st's loads are waited for
// (s_waitcnt vmcnt, own loads) just before that barrier.

TTT_DEV void dma16(const bf16_t* g, bf16_t* lds) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(g), (lds_void_t*)(lds), 16, 0, 0);
}

// KROW = false: LDS [R][32] with the 16-byte XOR swizzle of Opnd; lane l of
// load y of wave w fills row 64 y + 16 w + l / 4, position l % 4, i.e. the
// global chunk (l % 4) ^ swz(row).
// KROW = true: LDS [32][R] without pad; logical 16-byte chunk c of k row kk
// sits at position c ^ 2 (kk % 4), which keeps the transposing reads of four
// consecutive k rows on distinct banks.  Load y of wave w fills k rows
// (32 y + 8 w) / T + l / (8 T), lane l at position l % (8 T).
template <bool KROW, int T>
struct Dop {
    static constexpr int R = 64 * T;
    static constexpr int BUF = GM_BK * R;   // elements per LDS buffer, both layouts
    const bf16_t* gp[T];   // KROW = false: this lane's 16-byte piece at step 0
    const bf16_t* base;    // KROW = true: wave-uniform base
    uint32_t off[T];       // KROW = true: column offset of this lane's piece
    int kr[T];             // KROW = true: k row within a step
    int dst[T];            // wave's LDS offset (elements) within a buffer
    uint32_t ld;
    int lim;

    // KROW = false only: rowptr(r) is the start of the operand's row r
    // (r < R), already clamped by the caller.
    template <class F>
    TTT_DEV void init_rows(F rowptr, int tid) {
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
#pragma unroll
        for (int y = 0; y < T; ++y) {
            const int r = 64 * y + 16 * w + (l >> 2);
            gp[y] = rowptr(r) + 8 * ((l & 3) ^ swz(r));
            dst[y] = (64 * y + 16 * w) * GM_BK;
        }
    }
    // KROW = false: rows off0 .. off0 + R - 1 of a [rows][ld] matrix at b,
    // rows >= rowlim clamped.  KROW = true: columns off0 .. off0 + R - 1 of
    // a [k][ld] matrix at b, k rows >= rowlim clamped; offsets from b stay
    // below 2^31 elements.
    TTT_DEV void init(const bf16_t* b, int ld_, int off0, int rowlim, int tid) {
        if (!KROW) {
            init_rows([&](int r) { return b + (int64_t)min(off0 + r, rowlim - 1) * ld_; }, tid);
            return;
        }
        base = b;
        ld = (uint32_t)ld_;
        lim = rowlim;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
#pragma unroll
        for (int y = 0; y < T; ++y) {
            const int row0 = (32 * y + 8 * w) / T;
            const int kk = row0 + l / (8 * T), pos = l % (8 * T);
            off[y] = (uint32_t)(off0 + 8 * (pos ^ (2 * (kk & 3))));
            kr[y] = kk;
            dst[y] = row0 * R;
        }
    }
    TTT_DEV void load(int st, bf16_t* buf) const {
#pragma unroll
        for (int y = 0; y < T; ++y) {
            if (!KROW) dma16(gp[y] + st * GM_BK, buf + dst[y]);
            else dma16(base + (off[y] + (uint32_t)min(st * GM_BK + kr[y], lim - 1) * ld), buf + dst[y]);
        }
    }
    TTT_DEV bf16x8 frag(const bf16_t* s, int r0, int k0, int lane) const {
        if (!KROW) {
            const int row = r0 + (lane & 31);
            const int c = (k0 >> 3) + (lane >> 5);
            return *reinterpret_cast<const bf16x8*>(s + row * GM_BK + 8 * (c ^ swz(row)));
        }
        const int G = lane >> 4, a = lane & 15;
        const int rb = r0 + 16 * (G & 1) + 4 * (a & 3);
        const int kk = k0 + 8 * (G >> 1) + (a >> 2);
        const int pos = 8 * ((rb >> 3) ^ (2 * (kk & 3))) + (rb & 7);
        const u32x2 lo2 = ds_read_tr(s + (kk + 0) * R + pos);
        const u32x2 hi2 = ds_read_tr(s + (kk + 4) * R + pos);
        return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    }
};

template <bool AK, bool BKR, int TI, int TJ>
struct DLoop {
    using OA = Dop<AK, TI>;
    using OB = Dop<BKR, TJ>;
    static constexpr int NB = 3;
    static constexpr int LDS = NB * (OA::BUF + OB::BUF);
    static constexpr int NLOAD = TI + TJ;   // load instructions per thread and step

    TTT_DEV static void run(Acc<TI, TJ>& acc, int steps, const OA& a, const OB& b, bf16_t* smem, int tid) {
        bf16_t* sA = smem;
        bf16_t* sB = smem + NB * OA::BUF;
        const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
        // loads of step st into the stage buffers wa, wb
        auto issue = [&](int st, bf16_t* wa, bf16_t* wb) __attribute__((always_inline)) {
            const int s = min(st, steps - 1);
            a.load(s, wa);
            b.load(s, wb);
        };
        auto compute = [&](const bf16_t* A, const bf16_t* B) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < GM_BK; kk += 16) {
                bf16x8 af[TI], bfr[TJ];
#pragma unroll
                for (int i = 0; i < TI; ++i) af[i] = a.frag(A, 32 * TI * wm + 32 * i, kk, lane);
#pragma unroll
                for (int j = 0; j < TJ; ++j) bfr[j] = b.frag(B, 32 * TJ * wn + 32 * j, kk, lane);
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j) mma32(acc[i][j], af[i], bfr[j]);
            }
        };
        // vmcnt field of s_waitcnt on gfx9: bits 3..0 and 15..14; lgkmcnt and
        // expcnt left at their maxima (no wait)
        constexpr int WAIT_ONE_STEP = (NLOAD & 15) | ((NLOAD >> 4) << 14) | (0x7 << 4) | (0xf << 8);
        issue(0, sA, sB);
        issue(1, sA + OA::BUF, sB + OB::BUF);
        for (int st = 0; st < steps; ++st) {
            // this wave's loads of step st are done once only step st + 1's are
            // left; the barrier makes everyone's done and ends everyone's reads
            // of the buffer that step st + 2 refills
            __builtin_amdgcn_s_waitcnt(WAIT_ONE_STEP);
            __builtin_amdgcn_s_barrier();
            const int rd = st % NB, wr = (st + 2) % NB;
            ring_step(sA + wr * OA::BUF, sB + wr * OB::BUF, sA + rd * OA::BUF, sB + rd * OB::BUF,
                      [&](bf16_t* wa, bf16_t* wb) __attribute__((always_inline)) { issue(st + 2, wa, wb); }, compute);
        }
        // drain the clamped loads still in flight before the LDS is reused
        __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
        __builtin_amdgcn_s_barrier();
    }
};

// Workgroup -> (head, row tile, column tile).  Heads are contiguous ranges of
// logical ids (xcd_logical: one XCD runs one contiguous range); within a
// head, groups of 8 column tiles walk all row tiles.
TTT_DEV void tile_id(int nrow, int ncol, int* bh, int* rt, int* ct) {
    const int n = nrow * ncol;
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    *bh = lid / n;
    const int t = lid % n;
    constexpr int G = 8;
    const int group = t / (G * nrow), first = group * G;
    const int gsz = min(G, ncol - first);
    const int r = t % (G * nrow);
    *ct = first + r % gsz;
    *rt = r / gsz;
}

// accumulator (i, j, r) -> row 32 TI wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,
// column 32 TJ wn + 32 j + lane % 32 of the block tile
template <int TI>
TTT_DEV int acc_row(int wm, int i, int q, int lane) { return 32 * TI * wm + 32 * i + 8 * q + 4 * (lane >> 5); }
template <int TJ>
TTT_DEV int acc_col(int wn, int j, int lane) { return 32 * TJ * wn + 32 * j + (lane & 31); }

}  // namespace gemm
}  // namespace ttt
