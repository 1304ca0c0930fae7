// dual.hip -- TTT-Linear mini-batch forward (MSE reconstruction), dual form.
//
// [P4] ("RNN의 기억을 작은 모델로 바꾼다면: Test-Time Training 읽기", ariser.io),
// section on making the gradient an efficient layer: tokens are grouped in
// mini-batches, every gradient of mini-batch n is taken at W_n, and the dual
// form evaluates exactly that mini-batch update with matrix products.  For
// token t of mini-batch n (inner model f(k) = k W, loss 1/2||kW - v||^2):
//     W_{n,t} = W_n - eta sum_{s<=t in n} k_s^T (k_s W_n - v_s),  o_t = q_t W_{n,t}.
//
// Kernel form.  Inside a mini-batch the update is linear attention that
// starts from W_n with corrected values v~_s = -eta (k_s W_n - v_s): with the
// running state S~ (S~ = W_n at the mini-batch start), each sub-chunk of up
// to 32 tokens computes
//     E   = K W_n,        V~ = eta (V - E)
//     O^T = S~^T Q^T + V~^T P^T,   P^T = tril(K Q^T)
//     S~ += K^T V~
// and W_{n+1} is S~ at the end of the mini-batch.  This needs no b x b score
// matrix, so a 2048-token mini-batch costs what 64 sub-chunks cost.
//
// Mapping: one workgroup per (b, h); wave w owns output / state columns
// [16w, 16w+16).  W_n, S~, E and V~ never leave the VGPRs: accumulator
// tiles feed the next contraction in the accperm k-assignment (common.h),
// so the sequential chain of mini-batches has no LDS round trip for state.
// Q, K, K^T and V^T of a sub-chunk are staged in LDS by the whole group.
#include "common.h"
#include "internal.h"

#include <type_traits>
#include <utility>

namespace ttt {

template <typename T> struct DSeg;
template <> struct DSeg<bf16_t> { u32x4 w; };
template <> struct DSeg<float> { u32x4 w0, w1; };
TTT_DEV void dseg_load(DSeg<bf16_t>& s, const bf16_t* p) { s.w = *reinterpret_cast<const u32x4*>(p); }
TTT_DEV void dseg_load(DSeg<float>& s, const float* p) {
    s.w0 = reinterpret_cast<const u32x4*>(p)[0];
    s.w1 = reinterpret_cast<const u32x4*>(p)[1];
}
TTT_DEV void dseg_zero(DSeg<bf16_t>& s) { s.w = u32x4{0, 0, 0, 0}; }
TTT_DEV void dseg_zero(DSeg<float>& s) { s.w0 = s.w1 = u32x4{0, 0, 0, 0}; }
TTT_DEV void dseg_store(bf16_t* p, const DSeg<bf16_t>& s) { *reinterpret_cast<u32x4*>(p) = s.w; }
TTT_DEV void dseg_store(float* p, const DSeg<float>& s) {
    reinterpret_cast<u32x4*>(p)[0] = s.w0;
    reinterpret_cast<u32x4*>(p)[1] = s.w1;
}
TTT_DEV float dseg_elem(const DSeg<bf16_t>& s, int e) {
    return bf2f((uint16_t)(s.w[e >> 1] >> (16 * (e & 1))));
}
TTT_DEV float dseg_elem(const DSeg<float>& s, int e) {
    return __uint_as_float(e < 4 ? s.w0[e] : s.w1[e - 4]);
}
TTT_DEV void dst_col4(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2bf(a, b), pack2bf(c, d)};
}
TTT_DEV void dst_col4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
TTT_DEV f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
TTT_DEV f32x4 ld4(const bf16_t* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}
// accumulator tiles -> operand fragment for K-block kb (accperm)
TTT_DEV f32x4 tiles_frag(const f32x4* t, int kb, float) { return t[kb]; }
TTT_DEV bf16x8 tiles_frag(const f32x4* t, int kb, bf16_t) { return acc_to_frag_bf16(t[2 * kb], t[2 * kb + 1]); }

template <typename T, int D, int DV>
__global__ __launch_bounds__(DV / 16 * 64) void dual_fwd_kernel(DualParams p) {
    constexpr int SB = 32;                    // sub-chunk tokens
    constexpr int NW = DV / 16;
    constexpr int NT = NW * 64;
    constexpr int KB = Tr<T>::KB;
    constexpr int PR = 16 / sizeof(T);
    constexpr int LDQ = D + PR;
    constexpr int LDT = SB + PR;
    constexpr int NTD = D / 16;               // state tiles along d
    constexpr int NKB = D / KB;               // K-blocks along d
    constexpr int NJT = SB / 16;              // token tiles in a sub-chunk
    constexpr int NJB = SB / KB;              // K-blocks along tokens
    constexpr int NUQ = (SB / 4) * (D / 8);
    constexpr int NUV = (SB / 4) * (DV / 8);
    constexpr int UQ = (NUQ + NT - 1) / NT;
    constexpr int UV = (NUV + NT - 1) / NT;
    using frag = typename Tr<T>::frag;

    __shared__ __attribute__((aligned(16))) T sQ[SB * LDQ];
    __shared__ __attribute__((aligned(16))) T sK[SB * LDQ];
    __shared__ __attribute__((aligned(16))) T sKT[D * LDT];
    __shared__ __attribute__((aligned(16))) T sVT[DV * LDT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int bh = blockIdx.x;
    const int L = p.L, mb = p.minibatch;
    const float eta = p.eta;
    const T* Qg = reinterpret_cast<const T*>(p.q) + (int64_t)bh * L * D;
    const T* Kg = reinterpret_cast<const T*>(p.k) + (int64_t)bh * L * D;
    const T* Vg = reinterpret_cast<const T*>(p.v) + (int64_t)bh * L * DV;
    T* Og = reinterpret_cast<T*>(p.out) + (int64_t)bh * L * DV;

    // running state S~ (fp32 accumulators): S~[16t + 4g + r][16*wave + c16]
    f32x4 Sacc[NTD];
    {
        const float* W0 = p.W0 + (int64_t)bh * p.W0_stride;
        const int col = 16 * wave + c16;
        for (int t = 0; t < NTD; ++t)
            for (int r = 0; r < 4; ++r) Sacc[t][r] = W0[(16 * t + 4 * g + r) * DV + col];
    }
    frag Sop[NKB], Wop[NKB];
    for (int kb = 0; kb < NKB; ++kb) Sop[kb] = tiles_frag(Sacc, kb, T());
    for (int kb = 0; kb < NKB; ++kb) Wop[kb] = Sop[kb];

    DSeg<T> qreg[UQ][4], kreg[UQ][4], vreg[UV][4];

    auto load = [&](int s0, int s1) {
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT;
            if (u < NUQ) {
                const int tb = u / (D / 8), db = u % (D / 8);
                for (int r = 0; r < 4; ++r) {
                    const int t = s0 + 4 * tb + r;
                    if (t < s1) {
                        dseg_load(qreg[x][r], Qg + (int64_t)t * D + 8 * db);
                        dseg_load(kreg[x][r], Kg + (int64_t)t * D + 8 * db);
                    } else {
                        dseg_zero(qreg[x][r]);
                        dseg_zero(kreg[x][r]);
                    }
                }
            }
        }
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT;
            if (u < NUV) {
                const int tb = u / (DV / 8), db = u % (DV / 8);
                for (int r = 0; r < 4; ++r) {
                    const int t = s0 + 4 * tb + r;
                    if (t < s1) dseg_load(vreg[x][r], Vg + (int64_t)t * DV + 8 * db);
                    else dseg_zero(vreg[x][r]);
                }
            }
        }
    };
    auto stage = [&]() {
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT;
            if (u < NUQ) {
                const int tb = u / (D / 8), db = u % (D / 8);
                for (int r = 0; r < 4; ++r) {
                    dseg_store(&sQ[(4 * tb + r) * LDQ + 8 * db], qreg[x][r]);
                    dseg_store(&sK[(4 * tb + r) * LDQ + 8 * db], kreg[x][r]);
                }
                for (int e = 0; e < 8; ++e)
                    dst_col4(&sKT[(8 * db + e) * LDT + 4 * tb], dseg_elem(kreg[x][0], e),
                             dseg_elem(kreg[x][1], e), dseg_elem(kreg[x][2], e), dseg_elem(kreg[x][3], e));
            }
        }
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT;
            if (u < NUV) {
                const int tb = u / (DV / 8), db = u % (DV / 8);
                for (int e = 0; e < 8; ++e)
                    dst_col4(&sVT[(8 * db + e) * LDT + 4 * tb], dseg_elem(vreg[x][0], e),
                             dseg_elem(vreg[x][1], e), dseg_elem(vreg[x][2], e), dseg_elem(vreg[x][3], e));
            }
        }
    };

    // sub-chunk walk: [s0, s1) inside mini-batch ending at mend
    int s0 = 0, mend = min(mb, L), s1 = min(SB, mend);
    load(s0, s1);
    __syncthreads();
    stage();
    __syncthreads();
    while (s0 < L) {
        // next sub-chunk
        int ns0 = s1, nmend = mend;
        if (ns0 == mend) nmend = min(ns0 + mb, L);
        const int ns1 = min(ns0 + SB, nmend);
        if (ns0 < L) load(ns0, ns1);

        // E = K W_n ; V~ = eta (V - E)   (tiles over tokens, this wave's 16 columns)
        f32x4 Vt[NJT];
        {
            const T* vrow = &sVT[(16 * wave + c16) * LDT];
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                f32x4 e = zero4();
                const T* krow = &sK[(16 * jt + c16) * LDQ];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) mma(e, ld_accperm(krow, kb * KB, g), Wop[kb]);
                const f32x4 vv = ld4(vrow + 16 * jt + 4 * g);
                for (int r = 0; r < 4; ++r) Vt[jt][r] = eta * (vv[r] - e[r]);
            }
        }
        frag VB[NJB];
        for (int jb = 0; jb < NJB; ++jb) VB[jb] = tiles_frag(Vt, jb, T());

        // P^T = tril(K Q^T): tiles (jt, it), jt <= it, as accumulators
        f32x4 P[NJT][NJT];
#pragma unroll
        for (int it = 0; it < NJT; ++it) {
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) {
                P[jt][it] = zero4();
                if (jt > it) continue;
                const T* arow = &sK[(16 * jt + c16) * LDQ];
                const T* brow = &sQ[(16 * it + c16) * LDQ];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    mma(P[jt][it], ld_contig<T>(arow, kb * KB, g), ld_contig<T>(brow, kb * KB, g));
                if (jt == it) {
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r > c16) P[jt][it][r] = 0.f;
                }
            }
        }

        // O^T = S~^T Q^T + V~^T P^T
#pragma unroll
        for (int it = 0; it < NJT; ++it) {
            f32x4 acc = zero4();
            const T* qrow = &sQ[(16 * it + c16) * LDQ];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma(acc, Sop[kb], ld_accperm(qrow, kb * KB, g));
            f32x4 col[NJT];
            for (int jt = 0; jt < NJT; ++jt) col[jt] = P[jt][it];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) mma(acc, VB[jb], tiles_frag(col, jb, T()));
            const int t = s0 + 16 * it + c16;
            if (t < s1) st4(&Og[(int64_t)t * DV + 16 * wave + 4 * g], acc);
        }

        // S~ += K^T V~
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const T* krow = &sKT[(16 * t + c16) * LDT];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) mma(Sacc[t], ld_accperm(krow, jb * KB, g), VB[jb]);
        }
        for (int kb = 0; kb < NKB; ++kb) Sop[kb] = tiles_frag(Sacc, kb, T());
        if (s1 == mend) {  // mini-batch done: W_{n+1} = S~
            for (int kb = 0; kb < NKB; ++kb) Wop[kb] = Sop[kb];
        }

        __syncthreads();
        s0 = ns0;
        s1 = ns1;
        mend = nmend;
        if (s0 < L) {
            stage();
            __syncthreads();
        }
    }

    if (p.W_final) {
        float* Wf = p.W_final + (int64_t)bh * D * DV;
        const int col = 16 * wave + c16;
        for (int t = 0; t < NTD; ++t)
            for (int r = 0; r < 4; ++r) Wf[(16 * t + 4 * g + r) * DV + col] = Sacc[t][r];
    }
}

// ------------------------------------------------------------------------
// dual_ring_kernel: bf16, d = dv = 64, mini-batches of a multiple of 16.
//
// The columns of W evolve independently under the linear MSE update (column
// j of E, V~ and S~ only involves column j of W and V), so each wave owns 16
// state columns of one (b, h) and runs its own chain with no barriers: 4 x
// (B*H) independent waves.  A step covers 16 tokens (never across a
// mini-batch boundary):
//     E = K W_n,  V~ = eta (V - E),  P^T = tril(K Q^T),
//     O^T = S~^T Q^T + V~^T P^T,  S~ += K^T V~,
// with W_{n+1} = S~ at the mini-batch end.  The critical path per step is
// E -> V~ -> S~ -> bf16(S~) -> next E; everything else hangs off it.
//
// Feature order: accumulator row position p = 32kb + 16h + 4g + i of the
// state holds feature d(p) = 32kb + 8g + 4h + i.  With that order the
// operand fragment of lane (g, row) for feature block kb is the 16 contiguous
// bytes X[row][32kb + 8g .. +8], so K and Q rows are MFMA operands as they
// sit in a row-major tile, and the state accumulators feed the next
// contraction from registers.  The two transposes the chain needs (V in the
// E layout, K^T for the state update) are ds_read_b64_tr_b16 reads of the
// same tiles.
typedef short s16x4d __attribute__((ext_vector_type(4)));

TTT_DEV u32x2 tr_read_d(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4d lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
// 16 x 16 x 16 product (k = 4g + j in lane group g) issued as a 16x16x32 MFMA
// whose upper k half is zero: lane slot j < 4 of both operands carries k =
// 4g + j, slots 4..7 are 0
TTT_DEV void mma16(f32x4& acc, const u32x2& a, const u32x2& b) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], 0u, 0u});
    const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{b[0], b[1], 0u, 0u});
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
}
// 8-byte chunk swizzle of the [16 tokens][64] K tile (rows of 16 chunks; bit 0
// untouched so 16-byte pairs stay whole): conflict-free row writes, at most
// two-way conflicts on the transposing reads
TTT_DEV int kswz(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 3); }
// feature of state row position p
TTT_DEV int feat(int p) { return (p & ~31) + 8 * ((p >> 2) & 3) + 4 * ((p >> 4) & 1) + (p & 3); }


// Operands reach LDS through a wave-private ring of DR_R stages of 32 tokens
// (two steps), filled by 16-byte direct loads, so no VGPR holds data in
// flight and nothing of the prefetch crosses the loop.  A stage holds the Q
// and K rows [32][64], the 16-byte unit u of row r at position
// u ^ (kswz(r mod 16) / 2), which gives row-fragment reads (MFMA operands of
// K and Q) and the transposing K^T reads of the state update without bank
// conflicts beyond two-way, and the wave's V tile [32][16] (read transposed
// into the E layout).  Rows past L lie outside the buffer ranges: they load
// as zero (a zero K row gives E = 0 and V~ = 0, so it adds nothing) and
// their stores are dropped, so no step needs a clamp or a mask.
constexpr int DR_R = 5;                         // ring stages
constexpr int DR_T = 64;                        // tokens per stage (four steps)
constexpr int DR_QK = DR_T * 64;                // elements of the Q (or K) part
constexpr int DR_STAGE = 2 * DR_QK + DR_T * 16; // elements per stage (18 KB)
constexpr int DR_NL = 18;                       // load instructions per stage

// ONESTEP: every mini-batch is exactly one 16-token step (W_n is S~ itself);
// STAGEEND: mini-batches end only at ring-stage ends (b a multiple of 64), so
// W_{n+1} = S~ is taken once per stage instead of tested every step
template <bool ONESTEP, bool STAGEEND>
__global__ __launch_bounds__(64) void dual_ring_kernel(DualParams p) {
    constexpr int D = 64, DV = 64;
    __shared__ __attribute__((aligned(16))) bf16_t ring[DR_R * DR_STAGE];

    const int lane = threadIdx.x, g = lane >> 4, c16 = lane & 15;
    // the 4 column waves of a head run on one XCD (shared Q/K rows in its L2)
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int bh = lid >> 2, w = lid & 3;
    const int L = p.L, mb = p.minibatch;
    const float eta = p.eta;
    const bf16_t* Qg = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)bh * L * D;
    const bf16_t* Kg = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)bh * L * D;
    const bf16_t* Vg = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)bh * L * DV + 16 * w;
    bf16_t* Og = reinterpret_cast<bf16_t*>(p.out) + (int64_t)bh * L * DV + 16 * w;

    // S~[feat(16t + 4g + r)][16w + c16], fp32
    f32x4 Sacc[4];
    {
        const float* W0 = p.W0 + (int64_t)bh * p.W0_stride;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sacc[t][r] = W0[feat(16 * t + 4 * g + r) * DV + 16 * w + c16];
    }
    bf16x8 Sop[2], Wop[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Sop[kb] = Wop[kb] = acc_to_frag_bf16(Sacc[2 * kb], Sacc[2 * kb + 1]);

    // one buffer descriptor per tensor of this head (range: the head's rows)
    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)Qg, 0, L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, L * DV * 2 - 32 * w, 0x00020000);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc((void*)Og, 0, L * DV * 2 - 32 * w, 0x00020000);
    // direct-load lane offsets (bytes from a stage's first token row): load i
    // of Q or K fills rows 8i .. 8i + 7, lane l the position l % 8 of row
    // 8i + l / 8; the V load fills the [32][16] tile, lane l half l % 2 of row l / 2
    uint32_t qko[DR_T / 8];
#pragma unroll
    for (int i = 0; i < DR_T / 8; ++i) {
        const int row = 8 * i + (lane >> 3);
        qko[i] = (uint32_t)(row * D * 2 + 16 * ((lane & 7) ^ (kswz(row & 15) >> 1)));
    }
    const uint32_t vdo = (uint32_t)((lane >> 1) * DV * 2 + 16 * (lane & 1));
    const int nsteps = (L + 15) / 16, nst = (nsteps + DR_T / 16 - 1) / (DR_T / 16);
    auto issue = [&](int s, bf16_t* dst) __attribute__((always_inline)) {
        const int sq = min(s, nst - 1) * DR_T * D * 2;   // bytes (D == DV)
#pragma unroll
        for (int i = 0; i < DR_T / 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_void_t*)(dst + 512 * i), 16, qko[i], sq, 0, 0);
#pragma unroll
        for (int i = 0; i < DR_T / 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void_t*)(dst + DR_QK + 512 * i), 16, qko[i], sq, 0, 0);
#pragma unroll
        for (int i = 0; i < DR_T / 32; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void_t*)(dst + 2 * DR_QK + 512 * i), 16, vdo, sq + 32 * DV * 2 * i,
                                                     0, 0);
    };

    // causal mask of the packed bf16 P^T pieces (j = 4g + r <= i = c16), fixed per lane
    u32x2 pmask;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        pmask[h] = ((4 * g + 2 * h <= c16) ? 0x0000ffffu : 0u) | ((4 * g + 2 * h + 1 <= c16) ? 0xffff0000u : 0u);
    // LDS addresses (elements within a step's rows)
    const int fro = c16 * D, fsw = kswz(c16) >> 1;           // row fragments
    const int rr = 4 * g + (c16 >> 2), cq = c16 & 3;         // transposing reads: row, chunk quad
    const int vr = rr * 16 + 4 * cq;
    const int kr = rr * D, krs = kswz(rr);
    const int vo = (c16 * DV + 4 * g) * 2;                   // output store (bytes)

    // step s16 (tokens 16 s16 ..), rows 16 j .. of the stage at X
    auto step = [&](const bf16_t* X, int j, int s16) __attribute__((always_inline)) {
        const bf16_t* Qs = X + 16 * j * D;
        const bf16_t* Ks = X + DR_QK + 16 * j * D;
        const bf16_t* Vs = X + 2 * DR_QK + 256 * j;
        const bf16x8 Kf0 = *reinterpret_cast<const bf16x8*>(Ks + fro + 8 * (g ^ fsw));
        const bf16x8 Kf1 = *reinterpret_cast<const bf16x8*>(Ks + fro + 8 * ((4 + g) ^ fsw));
        const bf16x8 Qf0 = *reinterpret_cast<const bf16x8*>(Qs + fro + 8 * (g ^ fsw));
        const bf16x8 Qf1 = *reinterpret_cast<const bf16x8*>(Qs + fro + 8 * ((4 + g) ^ fsw));
        // E[token 4g+r][col c16] = K W_n
        f32x4 e = zero4();
        mma(e, Kf0, ONESTEP ? Sop[0] : Wop[0]);
        mma(e, Kf1, ONESTEP ? Sop[1] : Wop[1]);
        // P^T[j 4g+r][i c16] = K Q^T, causal j <= i
        f32x4 pt = zero4();
        mma(pt, Kf0, Qf0);
        mma(pt, Kf1, Qf1);
        // O^T partial: S~^T Q^T with S~ as of the step start
        f32x4 o = zero4();
        mma(o, Sop[0], Qf0);
        mma(o, Sop[1], Qf1);
        // V in the E layout; V~ = eta (V - E), zero past L
        const u32x2 vraw = tr_read_d(Vs + vr);
        f32x4 vt;
        vt[0] = __uint_as_float(vraw[0] << 16);
        vt[1] = __uint_as_float(vraw[0] & 0xffff0000u);
        vt[2] = __uint_as_float(vraw[1] << 16);
        vt[3] = __uint_as_float(vraw[1] & 0xffff0000u);
#pragma unroll
        for (int r = 0; r < 4; ++r) vt[r] = eta * (vt[r] - e[r]);
        const u32x2 VB = u32x2{pack2bf(vt[0], vt[1]), pack2bf(vt[2], vt[3])};
        // S~ += K^T V~ : K^T tile t (positions 16t..) through the transposing read
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int chunk = 8 * (t >> 1) + 2 * cq + (t & 1);
            mma16(Sacc[t], tr_read_d(Ks + kr + 4 * (chunk ^ krs)), VB);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Sop[kb] = acc_to_frag_bf16(Sacc[2 * kb], Sacc[2 * kb + 1]);
        if (!ONESTEP && !STAGEEND) {
            const int t1 = 16 * s16 + 16;
            if (t1 % mb == 0 || t1 >= L) {   // mini-batch end: W_{n+1} = S~
                Wop[0] = Sop[0];
                Wop[1] = Sop[1];
            }
        }
        // O^T += V~^T P^T, store O rows (4 consecutive columns per lane)
        mma16(o, VB, u32x2{pack2bf(pt[0], pt[1]) & pmask[0], pack2bf(pt[2], pt[3]) & pmask[1]});
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, u32x2{pack2bf(o[0], o[1]), pack2bf(o[2], o[3])}),
                                              rO, vo, 16 * s16 * DV * 2, 0);
    };

    // vmcnt of s_waitcnt (gfx9: bits 3..0 and 15..14): in iteration s, after
    // stage s's loads this wave issued (DR_R - 2) stages of loads, 2 stores
    // per finished iteration and the stores of iteration s - DR_R + 1, never
    // fewer than (DR_R - 2) * DR_NL operations: waiting for that many left
    // has stage s in LDS (memory operations of a wave complete in order)
    constexpr int NW = (DR_R - 2) * DR_NL;
    static_assert(NW <= 63, "vmcnt holds 6 bits");
    constexpr int WAIT_STAGE = (NW & 15) | ((NW >> 4) << 14) | (0x7 << 4) | (0xf << 8);
#pragma unroll
    for (int s = 0; s < DR_R - 1; ++s) issue(s, ring + s * DR_STAGE);
    // ring offsets (elements) of the stage read and the stage refilled,
    // advanced with scalar adds (a modulo would cost vector address math)
    int rdo = 0, wro = (DR_R - 1) * DR_STAGE;
    for (int s = 0; s < nst; ++s) {
        __builtin_amdgcn_s_waitcnt(WAIT_STAGE);
        const int rd_off = rdo, wr_off = wro;
        rdo = (rdo + DR_STAGE == DR_R * DR_STAGE) ? 0 : rdo + DR_STAGE;
        wro = (wro + DR_STAGE == DR_R * DR_STAGE) ? 0 : wro + DR_STAGE;
        // the stage refilled here was read in iteration s - 1 (its reads were
        // consumed there); this step's reads go through their own pointer
        ring_step1(ring + __builtin_amdgcn_readfirstlane(wr_off), ring + __builtin_amdgcn_readfirstlane(rd_off),
                   [&](bf16_t* dst) __attribute__((always_inline)) { issue(s + DR_R - 1, dst); },
                   [&](const bf16_t* X) __attribute__((always_inline)) {
#pragma unroll
                       for (int j = 0; j < DR_T / 16; ++j) step(X, j, (DR_T / 16) * s + j);
                   });
        if (STAGEEND) {
            const int t1 = DR_T * (s + 1);
            if (t1 % mb == 0 || t1 >= L) {   // mini-batch end: W_{n+1} = S~
                Wop[0] = Sop[0];
                Wop[1] = Sop[1];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));   // the clamped loads still in flight

    if (p.W_final) {
        float* Wf = p.W_final + (int64_t)bh * D * DV;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wf[feat(16 * t + 4 * g + r) * DV + 16 * w + c16] = Sacc[t][r];
    }
}

// ------------------------------------------------------------------------
// dual_seg_kernel: the same chain with every sequence cut into segments of
// whole mini-batches that run concurrently.
//
// Over one mini-batch the update is affine in the state,
//     W_{n+1} = (I - eta K_n^T K_n) W_n + eta K_n^T V_n,
// so a segment maps the state it starts from to A W + B.  One workgroup of
// four waves (wave w: columns [16w, 16w + 16)) runs one (b, h, segment):
//   1. Every segment but the last runs its mini-batch chain from K and V
//      alone, twice at once: from W = 0, which ends at B, and from W = I,
//      which ends at A.  The second chain carries Delta = A - I (the state
//      minus I): its products take bf16(Delta), so the rounding of the
//      operand applies to the small part and not to I, whose share of
//      E = K A is the exact column slice of K.  Delta and B are published
//      behind a flag.
//   2. It composes its start state W = f_{s-1}(... f_0(W0)), f_j(W) =
//      W + Delta_j W + B_j, in the order of the segments (results do not
//      depend on timing).  The products use split operands, x = hi + lo
//      with hi = bf16(x), lo = bf16(x - hi), and three products per pair
//      (hi hi, lo hi, hi lo): about 16 bits of each operand.
//   3. It runs the forward over its own tokens from that state, as the
//      sequential kernel does.
// Q, K and V reach LDS through a ring of stages of 64 tokens shared by the
// waves of the workgroup (direct 16-byte loads, one barrier per stage); a
// stage is [64][64] Q, K and V tiles, 24 KB.
// Workgroups take tickets in segment order, so a segment only waits for
// workgroups that already run.
// ring stages: 4 with one four-wave workgroup per CU (96 KB), 3 with two
// two-wave workgroups per CU (72 KB each)
constexpr int dual_ring_stages(int nw) { return nw == 4 ? 4 : 3; }
#ifndef DUAL_GROUPED
#define DUAL_GROUPED 1
#endif
constexpr int DS_T = 64;                       // tokens per stage (four steps)
constexpr int DS_TILE = DS_T * 64;             // elements of one [64][64] tile
constexpr int DS_STAGE = 3 * DS_TILE;          // Q | K | V, elements per stage
constexpr int DS_MAP = 2 * 64 * 64 * 2 + 64 * 64 * 4;   // bytes of one segment map (Delta hi, lo; B)
constexpr int DS_MB = 4;                       // maps staged in the ring at a time (16 KB each)
constexpr int DS_BOFF = 2 * 64 * 64 * 2;       // byte offset of B in a map block
constexpr int DS_SC1 = 16;                     // cache policy: device-coherent (sc1)

template <int N, class F, int... I>
TTT_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
TTT_DEV void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// V tile swizzle: the 16-byte unit u of row r sits at position u ^ vswz(r),
// which spreads the 16 rows of a step's transposing reads over all banks
TTT_DEV int vswz(int r) { return 2 * ((r >> 1) & 3); }

TTT_DEV void dma16(__amdgpu_buffer_rsrc_t r, bf16_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
// the same, device-coherent (sc1)
TTT_DEV void dma16_sc1(__amdgpu_buffer_rsrc_t r, bf16_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 16);
}
// x = hi + lo for the four values of an accumulator slice, both as bf16
TTT_DEV void split4(const f32x4& x, u32x2& hi, u32x2& lo) {
    hi = u32x2{pack2bf(x[0], x[1]), pack2bf(x[2], x[3])};
    const float h0 = __uint_as_float(hi[0] << 16), h1 = __uint_as_float(hi[0] & 0xffff0000u);
    const float h2 = __uint_as_float(hi[1] << 16), h3 = __uint_as_float(hi[1] & 0xffff0000u);
    lo = u32x2{pack2bf(x[0] - h0, x[1] - h1), pack2bf(x[2] - h2, x[3] - h3)};
}
TTT_DEV bf16x8 join2(const u32x2& a, const u32x2& b) { return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]}); }
// two 16-token products in one 16x16x32 MFMA: lane group g's k slots 0..3
// are tokens 4g..4g+3 of the first tile, slots 4..7 those of the second
// (operands a0|a1 and b0|b1 in the same order)
TTT_DEV void mma2x16(f32x4& acc, const u32x2& a0, const u32x2& a1, const u32x2& b0, const u32x2& b1) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(join2(a0, a1), join2(b0, b1), acc, 0, 0, 0);
}
TTT_DEV u32x2 pack4(const f32x4& x) { return u32x2{pack2bf(x[0], x[1]), pack2bf(x[2], x[3])}; }
// a pointer the compiler may not prove uniform, made scalar (buffer
// descriptors built from vector registers need a loop per access)
TTT_DEV void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}

// MBK: 0 = one-step mini-batches (b = 16), 1 = mini-batches ending only at
// stage ends (b a multiple of 64), 2 = any multiple of 16 (per-step test).
// NW: waves per workgroup (4 or 2); wave w owns NCB = 4 / NW column blocks
// of 16 (columns [16 NCB w, 16 NCB (w + 1))), whose chains share every K and
// Q fragment and the score tile and interleave in the issue stream.
template <int MBK, int NW>
__global__ __launch_bounds__(64 * NW) void dual_seg_kernel(DualParams p) {
    constexpr int D = 64, DV = 64;
    constexpr bool ONE = (MBK == 0), SEND = (MBK == 1);
    constexpr int NCB = 4 / NW;          // column blocks per wave
    constexpr int R = dual_ring_stages(NW);
    constexpr int NLQ = 8 / NW;          // direct loads per wave per [64][64] tile
    constexpr int MB = DS_MB / NCB;      // maps staged per batch of the composition
    // pass 1 takes a stage as one group of four tiles (see its group lambda)
    constexpr bool GROUPED = (MBK != 2) && (NCB == 1) && DUAL_GROUPED;
    // the only LDS array (see ring_step1); its first word carries the ticket
    __shared__ __attribute__((aligned(16))) bf16_t ring[R * DS_STAGE];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nheads = p.B * p.H, nseg = p.nseg;
    int ticket = blockIdx.x, seg_q = nheads, grp = 0, ngrp = 1;   // one segment per sequence: no tickets
    if (nseg > 1) {
        // Tickets hand out segments in order, so a workgroup only ever waits
        // for workgroups that took a ticket before it and are running.  With
        // B*H a multiple of 8, the workgroups form 8 groups by blockIdx % 8
        // (the XCD the dispatcher places them on), each with a counter of its
        // own and every segment of the heads bh = 8 i + group: when segment 0
        // runs only its forward, the CUs it frees are on the XCD that the
        // group's last segments are dispatched to
        ngrp = (nheads % 8 == 0) ? 8 : 1;
        grp = (int)(blockIdx.x % ngrp);
        seg_q = nheads / ngrp;
        if (tid == 0) {
            const int t = atomicAdd(p.flags + (int64_t)nheads * nseg + 2 + grp, 1);
            *reinterpret_cast<int*>(ring) = t;
            // started (bit 1 of the workgroup's flag)
            __hip_atomic_store(p.flags + (int64_t)((t % seg_q) * ngrp + grp) * nseg + t / seg_q, 2,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        ticket = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(ring));
        __syncthreads();   // every wave holds the ticket before the ring is filled
    }
    // (uniform values: buffer descriptors built from them stay scalar)
    const int seg = __builtin_amdgcn_readfirstlane(ticket / seg_q);
    const int bh = __builtin_amdgcn_readfirstlane((ticket % seg_q) * ngrp + grp);
    const int L = p.L, mb = p.minibatch;
    const int tok0 = seg * p.seg_len;
    const int len = min(p.seg_len, L - tok0);
    const float eta = p.eta;
    const int col0 = 16 * NCB * w;       // first column of this wave
    const bf16_t* Qg = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)bh * L * D;
    const bf16_t* Kg = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)bh * L * D;
    const bf16_t* Vg = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)bh * L * DV;
    bf16_t* Og = reinterpret_cast<bf16_t*>(p.out) + (int64_t)bh * L * DV + col0;
    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)Qg, 0, L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, L * DV * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc((void*)Og, 0, L * DV * 2 - 2 * col0, 0x00020000);

    // direct-load lane offsets (bytes from the stage's first row): load i of
    // wave w is the tile's wave-load j = NLQ w + i, which fills rows 8j .. 8j
    // + 7, lane l position l % 8 of row 8j + l / 8, fetching the unit that
    // belongs there
    uint32_t qko[NLQ], vdo[NLQ];
#pragma unroll
    for (int i = 0; i < NLQ; ++i) {
        const int row = 8 * (NLQ * w + i) + (lane >> 3);
        qko[i] = (uint32_t)(row * D * 2 + 16 * ((lane & 7) ^ (kswz(row & 15) >> 1)));
        vdo[i] = (uint32_t)(row * DV * 2 + 16 * ((lane & 7) ^ vswz(row)));
    }
    auto load_tile = [&](__amdgpu_buffer_rsrc_t r, bf16_t* tile, const uint32_t* off, int sq) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NLQ; ++i) dma16(r, tile + 512 * (NLQ * w + i), off[i], sq);
    };
    // LDS read offsets within a step's 16 rows (elements)
    const int fro = c16 * D, fsw = kswz(c16) >> 1;           // row fragments
    const int rr = 4 * g + (c16 >> 2), cq = c16 & 3;         // transposing reads: row, chunk quad
    const int kr = rr * D, krs = kswz(rr);
    int kro[NCB], vro[NCB];                                   // K[.][c + 4cq ..], V[.][c + 4cq ..] of column block c
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int c = NCB * w + cb;
        kro[cb] = kr + 4 * ((4 * c + cq) ^ krs);
        vro[cb] = rr * DV + 8 * ((2 * c + (cq >> 1)) ^ vswz(rr)) + 4 * (cq & 1);
    }
    const int vo = (c16 * DV + 4 * g) * 2;                    // output store (bytes)
    u32x2 pmask;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        pmask[h] = ((4 * g + 2 * h <= c16) ? 0x0000ffffu : 0u) | ((4 * g + 2 * h + 1 <= c16) ? 0xffff0000u : 0u);

    auto kfrag = [&](const bf16_t* Ks, int kb) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(Ks + fro + 8 * ((4 * kb + g) ^ fsw));
    };
    auto kT = [&](const bf16_t* Ks, int t) __attribute__((always_inline)) {
        const int chunk = 8 * (t >> 1) + 2 * cq + (t & 1);
        return tr_read_d(Ks + kr + 4 * (chunk ^ krs));
    };
    auto to4 = [](const u32x2& r) {
        return f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u), __uint_as_float(r[1] << 16),
                     __uint_as_float(r[1] & 0xffff0000u)};
    };
    auto mb_end = [&](int t1) { return t1 % mb == 0 || t1 >= L; };

    // vmcnt field of s_waitcnt on gfx9 (bits 3..0 and 15..14), no other wait
    auto wait_vm = [](auto N) __attribute__((always_inline)) {
        constexpr int n = decltype(N)::value;
        static_assert(n <= 63, "vmcnt holds 6 bits");
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    };
    using V0 = std::integral_constant<int, 0>;
    // the ring's scalar offsets of the stage read and the stage refilled
    auto advance = [](int& o) { o = (o + DS_STAGE == R * DS_STAGE) ? 0 : o + DS_STAGE; };

    // per (b, h, segment) map block of 32 KB: Delta as two bf16 [64][64]
    // row-major arrays (hi, lo: Delta = hi + lo to about 16 bits), then B
    // in accumulator slots (fp32): column block c, tile t, lane l at slot
    // (4c + t) * 64 + l
    const int64_t id = (int64_t)bh * nseg + seg;
    char* maps = reinterpret_cast<char*>(p.maps);

    // ================= pass 1: the segment's map (Delta, B).  The last
    // segment's map is never read; with seg0_state segment 0 hands on its end
    // state instead (after its forward)
    const bool from_w0 = (seg == 0) || !p.seg0_state;
    if ((seg > 0 || !p.seg0_state) && seg < nseg - 1) {
        f32x4 SB[NCB][4], SD[NCB][4];
        bf16x8 BopS[NCB][2], DopS[NCB][2], BopW[NCB][2], DopW[NCB][2];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int t = 0; t < 4; ++t) SB[cb][t] = SD[cb][t] = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) BopS[cb][kb] = DopS[cb][kb] = BopW[cb][kb] = DopW[cb][kb] = bf16x8{};
        }
        const int nst = len / DS_T;   // segments before the last hold whole stages
        auto issue = [&](int s, bf16_t* dst) __attribute__((always_inline)) {
            const int sq = (tok0 + DS_T * min(s, nst - 1)) * D * 2;
            load_tile(rK, dst + DS_TILE, qko, sq);
            load_tile(rV, dst + 2 * DS_TILE, vdo, sq);
        };
        auto step = [&](const bf16_t* X, int j, int s16) __attribute__((always_inline)) {
            const bf16_t* Ks = X + DS_TILE + 16 * j * D;
            const bf16_t* Vs = X + 2 * DS_TILE + 16 * j * DV;
            const bf16x8 Kf0 = kfrag(Ks, 0), Kf1 = kfrag(Ks, 1);
            u32x2 VBb[NCB], VDb[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 eB = zero4(), eD = zero4();
                mma(eB, Kf0, ONE ? BopS[cb][0] : BopW[cb][0]);
                mma(eB, Kf1, ONE ? BopS[cb][1] : BopW[cb][1]);
                mma(eD, Kf0, ONE ? DopS[cb][0] : DopW[cb][0]);
                mma(eD, Kf1, ONE ? DopS[cb][1] : DopW[cb][1]);
                const f32x4 ks = to4(tr_read_d(Ks + kro[cb]));   // the I share of K A: K[4g + r][c + c16]
                const f32x4 vv = to4(tr_read_d(Vs + vro[cb]));
                f32x4 vb, vd;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vb[r] = eta * (vv[r] - eB[r]);
                    vd[r] = -eta * (eD[r] + ks[r]);
                }
                VBb[cb] = u32x2{pack2bf(vb[0], vb[1]), pack2bf(vb[2], vb[3])};
                VDb[cb] = u32x2{pack2bf(vd[0], vd[1]), pack2bf(vd[2], vd[3])};
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x2 kt = kT(Ks, t);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    mma16(SB[cb][t], kt, VBb[cb]);
                    mma16(SD[cb][t], kt, VDb[cb]);
                }
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    BopS[cb][kb] = acc_to_frag_bf16(SB[cb][2 * kb], SB[cb][2 * kb + 1]);
                    DopS[cb][kb] = acc_to_frag_bf16(SD[cb][2 * kb], SD[cb][2 * kb + 1]);
                }
            if (MBK == 2 && mb_end(16 * s16 + 16)) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        BopW[cb][kb] = BopS[cb][kb];
                        DopW[cb][kb] = DopS[cb][kb];
                    }
            }
        };
        // One stage as a group of four 16-token tiles (one-step mini-batches,
        // or mini-batches that end only at stage ends, one column block per
        // wave).  Every E_j takes the state the group starts from, and with
        // one-step mini-batches the tiles before j add their share through
        // the Gram blocks G_ji = K_j K_i^T (state-free, off the chain):
        //     E_j = K_j W + sum_{i<j} G_ji V~_i,
        // the state takes all four tiles in two 32-token products and its
        // bf16 copies are refreshed once per stage.  (The same grouping of
        // pass 3, with the outputs as the start state read by Q plus causal
        // attention over the group, measured slower: its 28 independent
        // readout and score products per stage did not pay for the shorter
        // chain.)
        auto group = [&](const bf16_t* X) __attribute__((always_inline)) {
            const bf16_t* Ks = X + DS_TILE;
            const bf16_t* Vs = X + 2 * DS_TILE;
            bf16x8 Kf[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) Kf[j][kb] = kfrag(Ks + 16 * j * D, kb);
            u32x2 G[4][4];   // G[j][i], i < j: A operand of G_ji (row t_j = c16, k = t_i)
            if (ONE) {
#pragma unroll
                for (int j = 1; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < j; ++i) {
                        f32x4 gt = zero4();
                        mma(gt, Kf[i][0], Kf[j][0]);
                        mma(gt, Kf[i][1], Kf[j][1]);
                        G[j][i] = pack4(gt);
                    }
            }
            f32x4 eB[4], eD[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                eB[j] = eD[j] = zero4();
                mma(eB[j], Kf[j][0], ONE ? BopS[0][0] : BopW[0][0]);
                mma(eB[j], Kf[j][1], ONE ? BopS[0][1] : BopW[0][1]);
                mma(eD[j], Kf[j][0], ONE ? DopS[0][0] : DopW[0][0]);
                mma(eD[j], Kf[j][1], ONE ? DopS[0][1] : DopW[0][1]);
            }
            u32x2 VBb[4], VDb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (ONE) {
#pragma unroll
                    for (int i = 0; i < j; ++i) {
                        mma16(eB[j], G[j][i], VBb[i]);
                        mma16(eD[j], G[j][i], VDb[i]);
                    }
                }
                const f32x4 ks = to4(tr_read_d(Ks + 16 * j * D + kro[0]));   // the I share of K A
                const f32x4 vv = to4(tr_read_d(Vs + 16 * j * DV + vro[0]));
                f32x4 vb, vd;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    vb[r] = eta * (vv[r] - eB[j][r]);
                    vd[r] = -eta * (eD[j][r] + ks[r]);
                }
                VBb[j] = pack4(vb);
                VDb[j] = pack4(vd);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x2 k0 = kT(Ks, t), k1 = kT(Ks + 16 * D, t), k2 = kT(Ks + 32 * D, t), k3 = kT(Ks + 48 * D, t);
                mma2x16(SB[0][t], k0, k1, VBb[0], VBb[1]);
                mma2x16(SB[0][t], k2, k3, VBb[2], VBb[3]);
                mma2x16(SD[0][t], k0, k1, VDb[0], VDb[1]);
                mma2x16(SD[0][t], k2, k3, VDb[2], VDb[3]);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                BopS[0][kb] = acc_to_frag_bf16(SB[0][2 * kb], SB[0][2 * kb + 1]);
                DopS[0][kb] = acc_to_frag_bf16(SD[0][2 * kb], SD[0][2 * kb + 1]);
            }
        };
        // a wave issues 2 NLQ loads per stage; after the stage read in
        // iteration s it has issued the loads of the R - 2 stages that follow
#pragma unroll
        for (int s = 0; s < R - 1; ++s) issue(s, ring + s * DS_STAGE);
        int rdo = 0, wro = (R - 1) * DS_STAGE;
        for (int s = 0; s < nst; ++s) {
            wait_vm(std::integral_constant<int, 2 * NLQ * (R - 2)>{});
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            const int rd_off = rdo, wr_off = wro;
            advance(rdo);
            advance(wro);
            ring_step1(ring + __builtin_amdgcn_readfirstlane(wr_off), ring + __builtin_amdgcn_readfirstlane(rd_off),
                       [&](bf16_t* dst) __attribute__((always_inline)) { issue(s + R - 1, dst); },
                       [&](const bf16_t* X) __attribute__((always_inline)) {
                           if constexpr (GROUPED) {
                               group(X);
                           } else {
#pragma unroll
                               for (int j = 0; j < DS_T / 16; ++j) step(X, j, (tok0 >> 4) + 4 * s + j);
                           }
                       });
            if (SEND && mb_end(tok0 + DS_T * (s + 1))) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        BopW[cb][kb] = BopS[cb][kb];
                        DopW[cb][kb] = DopS[cb][kb];
                    }
            }
        }
        wait_vm(V0{});   // the clamped loads still in flight
        // publish: Delta row-major (row = feature of the state row, column =
        // the input feature c + c16) as hi and lo, B in accumulator slots.
        // The stores are device-coherent (sc1: written through to memory), so
        // once they are complete every XCD reads them with sc1 loads, and the
        // flag needs no release (which would write back this XCD's whole L2)
        const __amdgpu_buffer_rsrc_t rP =
            __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(maps + id * DS_MAP), 0, DS_MAP, 0x00020000);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int c = NCB * w + cb;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, SB[cb][t]), rP,
                                                       (uint32_t)(DS_BOFF + 16 * ((c * 4 + t) * 64 + lane)), 0, DS_SC1);
                u32x2 hi, lo;
                split4(SD[cb][t], hi, lo);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t e = 2u * (uint32_t)(feat(16 * t + 4 * g + r) * DV + 16 * c + c16);
                    const uint32_t sh = 16 * (r & 1);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hi[r >> 1] >> sh), rP, e, 0, DS_SC1);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(lo[r >> 1] >> sh), rP, e + 2 * D * DV, 0, DS_SC1);
                }
            }
        }
        wait_vm(V0{});   // this wave's stores are complete
        __syncthreads();
        if (tid == 0) __hip_atomic_store(p.flags + id, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Flags: bit 1 when the workgroup of (b, h, segment) has started, bit 0
    // when its map (or segment 0's end state) is published.  Waiting for
    // published flags of segments [0, j_end) of this head: one thread polls
    // with relaxed loads (an acquire in the loop would invalidate the XCD's
    // L2 on every poll, under the feet of the workgroups still computing);
    // the maps are then read with device-coherent loads (sc1), which see the
    // published stores, and the other waves' reads follow the barrier.  The
    // wait is bounded; one that gives up raises the error word (results are
    // then invalid)
    auto wait_published = [&](int j_end) __attribute__((always_inline)) {
        if (tid == 0) {
            bool all = true;
            for (int j = 0; j < j_end; ++j) {
                int v = 0;
                for (int spin = 0; spin < p.max_polls; ++spin) {
                    v = __hip_atomic_load(p.flags + (int64_t)bh * nseg + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (v & 1) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                all = all && (v & 1);
            }
            if (!all)
                __hip_atomic_store(p.flags + (int64_t)nheads * nseg + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    };
    // segment 0's end state sits in the B slots of its map block
    const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(maps + (int64_t)bh * nseg * DS_MAP), 0, nseg * DS_MAP, 0x00020000);
    constexpr int NMO = 16 / NW;   // direct loads per wave per map (1024 slots of 16 bytes)
    uint32_t mo[NMO];
#pragma unroll
    for (int i = 0; i < NMO; ++i) {
        const int slot = 64 * (NMO * w + i) + lane, row = (slot >> 3) & 63;
        // slots 0..511: hi rows, 512..1023: lo rows
        mo[i] = (uint32_t)((slot >> 9) * D * DV * 2 + row * DV * 2 + 16 * ((slot & 7) ^ (row & 7)));
    }
    f32x4 Sacc[NCB][4];
    // Sacc <- f_{j_end-1}(... f_{j_begin}(Sacc)), f_j(W) = W + Delta_j W + B_j:
    // Delta_j (hi, lo) of up to MB maps at a time go into the ring by direct
    // loads (16 KB per map; the 16-byte unit u of row r at position u ^ (r &
    // 7)), B_j into registers; then the maps are applied in order
    auto compose = [&](int j_begin, int j_end) __attribute__((always_inline)) {
        for (int j0 = j_begin; j0 < j_end; j0 += MB) {
            const int nb = min(MB, j_end - j0);
            f32x4 bj[MB][NCB][4];
#pragma unroll
            for (int x = 0; x < MB; ++x) {
                if (x < nb) {
#pragma unroll
                    for (int i = 0; i < NMO; ++i) dma16_sc1(rM, ring + x * 2 * D * DV + 512 * (NMO * w + i), mo[i], (j0 + x) * DS_MAP);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            bj[x][cb][t] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rM, (uint32_t)(DS_BOFF + 16 * (((NCB * w + cb) * 4 + t) * 64 + lane)),
                                           (j0 + x) * DS_MAP, DS_SC1));
                }
            }
            wait_vm(V0{});
            __syncthreads();
#pragma unroll
            for (int x = 0; x < MB; ++x) {
                if (x < nb) {
                    // Y = Delta_j W: A operand rows = state row positions
                    // 16t + c16, k = features 32kb + 8g ..; B operand = W in
                    // the accperm order, split into hi and lo
                    const bf16_t* Mh = ring + x * 2 * D * DV;
                    bf16x8 whi[NCB][2], wlo[NCB][2];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            u32x2 h0, l0, h1, l1;
                            split4(Sacc[cb][2 * kb], h0, l0);
                            split4(Sacc[cb][2 * kb + 1], h1, l1);
                            whi[cb][kb] = join2(h0, h1);
                            wlo[cb][kb] = join2(l0, l1);
                        }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int row = feat(16 * t + c16);
                        f32x4 y[NCB];
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) y[cb] = zero4();
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            const int e = row * DV + 8 * ((4 * kb + g) ^ (row & 7));
                            const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(Mh + e);
                            const bf16x8 alo = *reinterpret_cast<const bf16x8*>(Mh + D * DV + e);
#pragma unroll
                            for (int cb = 0; cb < NCB; ++cb) {
                                mma(y[cb], ahi, whi[cb][kb]);
                                mma(y[cb], alo, whi[cb][kb]);
                                mma(y[cb], ahi, wlo[cb][kb]);
                            }
                        }
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) Sacc[cb][t] += y[cb] + bj[x][cb][t];
                    }
                }
            }
            __syncthreads();   // the staged maps are read before the ring is refilled
        }
    };

    // ================= the start state: W0, then the maps of segments
    // 0 .. seg-1; with seg0_state, segment 0's end state, then the maps of
    // segments 1 .. seg-1
    if (from_w0) {
        const float* W0 = p.W0 + (int64_t)bh * p.W0_stride;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[cb][t][r] = W0[feat(16 * t + 4 * g + r) * DV + col0 + 16 * cb + c16];
    }
    if (seg > 0) {
        wait_published(seg);
        if (!from_w0) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    Sacc[cb][t] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rM, (uint32_t)(DS_BOFF + 16 * (((NCB * w + cb) * 4 + t) * 64 + lane)), 0, DS_SC1));
        }
        compose(from_w0 ? 0 : 1, seg);
    }

    // With seg0_state the last segment has no workgroup of its own: segment
    // 0's workgroup, which runs only its forward and finishes first, goes on
    // to it (composing the maps of segments 1 .. nseg-2 onto the end state it
    // holds), or, failing that, the workgroup of segment nseg-2, whose end
    // state is the last segment's start.  Segment 0 claims it only once every
    // workgroup it would wait for has started, so it never waits for one
    // that cannot run; segment nseg-2 waits for nothing.  A claim word (the
    // last segment's flag) makes exactly one of them run it.
    for (int cur = seg;;) {
        // ================= pass 3: the forward over segment cur's tokens
        const int ctok0 = cur * p.seg_len, clen = min(p.seg_len, L - ctok0);
        bf16x8 Sop[NCB][2], Wop[NCB][2];
    #pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
    #pragma unroll
            for (int kb = 0; kb < 2; ++kb) Sop[cb][kb] = Wop[cb][kb] = acc_to_frag_bf16(Sacc[cb][2 * kb], Sacc[cb][2 * kb + 1]);
        wait_vm(V0{});
        __syncthreads();   // every wave is past pass 1 before the ring is refilled
        const int nst = (clen + DS_T - 1) / DS_T;
        auto issue = [&](int s, bf16_t* dst) __attribute__((always_inline)) {
            const int sq = (ctok0 + DS_T * min(s, nst - 1)) * D * 2;
            load_tile(rQ, dst, qko, sq);
            load_tile(rK, dst + DS_TILE, qko, sq);
            load_tile(rV, dst + 2 * DS_TILE, vdo, sq);
        };
        auto step = [&](const bf16_t* X, int j, int s16) __attribute__((always_inline)) {
            const bf16_t* Qs = X + 16 * j * D;
            const bf16_t* Ks = X + DS_TILE + 16 * j * D;
            const bf16_t* Vs = X + 2 * DS_TILE + 16 * j * DV;
            const bf16x8 Kf0 = kfrag(Ks, 0), Kf1 = kfrag(Ks, 1);
            const bf16x8 Qf0 = kfrag(Qs, 0), Qf1 = kfrag(Qs, 1);
            // P^T = K Q^T (causal j <= i), shared by the column blocks
            f32x4 pt = zero4();
            mma(pt, Kf0, Qf0);
            mma(pt, Kf1, Qf1);
            u32x2 VB[NCB];
            f32x4 o[NCB];
    #pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                // E = K W_n;  O^T partial = S~^T Q^T
                f32x4 e = zero4();
                o[cb] = zero4();
                mma(e, Kf0, ONE ? Sop[cb][0] : Wop[cb][0]);
                mma(e, Kf1, ONE ? Sop[cb][1] : Wop[cb][1]);
                mma(o[cb], Sop[cb][0], Qf0);
                mma(o[cb], Sop[cb][1], Qf1);
                const f32x4 vv = to4(tr_read_d(Vs + vro[cb]));
                f32x4 vt;
    #pragma unroll
                for (int r = 0; r < 4; ++r) vt[r] = eta * (vv[r] - e[r]);
                VB[cb] = u32x2{pack2bf(vt[0], vt[1]), pack2bf(vt[2], vt[3])};
            }
    #pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x2 kt = kT(Ks, t);
    #pragma unroll
                for (int cb = 0; cb < NCB; ++cb) mma16(Sacc[cb][t], kt, VB[cb]);
            }
            const u32x2 pm = u32x2{pack2bf(pt[0], pt[1]) & pmask[0], pack2bf(pt[2], pt[3]) & pmask[1]};
    #pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb) Sop[cb][kb] = acc_to_frag_bf16(Sacc[cb][2 * kb], Sacc[cb][2 * kb + 1]);
                if (MBK == 2 && mb_end(16 * s16 + 16)) {
                    Wop[cb][0] = Sop[cb][0];
                    Wop[cb][1] = Sop[cb][1];
                }
                // O^T += V~^T P^T, store O rows (4 consecutive columns per lane)
                mma16(o[cb], VB[cb], pm);
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(u32x2, u32x2{pack2bf(o[cb][0], o[cb][1]), pack2bf(o[cb][2], o[cb][3])}), rO,
                    vo + 32 * cb, 16 * s16 * DV * 2, 0);
            }
        };
        // a wave issues NL3 loads and NST stores (one per step and column block)
        // per stage.  Operations issued after the loads of the stage read in
        // iteration s: for s < R - 1 (stages of the prologue) the loads of
        // prologue stages s + 1 .. R - 2 and iterations 0 .. s - 1,
        // NL3 (R - 2) + NST s; after that the stores of the iteration that
        // issued them and R - 2 whole iterations, NST + (NL3 + NST) (R - 2)
        constexpr int NL3 = 3 * NLQ, NST = 4 * NCB;
    #pragma unroll
        for (int s = 0; s < R - 1; ++s) issue(s, ring + s * DS_STAGE);
        int rdo = 0, wro = (R - 1) * DS_STAGE;
        auto wait_stage = [&](int s) __attribute__((always_inline)) {
            if (s >= R - 1) {
                wait_vm(std::integral_constant<int, NST + (NL3 + NST) * (R - 2)>{});
                return;
            }
            static_for<R - 1>([&](auto I) __attribute__((always_inline)) {
                constexpr int i = decltype(I)::value;
                if (s == i) wait_vm(std::integral_constant<int, NL3 * (R - 2) + NST * i>{});
            });
        };
        for (int s = 0; s < nst; ++s) {
            wait_stage(s);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            const int rd_off = rdo, wr_off = wro;
            advance(rdo);
            advance(wro);
            ring_step1(ring + __builtin_amdgcn_readfirstlane(wr_off), ring + __builtin_amdgcn_readfirstlane(rd_off),
                       [&](bf16_t* dst) __attribute__((always_inline)) { issue(s + R - 1, dst); },
                       [&](const bf16_t* X) __attribute__((always_inline)) {
    #pragma unroll
                           for (int j = 0; j < DS_T / 16; ++j) step(X, j, (ctok0 >> 4) + 4 * s + j);
                       });
            if (SEND && mb_end(ctok0 + DS_T * (s + 1))) {
    #pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    Wop[cb][0] = Sop[cb][0];
                    Wop[cb][1] = Sop[cb][1];
                }
            }
        }
        wait_vm(V0{});   // the clamped loads still in flight

        if (cur == 0 && nseg > 2 && p.seg0_state) {
            // segment 0's end state, for every later segment to start from: the
            // same device-coherent stores and relaxed flag as a map
            const __amdgpu_buffer_rsrc_t rP =
                __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(maps + id * DS_MAP), 0, DS_MAP, 0x00020000);
    #pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
    #pragma unroll
                for (int t = 0; t < 4; ++t)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Sacc[cb][t]), rP,
                                                           (uint32_t)(DS_BOFF + 16 * (((NCB * w + cb) * 4 + t) * 64 + lane)),
                                                           0, DS_SC1);
            wait_vm(V0{});   // this wave's stores are complete
            __syncthreads();
            if (tid == 0) __hip_atomic_store(p.flags + id, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        if (cur == nseg - 1 && p.W_final) {
            float* Wf = p.W_final + (int64_t)bh * D * DV;
    #pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
    #pragma unroll
                for (int t = 0; t < 4; ++t)
    #pragma unroll
                    for (int r = 0; r < 4; ++r) Wf[feat(16 * t + 4 * g + r) * DV + col0 + 16 * cb + c16] = Sacc[cb][t][r];
        }

        if (!p.seg0_state || cur == nseg - 1 || (cur != 0 && cur != nseg - 2)) break;
        __syncthreads();   // the ring is free (its first word carries the claim)
        if (tid == 0) {
            bool ok = true;
            for (int j = 1; cur == 0 && j < nseg - 1; ++j)
                ok = ok && (__hip_atomic_load(p.flags + (int64_t)bh * nseg + j, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) & 2);
            if (ok) ok = atomicCAS(p.flags + (int64_t)bh * nseg + nseg - 1, 0, 1) == 0;
            *reinterpret_cast<int*>(ring) = ok ? 1 : 0;
        }
        __syncthreads();
        const int go = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(ring));
        __syncthreads();
        if (!go) break;
        if (cur == 0 && nseg > 2) {
            wait_published(nseg - 1);
            compose(1, nseg - 1);
        }
        cur = nseg - 1;
    }
}

__global__ void dual_flags_clear_kernel(int* flags, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flags[i] = 0;
}

bool dual_supported(int dtype, int d, int dv, int minibatch) {
    return (dtype == 0 || dtype == 1) && d == 64 && dv == 64 && minibatch >= 1;
}

namespace {

// Segmented plan for bf16 mini-batches of a multiple of 16: enough segments
// to fill the CUs with workgroups (kDualNW waves each, one wave per SIMD),
// and one more, each a whole number of mini-batches and of 64-token stages,
// at least 256 tokens long.  Four waves of one column block each: a step is bound by
// instruction issue, so two column blocks per wave (two-wave workgroups,
// twice the segments) took twice as long per step and lost the time the
// shared fragments saved to the longer composition.
#ifndef DUAL_NW
#define DUAL_NW 4
#endif
constexpr int kDualNW = DUAL_NW;                  // waves per workgroup
constexpr int kCUs = 256;
constexpr int kDualSlots = kCUs * 4 / kDualNW;     // workgroups resident at once
constexpr int kDualMinSeg = 256;
constexpr int kDualPolls = 1 << 22;   // polls of ~0.1 us before a wait gives up
struct DualSegPlan {
    int nseg, seg_len, seg0_state;
};

// segment length (a whole number of units, at least the minimum) for about
// `want` segments over L tokens
int64_t dual_seg_len(int64_t L, int64_t want, int64_t unit) {
    int64_t seg = ((L + want - 1) / want + unit - 1) / unit * unit;
    const int64_t min_seg = (kDualMinSeg + unit - 1) / unit * unit;
    return seg < min_seg ? min_seg : seg;
}

DualSegPlan dual_seg_plan(int dtype, int B, int H, int L, int d, int dv, int mb) {
    DualSegPlan pl{1, L, 0};
    if (dtype != 1 || d != 64 || dv != 64 || mb % 16 != 0) return pl;
    if ((int64_t)L * 128 >= (int64_t)1 << 31) return pl;   // 32-bit buffer ranges
    const int64_t nheads = (int64_t)B * H;
    // with more sequences than half the slots there would be two segments,
    // the second waiting for the end of the first: no gain over one chain
    if (nheads * 2 > kDualSlots) return pl;
    int64_t gcd = 64, x = mb;
    while (x) {
        const int64_t t = gcd % x;
        gcd = x;
        x = t;
    }
    const int64_t unit = (int64_t)mb / gcd * 64;   // lcm(mb, 64)
    // Segment 0 may run only its forward and hand on its end state: it then
    // finishes first, and its workgroup goes on to one more segment than the
    // slots hold.  That pays when the extra segment exists; otherwise the
    // later segments would wait for segment 0's forward instead of its
    // shorter map pass, so segment 0 publishes a map like the others
    int64_t seg = dual_seg_len(L, kDualSlots / nheads + 1, unit);
    int64_t nseg = (L + seg - 1) / seg;
    if (nseg * nheads > kDualSlots) {
        pl.seg0_state = 1;
    } else {
        seg = dual_seg_len(L, (kDualSlots + nheads - 1) / nheads, unit);
        nseg = (L + seg - 1) / seg;
    }
    if (nseg <= 1) return pl;
    pl.nseg = (int)nseg;
    pl.seg_len = (int)seg;
    return pl;
}
// flags (one per (b, h, segment)), a spare word, the error word, 8 ticket counters
constexpr int kDualFlagWords = 10;
size_t dual_flag_bytes(int64_t n) { return (size_t)(((n + kDualFlagWords) * 4 + 255) / 256 * 256); }

void launch_dual_seg(const DualParams& p, unsigned nwg, hipStream_t s) {
    const dim3 grid(nwg), block(64 * kDualNW);
    if (p.minibatch == 16) hipLaunchKernelGGL((dual_seg_kernel<0, kDualNW>), grid, block, 0, s, p);
    else if (p.minibatch % DS_T == 0) hipLaunchKernelGGL((dual_seg_kernel<1, kDualNW>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dual_seg_kernel<2, kDualNW>), grid, block, 0, s, p);
}

}  // namespace

size_t dual_workspace(int dtype, int B, int H, int L, int d, int dv, int minibatch) {
    const DualSegPlan pl = dual_seg_plan(dtype, B, H, L, d, dv, minibatch);
    if (pl.nseg <= 1) return 0;
    const int64_t n = (int64_t)B * H * pl.nseg;
    return dual_flag_bytes(n) + (size_t)n * DS_MAP;
}

int64_t dual_error_word(int dtype, int B, int H, int L, int d, int dv, int minibatch) {
    const DualSegPlan pl = dual_seg_plan(dtype, B, H, L, d, dv, minibatch);
    if (pl.nseg <= 1) return -1;
    return (int64_t)B * H * pl.nseg + 1;
}

hipError_t launch_dual_fwd(const DualParams& pin, int dtype, hipStream_t s) {
    if (!dual_supported(dtype, pin.d, pin.dv, pin.minibatch)) return hipErrorInvalidValue;
    const bool ring_ok = (int64_t)pin.L * 128 < ((int64_t)1 << 31);
    if (dtype == 1 && pin.minibatch % 16 == 0 && ring_ok) {
        const DualSegPlan pl = dual_seg_plan(dtype, pin.B, pin.H, pin.L, pin.d, pin.dv, pin.minibatch);
        if (pl.nseg > 1 && pin.workspace) {
            DualParams p = pin;
            const int64_t n = (int64_t)p.B * p.H * pl.nseg;
            if (p.workspace_bytes < dual_workspace(dtype, p.B, p.H, p.L, p.d, p.dv, p.minibatch))
                return hipErrorInvalidValue;
            p.nseg = pl.nseg;
            p.seg_len = pl.seg_len;
            p.seg0_state = pl.seg0_state;
            p.flags = reinterpret_cast<int*>(p.workspace);
            p.maps = reinterpret_cast<float*>(reinterpret_cast<char*>(p.workspace) + dual_flag_bytes(n));
            if (p.max_polls <= 0) p.max_polls = kDualPolls;
            // flags, tickets and error word start at zero (a fill kernel, not a
            // memset node, so the call stays valid inside a captured graph)
            const int nflags = (int)n + kDualFlagWords;
            hipLaunchKernelGGL(dual_flags_clear_kernel, dim3((nflags + 255) / 256), dim3(256), 0, s, p.flags, nflags);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            // with seg0_state the last segment runs on segment 0's (or
            // segment nseg-2's) workgroup
            const int64_t nwg = p.seg0_state ? n - p.B * p.H : n;
            launch_dual_seg(p, (unsigned)nwg, s);
            return hipGetLastError();
        }
        const DualParams& p = pin;
        if ((int64_t)p.B * p.H > kCUs / 4) {
            // more sequences than the one-wave-per-CU chain kernel runs at
            // once: one workgroup per sequence, unsegmented
            DualParams q = p;
            q.nseg = 1;
            q.seg_len = q.L;
            q.seg0_state = 0;
            q.flags = nullptr;
            q.maps = nullptr;
            launch_dual_seg(q, (unsigned)(q.B * q.H), s);
            return hipGetLastError();
        }
        // one wave per (b, h, 16-column tile), one wave per CU (its ring takes 92 KB)
        if (p.minibatch == 16)
            hipLaunchKernelGGL((dual_ring_kernel<true, false>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        else if (p.minibatch % DR_T == 0)
            hipLaunchKernelGGL((dual_ring_kernel<false, true>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((dual_ring_kernel<false, false>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        return hipGetLastError();
    }
    const DualParams& p = pin;
    const int grid = p.B * p.H;
    if (dtype == 1)
        hipLaunchKernelGGL((dual_fwd_kernel<bf16_t, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((dual_fwd_kernel<float, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ttt
