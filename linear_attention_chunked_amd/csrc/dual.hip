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

bool dual_supported(int dtype, int d, int dv, int minibatch) {
    return (dtype == 0 || dtype == 1) && d == 64 && dv == 64 && minibatch >= 1;
}

hipError_t launch_dual_fwd(const DualParams& p, int dtype, hipStream_t s) {
    if (!dual_supported(dtype, p.d, p.dv, p.minibatch)) return hipErrorInvalidValue;
    if (dtype == 1 && p.minibatch % 16 == 0) {
        // one wave per (b, h, 16-column tile)
        if (p.minibatch == 16)
            hipLaunchKernelGGL((dual_ring_kernel<true, false>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        else if (p.minibatch % DR_T == 0)
            hipLaunchKernelGGL((dual_ring_kernel<false, true>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((dual_ring_kernel<false, false>), dim3(p.B * p.H * 4), dim3(64), 0, s, p);
        return hipGetLastError();
    }
    const int grid = p.B * p.H;
    if (dtype == 1)
        hipLaunchKernelGGL((dual_fwd_kernel<bf16_t, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((dual_fwd_kernel<float, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ttt
