// dbeta.hip -- dL/dbeta of the token-causal momentum forward.
//
// [P1] ("KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다",
// aitrends.kr/articles/4698), paragraph on momentum: the update carries a
// momentum m_t = beta m_{t-1} + g_t (g_t = eta_t k_t^T v_t) and the state
// S_t = S_{t-1} + m_t is read by o_t = q_t S_t.  [P4] ("RNN의 기억을 작은
// 모델로 바꾼다면: Test-Time Training 읽기", ariser.io), section on the two
// kinds of weights: the outer model learns through the inner updates, which
// includes beta when it is learned.
//
// Forward-mode derivative.  With the tangents m'_t = dm_t/dbeta and
// S'_t = dS_t/dbeta,
//     m'_t = beta m'_{t-1} + m_{t-1},   S'_t = S'_{t-1} + m'_t   (from 0),
//     dL/dbeta = sum_t q_t S'_t do_t^T + <dS_final, S'_{L-1}> + <dM_final, m'_{L-1}>.
// S0 does not enter.  Over a block of n tokens (local i, j) that starts from
// (M, M', T) = (m, m', S') before its first token, with w_i = 1 + .. + beta^i
// and F(d) = sum_{e=1..d} e beta^(e-1):
//     S'_i = T + beta w_i M' + F(i+1) M + sum_{j<i} F(i-j) g_j,
//     T   <- T + beta w_{n-1} M' + F(n) M + sum_j F(n-1-j) g_j,
//     M'  <- beta^n M' + n beta^(n-1) M + sum_j (n-1-j) beta^(n-2-j) g_j,
//     M   <- beta^n M + sum_j beta^(n-1-j) g_j,
// so a block needs three readouts Q [T | M' | M], the pairwise term
// F(i-j) eta_j (q_i . k_j)(do_i . v_j) and three weighted K^T V aggregates.
// Every column of the three states evolves on its own (column c only meets
// column c of v and do), so a wave owns 16 state columns of one (b, h) and
// walks the sequence in 16-token blocks.  The readouts and the scores are
// contractions over the state rows (features) and dL/dbeta is linear in
// them, so the rows split further: a wave holds a slice of 32 rows of its 16
// columns and adds its slice's share; with d_k = 128 four waves cover a
// column tile, which fills the chip at a few heads (one wave of all 128 rows
// per tile left three SIMDs in four idle at the momentum workload).  The
// per-wave sums are added up in a fixed order by a second kernel
// (deterministic).
//
// Data path: a wave-private ring of 32-token stages in LDS filled by 16-byte
// direct loads (no VGPR holds data in flight): the wave's slice of the Q and K
// rows [32][32] with the 16-byte units of row r rotated by XOR with r
// (bank-conflict-free row fragments), its V and dO tiles [32][16] and 32
// per-token rates.
// Rows past L load as zero: their q, do and eta are zero, so they add
// nothing; the last block takes its own length n in the state update.
#include "common.h"
#include "internal.h"

#include <cmath>

namespace ttt {

typedef short s16x4b __attribute__((ext_vector_type(4)));

TTT_DEV u32x2 tr_read_b(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4b lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
// 16 x 16 x 16 product (k = 4g + s in lane group g) as a 16x16x32 MFMA whose
// upper k half is zero
TTT_DEV void mma_k16(f32x4& acc, const u32x2& a, const u32x2& b) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], 0u, 0u});
    const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{b[0], b[1], 0u, 0u});
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
}
TTT_DEV f32x4 unpack4(const u32x2& w) {
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}

// 16-byte (4-byte) direct loads into LDS.  Kept out of the kernel template:
// the host-side pass rejects a dependent 16-byte form without a word and
// then drops the kernel's launch stub
TTT_DEV void dma_b128(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}
TTT_DEV void dma_b32(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

constexpr int DB_T = 32;   // tokens per ring stage (two 16-token blocks)

template <typename T, int DK>
struct DbGeo {
    static constexpr int ESZ = sizeof(T);
    static constexpr int ROWB = DK * ESZ;                  // bytes per Q/K row
    static constexpr int U = ROWB / 16;                    // 16-byte units per row
    static constexpr int QKB = DB_T * ROWB;                // bytes of the Q (or K) part
    static constexpr int VB = DB_T * 16 * ESZ;             // bytes of the V (or dO) tile
    static constexpr int NQ = QKB / 1024, NV = VB / 1024;  // load instructions per part
    static constexpr int STAGE = 2 * QKB + 2 * VB + 256;   // + 64 rates (32 used)
    static constexpr int NL = 2 * NQ + 2 * NV + 1;         // load instructions per stage
    // ring stages: as deep as vmcnt counts, and small enough for four
    // single-wave workgroups per CU (40 KB each)
    static constexpr int RV = (2 + 63 / NL) < 8 ? (2 + 63 / NL) : 8;
    static constexpr int R = RV * STAGE <= 40 * 1024 ? RV : 40 * 1024 / STAGE;
    static_assert(QKB % 1024 == 0 && VB % 1024 == 0, "whole 1 KB loads");
    static_assert((R - 2) * NL <= 63 && R >= 3, "vmcnt holds 6 bits");
};

// DK: the rows of this wave's slice; NSL slices make the head's d_k
template <typename T, int DK, int NSL>
__global__ __launch_bounds__(64) void dbeta_kernel(DbetaParams p) {
    using G = DbGeo<T, DK>;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int ROWG = DK * NSL * G::ESZ;   // bytes per Q/K row in memory
    __shared__ __attribute__((aligned(16))) char ring[G::R * G::STAGE];

    const int lane = threadIdx.x, g = lane >> 4, c16 = lane & 15;
    const int ntile = p.dv / 16;
    // the column tiles and row slices of a head on one XCD
    const int lid = xcd_logical(blockIdx.x, gridDim.x);
    const int bh = lid / (ntile * NSL), w = (lid / NSL) % ntile, sl = lid % NSL;
    const int row0 = DK * sl;   // first state row of this slice
    const int L = p.L, DV = p.dv;
    const char* Qg = reinterpret_cast<const char*>(p.q) + ((int64_t)bh * L * DK * NSL + row0) * G::ESZ;
    const char* Kg = reinterpret_cast<const char*>(p.k) + ((int64_t)bh * L * DK * NSL + row0) * G::ESZ;
    const char* Vg = reinterpret_cast<const char*>(p.v) + ((int64_t)bh * L * DV + 16 * w) * G::ESZ;
    const char* Dg = reinterpret_cast<const char*>(p.dout) + ((int64_t)bh * L * DV + 16 * w) * G::ESZ;
    const float* Eg = p.eta ? p.eta + (int64_t)bh * L : nullptr;

    // states: X[t][r] = X[16t + 4g + r][16w + c16], fp32
    constexpr int NT = DK / 16;
    f32x4 M[NT], Mp[NT], Tt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        Mp[t] = zero4();
        Tt[t] = zero4();
        M[t] = zero4();
        if (p.M0) {
            const float* m0 = p.M0 + (int64_t)bh * DK * NSL * DV + (int64_t)(row0 + 16 * t + 4 * g) * DV + 16 * w + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) M[t][r] = m0[(int64_t)r * DV];
        }
    }

    const __amdgpu_buffer_rsrc_t rQ =
        __builtin_amdgcn_make_buffer_rsrc((void*)Qg, 0, L * ROWG - row0 * G::ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t rK =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, L * ROWG - row0 * G::ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, (L * DV - 16 * w) * G::ESZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t rD =
        __builtin_amdgcn_make_buffer_rsrc((void*)Dg, 0, (L * DV - 16 * w) * G::ESZ, 0x00020000);
    // a scalar rate: a zero-range descriptor (every load returns 0, nothing is read)
    const __amdgpu_buffer_rsrc_t rE =
        __builtin_amdgcn_make_buffer_rsrc(Eg ? (void*)Eg : (void*)Qg, 0, Eg ? L * 4 : 0, 0x00020000);

    // direct-load lane offsets (bytes from the stage's first token row): LDS
    // slot (row, pos) of the slice holds its unit pos ^ (row % U)
    uint32_t qko[G::NQ], vdo[G::NV];
#pragma unroll
    for (int i = 0; i < G::NQ; ++i) {
        const int o = 1024 * i + 16 * lane, row = o / G::ROWB, pos = (o % G::ROWB) / 16;
        qko[i] = (uint32_t)(row * ROWG + 16 * (pos ^ (row % G::U)));
    }
#pragma unroll
    for (int i = 0; i < G::NV; ++i) {
        const int o = 1024 * i + 16 * lane, row = o / (16 * G::ESZ), piece = o % (16 * G::ESZ);
        vdo[i] = (uint32_t)(row * DV * G::ESZ + piece);
    }
    const int nblk = (L + 15) / 16, nst = (nblk + 1) / 2;
    auto issue = [&](int s, char* dst) __attribute__((always_inline)) {
        const int sc = min(s, nst - 1) * DB_T;   // first token of the stage
#pragma unroll
        for (int i = 0; i < G::NQ; ++i) dma_b128(rQ, dst + 1024 * i, qko[i], sc * ROWG);
#pragma unroll
        for (int i = 0; i < G::NQ; ++i) dma_b128(rK, dst + G::QKB + 1024 * i, qko[i], sc * ROWG);
#pragma unroll
        for (int i = 0; i < G::NV; ++i) dma_b128(rV, dst + 2 * G::QKB + 1024 * i, vdo[i], sc * DV * G::ESZ);
#pragma unroll
        for (int i = 0; i < G::NV; ++i) dma_b128(rD, dst + 2 * G::QKB + G::VB + 1024 * i, vdo[i], sc * DV * G::ESZ);
        dma_b32(rE, dst + 2 * G::QKB + 2 * G::VB, 4 * lane, sc * 4);
    };

    // element e of Q/K row r of a stage part X (swizzled 16-byte units)
    auto rowp = [&](const char* X, int r, int e) __attribute__((always_inline)) {
        const int byte = e * G::ESZ;
        return X + r * G::ROWB + 16 * ((byte / 16) ^ (r % G::U)) + (byte % 16);
    };
    // A/B operand of a contraction over features, k-block kb (the accperm
    // k-assignment, which is what a pair of state tiles holds per lane)
    auto feat_frag = [&](const char* X, int r, int kb) __attribute__((always_inline)) {
        if constexpr (BF) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(rowp(X, r, 32 * kb + 4 * g));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(rowp(X, r, 32 * kb + 16 + 4 * g));
            return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        } else {
            return *reinterpret_cast<const f32x4*>(rowp(X, r, 16 * kb + 4 * g));
        }
    };
    auto state_frag = [&](const f32x4* S, int kb) __attribute__((always_inline)) {
        if constexpr (BF) return acc_to_frag_bf16(S[2 * kb], S[2 * kb + 1]);
        else return S[kb];
    };
    // 4 consecutive rows 4g + s (s = 0..3) of column c of a [32][16] tile, fp32
    auto col4 = [&](const char* X, int r0, int c) __attribute__((always_inline)) {
        if constexpr (BF) {
            // transposing read: lane a of group g points at row r0 + 4g + a / 4, columns 4 (a % 4) ..
            const int a = lane & 15;
            return unpack4(tr_read_b(reinterpret_cast<const bf16_t*>(X) + (r0 + 4 * g + (a >> 2)) * 16 + 4 * (a & 3)));
        } else {
            const float* f = reinterpret_cast<const float*>(X);
            return f32x4{f[(r0 + 4 * g) * 16 + c], f[(r0 + 4 * g + 1) * 16 + c], f[(r0 + 4 * g + 2) * 16 + c],
                         f[(r0 + 4 * g + 3) * 16 + c]};
        }
    };
    // column 16t + c16 of K rows r0 + 4g + s, as the A operand of a K^T product
    auto kcol = [&](const char* X, int r0, int t) __attribute__((always_inline)) {
        if constexpr (BF) {
            const int a = lane & 15;
            return tr_read_b(reinterpret_cast<const bf16_t*>(rowp(X, r0 + 4 * g + (a >> 2), 16 * t + 4 * (a & 3))));
        } else {
            return f32x4{*reinterpret_cast<const float*>(rowp(X, r0 + 4 * g, 16 * t + c16)),
                         *reinterpret_cast<const float*>(rowp(X, r0 + 4 * g + 1, 16 * t + c16)),
                         *reinterpret_cast<const float*>(rowp(X, r0 + 4 * g + 2, 16 * t + c16)),
                         *reinterpret_cast<const float*>(rowp(X, r0 + 4 * g + 3, 16 * t + c16))};
        }
    };
    // 16 x 16 product over 16 k values (k = 4g + s): bf16 pieces or fp32
    auto mma16v = [&](f32x4& acc, const f32x4& a, const f32x4& b) __attribute__((always_inline)) {
        if constexpr (BF) mma_k16(acc, u32x2{pack2bf(a[0], a[1]), pack2bf(a[2], a[3])},
                                  u32x2{pack2bf(b[0], b[1]), pack2bf(b[2], b[3])});
        else mma(acc, a, b);
    };
    // the same with a raw bf16 A piece (K^T through the transposing read)
    auto mma16k = [&](f32x4& acc, const auto& kpiece, const f32x4& b) __attribute__((always_inline)) {
        if constexpr (BF) mma_k16(acc, kpiece, u32x2{pack2bf(b[0], b[1]), pack2bf(b[2], b[3])});
        else mma(acc, kpiece, b);
    };

    const float eta_s = p.eta_scalar;
    float acc = 0.f;   // this lane's share of sum_t <do_t, q_t S'_t>
    // this lane's weights, read once (LDS holds only the ring: a second LDS
    // array, or reads of one outside the ring's pointers, would make the
    // compiler wait for the ring's loads): readout rows i = 4g + r, score
    // (i, j = c16), and the update of a whole block for rows j = 4g + s
    float wP[4], wM[4], wS[4], u0[4], u1[4], u2[4], z0[4], z1[4], z2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        wP[r] = p.bw[i];
        wM[r] = p.F[i + 1];
        wS[r] = c16 < i ? p.F[i - c16] : 0.f;
        u0[r] = p.bp[15 - i];
        u1[r] = p.f1[15 - i];
        u2[r] = p.F[15 - i];
        z0[r] = p.lb[0][i];   // the last block's (length L - 16 (nblk - 1))
        z1[r] = p.lb[1][i];
        z2[r] = p.lb[2][i];
    }

    // one 16-token block: rows r0 .. r0 + 15 of the stage at X, tokens t0 ..
    auto block = [&](const char* X, int r0, int t0) __attribute__((always_inline)) {
        const char* Qs = X;
        const char* Ks = X + G::QKB;
        const char* Vs = X + 2 * G::QKB;
        const char* Ds = X + 2 * G::QKB + G::VB;
        const float* Es = reinterpret_cast<const float*>(X + 2 * G::QKB + 2 * G::VB);
        // readouts of the three states and the scores q_i . k_j
        f32x4 yT = zero4(), yP = zero4(), yM = zero4(), P = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / Tr<T>::KB; ++kb) {
            const auto qa = feat_frag(Qs, r0 + c16, kb);
            mma(yT, qa, state_frag(Tt, kb));
            mma(yP, qa, state_frag(Mp, kb));
            mma(yM, qa, state_frag(M, kb));
            mma(P, qa, feat_frag(Ks, r0 + c16, kb));
        }
        // R[i][j] = do_i . v_j over this wave's 16 columns (k = column 4g + s)
        f32x4 Rr = zero4();
        {
            f32x4 da, vb;
            if constexpr (BF) {
                da = unpack4(*reinterpret_cast<const u32x2*>(Ds + ((r0 + c16) * 16 + 4 * g) * 2));
                vb = unpack4(*reinterpret_cast<const u32x2*>(Vs + ((r0 + c16) * 16 + 4 * g) * 2));
            } else {
                da = *reinterpret_cast<const f32x4*>(Ds + ((r0 + c16) * 16 + 4 * g) * 4);
                vb = *reinterpret_cast<const f32x4*>(Vs + ((r0 + c16) * 16 + 4 * g) * 4);
            }
            mma16v(Rr, da, vb);
        }
        // lane (g, c16): token i = 4g + r (readout row, score row), column c16
        // for the readouts, key token j = c16 for the scores
        const f32x4 dcol = col4(Ds, r0, c16);
        const float ej = Eg ? Es[r0 + c16] : eta_s;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc += dcol[r] * (yT[r] + wP[r] * yP[r] + wM[r] * yM[r]) + wS[r] * ej * P[r] * Rr[r];
        // state update over the block's n tokens (a block past L changes nothing)
        const int n = min(16, L - t0);
        if (n <= 0) return;
        const f32x4 vcol = col4(Vs, r0, c16);
        f32x4 b0, b1, b2;   // rows j = 4g + s of diag(c_x eta) V
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float e = (Eg ? Es[r0 + 4 * g + s] : eta_s) * vcol[s];
            b0[s] = (n == 16 ? u0[s] : z0[s]) * e;
            b1[s] = (n == 16 ? u1[s] : z1[s]) * e;
            b2[s] = (n == 16 ? u2[s] : z2[s]) * e;
        }
        const float cT1 = p.bw[n - 1], cT2 = p.F[n], cB = p.bp[n], cB1 = p.f1[n];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const auto kp = kcol(Ks, r0, t);
            Tt[t] = Tt[t] + cT1 * Mp[t] + cT2 * M[t];
            mma16k(Tt[t], kp, b2);
            Mp[t] = cB * Mp[t] + cB1 * M[t];
            mma16k(Mp[t], kp, b1);
            M[t] = cB * M[t];
            mma16k(M[t], kp, b0);
        }
    };

    // vmcnt (gfx9: bits 3..0 and 15..14): after a stage's loads this wave
    // issued at least (R - 2) stages of loads, so waiting for that many left
    // has the stage in LDS (a wave's memory operations complete in order)
    constexpr int NW = (G::R - 2) * G::NL;
    constexpr int WAIT_STAGE = (NW & 15) | ((NW >> 4) << 14) | (0x7 << 4) | (0xf << 8);
    // the weights and M0 have landed: the compiler then sees nothing of its
    // own in flight inside the loop and adds no wait there
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
#pragma unroll
    for (int s = 0; s < G::R - 1; ++s) issue(s, ring + s * G::STAGE);
    for (int s = 0; s < nst; ++s) {
        __builtin_amdgcn_s_waitcnt(WAIT_STAGE);
        const int rd = s % G::R, wr = (s + G::R - 1) % G::R;
        // the stage refilled here was read in iteration s - 1 (its reads were consumed there)
        ring_step1(reinterpret_cast<bf16_t*>(ring + wr * G::STAGE), reinterpret_cast<const bf16_t*>(ring + rd * G::STAGE),
                   [&](bf16_t* dst) __attribute__((always_inline)) { issue(s + G::R - 1, reinterpret_cast<char*>(dst)); },
                   [&](const bf16_t* X) __attribute__((always_inline)) {
                       block(reinterpret_cast<const char*>(X), 0, DB_T * s);
                       block(reinterpret_cast<const char*>(X), 16, DB_T * s + 16);
                   });
    }
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));   // the clamped loads still in flight

    // boundary terms <dS_final, S'_{L-1}> + <dM_final, m'_{L-1}>
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t o = (int64_t)bh * DK * NSL * DV + (int64_t)(row0 + 16 * t + 4 * g) * DV + 16 * w + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (p.dS_final) acc += p.dS_final[o + (int64_t)r * DV] * Tt[t][r];
            if (p.dM_final) acc += p.dM_final[o + (int64_t)r * DV] * Mp[t][r];
        }
    }
    // wave sum in a fixed order
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) p.partial[lid] = acc;
}

// dbeta[bh] = the partial sums of its column tiles, in tile order
__global__ __launch_bounds__(256) void dbeta_finish_kernel(const float* partial, int ntile, int nbh, float* dbeta) {
    const int bh = blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= nbh) return;
    float s = 0.f;
    for (int t = 0; t < ntile; ++t) s += partial[bh * ntile + t];
    dbeta[bh] = s;
}

bool dbeta_supported(int dtype, int dk, int dv) {
    return (dtype == 0 || dtype == 1) && (dk == 32 || dk == 64 || dk == 128) && dv % 16 == 0 && dv >= 16 &&
           dv <= 1024;
}

// one partial sum per wave: up to 4 row slices per column tile
size_t dbeta_workspace(int B, int H, int dv) { return (size_t)B * H * (dv / 16) * 4 * sizeof(float); }

// weight tables in fp64 (sums, no closed forms: exact for beta near 1 too)
static void dbeta_tables(double beta, DbetaParams& p) {
    double pw[18];
    pw[0] = 1.0;
    for (int d = 1; d < 18; ++d) pw[d] = pw[d - 1] * beta;
    for (int d = 0; d <= 16; ++d) {
        p.bp[d] = (float)pw[d];
        p.f1[d] = d == 0 ? 0.f : (float)(d * pw[d - 1]);
        double F = 0.0;
        for (int e = 1; e <= d; ++e) F += e * pw[e - 1];
        p.F[d] = (float)F;
    }
    for (int i = 0; i < 16; ++i) {
        double s = 0.0;
        for (int l = 0; l <= i; ++l) s += pw[l];
        p.bw[i] = (float)(beta * s);
    }
    // the last block's token weights (zero past its end)
    const int n = p.L - 16 * ((p.L + 15) / 16 - 1);
    for (int j = 0; j < 16; ++j) {
        const int d = n - 1 - j;
        p.lb[0][j] = d >= 0 ? p.bp[d] : 0.f;
        p.lb[1][j] = d >= 0 ? p.f1[d] : 0.f;
        p.lb[2][j] = d >= 0 ? p.F[d] : 0.f;
    }
}

hipError_t launch_dbeta(DbetaParams p, int dtype, float beta, hipStream_t s) {
    if (!dbeta_supported(dtype, p.dk, p.dv)) return hipErrorInvalidValue;
    dbeta_tables(beta, p);
    // row slices of 32: one wave per (head, column tile, slice)
    const int nsl = p.dk / 32, ntile = p.dv / 16, nbh = p.B * p.H;
    const dim3 grid(nbh * ntile * nsl);
#define DB_LAUNCH(T, NSL) hipLaunchKernelGGL((dbeta_kernel<T, 32, NSL>), grid, dim3(64), 0, s, p)
    if (dtype == 1) {
        if (nsl == 1) DB_LAUNCH(bf16_t, 1);
        else if (nsl == 2) DB_LAUNCH(bf16_t, 2);
        else DB_LAUNCH(bf16_t, 4);
    } else {
        if (nsl == 1) DB_LAUNCH(float, 1);
        else if (nsl == 2) DB_LAUNCH(float, 2);
        else DB_LAUNCH(float, 4);
    }
#undef DB_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dbeta_finish_kernel, dim3((nbh + 255) / 256), dim3(256), 0, s, p.partial, ntile * nsl, nbh,
                       p.dbeta);
    return hipGetLastError();
}

}  // namespace ttt
