// swiglu.hip -- large-chunk SwiGLU fast weight (nonlinear fast-weight state).
//
// [P5] ("LaCT (Large Chunk Test-Time Training)", aisparkup.com/wiki/lact),
// section on the core idea: the fast weights are a nonlinear model whose
// state can grow to a large share of the model's parameters, and they take
// one update per large chunk whose tokens act as one big batch, which turns
// the update into GEMMs.  [P4] ("RNN의 기억을 작은 모델로 바꾼다면: Test-Time
// Training 읽기", ariser.io), section on the update rule: one gradient step
// on the inner loss, W <- W - eta grad l.  Per head and chunk i, with the
// weights left by chunks < i:
//
//     O_i = f_W(Q_i),   f_W(x) = W2 (silu(W1 x) * (W3 x))
//     W  <- W - grad_W sum_{t in i} eta_t l_t(W),
//     l_t = -<f_W(k_t), v_t>  (loss 0)   or   1/2 ||f_W(k_t) - v_t||^2  (loss 1)
//
// One chunk step is four launches over all heads, each a bf16 MFMA GEMM
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation, 2 x 2 waves per workgroup)
// with its elementwise work fused into the epilogue:
//
//   sw_fwd   [Q_i; K_i] x W13^T   (K = dk)  -> A = silu(H1) * H3 for the Q rows
//            (aq) and, for loss 1, the K rows (ak) with the two factors of
//            the SwiGLU derivative (cc): c1 = H3 silu'(H1), c3 = silu(H1).
//   sw_fwdk  loss 0, the K rows: K_i x W13^T and dA = V_i x W2 for the same
//            hidden units in one workgroup -> eta_t A and dH = -eta_t dA (c1, c3)
//            (dY = -eta_t V never formed, c1 and c3 never leave the chip).
//   sw_out   A x W2^T            (K = m)   -> O_i (Q rows); for loss 1 also
//            dY = eta_t (Y - V) (K rows).
//   sw_bwda  loss 1: dY x W2     (K = dv)  -> dA, then dH = (dA c1, dA c3).
//   sw_upd   dW2 = dY^T A_K and dW13 = dH^T K_i (K = chunk tokens), both in
//            one launch; the epilogue updates the fp32 master weights and
//            writes their bf16 copies for the next chunk.
//
// The GEMMs contracting over features stream their operands with gfx950's
// direct global-to-LDS loads (DLoop); the update, contracting over tokens,
// stages its loads through registers (Loop), which measured faster there.
//
// Layouts.  W13 interleaves the rows of W1 and W3 (row 2f = W1 row f,
// row 2f + 1 = W3 row f), so the gate and up values of one hidden unit land
// in consecutive accumulator registers of one lane and the SwiGLU epilogue
// needs no exchange; dH uses the same interleave, so dW13 = dH^T K comes out
// row-for-row in W13's layout.  The GEMMs contracting over features read
// both operands K-contiguous; those contracting over the chunk's tokens
// read token-major data through the gfx950 transposing LDS read.
//
// Tokens past the end of the sequence (a last, shorter chunk): loads are
// clamped to the last token, and the K-row epilogues write zero A and zero
// c1, c3 there, so those rows add nothing to the weight update.
#include "common.h"
#include "gemm.h"
#include "internal.h"

namespace ttt {

namespace {

using namespace gemm;

constexpr int SW_TILE = 128;   // dimensions are multiples of the small block tile
constexpr int SW_NT = GM_NT;
constexpr int SW_BK = GM_BK;


// Kernel arguments: base pointers (head 0) and per-head strides in elements.
struct SwDev {
    const bf16_t* q;
    const bf16_t* k;
    const bf16_t* v;
    const float* eta;
    float eta_scalar;
    float* W1;
    float* W3;
    float* W2;
    bf16_t* out;
    bf16_t* w13;   // [2m][dk]  W1 / W3 rows interleaved
    bf16_t* w2;    // [dv][m]
    bf16_t* w2t;   // [m][dv]
    bf16_t* aq;    // [C][m]    A of the Q rows
    bf16_t* ak;    // [C][m]    A of the K rows (times eta_t for loss 0)
    bf16_t* cc;    // [C][2m]   (c1, c3) per hidden unit, K rows
    bf16_t* dy;    // [C][dv]   loss 1 only
    bf16_t* dh;    // [C][2m]   (dH1, dH3) per hidden unit
    int64_t s_w13, s_w2, s_act, s_cc, s_dy;
    int L, dk, dv, m, C, c0, clen;
};

TTT_DEV float eta_at(const SwDev& p, int bh, int t) {
    return p.eta ? p.eta[(int64_t)bh * p.L + t] : p.eta_scalar;
}
// logistic sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of
// an IEEE division sequence; exp(-x) = inf gives 0
TTT_DEV float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// ------------------------------------------------------------ forward GEMM
// tile (row tile of W13, token tile of [Q_i; K_i]); K = dk
template <int LOSS, int TI, int TJ>
__global__ __launch_bounds__(SW_NT) void sw_fwd_kernel(SwDev p) {
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    using LP = DLoop<false, false, TI, TJ>;
    // epilogue staging: A [BN tokens][BM/2 + 4] and (K rows, loss 1) c1, c3 [BN][BM + 4]
    constexpr int AW = BM / 2, LA = AW + 4, LC = BM + 4;
    constexpr int STAGE = BN * (LA + (LOSS == 1 ? LC : 0));
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS > STAGE ? LP::LDS : STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int nct = p.C / BN;
    int bh, rt, ct;
    // the binding loss runs its K rows in sw_fwdk_kernel
    tile_id(2 * p.m / BM, (LOSS == 0 ? 1 : 2) * nct, &bh, &rt, &ct);
    const bool isK = ct >= nct;
    const int tok0 = (isK ? ct - nct : ct) * BN;
    Acc<TI, TJ> acc;
    zero(acc);
    if (tok0 < p.clen) {
        typename LP::OA a;
        typename LP::OB b;
        a.init(p.w13 + bh * p.s_w13, p.dk, rt * BM, 2 * p.m, tid);
        b.init((isK ? p.k : p.q) + ((int64_t)bh * p.L + p.c0) * p.dk, p.dk, tok0, p.L - p.c0, tid);
        LP::run(acc, p.dk / SW_BK, a, b, smem, tid);
    }
    // the SwiGLU values go through LDS ([token][feature]) so that the stores
    // to the token-major buffers are whole row segments
    __syncthreads();
    bf16_t* sA = smem;
    bf16_t* sC = smem + BN * LA;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int tl = acc_col<TJ>(wn, j, lane), tc = tok0 + tl;
        const bool live = tc < p.clen;
        // K rows: eta_t folded in for loss 0; zero past the sequence end
        const float e = !isK ? 1.f : !live ? 0.f : (LOSS == 0 ? eta_at(p, bh, p.c0 + tc) : 1.f);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int fl = acc_row<TI>(wm, i, q, lane) >> 1;   // local features fl, fl + 1
                const float g0 = acc[i][j][4 * q], u0 = acc[i][j][4 * q + 1];
                const float g1 = acc[i][j][4 * q + 2], u1 = acc[i][j][4 * q + 3];
                const float sg0 = sigm(g0), sg1 = sigm(g1);
                const float s0 = g0 * sg0, s1 = g1 * sg1;
                *reinterpret_cast<uint32_t*>(sA + tl * LA + fl) = pack2bf(e * s0 * u0, e * s1 * u1);
                if (isK) {
                    const float c10 = u0 * sg0 * (1.f + g0 * (1.f - sg0));
                    const float c11 = u1 * sg1 * (1.f + g1 * (1.f - sg1));
                    *reinterpret_cast<u32x2*>(sC + tl * LC + 2 * fl) =
                        live ? u32x2{pack2bf(c10, s0), pack2bf(c11, s1)} : u32x2{0u, 0u};
                }
            }
    }
    __syncthreads();
    // copy-out in 8-byte pieces, consecutive threads along a token's row
    // (K rows past the sequence end hold zeros; Q rows past it are not stored)
    const int f_base = rt * AW;
    bf16_t* dst = (isK ? p.ak : p.aq) + bh * p.s_act;
    constexpr int PA = AW / 4;
    for (int x = tid; x < BN * PA; x += SW_NT) {
        const int tl = x / PA, pc = x % PA, tc = tok0 + tl;
        if (!isK && tc >= p.clen) continue;
        *reinterpret_cast<u32x2*>(dst + (int64_t)tc * p.m + f_base + 4 * pc) =
            *reinterpret_cast<const u32x2*>(sA + tl * LA + 4 * pc);
    }
    if (isK) {
        bf16_t* ccb = p.cc + bh * p.s_cc;
        constexpr int PC = BM / 4;
        for (int x = tid; x < BN * PC; x += SW_NT) {
            const int tl = x / PC, pc = x % PC, tc = tok0 + tl;
            *reinterpret_cast<u32x2*>(ccb + (int64_t)tc * 2 * p.m + 2 * f_base + 4 * pc) =
                *reinterpret_cast<const u32x2*>(sC + tl * LC + 4 * pc);
        }
    }
}

// ---------------------------------------- K rows, binding loss: forward + dA
// For loss 0, dY = -eta_t V does not depend on the forward, so one workgroup
// computes for its 128 K tokens and 64 hidden units both H = K W13^T (K = dk)
// and dA = V W2 (K = dv, 64 x 128), and writes eta_t A and dH straight away:
// no (c1, c3) buffer and no separate dA launch.  dA goes through LDS to meet
// the forward's lane layout (a lane holds two hidden units of one token).
__global__ __launch_bounds__(SW_NT) void sw_fwdk_kernel(SwDev p) {
    constexpr int TI = 2, TJ = 2, BM = 128, BN = 128;
    using LH = DLoop<false, false, TI, TJ>;
    using LDa = DLoop<false, false, 1, TJ>;
    constexpr int AW = BM / 2, LA = AW + 4, LHD = BM + 4, LDD = AW + 4;
    constexpr int STAGE = BN * (LA + LHD);
    constexpr int SM = LH::LDS > STAGE ? LH::LDS : STAGE;
    static_assert(BN * LDD * 2 <= SM && LDa::LDS <= SM, "dA staging and its main loop fit");
    __shared__ __attribute__((aligned(16))) bf16_t smem[SM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    int bh, rt, ct;
    tile_id(2 * p.m / BM, p.C / BN, &bh, &rt, &ct);
    const int tok0 = ct * BN;
    Acc<TI, TJ> acc;
    Acc<1, TJ> dacc;
    zero(acc);
    zero(dacc);
    if (tok0 < p.clen) {
        {
            typename LH::OA a;
            typename LH::OB b;
            a.init(p.w13 + bh * p.s_w13, p.dk, rt * BM, 2 * p.m, tid);
            b.init(p.k + ((int64_t)bh * p.L + p.c0) * p.dk, p.dk, tok0, p.L - p.c0, tid);
            LH::run(acc, p.dk / SW_BK, a, b, smem, tid);
        }
        {
            typename LDa::OA a;
            typename LDa::OB b;
            a.init(p.w2t + bh * p.s_w2, p.dv, rt * AW, p.m, tid);
            b.init(p.v + ((int64_t)bh * p.L + p.c0) * p.dv, p.dv, tok0, p.L - p.c0, tid);
            LDa::run(dacc, p.dv / SW_BK, a, b, smem, tid);
        }
    }
    __syncthreads();
    float* sD = reinterpret_cast<float*>(smem);   // dA [token][unit]
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sD[acc_col<TJ>(wn, j, lane) * LDD + acc_row<1>(wm, 0, r >> 2, lane) + (r & 3)] = dacc[0][j][r];
    __syncthreads();
    uint32_t oa[TI][TJ][4];
    u32x2 oh[TI][TJ][4];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int tl = acc_col<TJ>(wn, j, lane), tc = tok0 + tl;
        const float e = tc < p.clen ? eta_at(p, bh, p.c0 + tc) : 0.f;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int fl = acc_row<TI>(wm, i, q, lane) >> 1;   // local units fl, fl + 1
                const f32x2 da = *reinterpret_cast<const f32x2*>(sD + tl * LDD + fl);
                const float g0 = acc[i][j][4 * q], u0 = acc[i][j][4 * q + 1];
                const float g1 = acc[i][j][4 * q + 2], u1 = acc[i][j][4 * q + 3];
                const float sg0 = sigm(g0), sg1 = sigm(g1);
                const float s0 = g0 * sg0, s1 = g1 * sg1;
                const float c10 = u0 * sg0 * (1.f + g0 * (1.f - sg0));
                const float c11 = u1 * sg1 * (1.f + g1 * (1.f - sg1));
                const float d0 = -e * da[0], d1 = -e * da[1];     // dA of the loss sum_t eta_t l_t
                oa[i][j][q] = pack2bf(e * s0 * u0, e * s1 * u1);
                oh[i][j][q] = u32x2{pack2bf(d0 * c10, d0 * s0), pack2bf(d1 * c11, d1 * s1)};
            }
    }
    __syncthreads();
    bf16_t* sA = smem;
    bf16_t* sH = smem + BN * LA;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int tl = acc_col<TJ>(wn, j, lane);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int fl = acc_row<TI>(wm, i, q, lane) >> 1;
                *reinterpret_cast<uint32_t*>(sA + tl * LA + fl) = oa[i][j][q];
                *reinterpret_cast<u32x2*>(sH + tl * LHD + 2 * fl) = oh[i][j][q];
            }
    }
    __syncthreads();
    const int f_base = rt * AW;
    bf16_t* ak = p.ak + bh * p.s_act;
    bf16_t* dh = p.dh + bh * p.s_cc;
    constexpr int PA = AW / 4, PH = BM / 4;
    for (int x = tid; x < BN * PA; x += SW_NT) {
        const int tl = x / PA, pc = x % PA;
        *reinterpret_cast<u32x2*>(ak + (int64_t)(tok0 + tl) * p.m + f_base + 4 * pc) =
            *reinterpret_cast<const u32x2*>(sA + tl * LA + 4 * pc);
    }
    for (int x = tid; x < BN * PH; x += SW_NT) {
        const int tl = x / PH, pc = x % PH;
        *reinterpret_cast<u32x2*>(dh + (int64_t)(tok0 + tl) * 2 * p.m + 2 * f_base + 4 * pc) =
            *reinterpret_cast<const u32x2*>(sH + tl * LHD + 4 * pc);
    }
}

// ------------------------------------------------------------- output GEMM
// tile (row tile of W2 = output features, token tile of A_Q, then of A_K for
// loss 1); K = m
template <int LOSS, int TI, int TJ>
__global__ __launch_bounds__(SW_NT) void sw_out_kernel(SwDev p) {
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    using LP = DLoop<false, false, TI, TJ>;
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int nct = p.C / BN;
    int bh, rt, ct;
    tile_id(p.dv / BM, LOSS ? 2 * nct : nct, &bh, &rt, &ct);
    const bool isK = ct >= nct;
    const int tok0 = (isK ? ct - nct : ct) * BN;
    Acc<TI, TJ> acc;
    zero(acc);
    if (tok0 < p.clen) {
        typename LP::OA a;
        typename LP::OB b;
        a.init(p.w2 + bh * p.s_w2, p.m, rt * BM, p.dv, tid);
        b.init((isK ? p.ak : p.aq) + bh * p.s_act, p.m, tok0, p.C, tid);
        LP::run(acc, p.m / SW_BK, a, b, smem, tid);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int tc = tok0 + acc_col<TJ>(wn, j, lane);
        const bool live = tc < p.clen;
        if (!isK) {
            if (!live) continue;
            bf16_t* orow = p.out + ((int64_t)bh * p.L + p.c0 + tc) * p.dv;
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = rt * BM + acc_row<TI>(wm, i, q, lane);
                    st4(orow + n, f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]});
                }
        } else {
            // dY = eta_t (Y - V); zero past the sequence end
            const float e = live ? eta_at(p, bh, p.c0 + tc) : 0.f;
            const bf16_t* vrow = p.v + ((int64_t)bh * p.L + p.c0 + min(tc, p.clen - 1)) * p.dv;
            bf16_t* yrow = p.dy + bh * p.s_dy + (int64_t)tc * p.dv;
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = rt * BM + acc_row<TI>(wm, i, q, lane);
                    const u32x2 vv = *reinterpret_cast<const u32x2*>(vrow + n);
                    f32x4 d;
                    d[0] = e * (acc[i][j][4 * q] - __uint_as_float(vv[0] << 16));
                    d[1] = e * (acc[i][j][4 * q + 1] - __uint_as_float(vv[0] & 0xffff0000u));
                    d[2] = e * (acc[i][j][4 * q + 2] - __uint_as_float(vv[1] << 16));
                    d[3] = e * (acc[i][j][4 * q + 3] - __uint_as_float(vv[1] & 0xffff0000u));
                    if (!live) d = zero4();
                    st4(yrow + n, d);
                }
        }
    }
}

// ----------------------------------------------------- dA and dH (K rows)
// tile (row tile of W2^T = hidden units, token tile); K = dv.  loss 0 reads
// V in place of dY and scales by -eta_t.
template <int LOSS, int TI, int TJ>
__global__ __launch_bounds__(SW_NT) void sw_bwda_kernel(SwDev p) {
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    using LP = DLoop<false, false, TI, TJ>;
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    int bh, rt, ct;
    tile_id(p.m / BM, p.C / BN, &bh, &rt, &ct);
    const int tok0 = ct * BN;
    Acc<TI, TJ> acc;
    zero(acc);
    if (tok0 < p.clen) {
        typename LP::OA a;
        typename LP::OB b;
        a.init(p.w2t + bh * p.s_w2, p.dv, rt * BM, p.m, tid);
        if (LOSS == 0) b.init(p.v + ((int64_t)bh * p.L + p.c0) * p.dv, p.dv, tok0, p.L - p.c0, tid);
        else b.init(p.dy + bh * p.s_dy, p.dv, tok0, p.C, tid);
        LP::run(acc, p.dv / SW_BK, a, b, smem, tid);
    }
    const bf16_t* ccb = p.cc + bh * p.s_cc;
    bf16_t* dhb = p.dh + bh * p.s_cc;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int tc = tok0 + acc_col<TJ>(wn, j, lane);
        const bool live = tc < p.clen;
        const float sc = !live ? 0.f : (LOSS == 0 ? -eta_at(p, bh, p.c0 + tc) : 1.f);
        const bf16_t* crow = ccb + (int64_t)tc * 2 * p.m;
        bf16_t* hrow = dhb + (int64_t)tc * 2 * p.m;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f0 = rt * BM + acc_row<TI>(wm, i, q, lane);   // hidden units f0 .. f0 + 3
                const u32x4 c = *reinterpret_cast<const u32x4*>(crow + 2 * f0);
                u32x4 o;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float da = sc * acc[i][j][4 * q + x];
                    o[x] = live ? pack2bf(da * __uint_as_float(c[x] << 16), da * __uint_as_float(c[x] & 0xffff0000u))
                                : 0u;
                }
                *reinterpret_cast<u32x4*>(hrow + 2 * f0) = o;
            }
    }
}

// ---------------------------------------------------------- weight update
// One launch, two problems per head (K = the chunk's tokens):
//   dW2[n][f]   = sum_t dY[t][n] A_K[t][f]   (loss 0: V and eta_t A_K, sign +)
//   dW13[r][c]  = sum_t dH[t][r] K[t][c]
// W <- W - dW in fp32, then the bf16 copies.
template <int LOSS, int TI, int TJ>
__global__ __launch_bounds__(SW_NT, 2) void sw_upd_kernel(SwDev p) {
    constexpr int BM = 64 * TI, BN = 64 * TJ;
    // register-staged loads (measured faster here than the direct-to-LDS
    // loop), three sets in flight; the launch bound asks for two waves per SIMD
    using LP = Loop<true, true, TI, TJ, (TI == 4 ? 3 : 4)>;
    __shared__ __attribute__((aligned(16))) bf16_t smem[LP::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int n4r = p.dv / BM, n4c = p.m / BN;
    const int n5r = 2 * p.m / BM, n5c = p.dk / BN;
    const int n4 = n4r * n4c, n5 = n5r * n5c;
    const int lid = xcd_logical(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    const int bh = lid / (n4 + n5), t = lid % (n4 + n5);
    const bool is5 = t >= n4;
    const int tt = is5 ? t - n4 : t, nc = is5 ? n5c : n4c;
    const int rt = tt / nc, ct = tt % nc;
    typename LP::OA a;
    typename LP::OB b;
    if (!is5) {
        if (LOSS == 0) a.init(p.v + ((int64_t)bh * p.L + p.c0) * p.dv, p.dv, rt * BM, p.L - p.c0, tid);
        else a.init(p.dy + bh * p.s_dy, p.dv, rt * BM, p.C, tid);
        b.init(p.ak + bh * p.s_act, p.m, ct * BN, p.C, tid);
    } else {
        a.init(p.dh + bh * p.s_cc, 2 * p.m, rt * BM, p.C, tid);
        b.init(p.k + ((int64_t)bh * p.L + p.c0) * p.dk, p.dk, ct * BN, p.L - p.c0, tid);
    }
    Acc<TI, TJ> acc;
    zero(acc);
    // tokens past the sequence end carry zero A_K and zero dH: the last,
    // shorter chunk still runs whole 128-token groups
    const int steps = ((p.clen + 127) / 128) * (128 / SW_BK);
    LP::run(acc, steps, a, b, smem, tid);

    // Epilogue, one accumulator row block i at a time through LDS (64 rows x
    // BN fp32): W_new = W + sign * dW with 16-byte read-modify-writes along
    // the master rows, the bf16 copies from the same values.
    constexpr int LDE = BN + 4;
    static_assert(64 * LDE * 4 <= LP::LDS * 2, "epilogue staging fits the main loop's LDS");
    float* sE = reinterpret_cast<float*>(smem);
    const float sgn = (!is5 && LOSS == 0) ? 1.f : -1.f;
    // staged row l (0..63) -> tile row: l < 32 from wave row 0, else wave row 1
    auto tile_row = [&](int l, int i) { return (l < 32 ? 0 : 32 * TI - 32) + 32 * i + l; };
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int l = 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                sE[l * LDE + acc_col<TJ>(wn, j, lane)] = acc[i][j][r];
            }
        __syncthreads();
        constexpr int P4 = BN / 4;
        for (int x = tid; x < 64 * P4; x += SW_NT) {
            const int l = x / P4, c4 = 4 * (x % P4);
            const int R = rt * BM + tile_row(l, i), col = ct * BN + c4;
            f32x4 d = *reinterpret_cast<const f32x4*>(sE + l * LDE + c4);
            float* wp;
            bf16_t* cp;
            if (!is5) {
                wp = p.W2 + (int64_t)bh * p.dv * p.m + (int64_t)R * p.m + col;
                cp = p.w2 + bh * p.s_w2 + (int64_t)R * p.m + col;
            } else {
                wp = ((R & 1) ? p.W3 : p.W1) + (int64_t)bh * p.m * p.dk + (int64_t)(R >> 1) * p.dk + col;
                cp = p.w13 + bh * p.s_w13 + (int64_t)R * p.dk + col;
            }
            const f32x4 w = *reinterpret_cast<const f32x4*>(wp) + sgn * d;
            *reinterpret_cast<f32x4*>(wp) = w;
            *reinterpret_cast<u32x2*>(cp) = u32x2{pack2bf(w[0], w[1]), pack2bf(w[2], w[3])};
            if (!is5) *reinterpret_cast<f32x4*>(sE + l * LDE + c4) = w;
        }
        if (!is5) {
            // W2^T copy: 4 consecutive rows n of one column f per 8-byte store
            __syncthreads();
            for (int x = tid; x < 16 * BN; x += SW_NT) {
                const int g = x % 16, fl = x / 16, l = 4 * g;
                const int n0 = rt * BM + tile_row(l, i), f = ct * BN + fl;
                const float* e = sE + l * LDE + fl;
                *reinterpret_cast<u32x2*>(p.w2t + bh * p.s_w2 + (int64_t)f * p.dv + n0) =
                    u32x2{pack2bf(e[0], e[LDE]), pack2bf(e[2 * LDE], e[3 * LDE])};
            }
        }
    }
}

// ------------------------------------------------------- bf16 weight copies
// w13 (interleaved W1 / W3 rows) and w2 from the fp32 weights; 4 elements per thread
__global__ __launch_bounds__(256) void sw_copy_kernel(SwDev p, int BH) {
    const int64_t n13 = (int64_t)BH * 2 * p.m * p.dk / 4, n2 = (int64_t)BH * p.dv * p.m / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n13) {
        const int64_t e = 4 * i;
        const int64_t per = (int64_t)2 * p.m * p.dk;
        const int64_t bh = e / per, rem = e % per;
        const int R = (int)(rem / p.dk), c = (int)(rem % p.dk);
        const float* src = ((R & 1) ? p.W3 : p.W1) + bh * p.m * p.dk + (int64_t)(R >> 1) * p.dk + c;
        const f32x4 w = *reinterpret_cast<const f32x4*>(src);
        *reinterpret_cast<u32x2*>(p.w13 + bh * p.s_w13 + rem) = u32x2{pack2bf(w[0], w[1]), pack2bf(w[2], w[3])};
    } else if (i < n13 + n2) {
        const int64_t e = 4 * (i - n13);
        const int64_t per = (int64_t)p.dv * p.m;
        const int64_t bh = e / per, rem = e % per;
        const f32x4 w = *reinterpret_cast<const f32x4*>(p.W2 + e);
        *reinterpret_cast<u32x2*>(p.w2 + bh * p.s_w2 + rem) = u32x2{pack2bf(w[0], w[1]), pack2bf(w[2], w[3])};
    }
}

// w2t = W2^T in bf16, 32 x 32 tiles through LDS; grid (dv/32 * m/32, BH)
__global__ __launch_bounds__(256) void sw_transpose_kernel(SwDev p) {
    __shared__ float tile[32][33];
    const int bh = blockIdx.y, nf = p.m / 32;
    const int n0 = (blockIdx.x / nf) * 32, f0 = (blockIdx.x % nf) * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const float* W = p.W2 + (int64_t)bh * p.dv * p.m;
    for (int r = ty; r < 32; r += 8) tile[r][tx] = W[(int64_t)(n0 + r) * p.m + f0 + tx];
    __syncthreads();
    bf16_t* o = p.w2t + bh * p.s_w2;
    for (int r = ty; r < 32; r += 8) o[(int64_t)(f0 + r) * p.dv + n0 + tx] = (bf16_t)tile[tx][r];
}

// workspace layout: eight regions, each 256-byte aligned
struct Layout {
    int64_t off[8];
    int64_t per[8];   // elements per head
    size_t bytes;
};
Layout layout(int BH, int dk, int dv, int m, int C) {
    Layout l{};
    const int64_t per[8] = {(int64_t)2 * m * dk, (int64_t)dv * m, (int64_t)dv * m, (int64_t)C * m,
                            (int64_t)C * m,      (int64_t)C * 2 * m, (int64_t)C * dv, (int64_t)C * 2 * m};
    size_t at = 0;
    for (int r = 0; r < 8; ++r) {
        l.per[r] = per[r];
        l.off[r] = (int64_t)at;
        at += ((size_t)BH * per[r] * 2 + 255) / 256 * 256;
    }
    l.bytes = at;
    return l;
}

// one chunk: forward (for loss 0 the Q rows here, the K rows fused with dA
// in sw_fwdk_kernel), output, dA / dH (loss 1), weight update.  The forward
// GEMMs run 128 x 128 tiles; with BIG the output and dA GEMMs run 256 x 256
// and the update 256 x 128 tiles (each measured fastest among 128 / 256
// choices for its kernel).
template <int LOSS, bool BIG>
hipError_t chunk_step(const SwDev& p, const SwParams& in, hipStream_t s) {
    constexpr int F = BIG ? 4 : 2;
    const dim3 blk(SW_NT);
    const int C = in.chunk;
    const dim3 g_fwd((2 * in.m / 128) * ((LOSS ? 2 : 1) * C / 128), in.BH);
    const dim3 g_out((in.dv / (64 * F)) * (LOSS ? 2 : 1) * (C / (64 * F)), in.BH);
    const dim3 g_bwda((in.m / (64 * F)) * (C / (64 * F)), in.BH);
    const dim3 g_upd((in.dv / (64 * F)) * (in.m / 128) + (2 * in.m / (64 * F)) * (in.dk / 128), in.BH);
    hipLaunchKernelGGL((sw_fwd_kernel<LOSS, 2, 2>), g_fwd, blk, 0, s, p);
    if (LOSS == 0) hipLaunchKernelGGL(sw_fwdk_kernel, dim3((2 * in.m / 128) * (C / 128), in.BH), blk, 0, s, p);
    hipLaunchKernelGGL((sw_out_kernel<LOSS, F, F>), g_out, blk, 0, s, p);
    if (LOSS == 1) hipLaunchKernelGGL((sw_bwda_kernel<LOSS, F, F>), g_bwda, blk, 0, s, p);
    hipLaunchKernelGGL((sw_upd_kernel<LOSS, F, 2>), g_upd, blk, 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool swiglu_supported(int dk, int dv, int m, int chunk) {
    return dk > 0 && dv > 0 && m > 0 && chunk > 0 && dk % SW_TILE == 0 && dv % SW_TILE == 0 && m % SW_TILE == 0 &&
           chunk % SW_TILE == 0;
}

size_t swiglu_workspace(int BH, int dk, int dv, int m, int chunk) { return layout(BH, dk, dv, m, chunk).bytes; }

hipError_t launch_swiglu(const SwParams& in, hipStream_t s) {
    if (!swiglu_supported(in.dk, in.dv, in.m, in.chunk) || (in.loss != 0 && in.loss != 1)) return hipErrorInvalidValue;
    const Layout l = layout(in.BH, in.dk, in.dv, in.m, in.chunk);
    char* ws = reinterpret_cast<char*>(in.workspace);
    SwDev p{};
    p.q = reinterpret_cast<const bf16_t*>(in.q);
    p.k = reinterpret_cast<const bf16_t*>(in.k);
    p.v = reinterpret_cast<const bf16_t*>(in.v);
    p.eta = in.eta;
    p.eta_scalar = in.eta_scalar;
    p.W1 = in.W1;
    p.W3 = in.W3;
    p.W2 = in.W2;
    p.out = reinterpret_cast<bf16_t*>(in.out);
    bf16_t** dst[8] = {&p.w13, &p.w2, &p.w2t, &p.aq, &p.ak, &p.cc, &p.dy, &p.dh};
    for (int r = 0; r < 8; ++r) *dst[r] = reinterpret_cast<bf16_t*>(ws + l.off[r]);
    p.s_w13 = l.per[0];
    p.s_w2 = l.per[1];
    p.s_act = l.per[3];
    p.s_cc = l.per[5];
    p.s_dy = l.per[6];
    p.L = in.L;
    p.dk = in.dk;
    p.dv = in.dv;
    p.m = in.m;
    p.C = in.chunk;

    const int64_t ncopy = ((int64_t)in.BH * 2 * in.m * in.dk + (int64_t)in.BH * in.dv * in.m) / 4;
    hipLaunchKernelGGL(sw_copy_kernel, dim3((unsigned)((ncopy + 255) / 256)), dim3(256), 0, s, p, in.BH);
    hipLaunchKernelGGL(sw_transpose_kernel, dim3((in.dv / 32) * (in.m / 32), in.BH), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // big tiles (256-row / 256-token blocks) where the sizes allow, else 128 x 128
    const bool big = in.m % 256 == 0 && in.dv % 256 == 0 && in.chunk % 256 == 0;
    for (int c0 = 0; c0 < in.L; c0 += in.chunk) {
        p.c0 = c0;
        p.clen = min(in.chunk, in.L - c0);
        if (in.loss == 0) e = big ? chunk_step<0, true>(p, in, s) : chunk_step<0, false>(p, in, s);
        else e = big ? chunk_step<1, true>(p, in, s) : chunk_step<1, false>(p, in, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ttt
