// tcb_fwd.hip -- bf16 chunked fast-weight forward for d_k in {64, 128} and
// d_v tiles of 64 (the LM-scale and momentum shapes).
//
// Same mathematics as tc_fwd.hip (see its header for the pages' passages and
// the momentum algebra); this is the gfx950-tuned form of it:
//   * Q, K, V chunks are staged in LDS as plain row copies; the transposed
//     operands K^T (state update) and V (intra term and update) are read out
//     of the row-major tiles with ds_read_b64_tr_b16, so staging is a copy.
//   * Rows are XOR-swizzled at 16-byte granularity (swz below), which makes
//     the row reads, the paired 8-byte reads, the transposing reads and the
//     staging writes all free of LDS bank conflicts.
//   * LDS is double-buffered: chunk c+1 is loaded into registers while chunk
//     c computes and written to the other buffer at the end, so each chunk
//     costs two barriers.
//   * eta (and the momentum weights) scale the V fragment in registers; the
//     same fragment feeds the intra-chunk term and the state update.
//   * The fp32 state lives in MFMA accumulators for the whole sequence and
//     feeds the readout straight from registers (accperm k-assignment).
// One workgroup = (b, h, 64-column dv tile), 4 waves; wave w owns state and
// output columns [16w, 16w+16) of the tile.  Chunk tile = 64 tokens.
#include "common.h"
#include "internal.h"

namespace ttt {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16-byte-chunk swizzle of a row-major bf16 tile with NCH chunks per row
template <int NCH> TTT_DEV int swz(int r);
template <> TTT_DEV int swz<16>(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
template <> TTT_DEV int swz<8>(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
template <int NCH> TTT_DEV int so(int r, int e) {       // element offset of (row r, element e)
    return r * (NCH * 8) + ((((e >> 3) ^ swz<NCH>(r))) << 3) + (e & 7);
}

// operand fragment, contig k-assignment: row r, k = kb0 + 8g .. +7
template <int NCH> TTT_DEV bf16x8 fr_contig(const bf16_t* t, int r, int kb0, int g) {
    return *reinterpret_cast<const bf16x8*>(t + so<NCH>(r, kb0 + 8 * g));
}
// operand fragment, accperm k-assignment: row r, k = kb0 + 4g + {0..3}, kb0 + 16 + 4g + {0..3}
template <int NCH> TTT_DEV bf16x8 fr_accperm(const bf16_t* t, int r, int kb0, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(t + so<NCH>(r, kb0 + 4 * g));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(t + so<NCH>(r, kb0 + 16 + 4 * g));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
TTT_DEV u32x2 tr_read(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
// Transposed operand: lane l <-> tile column c0 + l%16, k = tile rows in the
// accperm assignment starting at row kb0.  ds_read_b64_tr_b16: in each group
// of 16 lanes, lane a loads 4 consecutive values and lane i receives, in slot
// j, the value lane 4j + i/4 loaded in its slot i%4; lane a therefore points
// at row kb0 + 4g + a/4, columns c0 + 4(a%4) .. +3.
template <int NCH> TTT_DEV bf16x8 fr_tr(const bf16_t* t, int c0, int kb0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    const int col = c0 + 4 * (a & 3);
    const int r = kb0 + 4 * g + (a >> 2);
    const u32x2 lo = tr_read(t + so<NCH>(r, col));
    const u32x2 hi = tr_read(t + so<NCH>(r + 16, col));
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// scale the 8 bf16 values of a fragment by per-slot factors
TTT_DEV bf16x8 scale_frag(const bf16x8& f, const f32x4& s_lo, const f32x4& s_hi) {
    const u32x4 w = __builtin_bit_cast(u32x4, f);
    const u32x4 o = u32x4{pack2bf(__uint_as_float(w[0] << 16) * s_lo[0], __uint_as_float(w[0] & 0xffff0000u) * s_lo[1]),
                          pack2bf(__uint_as_float(w[1] << 16) * s_lo[2], __uint_as_float(w[1] & 0xffff0000u) * s_lo[3]),
                          pack2bf(__uint_as_float(w[2] << 16) * s_hi[0], __uint_as_float(w[2] & 0xffff0000u) * s_hi[1]),
                          pack2bf(__uint_as_float(w[3] << 16) * s_hi[2], __uint_as_float(w[3] & 0xffff0000u) * s_hi[3])};
    return __builtin_bit_cast(bf16x8, o);
}

}  // namespace

template <int DK, int MODE>
__global__ __launch_bounds__(256) void tcb_fwd_kernel(TcParams p) {
    constexpr int CS = 64, DVT = 64, NW = 4, NT = 256;
    constexpr int NCQ = DK / 8;             // 16-byte chunks per Q/K row
    constexpr int NCV = DVT / 8;            // ... per V row
    constexpr int LP = CS + 8;              // sP row stride (padded)
    constexpr bool MOM = (MODE == MODE_MOM);
    constexpr bool HAS_P = (MODE != MODE_CC);
    constexpr int NV = MOM ? 3 : 1;         // eta | eta*w_{n-1-j} | eta*beta^{n-1-j}
    constexpr int NTD = DK / 16;            // state tiles along dk
    constexpr int NKB = DK / 32;            // K-blocks along dk
    constexpr int UQ = CS * NCQ / NT;       // staged chunks per thread (Q and K each)
    constexpr int UV = CS * NCV / NT;

    __shared__ __attribute__((aligned(16))) bf16_t sQ[2][CS * DK];
    __shared__ __attribute__((aligned(16))) bf16_t sK[2][CS * DK];
    __shared__ __attribute__((aligned(16))) bf16_t sV[2][CS * DVT];
    __shared__ __attribute__((aligned(16))) float sE[2][NV][CS];
    __shared__ __attribute__((aligned(16))) bf16_t sP[HAS_P ? CS * LP : 8];
    __shared__ float sTab[3 * (CS + 1)];    // w_p | beta^p | a_p

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;

    int bh, vt;
    {
        const int i = blockIdx.x;
        if (p.xcd_map) {
            const int grp = i / (8 * p.n_vt), rem = i % (8 * p.n_vt);
            bh = grp * 8 + (rem & 7);
            vt = rem >> 3;
        } else {
            bh = i / p.n_vt;
            vt = i % p.n_vt;
        }
    }
    const int b = bh / p.H, h = bh % p.H;
    const int n0 = vt * DVT;
    const int L = p.L;
    const bf16_t* Qg = reinterpret_cast<const bf16_t*>(p.q) + b * p.qs[0] + h * p.qs[1];
    const bf16_t* Kg = reinterpret_cast<const bf16_t*>(p.k) + b * p.ks[0] + h * p.ks[1];
    const bf16_t* Vg = reinterpret_cast<const bf16_t*>(p.v) + b * p.vs[0] + h * p.vs[1] + n0;
    bf16_t* Og = reinterpret_cast<bf16_t*>(p.out) + b * p.os[0] + h * p.os[1] + n0;
    const float* Eg = p.eta ? p.eta + b * p.es[0] + h * p.es[1] : nullptr;
    const int64_t qL = p.qs[2], kL = p.ks[2], vL = p.vs[2], oL = p.os[2], eL = p.es[2];

    if (MOM) {
        for (int pp = tid; pp <= CS; pp += NT) {
            const double be = (double)p.beta;
            double bp = 1.0;
            for (int x = 0; x < pp; ++x) bp *= be;
            const double bp1 = bp * be;
            sTab[pp] = (float)((1.0 - bp1) / (1.0 - be));
            sTab[(CS + 1) + pp] = (float)bp;
            sTab[2 * (CS + 1) + pp] = (float)(be * (1.0 - bp1) / (1.0 - be));
        }
    }
    if (HAS_P) {  // strictly-upper P tiles stay zero
        for (int x = tid; x < CS * LP / 8; x += NT)
            reinterpret_cast<u32x4*>(sP)[x] = u32x4{0, 0, 0, 0};
    }

    // ---- state accumulators S[16t + 4g + r][16*wave + c16] (and m)
    f32x4 Sacc[NTD];
    f32x4 Macc[MOM ? NTD : 1];
    {
        const float* S0 = p.S0 ? p.S0 + b * p.s0s[0] + h * p.s0s[1] : nullptr;
        const float* M0 = (MOM && p.M0) ? p.M0 + b * p.m0s[0] + h * p.m0s[1] : nullptr;
        const int col = n0 + 16 * wave + c16;
#pragma unroll
        for (int t = 0; t < NTD; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * g + r;
                Sacc[t][r] = S0 ? S0[(int64_t)row * p.dv + col] : 0.f;
                if (MOM) Macc[t][r] = M0 ? M0[(int64_t)row * p.dv + col] : 0.f;
            }
    }
    bf16x8 Sop[NKB], Mop[MOM ? NKB : 1];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Sop[kb] = acc_to_frag_bf16(Sacc[2 * kb], Sacc[2 * kb + 1]);
    if (MOM) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) Mop[kb] = acc_to_frag_bf16(Macc[2 * kb], Macc[2 * kb + 1]);
    }

    // ---- staging registers
    u32x4 rq[UQ], rk[UQ], rv[UV];
    float re = 0.f;
    auto load = [&](int c) {
        const int t0 = c * CS;
#pragma unroll
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT, r = u / NCQ, ch = u % NCQ, t = t0 + r;
            const bool ok = t < L;
            rq[x] = ok ? *reinterpret_cast<const u32x4*>(Qg + t * qL + 8 * ch) : u32x4{0, 0, 0, 0};
            rk[x] = ok ? *reinterpret_cast<const u32x4*>(Kg + t * kL + 8 * ch) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT, r = u / NCV, ch = u % NCV, t = t0 + r;
            rv[x] = (t < L) ? *reinterpret_cast<const u32x4*>(Vg + t * vL + 8 * ch) : u32x4{0, 0, 0, 0};
        }
        if (tid < CS) {
            const int t = t0 + tid;
            re = (t < L) ? (Eg ? Eg[t * eL] : p.eta_scalar) : 0.f;
        }
    };
    auto store = [&](int c, int buf) {
#pragma unroll
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT, r = u / NCQ, ch = u % NCQ;
            *reinterpret_cast<u32x4*>(&sQ[buf][so<NCQ>(r, 8 * ch)]) = rq[x];
            *reinterpret_cast<u32x4*>(&sK[buf][so<NCQ>(r, 8 * ch)]) = rk[x];
        }
#pragma unroll
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT, r = u / NCV, ch = u % NCV;
            *reinterpret_cast<u32x4*>(&sV[buf][so<NCV>(r, 8 * ch)]) = rv[x];
        }
        if (tid < CS) {
            sE[buf][0][tid] = re;
            if (MOM) {
                const int n = min(CS, L - c * CS);
                const int pw = n - 1 - tid;
                sE[buf][1][tid] = (pw >= 0) ? re * sTab[pw] : 0.f;
                sE[buf][2][tid] = (pw >= 0) ? re * sTab[(CS + 1) + pw] : 0.f;
            }
        }
    };

    const int ntiles = (L + CS - 1) / CS;
    load(0);
    __syncthreads();  // tables ready
    store(0, 0);
    __syncthreads();

    for (int c = 0; c < ntiles; ++c) {
        const int cur = c & 1;
        const int tbase = c * CS;
        const int n = min(CS, L - tbase);
        if (c + 1 < ntiles) load(c + 1);
        const bf16_t* Q = sQ[cur];
        const bf16_t* K = sK[cur];
        const bf16_t* V = sV[cur];

        // ------------- intra scores P^T = K Q^T (lower-triangular 16x16 tiles)
        if (HAS_P) {
            // tiles grouped by query tile so a wave reuses its Q fragments:
            // w0: (1,3)(2,3)(3,3)  w1: (0,2)(1,2)(2,2)  w2: (0,1)(1,1)(0,0)  w3: (0,3)
            int ti, tj0, ntj;
            if (wave == 0) { ti = 3; tj0 = 1; ntj = 3; }
            else if (wave == 1) { ti = 2; tj0 = 0; ntj = 3; }
            else if (wave == 2) { ti = 1; tj0 = 0; ntj = 2; }
            else { ti = 3; tj0 = 0; ntj = 1; }
            for (int pass = 0; pass < 2; ++pass) {
                if (pass == 1) {                 // wave 2 also owns (0,0)
                    if (wave != 2) break;
                    ti = 0; tj0 = 0; ntj = 1;
                }
                f32x4 pa[3] = {zero4(), zero4(), zero4()};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 bq = fr_contig<NCQ>(Q, 16 * ti + c16, 32 * kb, g);
#pragma unroll
                    for (int x = 0; x < 3; ++x)
                        if (x < ntj) mma(pa[x], fr_contig<NCQ>(K, 16 * (tj0 + x) + c16, 32 * kb, g), bq);
                }
                const int i = 16 * ti + c16;
#pragma unroll
                for (int x = 0; x < 3; ++x) {
                    if (x >= ntj) break;
                    const int tj = tj0 + x;
                    f32x4 v = pa[x];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tj + 4 * g + r;
                        float val = (j <= i) ? v[r] : 0.f;
                        if (MOM && j <= i) val *= sTab[i - j];
                        v[r] = val;
                    }
                    st4(&sP[i * LP + 16 * tj + 4 * g], v);
                }
            }
            __syncthreads();
        }

        // ------------- value fragments: raw V^T (accperm over tokens), scaled in registers
        bf16x8 VB[2], VS[MOM ? 2 : 1], VM[MOM ? 2 : 1];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bf16x8 raw = fr_tr<NCV>(V, 16 * wave, 32 * jb, lane);
            const float* e0 = &sE[cur][0][32 * jb + 4 * g];
            VB[jb] = scale_frag(raw, *reinterpret_cast<const f32x4*>(e0), *reinterpret_cast<const f32x4*>(e0 + 16));
            if (MOM) {
                const float* e1 = &sE[cur][1][32 * jb + 4 * g];
                const float* e2 = &sE[cur][2][32 * jb + 4 * g];
                VS[jb] = scale_frag(raw, *reinterpret_cast<const f32x4*>(e1), *reinterpret_cast<const f32x4*>(e1 + 16));
                VM[jb] = scale_frag(raw, *reinterpret_cast<const f32x4*>(e2), *reinterpret_cast<const f32x4*>(e2 + 16));
            }
        }

        // ------------- readout O^T = S^T Q^T (+ a_i m^T Q^T) + V~^T P^T
        {
            f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
            f32x4 acc2[MOM ? 4 : 1];
            if (MOM) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) acc2[ti] = zero4();
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                bf16x8 bq[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) bq[ti] = fr_accperm<NCQ>(Q, 16 * ti + c16, 32 * kb, g);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    mma(acc[ti], Sop[kb], bq[ti]);
                    if (MOM) mma(acc2[ti], Mop[kb], bq[ti]);
                }
            }
            if (HAS_P) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const bf16_t* prow = &sP[(16 * ti + c16) * LP];
                    mma(acc[ti], VB[0], ld_accperm(prow, 0, g));
                    if (ti >= 2) mma(acc[ti], VB[1], ld_accperm(prow, 32, g));
                }
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int i = 16 * ti + c16;
                f32x4 o = acc[ti];
                if (MOM) {
                    const float a = sTab[2 * (CS + 1) + i];
                    for (int r = 0; r < 4; ++r) o[r] += a * acc2[ti][r];
                }
                if (i < n) st4(&Og[(int64_t)(tbase + i) * oL + 16 * wave + 4 * g], o);
            }
        }

        // ------------- state update S += K^T V~  (momentum: affine chunk transition)
        {
            if (MOM) {
                const float alpha = sTab[2 * (CS + 1) + (n - 1)];
                const float gamma = sTab[(CS + 1) + n];
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    Sacc[t] += alpha * Macc[t];
                    Macc[t] *= gamma;
                }
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const bf16x8 a = fr_tr<NCQ>(K, 16 * t, 32 * jb, lane);
                    mma(Sacc[t], a, MOM ? VS[jb] : VB[jb]);
                    if (MOM) mma(Macc[t], a, VM[jb]);
                }
            }
            bool refresh = true;
            if (MODE == MODE_CC) {
                const int end = tbase + CS;
                refresh = (end % p.chunk == 0) || (end >= L);
            }
            if (refresh) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) Sop[kb] = acc_to_frag_bf16(Sacc[2 * kb], Sacc[2 * kb + 1]);
                if (MOM) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) Mop[kb] = acc_to_frag_bf16(Macc[2 * kb], Macc[2 * kb + 1]);
                }
            }
        }
        if (c + 1 < ntiles) store(c + 1, cur ^ 1);
        __syncthreads();
    }

    const int col = n0 + 16 * wave + c16;
    if (p.S_final) {
        float* Sf = p.S_final + (int64_t)bh * p.dk * p.dv;
#pragma unroll
        for (int t = 0; t < NTD; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sf[(int64_t)(16 * t + 4 * g + r) * p.dv + col] = Sacc[t][r];
    }
    if (MOM && p.M_final) {
        float* Mf = p.M_final + (int64_t)bh * p.dk * p.dv;
#pragma unroll
        for (int t = 0; t < NTD; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Mf[(int64_t)(16 * t + 4 * g + r) * p.dv + col] = Macc[t][r];
    }
}

bool tcb_supported(int dtype, int dk, int dv) {
    return dtype == 1 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

hipError_t launch_tcb_fwd(const TcParams& pin, int mode, hipStream_t s) {
    TcParams p = pin;
    p.n_vt = p.dv / 64;
    p.xcd_map = ((p.B * p.H) % 8 == 0) ? 1 : 0;
    const dim3 grid(p.B * p.H * p.n_vt), block(256);
#define TTT_L(DK_, M_) hipLaunchKernelGGL((tcb_fwd_kernel<DK_, M_>), grid, block, 0, s, p)
    if (p.dk == 128) {
        if (mode == MODE_TC) TTT_L(128, MODE_TC);
        else if (mode == MODE_MOM) TTT_L(128, MODE_MOM);
        else TTT_L(128, MODE_CC);
    } else {
        if (mode == MODE_TC) TTT_L(64, MODE_TC);
        else if (mode == MODE_MOM) TTT_L(64, MODE_MOM);
        else TTT_L(64, MODE_CC);
    }
#undef TTT_L
    return hipGetLastError();
}

}  // namespace ttt
