// tcb_fwd.hip -- bf16 chunked fast-weight forward for d_k in {64, 128} and
// d_v tiles of 32 or 64 columns (the LM-scale and momentum shapes).
//
// Same mathematics as tc_fwd.hip (its header cites the pages' passages and
// derives the momentum algebra); this is the gfx950-tuned form:
//   * Wave w owns state columns [16(w%NNT), +16) of the column tile and one
//     half of the d_k rows (w/NNT); the two halves of a column tile add their
//     readout partial sums through LDS at the top of the next chunk, so no
//     extra barrier is needed.  Tiles: CS tokens x DVT columns; the 32 x 32
//     form (4 waves, ~50 KB LDS) runs two workgroups per CU with independent
//     barriers, the 64 x 64 form (8 waves) one.
//   * Q, K, V chunks are staged as plain row copies in a K-block-major
//     layout [block of 32 features][token][32] with a 16-byte XOR swizzle
//     (swz below): row reads, paired 8-byte reads and the transposing reads
//     (ds_read_b64_tr_b16, which give K^T and V operands straight from the
//     token-major tiles) are all bank-conflict free, and every fragment
//     address is a per-lane base computed once plus a compile-time offset.
//   * LDS is double-buffered; chunk c+2 is fetched into registers while c
//     computes, chunk c+1 is written to LDS at the end: two barriers per chunk.
//   * The output tile is summed over the two d_k halves, rounded and parked
//     in LDS, then written as full 128-byte row segments by all threads.
//   * eta and the momentum weights scale the V fragment in registers; the
//     fp32 state is held in MFMA accumulators for the whole sequence and
//     feeds the readout from registers.
#include "common.h"
#include "internal.h"

#include <type_traits>

namespace ttt {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Block strides (elements) of the [token][32] blocks: the pads keep the
// row-order staging writes conflict free; reads never cross a block within
// one instruction.
template <int CS> constexpr int blk_qk() { return CS * 32 + 32; }
template <int CS, int DVT> constexpr int blk_v() { return DVT == 64 ? CS * 32 + 64 : CS * 32; }
// output tile swizzle: 16-byte chunk position of row i (rows of DVT columns)
template <int DVT> TTT_DEV int oswz(int i) { return DVT == 64 ? ((i >> 1) & 7) : ((i >> 2) & 3); }

TTT_DEV int swz(int r) { return (((r >> 2) & 1) << 1) | ((r >> 3) & 1); }
// (row r, feature e) of a tile lives at element (e/32)*BLK + r*32 + 8*(((e/8)%4) ^ swz(r)) + e%8

TTT_DEV u32x2 tr_read(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}
TTT_DEV bf16x8 join(const u32x2& lo, const u32x2& hi) {
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}
// 8 bf16 values of one row times one scale, rounded back to bf16
TTT_DEV u32x4 scale_row(const u32x4& w, float e) {
    return u32x4{pack2bf(__uint_as_float(w[0] << 16) * e, __uint_as_float(w[0] & 0xffff0000u) * e),
                 pack2bf(__uint_as_float(w[1] << 16) * e, __uint_as_float(w[1] & 0xffff0000u) * e),
                 pack2bf(__uint_as_float(w[2] << 16) * e, __uint_as_float(w[2] & 0xffff0000u) * e),
                 pack2bf(__uint_as_float(w[3] << 16) * e, __uint_as_float(w[3] & 0xffff0000u) * e)};
}

}  // namespace

// OSC: output rows are scaled by per-token factors (a compile-time switch, so
// the forward carries no dead scaling code)
template <int DK, int MODE, int CS, int DVT, bool OSC>
__global__ __launch_bounds__(DVT / 16 * 128) void tcb_fwd_kernel(TcParams p) {
    constexpr int NNT = DVT / 16;           // column tiles per workgroup
    constexpr int NW = 2 * NNT, NT = 64 * NW;
    static_assert((CS == 64 && DVT == 64) || (CS == 32 && DVT == 32), "tile forms: 64x64, 32x32");
    constexpr int NTI = CS / 16;            // token tiles per chunk
    constexpr int NJB = CS / 32;            // token K-blocks per chunk
    constexpr int BLK = blk_qk<CS>();
    constexpr int BLKV = blk_v<CS, DVT>();
    constexpr int NVC = CS * DVT / 8;       // 16-byte chunks of a V tile
    constexpr int NKB = DK / 32;            // feature blocks of Q / K
    constexpr int DKH = DK / 2;             // d_k rows per wave
    constexpr int NTH = DKH / 16;           // state tiles per wave
    constexpr int NKH = DKH / 32;           // K-blocks per wave
    constexpr int LP = CS + 8;              // sP row stride
    constexpr bool MOM = (MODE == MODE_MOM);
    constexpr bool HAS_P = (MODE != MODE_CC);
    constexpr int NV = MOM ? 3 : 1;         // eta | eta*w_{n-1-j} | eta*beta^{n-1-j}
    constexpr int UQ = CS * DK / 8 / NT;    // 16-byte chunks per thread (Q and K each)

    __shared__ __attribute__((aligned(16))) bf16_t sQ[2][NKB * BLK];
    __shared__ __attribute__((aligned(16))) bf16_t sK[2][NKB * BLK];
    // V staged already scaled per token: eta | eta*w_{n-1-j} | eta*beta^{n-1-j}
    __shared__ __attribute__((aligned(16))) bf16_t sV[2][NV][(DVT / 32) * BLKV];
    __shared__ __attribute__((aligned(16))) float sOS[2][CS];     // output row scales
    // one barrier per chunk (64 x 64 form without momentum): the score, partial
    // and output tiles are double-buffered, see the chunk loop
    constexpr bool PIPE = (CS == 64) && !MOM;
    constexpr int NPB = PIPE ? 2 : 1;
    __shared__ __attribute__((aligned(16))) bf16_t sP[NPB][HAS_P ? CS * LP : 8];
    __shared__ __attribute__((aligned(16))) f32x4 sX[NPB][NNT][NTI][64];   // half-1 readout partials
    __shared__ __attribute__((aligned(16))) bf16_t sO[NPB][CS * DVT];  // finished output tile
    __shared__ float sTab[3 * (CS + 1)];                           // w_p | beta^p | a_p

    // the wave index is made uniform (scalar), so branches on it are scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int nt = wave % NNT, hf = wave / NNT;

    // ---- which (head, dv tile, segment) this workgroup runs
    const int ntiles = (p.L + CS - 1) / CS;
    const int nbv = p.B * p.H * p.n_vt;
    const bool segmented = p.nseg > 1;
    int bh, vt, seg = 0, c_begin = 0, c_end = ntiles;
    __shared__ int sTicket;
    if (segmented) {
        // Tickets hand out segments in order, so a workgroup only ever waits
        // for workgroups that took a ticket before it and are running.  With
        // xcd_map the workgroups form 8 groups by blockIdx % 8 (the XCD the
        // dispatcher places them on), each with a counter of its own and
        // every (segment, dv tile) of the heads bh = 8 i + group: the tiles
        // of a head then read its K and Q through one XCD's L2, and all a
        // workgroup waits for is in its own group, ahead of it in segment
        // order.  Correctness needs only the group's own counts, which
        // blockIdx fixes, not where the hardware puts the workgroups.
        const int G = p.xcd_map ? 8 : 1, grp = (int)(blockIdx.x % G);
        if (tid == 0) sTicket = atomicAdd(p.lb_flags + (int64_t)nbv * p.nseg + 2 + grp, 1);
        __syncthreads();
        const int per = nbv / G, t = sTicket, r = t % per;
        seg = t / per;
        bh = (r / p.n_vt) * G + grp;
        vt = r % p.n_vt;
        c_begin = seg * p.seg_tiles;
        c_end = min(c_begin + p.seg_tiles, ntiles);
    } else {
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
    if (HAS_P) {
        for (int x = tid; x < NPB * CS * LP / 8; x += NT) reinterpret_cast<u32x4*>(&sP[0][0])[x] = u32x4{0, 0, 0, 0};
    }

    // ---- per-lane LDS bases (elements)
    // row reads of rows r0 + c16: contig k = 8g..; accperm k = 4g.., 16 + 4g..
    const int sw_l = swz(c16);
    const int b_contig = c16 * 32 + 8 * (g ^ sw_l);
    const int b_ap0 = c16 * 32 + 8 * ((g >> 1) ^ sw_l) + 4 * (g & 1);
    const int b_ap1 = c16 * 32 + 8 * ((2 + (g >> 1)) ^ sw_l) + 4 * (g & 1);
    // transposing reads: lane (g, a) -> row 4g + a/4, column 16*par + 4(a%4) of a block
    const int a_tr = lane & 15;
    const int r_tr = 4 * g + (a_tr >> 2);
    const int b_tr0 = r_tr * 32 + 8 * ((0 | ((a_tr & 3) >> 1)) ^ swz(r_tr)) + 4 * (a_tr & 1);
    const int b_tr1 = r_tr * 32 + 8 * ((2 | ((a_tr & 3) >> 1)) ^ swz(r_tr)) + 4 * (a_tr & 1);
    // V fragment of this wave's columns 16*nt: block nt/2, parity nt&1
    const int b_v = (nt >> 1) * BLKV + ((nt & 1) ? b_tr1 : b_tr0);

    // ---- state accumulators S[DKH*hf + 16t + 4g + r][16*nt + c16]
    f32x4 Sacc[NTH];
    f32x4 Macc[MOM ? NTH : 1];
    auto load_initial = [&](f32x4* S, f32x4* M) {
        const float* S0 = p.S0 ? p.S0 + b * p.s0s[0] + h * p.s0s[1] : nullptr;
        const float* M0 = (MOM && p.M0) ? p.M0 + b * p.m0s[0] + h * p.m0s[1] : nullptr;
        const int col = n0 + 16 * nt + c16;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = DKH * hf + 16 * t + 4 * g + r;
                const int64_t e = p.s0_trans ? (int64_t)col * p.dk + row : (int64_t)row * p.dv + col;
                S[t][r] = S0 ? S0[e] : 0.f;
                if (MOM) M[t][r] = M0 ? M0[e] : 0.f;
            }
    };
    if (!segmented) load_initial(Sacc, Macc);
    bf16x8 Sop[NKH], Mop[MOM ? NKH : 1];

    // ---- staging: each 16-byte piece of a row goes to its swizzled slot of the
    // K-block-major layout (16 lanes cover one 256-byte Q/K row)
    // register sets for chunks in flight: chunk c+PF is requested after the
    // output store of iteration c (the memory counter retires in order, so a
    // later wait on the store leaves these loads in flight); momentum keeps
    // one set, its VGPRs are taken by the second state
    constexpr int PF = MOM ? 1 : 2;
    u32x4 rq[PF][UQ], rk[PF][UQ], rv[PF];
    float re[PF], ros[PF];
    const float* OSg = p.oscale ? p.oscale + b * p.ocs[0] + h * p.ocs[1] : nullptr;
    // staging: 16 lanes load one 256-byte Q/K row (8 lanes one 128-byte V row);
    // chunk c of row r lands in block c/4 at swizzled position (c%4)^swz(r)
    int loff_q[UQ], loff_v;
#pragma unroll
    for (int x = 0; x < UQ; ++x) {
        const int u = tid + x * NT, row = u / (DK / 8), ch = u % (DK / 8);
        loff_q[x] = (ch >> 2) * BLK + row * 32 + 8 * ((ch & 3) ^ swz(row));
    }
    {
        const int row = tid / (DVT / 8), ch = tid % (DVT / 8);
        loff_v = (ch >> 2) * BLKV + row * 32 + 8 * ((ch & 3) ^ swz(row));
    }
    // Every lane issues the same loads for every chunk: rows past L read row
    // L-1 again (their eta is zero, so they add nothing; their outputs are
    // never stored) and a chunk index past the end refetches the last chunk.
    // With no load under a branch, the memory counter advances uniformly and
    // the compiler's waits before the LDS writes drain only the oldest set.
    // The chunk base is a scalar 64-bit pointer; a lane's offset within the
    // chunk is a signed 24-bit product (|L stride| < 2^23 elements; a
    // negative stride walks the sequence backwards).
    int row_q[UQ], pc_q[UQ];
#pragma unroll
    for (int x = 0; x < UQ; ++x) {
        row_q[x] = (tid + x * NT) / (DK / 8);
        pc_q[x] = 8 * ((tid + x * NT) % (DK / 8));
    }
    const int row_v = (tid % NVC) / (DVT / 8), pc_v = 8 * ((tid % NVC) % (DVT / 8));
    const int qL24 = (int)qL, kL24 = (int)kL, vL24 = (int)vL, eL24 = (int)eL;
    auto load = [&](int c, auto SET, auto WITHQ) {
        constexpr int st = decltype(SET)::value;
        constexpr bool wq = decltype(WITHQ)::value;
        const int t0 = min(c, ntiles - 1) * CS;
        const int lim = min(CS, L - t0) - 1;      // last row of this chunk
        const bf16_t* Qc = Qg + (int64_t)t0 * qL;
        const bf16_t* Kc = Kg + (int64_t)t0 * kL;
        const bf16_t* Vc = Vg + (int64_t)t0 * vL;
#pragma unroll
        for (int x = 0; x < UQ; ++x) {
            const int rr = min(row_q[x], lim);
            if (wq) rq[st][x] = *reinterpret_cast<const u32x4*>(Qc + (__mul24(rr, qL24) + pc_q[x]));
            rk[st][x] = *reinterpret_cast<const u32x4*>(Kc + (__mul24(rr, kL24) + pc_q[x]));
        }
        // V rows are read by this workgroup alone (Q and K rows also by the
        // other d_v tiles of the head, through L2), output rows are written
        // once: both stream past the caches (non-temporal)
        rv[st] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vc + (__mul24(min(row_v, lim), vL24) + pc_v)));
        // (tokens past L get eta 0 when the chunk is written to LDS: a select
        // here would make the compiler wait for this load right away)
        re[st] = Eg ? (Eg + (int64_t)t0 * eL)[__mul24(min(tid % CS, lim), eL24)] : p.eta_scalar;
        if (OSC) ros[st] = OSg ? OSg[(int64_t)(t0 + min(tid % CS, lim)) * p.ocs[2]] : p.oscale_scalar;
    };
    // one 16-byte piece of a V row (8 columns of token row_v) into the staged
    // copies: times eta (e), and with momentum also times eta*w_{n-1-j} and
    // eta*beta^{n-1-j}, each rounded to bf16 once
    auto stage_v = [&](int buf, const u32x4& raw, float e, int n) {
        *reinterpret_cast<u32x4*>(&sV[buf][0][loff_v]) = scale_row(raw, e);
        if (MOM) {
            const int pw = max(n - 1 - row_v, 0);   // rows past the end have e = 0
            *reinterpret_cast<u32x4*>(&sV[buf][1 % NV][loff_v]) = scale_row(raw, e * sTab[pw]);
            *reinterpret_cast<u32x4*>(&sV[buf][2 % NV][loff_v]) = scale_row(raw, e * sTab[(CS + 1) + pw]);
        }
    };
    auto store = [&](int c, int buf, auto SET, auto WITHQ) {
        constexpr int st = decltype(SET)::value;
        constexpr bool wq = decltype(WITHQ)::value;
#pragma unroll
        for (int x = 0; x < UQ; ++x) {
            if (wq) *reinterpret_cast<u32x4*>(&sQ[buf][loff_q[x]]) = rq[st][x];
            *reinterpret_cast<u32x4*>(&sK[buf][loff_q[x]]) = rk[st][x];
        }
        if (tid < NVC) {
            // the eta of token r sits in lane r of every wave; zero past the end
            const int n = min(CS, L - c * CS);
            const float e = __shfl(re[st], row_v);
            stage_v(buf, rv[st], row_v < n ? e : 0.f, n);
        }
        if (OSC && tid < CS) sOS[buf][tid] = ros[st];
    };

    // P^T tile assignment (query tile ti; key tiles tjA, tjB; -1 = none), grouped by
    // query tile so a wave reuses its Q fragments.  The waves of d_k half 1
    // take the pairs: half 0 also sums the previous output tile before the
    // first barrier, so it gets at most one tile.
    int p_ti = -1, p_tjA = -1, p_tjB = -1;
    if (CS == 64) {
        switch (wave) {
            case 4: p_ti = 3; p_tjA = 1; p_tjB = 2; break;
            case 5: p_ti = 3; p_tjA = 0; p_tjB = 3; break;
            case 6: p_ti = 2; p_tjA = 0; p_tjB = 1; break;
            case 7: p_ti = 1; p_tjA = 0; p_tjB = 1; break;
            case 0: p_ti = 2; p_tjA = 2; break;
            case 1: p_ti = 0; p_tjA = 0; break;
            default: break;
        }
    } else {
        if (wave == 2) { p_ti = 1; p_tjA = 0; p_tjB = 1; }
        else if (wave == 3) { p_ti = 0; p_tjA = 0; }
    }

    f32x4 oacc[NTI];  // this wave's readout partial of the previous chunk (half 0 keeps it)
    int prev_base = 0, prev_n = 0, prev_buf = 0;
    // half 0: add half 1's partial, round, and park the tile in sO (rows of 128 B,
    // 16-byte chunks swizzled by (row/2)%8: conflict-free for both sides)
    auto combine = [&]() {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) {
            const int i = 16 * ti + c16;
            f32x4 o = oacc[ti] + sX[0][nt][ti][lane];
            if (OSC) o *= sOS[prev_buf][i];
            const int ch = (2 * nt + (g >> 1)) ^ oswz<DVT>(i);
            st4(&sO[0][i * DVT + 8 * ch + 4 * (g & 1)], o);
        }
    };
    // all threads: write the parked tile out as full 128-byte row segments
    auto write_out = [&]() {
        const int row = tid / (DVT / 8), ch = tid % (DVT / 8);
        if (tid < NVC && row < prev_n) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(&sO[0][row * DVT + 8 * (ch ^ oswz<DVT>(row))]);
            bf16_t* Oc = Og + (int64_t)prev_base * oL;
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(Oc + (__mul24(row, (int)oL) + 8 * ch)));
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, PF - 1>;
    using WQ = std::true_type;
    using NQ = std::false_type;

    // value fragments of the staged chunk (tokens in accperm order), staged
    // already scaled by eta (VB) and, with momentum, eta*w_{n-1-j} (VS) and
    // eta*beta^{n-1-j} (VM)
    auto vfrags = [&](int cur, bf16x8* VB, bf16x8* VS, bf16x8* VM) {
        auto frag = [&](int k, int jb) {
            const bf16_t* V = sV[cur][k];
            return join(tr_read(V + b_v + (32 * jb) * 32), tr_read(V + b_v + (32 * jb + 16) * 32));
        };
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            VB[jb] = frag(0, jb);
            if (MOM) {
                VS[jb] = frag(1 % NV, jb);
                VM[jb] = frag(2 % NV, jb);
            }
        }
    };
    // S (and m) over one staged chunk of n tokens, this wave's d_k half
    auto state_update = [&](int cur, int n, const bf16x8* VB, const bf16x8* VS, const bf16x8* VM) {
        if (MOM) {
            const float alpha = sTab[2 * (CS + 1) + (n - 1)];
            const float gamma = sTab[(CS + 1) + n];
#pragma unroll
            for (int t = 0; t < NTH; ++t) {
                Sacc[t] += alpha * Macc[t];
                Macc[t] *= gamma;
            }
        }
        const bf16_t* Kh = sK[cur] + (hf * NTH / 2) * BLK;   // d_k half -> feature blocks
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
            for (int t = 0; t < NTH; ++t) {
                const int base = (t >> 1) * BLK + ((t & 1) ? b_tr1 : b_tr0) + (32 * jb) * 32;
                const bf16x8 a = join(tr_read(Kh + base), tr_read(Kh + base + 16 * 32));
                mma(Sacc[t], a, MOM ? VS[jb] : VB[jb]);
                if (MOM) mma(Macc[t], a, VM[jb]);
            }
        }
    };
    auto refresh_ops = [&]() {
#pragma unroll
        for (int kk = 0; kk < NKH; ++kk) Sop[kk] = acc_to_frag_bf16(Sacc[2 * kk], Sacc[2 * kk + 1]);
        if (MOM) {
#pragma unroll
            for (int kk = 0; kk < NKH; ++kk) Mop[kk] = acc_to_frag_bf16(Macc[2 * kk], Macc[2 * kk + 1]);
        }
    };

    if (segmented) {
        // ================= look-back over sequence segments =================
        // A segment of n tokens maps the state (S, m) it starts from to
        //     (S + a_n m + X, beta^n m + Y),  a_n = beta + ... + beta^n,
        // where (X, Y) is the segment's own result from a zero start (its
        // aggregate).  Segment s publishes its aggregate, then walks back over
        // segments s-1, s-2, ..., composing their aggregates into the running
        // map T.  The walk has a fixed shape, so results never depend on
        // timing: it ends at the inclusive state of segment s - kChain (the
        // state after that segment, which it publishes once its own walk is
        // done), or past segment 0, where T is applied to (S0, M0).  So a
        // segment reads at most kChain - 1 aggregates and one inclusive
        // state, and inclusive states form a chain of nseg / kChain links.
        // Exchange blocks use the accumulator layout itself (lane-private
        // f32x4 slots), so publishing and reading are coalesced 16-byte
        // accesses with no reshuffle.
        constexpr int NSTATE = MOM ? 2 : 1;
        constexpr int kChain = 8;   // segments per link of the inclusive-state chain
        const int my_id = seg * nbv + bh * p.n_vt + vt;
        auto slot = [&](int id, int which, int st, int t) -> f32x4* {
            return reinterpret_cast<f32x4*>(p.lb_data + ((int64_t)id * 2 + which) * p.lb_stride) +
                   ((wave * NSTATE + st) * NTH + t) * 64 + lane;
        };
        // Publishing: every wave waits for its own stores to reach L2, then one
        // thread makes them visible device-wide (one agent-scope release: an
        // L2 write-back) and raises the flag.  Agent-scope fences in every wave
        // would write back and invalidate the XCD's L2 once per wave.
        auto publish = [&](int which, const f32x4* S, const f32x4* M) {
#pragma unroll
            for (int t = 0; t < NTH; ++t) {
                *slot(my_id, which, 0, t) = S[t];
                if (MOM) *slot(my_id, which, 1, t) = M[t];
            }
            __builtin_amdgcn_s_waitcnt(0);   // this wave's stores are complete
            __syncthreads();
            if (tid == 0) __hip_atomic_store(p.lb_flags + my_id, which + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        };
        // Waiting: one thread polls the flag with relaxed agent-scope loads
        // until it reaches `want` (1: aggregate published, 2: inclusive state
        // too), then acquires once: the acquire invalidates this CU's L1 and
        // the stale lines of the XCD's L2, which the other waves' loads go
        // through after the barrier.  (An acquire load in the loop would
        // invalidate the XCD's L2 on every poll, under the feet of every
        // workgroup still computing there.)  The wait is bounded by
        // p.lb_max_polls: a flag that never arrives ends it, the error word in
        // the workspace is raised (the host reads it back) and every wave
        // still finishes, with wrong results.
        auto wait_flag = [&](int id, int want) {
            if (tid == 0) {
                int v = 0;
                for (int spin = 0; spin < p.lb_max_polls; ++spin) {
                    v = __hip_atomic_load(p.lb_flags + id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (v >= want) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if (v < want) __hip_atomic_store(p.lb_error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        };
        const int seg_len = p.seg_tiles * CS;           // every segment but the last is full
        float a_seg = 0.f, g_seg = 1.f;
        if (MOM) {
            const double be = (double)p.beta, bn = pow(be, (double)seg_len);
            a_seg = (float)(be * (1.0 - bn) / (1.0 - be));
            g_seg = (float)bn;
        }

        // ---- pass 1: this segment's aggregate (K, V, eta only)
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
            Sacc[t] = zero4();
            if (MOM) Macc[t] = zero4();
        }
        __syncthreads();   // tables ready
        const bool last = (seg == p.nseg - 1);
        if (!last) {
            // K, V and eta only, three chunks in flight: register set k % 3
            // carries chunk c_begin + k until it is written to LDS buffer k % 2
            constexpr int D = 3;
            u32x4 ak[D][UQ], av[D];
            float ae[D];
            // Every lane issues the same loads in every step (past the segment end
            // the last chunk is fetched again, V and eta lanes wrap): the memory
            // counter then advances uniformly and a wait before an LDS write
            // only drains the oldest set instead of all three.
            auto kv_load = [&](int c, auto SET) {
                constexpr int st = decltype(SET)::value;
                const int t0 = min(c, c_end - 1) * CS;   // segments before the last hold only whole chunks
                const bf16_t* Kc = Kg + (int64_t)t0 * kL;
#pragma unroll
                for (int x = 0; x < UQ; ++x) {
                    const int row = (tid + x * NT) / (DK / 8);
                    const int64_t ko = (int64_t)row * kL + 8 * ((tid + x * NT) % (DK / 8));
                    ak[st][x] = *reinterpret_cast<const u32x4*>(Kc + ko);
                }
                {
                    const int u = tid % NVC, row = u / (DVT / 8), ch = u % (DVT / 8);
                    av[st] = *reinterpret_cast<const u32x4*>(Vg + (int64_t)(t0 + row) * vL + 8 * ch);
                }
                ae[st] = Eg ? Eg[(t0 + (tid % CS)) * eL] : p.eta_scalar;
            };
            auto kv_store = [&](int buf, auto SET) {
                constexpr int st = decltype(SET)::value;
#pragma unroll
                for (int x = 0; x < UQ; ++x) *reinterpret_cast<u32x4*>(&sK[buf][loff_q[x]]) = ak[st][x];
                if (tid < NVC) stage_v(buf, av[st], __shfl(ae[st], row_v), CS);
            };
            using J0 = std::integral_constant<int, 0>;
            using J1 = std::integral_constant<int, 1>;
            using J2 = std::integral_constant<int, 2>;
            kv_load(c_begin, J0{});
            kv_load(c_begin + 1, J1{});
            kv_load(c_begin + 2, J2{});
            kv_store(0, J0{});
            __syncthreads();
            auto step = [&](int c, auto CUR, auto NXT) {
                const int buf = (c - c_begin) & 1;
                kv_load(c + 3, CUR);
                bf16x8 VB[NJB], VS[MOM ? NJB : 1], VM[MOM ? NJB : 1];
                vfrags(buf, VB, VS, VM);
                state_update(buf, CS, VB, VS, VM);
                if (c + 1 < c_end) kv_store(buf ^ 1, NXT);
                __syncthreads();
            };
            // With momentum (beta <= 0.95) the aggregate of the segment's n
            // tokens is X = sum_s w_{n-1-s} g_s = (U - beta Y) / (1 - beta)
            // (w_m = (1 - beta^{m+1}) / (1 - beta)), with U = sum_s g_s and
            // Y = sum_s beta^{n-1-s} g_s the momentum aggregate.  So every
            // chunk stages only the eta-scaled copy of V and adds to U, and Y,
            // whose weights fall below 2^-30 within 30 / -log2(beta) tokens,
            // runs its recurrence over the last chunks only.  (Closer to 1,
            // the 1 / (1 - beta) factor would amplify rounding; those betas
            // take the chunk recurrence of S and m above.)
            const bool split = MOM && p.beta <= 0.95f;
            const int tail_from = split ? c_end - min(c_end - c_begin, (int)ceil(30.0 / -log2((double)p.beta) / CS))
                                        : c_end;
            auto kv_store_split = [&](int buf, auto SET, bool tail) {
                constexpr int st = decltype(SET)::value;
#pragma unroll
                for (int x = 0; x < UQ; ++x) *reinterpret_cast<u32x4*>(&sK[buf][loff_q[x]]) = ak[st][x];
                if (tid < NVC) {
                    const float e = __shfl(ae[st], row_v);
                    *reinterpret_cast<u32x4*>(&sV[buf][0][loff_v]) = scale_row(av[st], e);
                    if (tail)
                        *reinterpret_cast<u32x4*>(&sV[buf][2 % NV][loff_v]) =
                            scale_row(av[st], e * sTab[(CS + 1) + (CS - 1 - row_v)]);
                }
            };
            auto step_split = [&](int c, auto CUR, auto NXT) {
                const int buf = (c - c_begin) & 1;
                const bool tail = c >= tail_from;
                kv_load(c + 3, CUR);
                bf16x8 VB[NJB], VM[NJB];
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    const bf16_t* V0 = sV[buf][0];
                    VB[jb] = join(tr_read(V0 + b_v + (32 * jb) * 32), tr_read(V0 + b_v + (32 * jb + 16) * 32));
                }
                if (tail) {
                    const float gamma = sTab[(CS + 1) + CS];
#pragma unroll
                    for (int t = 0; t < NTH; ++t) Macc[t] *= gamma;
#pragma unroll
                    for (int jb = 0; jb < NJB; ++jb) {
                        const bf16_t* V2 = sV[buf][2 % NV];
                        VM[jb] = join(tr_read(V2 + b_v + (32 * jb) * 32), tr_read(V2 + b_v + (32 * jb + 16) * 32));
                    }
                }
                const bf16_t* Kh = sK[buf] + (hf * NTH / 2) * BLK;
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
#pragma unroll
                    for (int t = 0; t < NTH; ++t) {
                        const int base = (t >> 1) * BLK + ((t & 1) ? b_tr1 : b_tr0) + (32 * jb) * 32;
                        const bf16x8 a = join(tr_read(Kh + base), tr_read(Kh + base + 16 * 32));
                        mma(Sacc[t], a, VB[jb]);
                        if (tail) mma(Macc[t], a, VM[jb]);
                    }
                }
                if (c + 1 < c_end) kv_store_split(buf ^ 1, NXT, c + 1 >= tail_from);
                __syncthreads();
            };
            if (split) {
                __syncthreads();   // the first chunk was staged with all copies: restage
                kv_store_split(0, J0{}, c_begin >= tail_from);
                __syncthreads();
                for (int c = c_begin; c < c_end; c += D) {
                    step_split(c, J0{}, J1{});
                    if (c + 1 < c_end) step_split(c + 1, J1{}, J2{});
                    if (c + 2 < c_end) step_split(c + 2, J2{}, J0{});
                }
                const float beta = p.beta, inv = (float)(1.0 / (1.0 - (double)p.beta));
#pragma unroll
                for (int t = 0; t < NTH; ++t) Sacc[t] = (Sacc[t] - beta * Macc[t]) * inv;
            } else {
                for (int c = c_begin; c < c_end; c += D) {
                    step(c, J0{}, J1{});
                    if (c + 1 < c_end) step(c + 1, J1{}, J2{});
                    if (c + 2 < c_end) step(c + 2, J2{}, J0{});
                }
            }
            publish(0, Sacc, Macc);
        }

        // ---- look-back: T(S, m) = (S + aT m + XT, gT m + YT)
        f32x4 XT[NTH], YT[MOM ? NTH : 1];
        float aT = 0.f, gT = 1.f;
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
            XT[t] = zero4();
            if (MOM) YT[t] = zero4();
        }
        bool have_base = false;
        for (int j = seg - 1; j >= 0 && !have_base; --j) {
            const int id = j * nbv + bh * p.n_vt + vt;
            const bool base = (seg - j == kChain);
            wait_flag(id, base ? 2 : 1);
            if (base) {
                // inclusive state after segment j: the base of the walk
#pragma unroll
                for (int t = 0; t < NTH; ++t) {
                    const f32x4 Sb = *slot(id, 1, 0, t);
                    if (MOM) {
                        const f32x4 Mb = *slot(id, 1, 1, t);
                        XT[t] += Sb + aT * Mb;
                        YT[t] += gT * Mb;
                    } else {
                        XT[t] += Sb;
                    }
                }
                have_base = true;
            } else {
                // aggregate of segment j: T <- T o f_j
#pragma unroll
                for (int t = 0; t < NTH; ++t) {
                    const f32x4 X = *slot(id, 0, 0, t);
                    if (MOM) {
                        const f32x4 Y = *slot(id, 0, 1, t);
                        XT[t] += X + aT * Y;
                        YT[t] += gT * Y;
                    } else {
                        XT[t] += X;
                    }
                }
                aT = a_seg + aT * g_seg;
                gT = gT * g_seg;
            }
        }
        if (!have_base) {
            // past segment 0: apply T to the initial state
            f32x4 S0v[NTH], M0v[MOM ? NTH : 1];
            load_initial(S0v, M0v);
#pragma unroll
            for (int t = 0; t < NTH; ++t) {
                if (MOM) {
                    XT[t] += S0v[t] + aT * M0v[t];
                    YT[t] += gT * M0v[t];
                } else {
                    XT[t] += S0v[t];
                }
            }
        }
        // XT, YT = state at the segment start; publish the state at its end
        // (read only by segment seg + kChain)
        if (seg + kChain < p.nseg) {
#pragma unroll
            for (int t = 0; t < NTH; ++t) {
                if (MOM) {
                    Sacc[t] += XT[t] + a_seg * YT[t];
                    Macc[t] += g_seg * YT[t];
                } else {
                    Sacc[t] += XT[t];
                }
            }
            publish(1, Sacc, Macc);
        }
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
            Sacc[t] = XT[t];
            if (MOM) Macc[t] = YT[t];
        }
    }
    refresh_ops();

    load(c_begin, I0{}, WQ{});
    __syncthreads();   // tables ready
    store(c_begin, 0, I0{}, WQ{});
    load(c_begin + 1, I1{}, WQ{});
    __syncthreads();

    // intra scores P^T = K Q^T of one staged chunk (lower-triangular 16x16
    // tiles) into the score tile P
    auto scores = [&](const bf16_t* Q, const bf16_t* K, bf16_t* P) {
        if (HAS_P && p_ti >= 0) {
            // all fragments are read before the first product (a wave with one
            // key tile computes its tile twice rather than branch in between)
            const int tjB = p_tjB >= 0 ? p_tjB : p_tjA;
            bf16x8 fq[NKB], fa[NKB], fb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                fq[kb] = *reinterpret_cast<const bf16x8*>(Q + kb * BLK + p_ti * 512 + b_contig);
                fa[kb] = *reinterpret_cast<const bf16x8*>(K + kb * BLK + p_tjA * 512 + b_contig);
                fb[kb] = *reinterpret_cast<const bf16x8*>(K + kb * BLK + tjB * 512 + b_contig);
            }
            f32x4 pa = zero4(), pb = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                mma(pa, fa[kb], fq[kb]);
                mma(pb, fb[kb], fq[kb]);
            }
            const int i = 16 * p_ti + c16;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int tj = x ? p_tjB : p_tjA;
                if (tj < 0) break;
                f32x4 v = x ? pb : pa;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * tj + 4 * g + r;
                    float val = (j <= i) ? v[r] : 0.f;
                    if (MOM && j <= i) val *= sTab[i - j];
                    v[r] = val;
                }
                st4(&P[i * LP + 16 * tj + 4 * g], v);
            }
        }
    };

    // chunk c_begin + k travels in register set k % PF; chunk c+1 is written
    // to the other LDS buffer at the end of iteration c
    auto iter = [&](int c, auto LSET, auto SSET) {
        const int cur = (c - c_begin) & 1;
        const int tbase = c * CS;
        const int n = min(CS, L - tbase);
        const bf16_t* Q = sQ[cur];
        const bf16_t* K = sK[cur];

        if (hf == 0 && c > c_begin) combine();

        scores(Q, K, sP[0]);
        // P^T complete; the previous chunk's output tile is parked in sO and
        // half 0 has read half 1's partials before they are overwritten below
        __syncthreads();
        if (c > c_begin) write_out();
        if (PF == 2) load(c + 2, LSET, WQ{});

        bf16x8 VB[NJB], VS[MOM ? NJB : 1], VM[MOM ? NJB : 1];
        vfrags(cur, VB, VS, VM);

        // ------------- readout partial: O^T = S_h^T Q_h^T (+ a_i m_h^T Q_h^T) (+ V~^T P^T share)
        {
            f32x4 acc[NTI];
            f32x4 acc2[MOM ? NTI : 1];
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                acc[ti] = zero4();
                if (MOM) acc2[ti] = zero4();
            }
            const bf16_t* Qh = Q + hf * NKH * BLK;
#pragma unroll
            for (int kk = 0; kk < NKH; ++kk) {
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(Qh + kk * BLK + ti * 512 + b_ap0);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(Qh + kk * BLK + ti * 512 + b_ap1);
                    asm volatile("" ::: "memory");   // no pairing across tiles (see below)
                    const bf16x8 bq = join(lo, hi);
                    mma(acc[ti], Sop[kk], bq);
                    if (MOM) mma(acc2[ti], Mop[kk], bq);
                }
            }
            if (HAS_P) {
                // half 0 takes key block 0 of every query tile, half 1 key block 1
                // (query tiles 2, 3 only); score fragments are read first
                const int pc = (NJB > 1 && hf) ? 32 : 0;
                bf16x8 pf[NTI];
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) pf[ti] = ld_accperm(&sP[0][(16 * ti + c16) * LP], pc, g);
                const bf16x8 vb = (NJB > 1 && hf) ? VB[NJB - 1] : VB[0];
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti)
                    if (hf == 0 || (NJB > 1 && ti >= 2)) mma(acc[ti], vb, pf[ti]);
            }
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                f32x4 o = acc[ti];
                if (MOM) o += sTab[2 * (CS + 1) + 16 * ti + c16] * acc2[ti];
                if (hf == 0) oacc[ti] = o;
                else sX[0][nt][ti][lane] = o;
            }
        }
        // (prev_* are read by write_out above, so they advance only here)
        prev_base = tbase;
        prev_n = n;
        prev_buf = cur;

        // ------------- state update (own d_k half)
        state_update(cur, n, VB, VS, VM);
        bool refresh = true;
        if (MODE == MODE_CC) {
            const int end = tbase + CS;
            refresh = (end % p.chunk == 0) || (end >= L);
        }
        if (refresh) refresh_ops();
        // unconditional: after the last chunk it stages the refetched last
        // chunk into the idle buffer (zero eta, never read).  A conditional
        // store leaves a path on which this register set's loads are never
        // waited for, and the compiler then drains every load in flight
        // before the next reuse of those registers (the score reads).
        store(c + 1, cur ^ 1, SSET, WQ{});
        if (PF == 1) load(c + 2, LSET, WQ{});
        __syncthreads();
    };
    // pairs of chunks with no branch inside the loop body; an odd last chunk after it
    if constexpr (!PIPE) {
        int c = c_begin;
        for (; c + 1 < c_end; c += 2) {
            iter(c, I0{}, I1{});
            iter(c + 1, I1{}, I0{});
        }
        if (c < c_end) iter(c, I0{}, I1{});
        if (hf == 0) combine();
        __syncthreads();
        write_out();
    } else {
        // One barrier per chunk.  The interval that ends with the barrier of
        // chunk c runs, in this order:
        //   half 0: adds half 1's partial of chunk c-2 to its own, into sO[c-2]
        //   all:    write chunk c-3's output tile from sO[c-3]
        //   all:    the intra term of chunk c-1 (scores sP[c-1], its V
        //           fragments kept in registers); half 1 parks its partial
        //           in sX[c-1], half 0 keeps its own
        //   all:    chunk c's readout with the state after chunk c-1, the
        //           state update, its scores into sP[c], and staging of c+1
        // (buffer index: chunk parity from c_begin).  Every tile is read in
        // the interval after the one that writes it and written again only
        // one interval later, so a double buffer of sP, sX and sO suffices.
        // The row scales of chunk c are read in chunk c's interval, since its
        // staging buffer is refilled in the next one.
        // readout partials by chunk parity (compile-time in the loop unrolled
        // by two): a chunk's partial is started in its own interval, finished
        // in the next and, in half 0, summed two intervals later, before the
        // chunk two ahead restarts the same registers
        f32x4 accs[2][NTI];
        bf16x8 VB_p[NJB];     // its eta-scaled V fragments
        float os_p[NTI];      // its output row scales
        bf16x8 VS_p[1], VM_p[1];
        auto rel = [&](int cc) { return (cc - c_begin) & 1; };
        auto combine_p = [&](int cc, auto PAR) {
            constexpr int q = decltype(PAR)::value;
            const int xb = rel(cc);
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                const int i = 16 * ti + c16;
                const f32x4 o = accs[q][ti] + sX[xb][nt][ti][lane];
                const int ch = (2 * nt + (g >> 1)) ^ oswz<DVT>(i);
                st4(&sO[xb][i * DVT + 8 * ch + 4 * (g & 1)], o);
            }
        };
        auto write_out_p = [&](int cc) {
            const int ob = rel(cc), base = cc * CS, nn = min(CS, L - base);
            const int row = tid / (DVT / 8), ch = tid % (DVT / 8);
            if (tid < NVC && row < nn) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(&sO[ob][row * DVT + 8 * (ch ^ oswz<DVT>(row))]);
                bf16_t* Oc = Og + (int64_t)base * oL;
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(Oc + (__mul24(row, (int)oL) + 8 * ch)));
            }
        };
        auto intra_p = [&](int cc, auto PAR) {
            constexpr int q = decltype(PAR)::value;
            f32x4* acc_p = accs[q];
            const int xb = rel(cc);
            if (HAS_P) {
                // half 0 takes key block 0 of every query tile, half 1 key
                // block 1 (query tiles 2, 3 only)
                const int pc = (NJB > 1 && hf) ? 32 : 0;
                bf16x8 pf[NTI];
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) pf[ti] = ld_accperm(&sP[xb][(16 * ti + c16) * LP], pc, g);
                const bf16x8 vb = (NJB > 1 && hf) ? VB_p[NJB - 1] : VB_p[0];
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti)
                    if (hf == 0 || (NJB > 1 && ti >= 2)) mma(acc_p[ti], vb, pf[ti]);
            }
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) {
                if (OSC) acc_p[ti] *= os_p[ti];
                if (hf != 0) sX[xb][nt][ti][lane] = acc_p[ti];
            }
        };
        auto iter_p = [&](int c, auto LSET, auto SSET) {
            constexpr int q = decltype(LSET)::value;   // parity of c - c_begin
            using Q0 = std::integral_constant<int, q>;
            using Q1 = std::integral_constant<int, q ^ 1>;
            f32x4* acc_p = accs[q];
            const int cur = rel(c);
            const int tbase = c * CS;
            const int n = min(CS, L - tbase);
            if (hf == 0 && c - 2 >= c_begin) combine_p(c - 2, Q0{});
            // the output store goes before this interval's loads: the memory
            // counter retires in order, so a later wait on the store leaves
            // the loads in flight
            if (c - 3 >= c_begin) write_out_p(c - 3);
            if (c - 1 >= c_begin) intra_p(c - 1, Q1{});
            load(c + 2, LSET, WQ{});
            vfrags(cur, VB_p, VS_p, VM_p);
            // readout partial with the state after chunk c-1: O^T = S_h^T Q_h^T
#pragma unroll
            for (int ti = 0; ti < NTI; ++ti) acc_p[ti] = zero4();
            const bf16_t* Qh = sQ[cur] + hf * NKH * BLK;
#pragma unroll
            for (int kk = 0; kk < NKH; ++kk) {
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) {
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(Qh + kk * BLK + ti * 512 + b_ap0);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(Qh + kk * BLK + ti * 512 + b_ap1);
                    // keep each fragment's two reads apart from the next
                    // tile's: left alone, the compiler pairs the reads of
                    // neighbouring tiles (a constant 1 KB apart) into one
                    // instruction and then shuffles the halves back into
                    // operand order with 50 moves per two chunks
                    asm volatile("" ::: "memory");
                    mma(acc_p[ti], Sop[kk], join(lo, hi));
                }
            }
            if (OSC) {
#pragma unroll
                for (int ti = 0; ti < NTI; ++ti) os_p[ti] = sOS[cur][16 * ti + c16];
            }
            state_update(cur, n, VB_p, VS_p, VM_p);
            bool refresh = true;
            if (MODE == MODE_CC) {
                const int end = tbase + CS;
                refresh = (end % p.chunk == 0) || (end >= L);
            }
            if (refresh) refresh_ops();
            // the scores go last: the readout and the state update, which
            // the next interval waits on, start first
            scores(sQ[cur], sK[cur], sP[cur]);
            // unconditional, as in the two-barrier loop above
            store(c + 1, cur ^ 1, SSET, WQ{});
            __syncthreads();
        };
        int c = c_begin;
        for (; c + 1 < c_end; c += 2) {
            iter_p(c, I0{}, I1{});
            iter_p(c + 1, I1{}, I0{});
        }
        if (c < c_end) iter_p(c, I0{}, I1{});
        // drain: the last three chunks' remaining stages
        auto drain = [&](auto PAR) {   // parity of the last chunk
            using QL = decltype(PAR);
            using QP = std::integral_constant<int, QL::value ^ 1>;
            if (hf == 0 && c_end - 2 >= c_begin) combine_p(c_end - 2, QP{});
            if (c_end - 3 >= c_begin) write_out_p(c_end - 3);
            intra_p(c_end - 1, QL{});
            __syncthreads();
            if (hf == 0) combine_p(c_end - 1, QL{});
            if (c_end - 2 >= c_begin) write_out_p(c_end - 2);
            __syncthreads();
            write_out_p(c_end - 1);
        };
        if ((c_end - 1 - c_begin) & 1) drain(std::integral_constant<int, 1>{});
        else drain(std::integral_constant<int, 0>{});
    }

    if (segmented && seg != p.nseg - 1) return;   // final states come from the last segment
    const int col = n0 + 16 * nt + c16;
    if (p.S_final) {
        float* Sf = p.S_final + (int64_t)bh * p.dk * p.dv;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sf[(int64_t)(DKH * hf + 16 * t + 4 * g + r) * p.dv + col] = Sacc[t][r];
    }
    if (MOM && p.M_final) {
        float* Mf = p.M_final + (int64_t)bh * p.dk * p.dv;
#pragma unroll
        for (int t = 0; t < NTH; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Mf[(int64_t)(DKH * hf + 16 * t + 4 * g + r) * p.dv + col] = Macc[t][r];
    }
}

bool tcb_supported(int dtype, int dk, int dv) {
    return dtype == 1 && (dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
}

namespace {

// Launch plan: tile form, and how many segments each (head, dv tile) is cut
// into.  The grid should cover the chip (256 CUs; the 32 x 32 form runs two
// workgroups per CU); a segment costs one extra pass over its K and V, so
// segments are only used when the (head, dv tile) grid is short of that and
// each segment keeps at least 1024 tokens.
struct TcbPlan {
    int cs, dvt, n_vt, nseg, seg_tiles;
};
constexpr int kCUs = 256;
constexpr int kMinSegTokens = 1024;
// polls of a look-back wait before it gives up (each poll sleeps ~0.1 us):
// far beyond any real wait, which is bounded by one segment's first pass
constexpr int kDefaultPolls = 1 << 22;

TcbPlan tcb_plan(int B, int H, int L, int dv, int mode, int chunk) {
    TcbPlan pl{};
    // chunk-causal needs the tile to divide the semantic chunk; 64 x 64 tiles
    // whenever they fit (measured faster than 32 x 32 with two workgroups
    // per CU: the 32-token tile doubles the per-chunk synchronisation)
    const bool cc32 = (mode == MODE_CC) && (chunk % 64 != 0);
    pl.cs = pl.dvt = (dv % 64 != 0 || cc32) ? 32 : 64;
    pl.n_vt = dv / pl.dvt;
    const int ntiles = (L + pl.cs - 1) / pl.cs;
    const int64_t nbv = (int64_t)B * H * pl.n_vt;
    const int slots = kCUs * (pl.cs == 32 ? 2 : 1);
    pl.nseg = 1;
    pl.seg_tiles = ntiles;
    if (nbv < slots) {
        // segment length: a whole number of tiles (and of chunks when the
        // chunk is part of the semantics)
        int unit = 1;
        if (mode == MODE_CC) unit = chunk / pl.cs;
        const int min_tiles = ((kMinSegTokens / pl.cs + unit - 1) / unit) * unit;
        const int want = (int)((slots + nbv - 1) / nbv);
        int seg_tiles = (ntiles + want - 1) / want;
        seg_tiles = ((seg_tiles + unit - 1) / unit) * unit;
        if (seg_tiles < min_tiles) seg_tiles = min_tiles;
        const int nseg = (ntiles + seg_tiles - 1) / seg_tiles;
        if (nseg > 1) {
            pl.nseg = nseg;
            pl.seg_tiles = seg_tiles;
        }
    }
    return pl;
}

// floats per workgroup state block (S, and m with momentum)
int64_t lb_block(int dk, int dvt, int mode) { return (int64_t)dk * dvt * (mode == MODE_MOM ? 2 : 1); }

// flags (one per workgroup), a spare word, the error word and 8 ticket counters
constexpr int kLbWords = 10;
size_t lb_flag_bytes(int64_t nwg) { return (size_t)(((nwg + kLbWords) * 4 + 255) / 256 * 256); }

__global__ void lb_clear_kernel(int* flags, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) flags[i] = 0;
}

}  // namespace

int64_t tcb_error_word(int B, int H, int L, int dv, int mode, int chunk) {
    const TcbPlan pl = tcb_plan(B, H, L, dv, mode, chunk);
    if (pl.nseg <= 1) return -1;
    return (int64_t)B * H * pl.n_vt * pl.nseg + 1;
}

size_t tcb_workspace(int B, int H, int L, int dk, int dv, int mode, int chunk) {
    const TcbPlan pl = tcb_plan(B, H, L, dv, mode, chunk);
    if (pl.nseg <= 1) return 0;
    const int64_t nwg = (int64_t)B * H * pl.n_vt * pl.nseg;
    return lb_flag_bytes(nwg) + (size_t)nwg * 2 * lb_block(dk, pl.dvt, mode) * sizeof(float);
}

hipError_t launch_tcb_fwd(const TcParams& pin, int mode, hipStream_t s) {
    TcParams p = pin;
    const TcbPlan pl = tcb_plan(p.B, p.H, p.L, p.dv, mode, p.chunk);
    p.n_vt = pl.n_vt;
    p.nseg = pl.nseg;
    p.seg_tiles = pl.seg_tiles;
    p.xcd_map = ((p.B * p.H) % 8 == 0) ? 1 : 0;
    const int64_t nwg = (int64_t)p.B * p.H * pl.n_vt * pl.nseg;
    if (pl.nseg > 1) {
        if (!p.workspace) return hipErrorInvalidValue;
        p.lb_flags = reinterpret_cast<int*>(p.workspace);
        p.lb_data = reinterpret_cast<float*>(reinterpret_cast<char*>(p.workspace) + lb_flag_bytes(nwg));
        p.lb_stride = lb_block(p.dk, pl.dvt, mode);
        p.lb_error = p.lb_flags + nwg + 1;
        if (p.lb_max_polls == 0) p.lb_max_polls = kDefaultPolls;
        else if (p.lb_max_polls < 0) p.lb_max_polls = 0;
        // flags, the ticket counters and the error word start at zero (a
        // fill kernel, not a memset node, so the call stays valid inside a
        // captured graph)
        const int nflags = (int)nwg + kLbWords;
        hipLaunchKernelGGL(lb_clear_kernel, dim3((nflags + 255) / 256), dim3(256), 0, s, p.lb_flags, nflags);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)nwg), block(pl.dvt / 16 * 128);
    // row scales come only with the token-causal forms (the backward's passes)
    if (mode == MODE_CC && p.use_oscale) return hipErrorInvalidValue;
#define TTT_L(DK_, M_, CS_, DVT_, OS_) \
    hipLaunchKernelGGL((tcb_fwd_kernel<DK_, M_, CS_, DVT_, OS_>), grid, block, 0, s, p)
#define TTT_O(DK_, M_, CS_, DVT_)                  \
    if (p.use_oscale) TTT_L(DK_, M_, CS_, DVT_, true); \
    else TTT_L(DK_, M_, CS_, DVT_, false)
#define TTT_M(CS_, DVT_)                                               \
    if (pl.cs == CS_ && pl.dvt == DVT_) {                               \
        if (p.dk == 128) {                                              \
            if (mode == MODE_TC) { TTT_O(128, MODE_TC, CS_, DVT_); }     \
            else if (mode == MODE_MOM) { TTT_O(128, MODE_MOM, CS_, DVT_); } \
            else TTT_L(128, MODE_CC, CS_, DVT_, false);                 \
        } else {                                                        \
            if (mode == MODE_TC) { TTT_O(64, MODE_TC, CS_, DVT_); }      \
            else if (mode == MODE_MOM) { TTT_O(64, MODE_MOM, CS_, DVT_); } \
            else TTT_L(64, MODE_CC, CS_, DVT_, false);                  \
        }                                                               \
        return hipGetLastError();                                       \
    }
    TTT_M(64, 64)
    TTT_M(32, 32)
#undef TTT_M
#undef TTT_O
#undef TTT_L
    return hipErrorInvalidValue;
}

}  // namespace ttt
