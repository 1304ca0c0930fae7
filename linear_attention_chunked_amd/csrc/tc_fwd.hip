// tc_fwd.hip -- chunked fast-weight forward for small heads (dk, dv <= 128).
//
// One workgroup owns one (batch, head, dv-tile) and walks the sequence chunk
// tile by chunk tile; the fp32 state tile stays in VGPRs (MFMA accumulators)
// for the whole sequence, so HBM sees every input byte once and every output
// byte once.  Wave w of the workgroup owns state columns [16w, 16w+16) of the
// tile and the matching output columns.
//
// Per chunk tile of CS tokens (c = chunk index, i, j = token in the tile):
//   stage     Q_c, K_c row-major and K_c^T, V~_c^T = (diag(eta) V_c)^T in LDS
//             (register prefetch of tile c+1 overlaps tile c's math)
//   intra     P^T = K_c Q_c^T, causal mask j <= i (momentum: x w_{i-j}),
//             lower-triangular tiles only, to LDS                (token-causal)
//   readout   O_c^T = S^T Q_c^T (+ a_i m^T Q_c^T) + V~_c^T P^T, S^T straight
//             from the accumulators (bf16 copy), stored once
//   update    S += K_c^T V~_c   (momentum: S += alpha m + K_c^T diag(w) V~_c,
//             m = gamma m + K_c^T diag(beta^.) V~_c)
//
// Sources ([P1] "KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다",
// aitrends.kr/articles/4698; [P2] "In-Place 테스트 시점 학습",
// aitrends.kr/articles/40879):
//   state update S += eta k^T v and the readout o = q S    [P1] paragraphs on
//       the state-matrix update and the one-step output identity
//   per-token eta folded into the values                  [P1] paragraph on
//       per-token learning rates being absorbable into V
//   momentum as a weighted linear attention               [P1] momentum paragraph
//   associative chunk combination                         [P1] weight-norm paragraph
//   chunk-causal readout o_t = q_t S_{i-1}                [P2] chunk-wise update
//
// Momentum algebra (derived from m_t = beta m_{t-1} + g_t, S_t = S_{t-1} + m_t):
// for local token i of a chunk that starts with (S, m),
//   S_i = S + a_i m + sum_{j<=i} w_{i-j} g_j,  a_i = beta(1-beta^{i+1})/(1-beta),
//   w_n = (1-beta^{n+1})/(1-beta);  a chunk of n tokens moves
//   S -> S + a_{n-1} m + sum_j w_{n-1-j} g_j,  m -> beta^n m + sum_j beta^{n-1-j} g_j.
#include "common.h"
#include "internal.h"

namespace ttt {

// One staging unit = 4 consecutive tokens x 8 consecutive features.
template <typename T> struct Seg;          // 8 elements of one row
template <> struct Seg<bf16_t> { u32x4 w; };
template <> struct Seg<float> { u32x4 w0, w1; };

TTT_DEV void seg_load(Seg<bf16_t>& s, const bf16_t* p) { s.w = *reinterpret_cast<const u32x4*>(p); }
TTT_DEV void seg_load(Seg<float>& s, const float* p) {
    s.w0 = reinterpret_cast<const u32x4*>(p)[0];
    s.w1 = reinterpret_cast<const u32x4*>(p)[1];
}
TTT_DEV void seg_zero(Seg<bf16_t>& s) { s.w = u32x4{0, 0, 0, 0}; }
TTT_DEV void seg_zero(Seg<float>& s) { s.w0 = s.w1 = u32x4{0, 0, 0, 0}; }
TTT_DEV void seg_store(bf16_t* p, const Seg<bf16_t>& s) { *reinterpret_cast<u32x4*>(p) = s.w; }
TTT_DEV void seg_store(float* p, const Seg<float>& s) {
    reinterpret_cast<u32x4*>(p)[0] = s.w0;
    reinterpret_cast<u32x4*>(p)[1] = s.w1;
}
TTT_DEV float seg_elem(const Seg<bf16_t>& s, int e) {
    return bf2f((uint16_t)(s.w[e >> 1] >> (16 * (e & 1))));
}
TTT_DEV float seg_elem(const Seg<float>& s, int e) {
    return __uint_as_float(e < 4 ? s.w0[e] : s.w1[e - 4]);
}
// 4 values (tokens t0..t0+3 of one feature) -> 4 consecutive LDS elements
TTT_DEV void st_col4(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack2bf(a, b), pack2bf(c, d)};
}
TTT_DEV void st_col4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// S^T operand fragments from the fp32 accumulators (accperm assignment)
TTT_DEV void pack_state(f32x4* op, const f32x4* acc, int nkb) {
    for (int kb = 0; kb < nkb; ++kb) op[kb] = acc[kb];
}
TTT_DEV void pack_state(bf16x8* op, const f32x4* acc, int nkb) {
    for (int kb = 0; kb < nkb; ++kb) op[kb] = acc_to_frag_bf16(acc[2 * kb], acc[2 * kb + 1]);
}

template <typename T, int DK, int DVT, int CS, int MODE>
__global__ __launch_bounds__(DVT / 16 * 64) void tc_fwd_kernel(TcParams p) {
    constexpr int NW = DVT / 16;               // waves; wave w owns 16 state columns
    constexpr int NT = NW * 64;
    constexpr int KB = Tr<T>::KB;
    constexpr int PR = 16 / sizeof(T);          // LDS row padding (16 bytes)
    constexpr int LDQ = DK + PR;                // sQ / sK row stride
    constexpr int LDT = CS + PR;                // sKT / sVT / sP row stride
    constexpr bool MOM = (MODE == MODE_MOM);
    constexpr bool HAS_P = (MODE != MODE_CC);
    constexpr int NV = MOM ? 3 : 1;             // scaled copies of V~^T
    constexpr int NTD = DK / 16;                // accumulator tiles along dk
    constexpr int NKB = DK / KB;                // operand K-blocks along dk
    constexpr int NTI = CS / 16;                // 16-token tiles per chunk tile
    constexpr int NUQ = (CS / 4) * (DK / 8);    // staging units of Q and K
    constexpr int NUV = (CS / 4) * (DVT / 8);   // staging units of V
    constexpr int UQ = (NUQ + NT - 1) / NT;
    constexpr int UV = (NUV + NT - 1) / NT;
    using frag = typename Tr<T>::frag;

    __shared__ __attribute__((aligned(16))) T sQ[CS * LDQ];
    __shared__ __attribute__((aligned(16))) T sK[HAS_P ? CS * LDQ : 8];
    __shared__ __attribute__((aligned(16))) T sKT[DK * LDT];
    __shared__ __attribute__((aligned(16))) T sVT[NV * DVT * LDT];
    __shared__ __attribute__((aligned(16))) T sP[HAS_P ? CS * LDT : 8];
    __shared__ float sTab[3 * (CS + 1)];        // w_p | beta^p | a_p

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;

    // ---- workgroup -> (b, h, dv tile); dv tiles of one head share an XCD
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
    const T* Qg = reinterpret_cast<const T*>(p.q) + b * p.qs[0] + h * p.qs[1];
    const T* Kg = reinterpret_cast<const T*>(p.k) + b * p.ks[0] + h * p.ks[1];
    const T* Vg = reinterpret_cast<const T*>(p.v) + b * p.vs[0] + h * p.vs[1] + n0;
    T* Og = reinterpret_cast<T*>(p.out) + b * p.os[0] + h * p.os[1] + n0;
    const float* Eg = p.eta ? p.eta + b * p.es[0] + h * p.es[1] : nullptr;
    const int64_t qL = p.qs[2], kL = p.ks[2], vL = p.vs[2], oL = p.os[2];
    const int64_t eL = p.es[2];

    // ---- momentum tables (computed in fp64, stored fp32)
    if (MOM) {
        for (int pp = tid; pp <= CS; pp += NT) {
            const double be = (double)p.beta;
            double bp = 1.0;
            for (int x = 0; x < pp; ++x) bp *= be;            // beta^pp
            const double bp1 = bp * be;                       // beta^(pp+1)
            sTab[pp] = (float)((1.0 - bp1) / (1.0 - be));     // w_pp
            sTab[(CS + 1) + pp] = (float)bp;                  // beta^pp
            sTab[2 * (CS + 1) + pp] = (float)(be * (1.0 - bp1) / (1.0 - be));  // a_pp
        }
    }
    // the strictly-upper tiles of P^T are never written: zero them once
    if (HAS_P) {
        for (int x = tid; x < CS * LDT; x += NT) sP[x] = (T)0.f;
    }

    // ---- state accumulators: S[16t + 4g + r][16*wave + c16]
    f32x4 Sacc[NTD];
    f32x4 Macc[MOM ? NTD : 1];
    {
        const float* S0 = p.S0 ? p.S0 + b * p.s0s[0] + h * p.s0s[1] : nullptr;
        const float* M0 = (MOM && p.M0) ? p.M0 + b * p.m0s[0] + h * p.m0s[1] : nullptr;
        const int col = n0 + 16 * wave + c16;
        for (int t = 0; t < NTD; ++t) {
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * g + r;
                const int64_t e = p.s0_trans ? (int64_t)col * p.dk + row : (int64_t)row * p.dv + col;
                Sacc[t][r] = S0 ? S0[e] : 0.f;
                if (MOM) Macc[t][r] = M0 ? M0[e] : 0.f;
            }
        }
    }
    frag Sop[NKB];
    frag Mop[MOM ? NKB : 1];
    pack_state(Sop, Sacc, NKB);
    if (MOM) pack_state(Mop, Macc, NKB);

    // ---- staging registers (tile prefetch)
    Seg<T> qreg[UQ][4], kreg[UQ][4], vreg[UV][4];
    float ereg[UV][4];

    auto load_tile = [&](int c) {
        const int t0 = c * CS;
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT;
            if (u < NUQ) {
                const int tb = u / (DK / 8), db = u % (DK / 8);
                for (int r = 0; r < 4; ++r) {
                    const int t = t0 + 4 * tb + r;
                    if (t < L) {
                        seg_load(qreg[x][r], Qg + t * qL + 8 * db);
                        seg_load(kreg[x][r], Kg + t * kL + 8 * db);
                    } else {
                        seg_zero(qreg[x][r]);
                        seg_zero(kreg[x][r]);
                    }
                }
            }
        }
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT;
            if (u < NUV) {
                const int tb = u / (DVT / 8), db = u % (DVT / 8);
                for (int r = 0; r < 4; ++r) {
                    const int t = t0 + 4 * tb + r;
                    if (t < L) {
                        seg_load(vreg[x][r], Vg + t * vL + 8 * db);
                        ereg[x][r] = Eg ? Eg[t * eL] : p.eta_scalar;
                    } else {
                        seg_zero(vreg[x][r]);
                        ereg[x][r] = 0.f;
                    }
                }
            }
        }
    };

    auto store_tile = [&](int c) {
        const int n = min(CS, L - c * CS);  // valid tokens in this tile
        for (int x = 0; x < UQ; ++x) {
            const int u = tid + x * NT;
            if (u < NUQ) {
                const int tb = u / (DK / 8), db = u % (DK / 8);
                for (int r = 0; r < 4; ++r) {
                    seg_store(&sQ[(4 * tb + r) * LDQ + 8 * db], qreg[x][r]);
                    if (HAS_P) seg_store(&sK[(4 * tb + r) * LDQ + 8 * db], kreg[x][r]);
                }
                for (int e = 0; e < 8; ++e) {
                    st_col4(&sKT[(8 * db + e) * LDT + 4 * tb], seg_elem(kreg[x][0], e),
                            seg_elem(kreg[x][1], e), seg_elem(kreg[x][2], e), seg_elem(kreg[x][3], e));
                }
            }
        }
        for (int x = 0; x < UV; ++x) {
            const int u = tid + x * NT;
            if (u < NUV) {
                const int tb = u / (DVT / 8), db = u % (DVT / 8);
                float s[NV][4];
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * tb + r;
                    s[0][r] = ereg[x][r];
                    if (MOM) {
                        const int pw = n - 1 - j;   // exponent within this tile
                        s[1][r] = (pw >= 0) ? ereg[x][r] * sTab[pw] : 0.f;
                        s[2][r] = (pw >= 0) ? ereg[x][r] * sTab[(CS + 1) + pw] : 0.f;
                    }
                }
                for (int vv = 0; vv < NV; ++vv) {
                    for (int e = 0; e < 8; ++e) {
                        st_col4(&sVT[(vv * DVT + 8 * db + e) * LDT + 4 * tb],
                                s[vv][0] * seg_elem(vreg[x][0], e), s[vv][1] * seg_elem(vreg[x][1], e),
                                s[vv][2] * seg_elem(vreg[x][2], e), s[vv][3] * seg_elem(vreg[x][3], e));
                    }
                }
            }
        }
    };

    const int ntiles = (L + CS - 1) / CS;
    load_tile(0);
    __syncthreads();
    store_tile(0);
    __syncthreads();

    for (int c = 0; c < ntiles; ++c) {
        const int tbase = c * CS;
        const int n = min(CS, L - tbase);
        if (c + 1 < ntiles) load_tile(c + 1);

        // ---------------- intra-chunk scores P^T = K Q^T (lower-triangular tiles)
        if (HAS_P) {
            int idx = 0;
            for (int ti = 0; ti < NTI; ++ti) {
                for (int tj = 0; tj <= ti; ++tj, ++idx) {
                    if (idx % NW != wave) continue;
                    f32x4 acc = zero4();
                    const T* arow = &sK[(16 * tj + c16) * LDQ];
                    const T* brow = &sQ[(16 * ti + c16) * LDQ];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
                        mma(acc, ld_contig<T>(arow, kb * KB, g), ld_contig<T>(brow, kb * KB, g));
                    const int i = 16 * ti + c16;
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tj + 4 * g + r;
                        float val = (j <= i) ? acc[r] : 0.f;
                        if (MOM && j <= i) val *= sTab[i - j];
                        acc[r] = val;
                    }
                    st4(&sP[i * LDT + 16 * tj + 4 * g], acc);
                }
            }
            __syncthreads();
        }

        // ---------------- readout O^T = S^T Q^T (+ a_i m^T Q^T) + V~^T P^T
        {
            const T* vrow = &sVT[(16 * wave + c16) * LDT];
            for (int ti = 0; ti < NTI; ++ti) {
                f32x4 acc = zero4();
                f32x4 acc2 = zero4();
                const T* qrow = &sQ[(16 * ti + c16) * LDQ];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const frag bq = ld_accperm(qrow, kb * KB, g);
                    mma(acc, Sop[kb], bq);
                    if (MOM) mma(acc2, Mop[kb], bq);
                }
                if (HAS_P) {
                    const T* prow = &sP[(16 * ti + c16) * LDT];
                    const int njb = (16 * (ti + 1) + KB - 1) / KB;
                    for (int jb = 0; jb < njb; ++jb)
                        mma(acc, ld_contig<T>(vrow, jb * KB, g), ld_contig<T>(prow, jb * KB, g));
                }
                const int i = 16 * ti + c16;
                if (MOM) {
                    const float a = sTab[2 * (CS + 1) + i];
                    for (int r = 0; r < 4; ++r) acc[r] += a * acc2[r];
                }
                if (i < n) {
                    if (p.use_oscale)
                        acc *= p.oscale ? p.oscale[b * p.ocs[0] + h * p.ocs[1] + (int64_t)(tbase + i) * p.ocs[2]]
                                        : p.oscale_scalar;
                    st4(&Og[(int64_t)(tbase + i) * oL + 16 * wave + 4 * g], acc);
                }
            }
        }

        // ---------------- state update S += K^T V~ (momentum: affine pair)
        {
            if (MOM) {
                const float alpha = sTab[2 * (CS + 1) + (n - 1)];
                const float gamma = sTab[(CS + 1) + n];
                for (int t = 0; t < NTD; ++t) {
                    for (int r = 0; r < 4; ++r) {
                        Sacc[t][r] += alpha * Macc[t][r];
                        Macc[t][r] *= gamma;
                    }
                }
            }
            const T* vS = &sVT[((MOM ? 1 : 0) * DVT + 16 * wave + c16) * LDT];
            const T* vM = &sVT[(2 * DVT + 16 * wave + c16) * LDT];
#pragma unroll
            for (int jb = 0; jb < CS / KB; ++jb) {
                const frag bS = ld_contig<T>(vS, jb * KB, g);
                frag bM;
                if (MOM) bM = ld_contig<T>(vM, jb * KB, g);
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const frag a = ld_contig<T>(&sKT[(16 * t + c16) * LDT], jb * KB, g);
                    mma(Sacc[t], a, bS);
                    if (MOM) mma(Macc[t], a, bM);
                }
            }
            bool refresh = true;
            if (MODE == MODE_CC) {
                const int end = tbase + CS;
                refresh = (end % p.chunk == 0) || (end >= L);
            }
            if (refresh) {
                pack_state(Sop, Sacc, NKB);
                if (MOM) pack_state(Mop, Macc, NKB);
            }
        }
        __syncthreads();
        if (c + 1 < ntiles) {
            store_tile(c + 1);
            __syncthreads();
        }
    }

    // ---- final state
    const int col = n0 + 16 * wave + c16;
    if (p.S_final) {
        float* Sf = p.S_final + (int64_t)bh * p.dk * p.dv;
        for (int t = 0; t < NTD; ++t)
            for (int r = 0; r < 4; ++r) Sf[(int64_t)(16 * t + 4 * g + r) * p.dv + col] = Sacc[t][r];
    }
    if (MOM && p.M_final) {
        float* Mf = p.M_final + (int64_t)bh * p.dk * p.dv;
        for (int t = 0; t < NTD; ++t)
            for (int r = 0; r < 4; ++r) Mf[(int64_t)(16 * t + 4 * g + r) * p.dv + col] = Macc[t][r];
    }
}

// ------------------------------------------------------------------ dispatch
template <typename T, int DK, int DVT, int CS, int MODE>
static hipError_t launch_one(const TcParams& p, hipStream_t s) {
    const int grid = p.B * p.H * p.n_vt;
    hipLaunchKernelGGL((tc_fwd_kernel<T, DK, DVT, CS, MODE>), dim3(grid), dim3(DVT / 16 * 64), 0, s, p);
    return hipGetLastError();
}

template <typename T, int CS, int MODE>
static hipError_t dispatch_dims(const TcParams& p, int dvt, hipStream_t s) {
#define TTT_CASE(DK_, DVT_) \
    if (p.dk == DK_ && dvt == DVT_) return launch_one<T, DK_, DVT_, CS, MODE>(p, s);
    TTT_CASE(32, 32) TTT_CASE(32, 64)
    TTT_CASE(64, 32) TTT_CASE(64, 64)
    TTT_CASE(128, 32) TTT_CASE(128, 64)
#undef TTT_CASE
    return hipErrorInvalidValue;
}

static int tile_chunk(int dtype) { return dtype == 1 ? 64 : 32; }

static int pick_dvt(int dv) { return dv >= 64 ? 64 : 32; }

bool tc_fwd_supported(int dtype, int mode, int dk, int dv, int chunk) {
    if (dtype != 0 && dtype != 1) return false;
    if (dk != 32 && dk != 64 && dk != 128) return false;
    if (dv != 32 && dv != 64 && dv != 128) return false;
    if (mode == MODE_CC && chunk % tile_chunk(dtype) != 0) return false;
    return true;
}

hipError_t launch_tc_fwd(const TcParams& pin, int dtype, int mode, hipStream_t s) {
    if (!tc_fwd_supported(dtype, mode, pin.dk, pin.dv, pin.chunk)) return hipErrorInvalidValue;
    if (tcb_supported(dtype, pin.dk, pin.dv)) return launch_tcb_fwd(pin, mode, s);
    TcParams p = pin;
    const int dvt = pick_dvt(p.dv);
    p.n_vt = p.dv / dvt;
    p.xcd_map = ((p.B * p.H) % 8 == 0) ? 1 : 0;
    if (dtype == 1) {
        if (mode == MODE_TC) return dispatch_dims<bf16_t, 64, MODE_TC>(p, dvt, s);
        if (mode == MODE_MOM) return dispatch_dims<bf16_t, 64, MODE_MOM>(p, dvt, s);
        return dispatch_dims<bf16_t, 64, MODE_CC>(p, dvt, s);
    }
    if (mode == MODE_TC) return dispatch_dims<float, 32, MODE_TC>(p, dvt, s);
    if (mode == MODE_MOM) return dispatch_dims<float, 32, MODE_MOM>(p, dvt, s);
    return dispatch_dims<float, 32, MODE_CC>(p, dvt, s);
}

}  // namespace ttt
