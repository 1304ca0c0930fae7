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

bool dual_supported(int dtype, int d, int dv, int minibatch) {
    return (dtype == 0 || dtype == 1) && d == 64 && dv == 64 && minibatch >= 1;
}

hipError_t launch_dual_fwd(const DualParams& p, int dtype, hipStream_t s) {
    if (!dual_supported(dtype, p.d, p.dv, p.minibatch)) return hipErrorInvalidValue;
    const int grid = p.B * p.H;
    if (dtype == 1)
        hipLaunchKernelGGL((dual_fwd_kernel<bf16_t, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((dual_fwd_kernel<float, 64, 64>), dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ttt
