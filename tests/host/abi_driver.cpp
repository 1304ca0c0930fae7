// abi_driver.cpp -- the C-ABI's argument validation under AddressSanitizer
// and UndefinedBehaviorSanitizer (CPU only, test code).
//
// api.cpp is compiled for the host with the launchers and planners of the
// kernel translation units replaced by stubs below: the stubs launch nothing
// and answer the planning questions with simple fixed rules, so that every
// validation branch of api.cpp can be reached with fake device addresses.
// The driver calls every entry point with valid and invalid arguments,
// including extreme sizes and strides, and checks that each call returns a
// status of the enum (the sanitizers abort on any out-of-bounds access,
// signed overflow or other undefined behaviour on the way).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/ttt.h"
#include "../../linear_attention_chunked_amd/csrc/internal.h"

namespace ttt {
bool tc_fwd_supported(int, int, int dk, int dv, int chunk) {
    auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
    return ok(dk) && ok(dv) && chunk >= 1;
}
bool tcb_supported(int dtype, int dk, int dv) { return dtype == 1 && (dk == 64 || dk == 128) && dv >= 32 && dv <= 128; }
size_t tcb_workspace(int B, int H, int L, int, int, int, int) { return ((int64_t)B * H < 64 && L > 2048) ? 1 << 20 : 0; }
int64_t tcb_error_word(int B, int H, int L, int, int, int) { return ((int64_t)B * H < 64 && L > 2048) ? 5 : -1; }
hipError_t launch_tc_fwd(const TcParams&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_tcb_fwd(const TcParams&, int, hipStream_t) { return hipSuccess; }
bool inplace_supported(int dtype, int dk, int dv, int chunk) {
    return dtype == 1 && dk % 256 == 0 && dv % 256 == 0 && chunk % 256 == 0;
}
size_t inplace_workspace(int, int, int L, int dk, int dv, int chunk) {
    return (size_t)((L + chunk - 1) / chunk) * dk * dv * 2;
}
hipError_t launch_inplace(const TcParams&, void*, hipStream_t) { return hipSuccess; }
bool inplace_strides_ok(int64_t q, int64_t k, int64_t v) {
    const int64_t lim = (int64_t(1) << 31) / 512;
    return q < lim && k < lim && v < lim;
}
// a host stand-in for the device array: validation never dereferences it
hipError_t noalloc_scratch(void** ptr) {
    static char stand_in[16];
    *ptr = stand_in;
    return hipSuccess;
}
hipError_t launch_state_scan(int, int, int, int, int, int, const float*, const float*, float, const float*,
                             const float*, float*, float*, float*, float*, hipStream_t) {
    return hipSuccess;
}
hipError_t launch_dual_fwd(const DualParams&, int, hipStream_t) { return hipSuccess; }
bool dual_supported(int, int d, int dv, int mb) { return d == 64 && dv == 64 && mb >= 1; }
size_t dual_workspace(int dtype, int B, int H, int, int d, int dv, int mb) {
    return (dtype == 1 && d == 64 && dv == 64 && mb % 16 == 0 && B * H <= 128) ? 4096 : 0;
}
int64_t dual_error_word(int dtype, int B, int H, int L, int d, int dv, int mb) {
    return dual_workspace(dtype, B, H, L, d, dv, mb) ? 1 : -1;
}
hipError_t launch_decode(const DecodeParams&, int, hipStream_t) { return hipSuccess; }
bool decode_supported(int, int dk, int dv) { return dk >= 1 && dk <= 1024 && dv % 4 == 0; }
bool bwd_supported(int, int dk, int dv) { return tc_fwd_supported(0, 0, dk, dv, 64); }
size_t bwd_workspace(int B, int H, int, int dk, int dv, int, bool mom) { return mom ? (size_t)4 * B * H * dk * dv * 4 : 0; }
hipError_t launch_bwd(const BwdParams&, hipStream_t, hipStream_t) { return hipSuccess; }
bool dbeta_supported(int dtype, int dk, int dv) {
    return (dtype == 0 || dtype == 1) && (dk == 32 || dk == 64 || dk == 128) && dv % 16 == 0 && dv >= 16 &&
           dv <= 1024;
}
size_t dbeta_workspace(int B, int H, int dv) { return (size_t)B * H * (dv / 16) * 4 * 4; }
hipError_t launch_dbeta(DbetaParams, int, float, hipStream_t) { return hipSuccess; }
bool fe_gemm_supported(int K, int rows) { return K % 128 == 0 && rows % 128 == 0; }
hipError_t launch_fe_gemm(const FeGemmParams&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_fe_conv(const FeConvParams&, hipStream_t) { return hipSuccess; }
int fe_gram_pairs(int chunk) { return (chunk / 128) * (chunk / 128 + 1) / 2 + 1; }
hipError_t launch_fe_clip(const FeGramParams&, hipStream_t) { return hipSuccess; }
bool swiglu_supported(int dk, int dv, int m, int chunk) {
    return dk % 128 == 0 && dv % 128 == 0 && m % 128 == 0 && chunk % 128 == 0;
}
size_t swiglu_workspace(int BH, int dk, int dv, int m, int chunk) {
    return (size_t)BH * ((size_t)4 * m * dk + 2 * (size_t)dv * m + (size_t)chunk * (6 * m + dv)) * 2;
}
hipError_t launch_swiglu(const SwParams&, hipStream_t) { return hipSuccess; }
}  // namespace ttt

namespace {

int n_calls = 0, n_bad = 0;
void expect_status(ttt_status_t s, const char* what) {
    ++n_calls;
    if ((int)s < 0 || (int)s > TTT_ERR_TIMEOUT) {
        std::fprintf(stderr, "%s: status %d is not in the enum\n", what, (int)s);
        ++n_bad;
    }
}

char* fake(int64_t off) { return reinterpret_cast<char*>((uintptr_t)1 << 40) + off; }

ttt_fwd_args base_args(int B, int H, int L, int dk, int dv) {
    ttt_fwd_args a;
    std::memset(&a, 0, sizeof(a));
    a.B = B; a.H = H; a.L = L; a.dk = dk; a.dv = dv; a.chunk = 64; a.dtype = TTT_BF16;
    const int64_t nq = (int64_t)B * H * L * dk * 2, nv = (int64_t)B * H * L * dv * 2;
    a.q = fake(0); a.k = fake(nq + 4096); a.v = fake(2 * (nq + 4096)); a.out = fake(2 * (nq + 4096) + nv + 4096);
    const int64_t sq[3] = {(int64_t)H * L * dk, (int64_t)L * dk, dk}, sv[3] = {(int64_t)H * L * dv, (int64_t)L * dv, dv};
    for (int i = 0; i < 3; ++i) { a.q_stride[i] = a.k_stride[i] = sq[i]; a.v_stride[i] = a.out_stride[i] = sv[i]; }
    a.eta_scalar = 0.1f;
    return a;
}

}  // namespace

int main() {
    const int sizes[] = {INT_MIN, -1, 0, 1, 7, 64, 128, 256, 4096, INT_MAX};
    const int64_t strides[] = {INT64_MIN, -8, 0, 8, 64, (int64_t)1 << 22, (int64_t)1 << 23, (int64_t)1 << 40,
                               (int64_t)1 << 62, INT64_MAX};
    const float scalars[] = {-1.f, 0.f, 1e-30f, 0.5f, 0.9999f, 1.f, 2.f, __builtin_nanf(""), __builtin_inff()};
    size_t ws = 0;
    int32_t flag = 0;
    // forward: every size in every position, then strides and scalars
    for (int x : sizes)
        for (int pos = 0; pos < 6; ++pos) {
            ttt_fwd_args a = base_args(2, 2, 128, 64, 64);
            int* f[6] = {&a.B, &a.H, &a.L, &a.dk, &a.dv, &a.chunk};
            *f[pos] = x;
            expect_status(ttt_fwd_chunked(&a), "fwd size");
            expect_status(ttt_fwd_workspace_size(&a, &ws), "fwd ws size");
            expect_status(ttt_fwd_lookback_status(&a, &flag), "lookback size");
            a.mode = TTT_CHUNK_CAUSAL;
            expect_status(ttt_fwd_chunked(&a), "fwd size cc");
        }
    for (int64_t st : strides)
        for (int which = 0; which < 12; ++which) {
            ttt_fwd_args a = base_args(3, 3, 200, 64, 128);
            int64_t* f[12] = {&a.q_stride[0], &a.q_stride[1], &a.q_stride[2], &a.k_stride[0], &a.v_stride[1],
                              &a.out_stride[0], &a.out_stride[1], &a.out_stride[2], &a.eta_stride[0],
                              &a.eta_stride[2], &a.S0_stride[0], &a.M0_stride[1]};
            *f[which] = st;
            a.eta = reinterpret_cast<const float*>(fake(1LL << 36));
            a.S0 = reinterpret_cast<const float*>(fake(1LL << 37));
            a.M0 = reinterpret_cast<const float*>(fake(3LL << 36));
            a.S_final = reinterpret_cast<float*>(fake(1LL << 38));
            a.beta = 0.5f;
            expect_status(ttt_fwd_chunked(&a), "fwd stride");
        }
    for (float b : scalars) {
        ttt_fwd_args a = base_args(1, 1, 5000, 128, 128);
        a.beta = b;
        expect_status(ttt_fwd_chunked(&a), "fwd beta");
        expect_status(ttt_fwd_workspace_size(&a, &ws), "fwd ws beta");
        a.workspace = fake(1LL << 39);
        a.workspace_bytes = 1 << 20;
        a.lookback_polls = -1;
        expect_status(ttt_fwd_chunked(&a), "fwd beta ws");
    }
    {   // In-Place sizes: large, chunk multiple of 256
        ttt_fwd_args a = base_args(1, 1, 32768, 9728, 2560);
        a.mode = TTT_CHUNK_CAUSAL; a.chunk = 1024; a.k = a.q;
        expect_status(ttt_fwd_workspace_size(&a, &ws), "inplace ws");
        a.workspace = fake(1LL << 41);
        a.workspace_bytes = ws;
        expect_status(ttt_fwd_chunked(&a), "inplace");
    }
    expect_status(ttt_fwd_chunked(nullptr), "fwd null");
    expect_status(ttt_fwd_workspace_size(nullptr, &ws), "ws null");
    // scan, dual, decode, bwd, front end, SwiGLU: sizes and scalars
    for (int x : sizes)
        for (float b : scalars) {
            const float* F = reinterpret_cast<const float*>(fake(0));
            float* O = reinterpret_cast<float*>(fake(1LL << 38));
            expect_status(ttt_chunk_state_scan(x, 2, 300, 64, 8, 8, F, F, b, nullptr, nullptr, O, nullptr, nullptr,
                                               nullptr, nullptr, 0, nullptr), "scan");
            expect_status(ttt_chunk_state_scan(1, 1, x, x, 4, x, F, F, b, F, F, O, O, O, O, nullptr, 0, nullptr),
                          "scan 2");
            expect_status(ttt_dual_form_fwd(2, 2, x, 64, 64, x, TTT_BF16, fake(0), fake(1LL << 32), fake(2LL << 32),
                                            F + (3LL << 30), x, b, fake(4LL << 32), O, nullptr, 0, nullptr),
                          "dual");
            expect_status(ttt_decode_step(x, 2, 64, 64, TTT_BF16, fake(0), fake(1 << 20), fake(2 << 20), nullptr, b,
                                          b, O, O + (1 << 22), fake(6 << 20), nullptr), "decode");
            expect_status(ttt_bwd_workspace_size(2, 2, x, 64, 64, TTT_BF16, b, &ws), "bwd ws");
            expect_status(ttt_bwd_chunked(2, 2, x, 64, 64, TTT_BF16, fake(0), fake(1LL << 32), fake(2LL << 32),
                                          nullptr, b, b, nullptr, nullptr, fake(3LL << 32), nullptr, nullptr,
                                          fake(4LL << 32), fake(5LL << 32), fake(6LL << 32), nullptr, nullptr, nullptr,
                                          fake(7LL << 32), 1LL << 31, nullptr, nullptr), "bwd");
            expect_status(ttt_inplace_gated_input(x, 256, 512, fake(0), fake(1LL << 32), fake(2LL << 32),
                                                  fake(3LL << 32), nullptr), "gated");
            expect_status(ttt_inplace_lm_target_workspace_size(1, x, 256, &ws), "lm ws");
            expect_status(ttt_inplace_lm_target(1, x, 256, 4, fake(0), F + (1LL << 30), fake(2LL << 32),
                                                fake(3LL << 32), fake(4LL << 32), 1LL << 32, nullptr), "lm");
            expect_status(ttt_inplace_clip_eta_workspace_size(1, x, 1024, &ws), "clip ws");
            expect_status(ttt_inplace_clip_eta(1, x, 256, 256, 1024, fake(0), fake(1LL << 32), b, b, O,
                                               fake(3LL << 32), 1LL << 30, nullptr), "clip");
            expect_status(ttt_swiglu_workspace_size(1, 2, x, 128, 128, 256, 256, &ws), "swiglu ws");
            expect_status(ttt_swiglu_fwd_chunked(1, 2, 300, 128, 128, 256, x, 0, fake(0), fake(1LL << 32),
                                                 fake(2LL << 32), nullptr, b, O, O + (1LL << 30), O + (2LL << 30),
                                                 fake(6LL << 32), fake(7LL << 32), 1LL << 33, nullptr), "swiglu");
        }
    for (int s = -1; s <= TTT_ERR_TIMEOUT + 1; ++s)
        if (!ttt_status_string((ttt_status_t)s)) ++n_bad;
    std::printf("abi validation driver: %d calls, %d bad statuses, args size %zu\n", n_calls, n_bad,
                ttt_fwd_args_size());
    return n_bad ? 1 : 0;
}
