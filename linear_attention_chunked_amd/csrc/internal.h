// internal.h -- launcher interfaces between the C-ABI layer (api.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttt {

enum { MODE_TC = 0, MODE_MOM = 1, MODE_CC = 2 };

// Arguments of the small-head token-/chunk-causal kernel (dk, dv <= 128).
struct TcParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int64_t qs[3], ks[3], vs[3], os[3];
    const float* eta;
    int64_t es[3];
    float eta_scalar;
    float beta;
    const float* S0;
    int64_t s0s[2];
    const float* M0;
    int64_t m0s[2];
    float* S_final;
    float* M_final;
    int B, H, L, dk, dv, chunk;
    int n_vt;     // dv tiles per head
    int xcd_map;  // 1: keep the dv tiles (and segments) of one head on one XCD
    // sequence segmentation with decoupled look-back (bf16 kernel only):
    // nseg segments of seg_tiles chunk tiles per (head, dv tile); lb_flags
    // holds one flag per workgroup, a spare word, the error word and eight
    // ticket counters, lb_data two state blocks (aggregate, inclusive) of
    // lb_stride floats per workgroup
    int nseg, seg_tiles;
    int* lb_flags;
    float* lb_data;
    int64_t lb_stride;
    // a look-back wait gives up after lb_max_polls polls (0 on input: the
    // default bound; negative: give up at once) and then raises *lb_error
    int lb_max_polls;
    int* lb_error;
    void* workspace;
    // S0 (and M0) stored transposed: element (i, j) of a head's [dk, dv]
    // state at j * dk + i (the backward pass reads a state this way)
    int s0_trans;
    // output rows scaled by a per-token factor (use_oscale = 1): oscale
    // [B,H,L] with strides ocs, or oscale_scalar when oscale is NULL
    int use_oscale;
    const float* oscale;
    int64_t ocs[3];
    float oscale_scalar;
};

// dtype: 0 fp32, 1 bf16.  mode: MODE_*.  Returns hipSuccess or the launch error;
// hipErrorInvalidValue when no kernel is instantiated for the shape.
hipError_t launch_tc_fwd(const TcParams& p, int dtype, int mode, hipStream_t stream);
bool tc_fwd_supported(int dtype, int mode, int dk, int dv, int chunk);
// gfx950-tuned bf16 variant (dk in {64,128}, dv in {64,128}); chosen by launch_tc_fwd
bool tcb_supported(int dtype, int dk, int dv);
hipError_t launch_tcb_fwd(const TcParams& p, int mode, hipStream_t stream);
// workspace of the bf16 kernel (look-back flags and states when the sequence
// is segmented; 0 otherwise)
size_t tcb_workspace(int B, int H, int L, int dk, int dv, int mode, int chunk);
// index (in ints from the workspace start) of the look-back error word, or
// -1 when the call is not segmented
int64_t tcb_error_word(int B, int H, int L, int dv, int mode, int chunk);

// Allocation-free forward: the look-back scratch in a static device array of
// kNoAllocScratchBytes per GPU; noalloc_scratch gives its device address on
// the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// Chunk-causal forward for large fast weights (dk, dv multiples of 256, bf16):
// update walk with bf16 W snapshots in `workspace`, then a batched readout.
bool inplace_supported(int dtype, int dk, int dv, int chunk);
// row strides (elements) the In-Place kernels address with 32-bit lane offsets
bool inplace_strides_ok(int64_t q_row, int64_t k_row, int64_t v_row);
size_t inplace_workspace(int B, int H, int L, int dk, int dv, int chunk);
hipError_t launch_inplace(const TcParams& p, void* workspace, hipStream_t stream);

// Chunk-state scan: element-parallel walk over chunks.
hipError_t launch_state_scan(int B, int H, int L, int chunk, int dk, int dv,
                             const float* dS, const float* dM, float beta,
                             const float* S0, const float* M0,
                             float* S_excl, float* M_excl, float* S_final, float* M_final,
                             hipStream_t stream);

// Dual form (TTT-Linear mini-batch, MSE).
struct DualParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const float* W0;
    int64_t W0_stride;
    float* W_final;
    float eta;
    int B, H, L, d, dv, minibatch;
    // segmented form (set by launch_dual_fwd from the workspace): flags (one
    // per (b, h, segment), then a spare word, the error word and eight ticket
    // counters) and the per-segment maps; seg0_state: segment 0 runs only its
    // forward and hands on its end state in place of a map
    void* workspace;            // null: the sequential form
    size_t workspace_bytes;
    int* flags;
    float* maps;
    int nseg, seg_len, max_polls, seg0_state;
};
hipError_t launch_dual_fwd(const DualParams& p, int dtype, hipStream_t stream);
bool dual_supported(int dtype, int d, int dv, int minibatch);
// workspace bytes of the segmented form (0: the shape runs sequentially)
size_t dual_workspace(int dtype, int B, int H, int L, int d, int dv, int minibatch);
// int index of the look-back error word in the workspace, or -1 (sequential)
int64_t dual_error_word(int dtype, int B, int H, int L, int d, int dv, int minibatch);

// dL/dbeta of the token-causal momentum forward (contiguous tensors).
struct DbetaParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* eta;          // [B,H,L] or null (eta_scalar)
    float eta_scalar;
    const float* M0;           // [B,H,dk,dv] or null
    const float* dS_final;     // [B,H,dk,dv] or null
    const float* dM_final;     // [B,H,dk,dv] or null
    float* partial;            // [B*H][dv/16] workspace
    float* dbeta;              // [B,H]
    int B, H, L, dk, dv;
    // weight tables filled by launch_dbeta: beta^d, d beta^(d-1),
    // F(d) = sum_{e<=d} e beta^(e-1) (d <= 16), beta (1 + .. + beta^i) (i < 16)
    float bp[17], f1[17], F[17], bw[16];
    float lb[3][16];   // the last block's token weights (bp, f1, F at n - 1 - j)
};
bool dbeta_supported(int dtype, int dk, int dv);
size_t dbeta_workspace(int B, int H, int dv);
hipError_t launch_dbeta(DbetaParams p, int dtype, float beta, hipStream_t stream);

// Recurrent decode step (one token per (b, h), state in place).
struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const float* eta;
    float eta_scalar;
    float beta;
    float* S;
    float* M;
    int B, H, dk, dv;
};
hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream);

// Backward of the token-causal forward (with or without momentum), contiguous [B,H,L,d]
// tensors.  dk and dv (the gradient buffers) receive intermediate results
// before the final scaling, so they must not alias any input.
struct BwdParams {
    int B, H, L, dk_dim, dv_dim, dtype;
    const void* q;
    const void* k;
    const void* v;
    const float* eta;
    float eta_scalar;
    float beta;
    const float* S0;
    const float* M0;
    const void* dout;
    const float* dS_final;
    const float* dM_final;
    void* dq;
    void* dk;
    void* dv;
    float* deta;
    float* dS0;
    float* dM0;
    void* workspace;
};
// In-Place front end (bf16).  Projections: out[t][f] from weight rows A
// (K elements each; gated: A0 = Wgate, A1 = Wup, arows = 2 d_ff) and token
// rows B (row stride ldb); out row stride ldo.
struct FeGemmParams {
    const void* A0;
    const void* A1;
    const void* B;
    void* out;
    int arows, K, T;
    int64_t ldb, ldo;
};
struct FeConvParams {
    const void* X;      // [B, L, d] bf16
    const float* w;     // [K, d]
    void* Y;            // [B, L, d] bf16
    int B, L, d, K;
};
struct FeGramParams {
    const void* Z;      // [B, L, dz] bf16
    const void* V;      // [B, L, dv] bf16
    int B, L, chunk, dz, dv, ntiles;
    float eta, tau;
    float* partial;     // [B, chunks, pairs]
    float* eta_out;     // [B, L]
};
bool fe_gemm_supported(int K, int nfeat_rows);
hipError_t launch_fe_gemm(const FeGemmParams& p, bool gated, hipStream_t stream);
hipError_t launch_fe_conv(const FeConvParams& p, hipStream_t stream);
int fe_gram_pairs(int chunk);
hipError_t launch_fe_clip(const FeGramParams& p, hipStream_t stream);

bool bwd_supported(int dtype, int dk, int dv);
size_t bwd_workspace(int B, int H, int L, int dk, int dv, int dtype, bool momentum);
// side: a second stream of the caller for the dv/deta step beside the R pass
// (NULL or equal to `stream`: everything runs on `stream`)
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream, hipStream_t side);
bool decode_supported(int dtype, int dk, int dv);

// Large-chunk SwiGLU fast weight (bf16 activations, fp32 master weights).
// Per head: W1, W3 [m][dk] and W2 [dv][m] fp32, updated in place; the
// workspace holds bf16 copies of the weights and one chunk's activations.
struct SwParams {
    const void* q;      // [BH][L][dk] bf16
    const void* k;      // [BH][L][dk]
    const void* v;      // [BH][L][dv]
    const float* eta;   // [BH][L] or null (eta_scalar)
    float eta_scalar;
    float* W1;          // [BH][m][dk]
    float* W3;          // [BH][m][dk]
    float* W2;          // [BH][dv][m]
    void* out;          // [BH][L][dv] bf16
    void* workspace;
    int BH, L, dk, dv, m, chunk, loss;   // loss: 0 = -<f(k), v>, 1 = 1/2 ||f(k) - v||^2
};
bool swiglu_supported(int dk, int dv, int m, int chunk);
size_t swiglu_workspace(int BH, int dk, int dv, int m, int chunk);
hipError_t launch_swiglu(const SwParams& p, hipStream_t stream);

}  // namespace ttt
