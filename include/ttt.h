/*
 * ttt.h -- C ABI of the MI355X (gfx950) chunked TTT fast-weight forward.
 *
 * The library computes the forward pass of a test-time-training fast-weight
 * layer read as linear attention.  Per (batch b, head h) a state S (dk x dv,
 * fp32) takes one gradient step per token or per chunk; outputs read the
 * state.  Three entry points:
 *
 *   ttt_fwd_chunked       token-causal (optionally with momentum) and
 *                         chunk-causal (In-Place TTT) forward
 *   ttt_chunk_state_scan  the associative scan over per-chunk state deltas
 *   ttt_dual_form_fwd     the non-associative TTT-Linear mini-batch update
 *                         (MSE reconstruction loss), dual form
 *   ttt_decode_step       one recurrent token per sequence (inference):
 *                         state update and readout with the state in HBM
 *   ttt_bwd_chunked       backward pass of the token-causal forward
 *   ttt_bwd_dbeta         gradient of the momentum coefficient
 *   ttt_inplace_*         In-Place TTT front end: gated input Z, LM-aligned
 *                         target V-hat, clipped per-token rates
 *
 * Sources (cited by page title and paragraph or section):
 *  [P1] "KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다"
 *       (aitrends.kr/articles/4698)
 *  [P2] "In-Place 테스트 시점 학습: LLM을 위한 원활한 동적 적응 프레임워크"
 *       (aitrends.kr/articles/40879)
 *  [P4] "RNN의 기억을 작은 모델로 바꾼다면: Test-Time Training 읽기" (ariser.io)
 *  [P5] "LaCT (Large Chunk Test-Time Training)" (aisparkup.com/wiki/lact)
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers (hipMalloc'd or equivalent) owned by the
 *    caller; the library never allocates, frees or keeps a pointer after the
 *    call returns.  Scratch memory comes in through `workspace`.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL =
 *    the default stream).  Argument validation is synchronous and happens
 *    before any launch: on any error nothing has been enqueued.
 *  - Row vectors: q_t, k_t in R^dk, v_t, o_t in R^dv; S in R^{dk x dv}, stored
 *    row-major (dv contiguous).  Activations are [B,H,L,d] tensors addressed
 *    through element strides for the B, H and L dimensions; the last
 *    dimension must be contiguous.
 *  - Base pointers must be 16-byte aligned; the L strides of q, k, v and out
 *    must be multiples of 8 elements (16 bytes of bf16) and below 2^23
 *    elements (eta's L stride too); S0/M0/W0/S_final
 *    etc. are contiguous [dk, dv] fp32 blocks per (b, h).
 *  - Size limits (TTT_ERR_SHAPE beyond them): sequence lengths, chunks,
 *    mini-batches and token counts up to 2^30; up to 2^24 sequences
 *    (B * H); head and feature sizes up to 2^16; no tensor spanning more
 *    than 2^48 bytes through its strides.
 *  - Written buffers (outputs, final states, the workspace) must not overlap
 *    any input, each other, or themselves (an output's strides must give
 *    every (b, h, t) its own row); TTT_ERR_ALIAS otherwise.  Inputs may
 *    overlap each other (q and k may be the same tensor; a state may be
 *    broadcast with stride 0).  In-place use is supported only where an
 *    entry point says so (ttt_decode_step's S and M).
 *  - Errors never abort and never throw across the ABI; launch failures are
 *    reported as TTT_ERR_HIP.  Calls on different streams with different
 *    workspaces may run concurrently; the library creates no streams of its
 *    own and holds no global or static state, except the scratch array of
 *    ttt_fwd_chunked_noalloc and its device address per GPU.
 */
#ifndef TTT_MI355X_H
#define TTT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TTT_OK = 0,
    TTT_ERR_NULL = 1,        /* a required pointer is NULL                       */
    TTT_ERR_SHAPE = 2,       /* a size or stride is out of range / inconsistent  */
    TTT_ERR_DTYPE = 3,       /* unknown dtype value                              */
    TTT_ERR_ALIGN = 4,       /* pointer or stride misaligned                     */
    TTT_ERR_UNSUPPORTED = 5, /* valid arguments the library has no kernel for    */
    TTT_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
    TTT_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed       */
    TTT_ERR_ALIAS = 8,       /* a written buffer overlaps an input or another    */
    TTT_ERR_VALUE = 9,       /* a scalar is out of range (beta not in [0,1), ...) */
    TTT_ERR_TIMEOUT = 10     /* a look-back wait gave up: results are invalid    */
} ttt_status_t;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype_t;

typedef enum {
    /* o_t reads the state after token t's own update: S_t = S_{t-1} + m_t,
     * m_t = beta m_{t-1} + eta_t k_t^T v_t, o_t = q_t S_t.  The chunk length
     * is only a tiling choice here: results do not depend on it. */
    TTT_TOKEN_CAUSAL = 0,
    /* In-Place TTT ([P2], paragraphs on the chunk-wise Wdown update and on
     * the associative scan): token t of chunk i reads the state left by the
     * previous chunks, o_t = q_t S_{i-1}, then S_i = S_{i-1} + K_i^T diag(eta_i) V_i.
     * The chunk length is part of the semantics.  beta must be 0. */
    TTT_CHUNK_CAUSAL = 1
} ttt_mode_t;

/* Arguments of ttt_fwd_chunked.  All strides are in elements. */
typedef struct ttt_fwd_args {
    int32_t B, H, L;          /* batch, heads, sequence length (L >= 1)          */
    int32_t dk, dv;           /* key / value head dims                           */
    int32_t chunk;            /* chunk length C >= 1                             */
    int32_t mode;             /* ttt_mode_t                                      */
    int32_t dtype;            /* ttt_dtype_t of q, k, v and out                  */
    const void* q;            /* [B,H,L,dk]                                      */
    const void* k;            /* [B,H,L,dk]                                      */
    const void* v;            /* [B,H,L,dv]                                      */
    int64_t q_stride[3];      /* strides of the B, H, L dims                     */
    int64_t k_stride[3];
    int64_t v_stride[3];
    const float* eta;         /* [B,H,L] fp32 per-token step size, or NULL       */
    int64_t eta_stride[3];    /* strides of eta (ignored when eta is NULL)       */
    float eta_scalar;         /* step size of every token when eta == NULL       */
    float beta;               /* momentum in [0,1); 0 = plain update             */
    const float* S0;          /* [B,H,dk,dv] initial state, NULL = zero          */
    int64_t S0_stride[2];     /* B, H strides of S0; 0 broadcasts                */
    const float* M0;          /* [B,H,dk,dv] initial momentum, NULL = zero       */
    int64_t M0_stride[2];
    void* out;                /* [B,H,L,dv], dtype `dtype`                       */
    int64_t out_stride[3];
    float* S_final;           /* [B,H,dk,dv] contiguous, NULL = not written      */
    float* M_final;           /* [B,H,dk,dv] contiguous, NULL = not written;
                                 only written when beta != 0                    */
    void* workspace;          /* device scratch, >= ttt_fwd_workspace_size bytes */
    size_t workspace_bytes;
    void* stream;             /* hipStream_t                                     */
    int32_t lookback_polls;   /* bound of each look-back wait of a segmented
                                 call, in polls of ~0.1 us: 0 = the default
                                 (2^22); < 0 = give up without polling (for
                                 tests of the failure report)                   */
} ttt_fwd_args;

/*
 * ttt_fwd_chunked -- chunked forward of the fast-weight layer.
 *
 * TOKEN_CAUSAL ([P1], paragraphs on the state-matrix update, momentum SGD as
 * weighted linear attention, associativity without weight normalisation,
 * per-token rates folded into the values; [P4] section on the inner update
 * rule): with g_t = eta_t k_t^T v_t,
 *     m_t = beta m_{t-1} + g_t,  S_t = S_{t-1} + m_t,  o_t = q_t S_t,
 * S_{-1} = S0, m_{-1} = M0.  Computed chunk by chunk: the readout of the
 * state at the chunk start, a causal intra-chunk term, then the chunk's
 * aggregate update; equal (up to rounding) to the per-token recurrence.
 *
 * CHUNK_CAUSAL ([P2]): o_t = q_t S_{i-1} for t in chunk i, then
 *     S_i = S_{i-1} + K_i^T diag(eta_i) V_i.
 * For the In-Place setting pass q = k = Z (activations), v = V-hat, S0 = W0.
 *
 * Precision: bf16 inputs are contracted on bf16 MFMA with fp32
 * accumulation; the state is accumulated in fp32 and read through a bf16
 * copy; out is rounded once to the input dtype.  fp32 inputs use fp32 MFMA
 * end to end.
 *
 * Supported (else TTT_ERR_UNSUPPORTED): dk, dv in {32, 64, 128} for both
 * dtypes and both modes; CHUNK_CAUSAL with bf16 also dk, dv multiples of 256
 * (large fast weights, e.g. the In-Place Wdown) with chunk a multiple of 256
 * and row strides of q, k and v below 2^22 elements.
 * CHUNK_CAUSAL with small dims needs chunk a multiple of 64 (bf16) or 32
 * (fp32).  Returns TTT_ERR_WORKSPACE if the workspace is too small, and
 * TTT_ERR_ALIAS if out, S_final, M_final or the workspace overlaps an input
 * (q, k, v, eta, S0, M0) or another of them, or if out's strides map two
 * (b, h, t) onto overlapping rows.
 */
ttt_status_t ttt_fwd_chunked(const ttt_fwd_args* args);

/* Bytes of workspace ttt_fwd_chunked needs for these arguments (pointers
 * need not be set).  0 is a valid answer (workspace may then be NULL). */
ttt_status_t ttt_fwd_workspace_size(const ttt_fwd_args* args, size_t* bytes);

/*
 * ttt_fwd_chunked_noalloc -- ttt_fwd_chunked for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and kernels, with
 * the look-back scratch of segmented calls in a static device array of
 * TTT_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The caller still passes every input and output;
 * args->workspace and args->workspace_bytes are ignored.
 * Calls whose scratch need (ttt_fwd_workspace_size) exceeds the array
 * return TTT_ERR_WORKSPACE before anything is enqueued: every token-causal
 * and small-head chunk-causal call fits (their look-back needs < 64 MiB);
 * the large-fast-weight chunk-causal (In-Place) path fits only while its
 * bf16 weight snapshots do (not at the 9728 x 2560 In-Place sizes).  All calls on one GPU share its array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must be serialised by the caller.  The first call on a device
 * looks up the array's device address (hipGetSymbolAddress); nothing is ever
 * allocated or freed.  Other errors as ttt_fwd_chunked.
 */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ttt_status_t ttt_fwd_chunked_noalloc(const ttt_fwd_args* args);

/*
 * ttt_fwd_lookback_status -- whether the last ttt_fwd_chunked call with
 * these arguments and this workspace gave up a look-back wait.
 *
 * When the (head, value-column tile) grid is short of the chip, a long
 * sequence is cut into segments that run concurrently and hand their states
 * on through flags in the workspace ([P1] paragraph on associativity: the
 * segment states compose; [P2] paragraph on the associative scan).  Each
 * wait for a flag is bounded (args->lookback_polls); a wait that gives up
 * lets the kernel finish with invalid results and raises an error word in
 * the workspace.  This call waits for `args->stream`, reads that word and
 * sets *gave_up to 1 if it was raised (0 otherwise, and always 0 for calls
 * that were not segmented).  Not callable inside a graph capture (it
 * synchronises the stream).  Errors: TTT_ERR_NULL, the shape errors of
 * ttt_fwd_workspace_size, TTT_ERR_WORKSPACE (segmented and no workspace),
 * TTT_ERR_HIP.
 */
ttt_status_t ttt_fwd_lookback_status(const ttt_fwd_args* args, int32_t* gave_up);

/*
 * ttt_chunk_state_scan -- exclusive scan of per-chunk state deltas.
 *
 * [P1] paragraph on removing weight normalisation: state updates become
 * associative and a parallel prefix scan replaces the sequential walk; [P2]
 * paragraph on the associative scan: chunk updates computed independently
 * are combined by a prefix sum, identical to the sequential update.
 *
 * Inputs dS, dM [B,H,N,dk,dv] fp32 (contiguous) are the change of (S, m)
 * over chunk c when that chunk starts from S = m = 0.  The chunk transition
 * for a chunk of n tokens is
 *     S' = S + alpha_n m + dS_c,  alpha_n = beta + ... + beta^n
 *     m' = beta^n m + dM_c
 * (beta = 0: S' = S + dS_c and dM is ignored, may be NULL).  Chunks hold
 * `chunk` tokens except the last, which holds L - (N-1)*chunk; N must equal
 * ceil(L / chunk).  Outputs the state at the start of every chunk, S_excl /
 * M_excl [B,H,N,dk,dv] (M_excl may be NULL), and the state after the last
 * chunk, S_final / M_final [B,H,dk,dv] (each may be NULL).  S0 / M0 are the
 * incoming state (NULL = zero).  fp32 throughout.  Any dk, dv >= 1 with
 * dk*dv a multiple of 4.  Needs no workspace (ws may be NULL).  The outputs
 * must not overlap the inputs or each other (no in-place scan):
 * TTT_ERR_ALIAS.
 */
ttt_status_t ttt_chunk_state_scan(int32_t B, int32_t H, int32_t L, int32_t chunk,
                                  int32_t dk, int32_t dv,
                                  const float* dS, const float* dM, float beta,
                                  const float* S0, const float* M0,
                                  float* S_excl, float* M_excl,
                                  float* S_final, float* M_final,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ttt_dual_form_fwd -- TTT-Linear mini-batch forward, dual form.
 *
 * [P4] section on turning the gradient into an efficient layer: tokens are
 * grouped into mini-batches of `minibatch` tokens; inside a mini-batch every
 * gradient is taken at the weights W_n the mini-batch started from, and the
 * output of token t uses the gradient of the mini-batch prefix up to t:
 *     W_{n,t} = W_n - eta sum_{s<=t, s in n} k_s^T (k_s W_n - v_s),  o_t = q_t W_{n,t},
 *     W_{n+1} = W_{n,last}.
 * Inner model f(k) = k W (linear, no bias, no normalisation); loss
 * 1/2 ||k W - v||^2.  This update is not associative; the mini-batches run
 * in order ([P5] background: small online mini-batches; key idea: large
 * chunks).
 *
 * q, k [B,H,L,d], v, out [B,H,L,dv] contiguous, dtype `dtype`; W0
 * [B,H,d,dv] fp32 (W0_stride_bh elements between heads, 0 broadcasts one
 * W0); W_final [B,H,d,dv] fp32 contiguous or NULL; out, W_final and the
 * workspace overlap no input (q, k, v, W0) and not each other
 * (TTT_ERR_ALIAS).  Supported: d = 64, dv = 64, bf16 or fp32, any
 * minibatch >= 1 (the last mini-batch holds the remaining
 * L - (ceil(L/minibatch)-1)*minibatch tokens).
 *
 * Segments.  Over one mini-batch the update is affine in the state,
 * W_{n+1} = (I - eta K_n^T K_n) W_n + eta K_n^T V_n, so a run of whole
 * mini-batches maps its start state W to A W + B.  For bf16 with minibatch
 * a multiple of 16 and few sequences (B*H <= 128), a call given a workspace
 * of at least ttt_dual_form_workspace_size bytes cuts every sequence into
 * segments of whole mini-batches that run concurrently: each segment
 * computes its (A - I, B) from K and V alone, composes the maps of the
 * segments before it onto W0 in order, then runs its own tokens.  When
 * that yields one more segment than the GPU holds at once, segment 0
 * instead runs only its tokens and hands on its end state, onto which the
 * later segments compose, and its workgroup then runs the last segment.
 * The result equals the one-chain result up to fp32 rounding (the composed
 * start states are not bit-identical to the chained ones; repeated calls
 * are).  workspace NULL runs each sequence as one chain; a non-NULL
 * workspace smaller than needed is TTT_ERR_WORKSPACE.  The waits between
 * segments are bounded; ttt_dual_form_lookback_status reports one that gave
 * up (TTT_ERR_TIMEOUT in the binding; its results are invalid).
 */
ttt_status_t ttt_dual_form_fwd(int32_t B, int32_t H, int32_t L, int32_t d, int32_t dv,
                               int32_t minibatch, int32_t dtype,
                               const void* q, const void* k, const void* v,
                               const float* W0, int64_t W0_stride_bh, float eta,
                               void* out, float* W_final,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace ttt_dual_form_fwd uses to run these sizes in segments;
 * 0 when the shape runs as one chain anyway.  Sizes only, no GPU needed.
 * Errors: TTT_ERR_NULL, TTT_ERR_DTYPE, TTT_ERR_SHAPE, TTT_ERR_UNSUPPORTED. */
ttt_status_t ttt_dual_form_workspace_size(int32_t B, int32_t H, int32_t L, int32_t d, int32_t dv,
                                          int32_t minibatch, int32_t dtype, size_t* bytes);

/* After a segmented ttt_dual_form_fwd with the same sizes and workspace:
 * waits for `stream` and sets *gave_up to 1 if a wait between segments gave
 * up (the outputs are then invalid), else 0 (also when the call ran as one
 * chain or workspace is NULL).  Errors: TTT_ERR_NULL (gave_up), the size
 * errors of ttt_dual_form_workspace_size, TTT_ERR_WORKSPACE (too small),
 * TTT_ERR_HIP. */
ttt_status_t ttt_dual_form_lookback_status(int32_t B, int32_t H, int32_t L, int32_t d, int32_t dv,
                                           int32_t minibatch, int32_t dtype, const void* workspace,
                                           size_t workspace_bytes, void* stream, int32_t* gave_up);

/*
 * ttt_decode_step -- one token of the token-causal recurrence per (b, h),
 * with the state updated in place.
 *
 * [P1] paragraphs on the state-matrix update and the one-step output
 * identity; [P4] section on the inner update rule and the fixed-size state
 * that replaces a growing cache.  With g = eta k^T v:
 *     m <- beta m + g,  S <- S + m,  o = q S   (o reads the updated state),
 * i.e. exactly ttt_fwd_chunked in TOKEN_CAUSAL mode for L = 1 with
 * S0 = S, M0 = M and S_final = S.  Calling it for t = 0..L-1 reproduces the
 * chunked forward over the L tokens.
 *
 * q, k [B,H,dk] and v, out [B,H,dv] are contiguous, dtype `dtype` (out in
 * that dtype).  eta [B,H] fp32 or NULL (eta_scalar for every sequence).
 * S [B,H,dk,dv] fp32 contiguous, read and written in place; M the same shape,
 * required when beta != 0 (ignored and may be NULL otherwise).  out, S and M
 * (the written buffers) must not overlap q, k, v, eta or each other.
 * Supported: dk in [1, 1024], dv a multiple of 4.
 * The state is read and written once (memory-bound); the update is fp32.
 * All pointers are caller-owned device memory, 16-byte aligned; stream is a
 * hipStream_t (NULL = default stream).  Nothing is allocated.
 *
 * Errors (checked before anything is enqueued): TTT_ERR_DTYPE, TTT_ERR_SHAPE
 * (a size < 1), TTT_ERR_VALUE (beta outside [0, 1)), TTT_ERR_NULL (q, k, v, S
 * or out NULL, or M NULL with beta != 0), TTT_ERR_ALIGN, TTT_ERR_UNSUPPORTED
 * (dk or dv outside the supported set), TTT_ERR_ALIAS (out overlaps an input,
 * or S overlaps M with beta != 0); TTT_ERR_HIP if the launch fails.
 */
ttt_status_t ttt_decode_step(int32_t B, int32_t H, int32_t dk, int32_t dv, int32_t dtype,
                             const void* q, const void* k, const void* v,
                             const float* eta, float eta_scalar, float beta,
                             float* S, float* M, void* out, void* stream);

/*
 * ttt_bwd_chunked -- backward pass of ttt_fwd_chunked in TOKEN_CAUSAL mode,
 * with or without momentum.
 *
 * [P1] paragraphs on the state-matrix update, on the one-step output
 * identity and on momentum give the forward g_t = eta_t k_t^T v_t,
 * m_t = beta m_{t-1} + g_t, S_t = S_{t-1} + m_t, o_t = q_t S_t (from S0, M0);
 * [P4] section on the two kinds of weights trains the outer model through
 * these updates, which needs their gradients.  Given dout = dL/do,
 * dS_final = dL/dS_final and dM_final = dL/dM_final (NULL: zero), with
 * A_t the adjoint of m_t (the sum over u >= t of the momentum-weighted
 * q_u^T do_u plus the boundary terms; beta = 0: dS_final + sum_{u>=t} q_u^T do_u):
 *     dq_t = do_t S_t^T,  dk_t = eta_t A_t v_t^T,  dv_t = eta_t k_t A_t,
 *     deta_t = k_t A_t v_t^T (per token, also for a scalar eta: its gradient
 *     is the sum over tokens),  dS0 = dL/dS0,  dM0 = beta A_0.
 * Every beta in [0, 1) is handled without dividing by beta.  The gradient
 * with respect to beta comes from ttt_bwd_dbeta (same inputs).
 *
 * All tensors are contiguous: q, k, dq, dk [B,H,L,dk]; v, dout, dv
 * [B,H,L,dv] in `dtype`; eta [B,H,L] fp32 or NULL (eta_scalar); S0, M0,
 * dS_final, dM_final, dS0, dM0 [B,H,dk,dv] fp32 or NULL (inputs: zero; M0
 * and dM_final ignored when beta = 0).  deta, dS0 and dM0 may be NULL (not
 * computed).  beta in [0, 1).  Supported: dk, dv in {32, 64, 128}.  Outputs
 * must not overlap any input or each other.  workspace: device memory of
 * ttt_bwd_workspace_size bytes (0 possible), caller-owned.
 * Errors (before anything is enqueued): TTT_ERR_NULL, TTT_ERR_DTYPE,
 * TTT_ERR_SHAPE, TTT_ERR_VALUE (beta), TTT_ERR_ALIGN (16 bytes),
 * TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_ALIAS; TTT_ERR_HIP if a
 * launch fails.
 * Streams: everything runs on `stream` when side_stream is NULL (or equal
 * to `stream`).  Otherwise side_stream, a second stream of the caller on
 * the same device, runs the dv/deta step beside the last pass: it is forked
 * from `stream` by an event and joined back before the call returns, also
 * on an error return after the fork, so all of the call's work is ordered
 * before anything enqueued on `stream` afterwards, also inside a captured
 * graph.  Work the caller enqueues on side_stream during the call runs
 * after the fork point, like any other work ordered behind an event.
 */
ttt_status_t ttt_bwd_workspace_size(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t dtype,
                                    float beta, size_t* bytes);
ttt_status_t ttt_bwd_chunked(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t dtype,
                             const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                             float beta, const float* S0, const float* M0, const void* dout,
                             const float* dS_final, const float* dM_final,
                             void* dq, void* dk_out, void* dv_out, float* deta, float* dS0, float* dM0,
                             void* workspace, size_t workspace_bytes, void* stream, void* side_stream);

/*
 * ttt_bwd_dbeta -- dL/dbeta, the gradient of the momentum coefficient, for
 * the token-causal forward with momentum ([P1] paragraph on momentum: the
 * update m_t = beta m_{t-1} + g_t; [P4] section on the two kinds of weights:
 * the outer model learns through the inner updates, beta included when it
 * is learned).  For L = sum_t <dout_t, o_t> + <dS_final, S_final> +
 * <dM_final, M_final> it returns, per (b, h),
 *     dbeta = sum_t q_t S'_t dout_t^T + <dS_final, S'_{L-1}> + <dM_final, m'_{L-1}>
 * with the derivatives of the states m'_t = beta m'_{t-1} + m_{t-1},
 * S'_t = S'_{t-1} + m'_t (from zero), i.e. the plain derivative of the
 * recurrence; S0 does not enter.  It is a call of its own beside
 * ttt_bwd_chunked (same inputs, same layouts: contiguous q, k [B,H,L,dk],
 * v, dout [B,H,L,dv] in dtype, eta [B,H,L] fp32 or NULL (eta_scalar), M0,
 * dS_final, dM_final fp32 [B,H,dk,dv] or NULL = zero).  Any beta in [0, 1)
 * (the derivative at beta = 0 is defined too).  Output dbeta: fp32 [B,H],
 * written in full; the sum over columns and tokens is taken in a fixed
 * order (repeated calls agree bit for bit).  workspace: device memory of
 * ttt_bwd_dbeta_workspace_size bytes, caller-owned, overwritten.
 * Supported: dk in {32, 64, 128}, dv a multiple of 16 up to 1024, a head's
 * rows below 2^31 bytes.  Errors (before anything is enqueued):
 * TTT_ERR_NULL, TTT_ERR_DTYPE, TTT_ERR_SHAPE, TTT_ERR_VALUE (beta),
 * TTT_ERR_ALIGN (16 bytes), TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE,
 * TTT_ERR_ALIAS (dbeta or the workspace overlapping an input or each
 * other); TTT_ERR_HIP if a launch fails.  Runs on `stream`.
 */
ttt_status_t ttt_bwd_dbeta_workspace_size(int32_t B, int32_t H, int32_t dv, size_t* bytes);
ttt_status_t ttt_bwd_dbeta(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t dtype,
                           const void* q, const void* k, const void* v, const float* eta, float eta_scalar,
                           float beta, const float* M0, const void* dout, const float* dS_final,
                           const float* dM_final, float* dbeta, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * In-Place TTT front end ([P2] "In-Place 테스트 시점 학습: LLM을 위한 원활한
 * 동적 적응 프레임워크", aitrends.kr/articles/40879).  These produce the
 * inputs of ttt_fwd_chunked in CHUNK_CAUSAL mode with q = k = Z, v = V-hat,
 * S0 = Wdown and per-token eta.  All activations are bf16 and contiguous;
 * weights use the row = output feature layout ([out, in], K contiguous).
 *
 * ttt_inplace_gated_input ([P2] paragraph on the Gated-MLP structure: Wgate
 * and Wup are fixed slow weights, Wdown the fast weight that multiplies
 * their output):
 *     Z = silu(X Wg^T) * (X Wu^T),  silu(a) = a / (1 + exp(-a))
 *   X [T, d_model], Wg, Wu [d_ff, d_model], Z [T, d_ff].  fp32 accumulation,
 *   one rounding of Z to bf16.  Supported: d_model a multiple of 128, d_ff
 *   a multiple of 128.  Z must not overlap the inputs.
 *
 * ttt_inplace_lm_target ([P2] paragraph on the LM-aligned objective: a 1D
 * convolution over the current and following tokens, then a projection):
 *     Y[b, t] = sum_{j < taps, t + j < L} conv_w[j] * X[b, t + j]   (depthwise)
 *     V-hat = Y Wv^T
 *   X, V-hat [B, L, d_model]; conv_w [taps, d_model] fp32 (1 <= taps <= 16);
 *   Wv [d_model, d_model].  Y is kept in bf16 in `workspace`
 *   (ttt_inplace_lm_target_workspace_size bytes).  Supported: d_model a
 *   multiple of 256.
 *
 * ttt_inplace_clip_eta ([P2] paragraph on the limitations: clipping keeps
 * accumulated updates stable): for each chunk i of each sequence,
 *     eta_out[t] = eta * min(1, tau / ||eta Z_i^T V_i||_F)   (t in chunk i)
 *   computed from the chunk's Gram products (Z_i Z_i^T, V_i V_i^T), without
 *   forming the d_ff x d_model update.  Z [B, L, d_ff], V-hat [B, L, d_model],
 *   eta_out [B, L] fp32; tau > 0.  workspace: ttt_inplace_clip_eta_workspace_size
 *   bytes.  Supported: d_ff, d_model multiples of 128.
 *
 * Errors (before anything is enqueued): TTT_ERR_NULL, TTT_ERR_SHAPE,
 * TTT_ERR_VALUE, TTT_ERR_ALIGN (16 bytes), TTT_ERR_UNSUPPORTED,
 * TTT_ERR_WORKSPACE, TTT_ERR_ALIAS (an output overlaps an input or the
 * workspace); TTT_ERR_HIP if a launch fails.  All pointers are caller-owned
 * device memory; stream is a hipStream_t (NULL: default stream).
 */
ttt_status_t ttt_inplace_gated_input(int32_t T, int32_t d_model, int32_t d_ff, const void* X, const void* Wg,
                                     const void* Wu, void* Z, void* stream);
ttt_status_t ttt_inplace_lm_target_workspace_size(int32_t B, int32_t L, int32_t d_model, size_t* bytes);
ttt_status_t ttt_inplace_lm_target(int32_t B, int32_t L, int32_t d_model, int32_t taps, const void* X,
                                   const float* conv_w, const void* Wv, void* Vhat, void* workspace,
                                   size_t workspace_bytes, void* stream);
ttt_status_t ttt_inplace_clip_eta_workspace_size(int32_t B, int32_t L, int32_t chunk, size_t* bytes);
ttt_status_t ttt_inplace_clip_eta(int32_t B, int32_t L, int32_t d_ff, int32_t d_model, int32_t chunk,
                                  const void* Z, const void* Vhat, float eta, float tau, float* eta_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Large-chunk SwiGLU fast weight ([P5] "LaCT (Large Chunk Test-Time
 * Training)" wiki, aisparkup.com/wiki/lact, section on the core idea:
 * nonlinear fast weights updated once per large chunk, the chunk's tokens
 * forming one batch; [P4] "RNN의 기억을 작은 모델로 바꾼다면: Test-Time
 * Training 읽기", ariser.io, section on the update rule: the state is the
 * weights of a small model and takes gradient steps on an inner loss).
 * Per (b, h) and chunk i of `chunk` tokens (the last one may be shorter),
 * with W = (W1, W3, W2) the weights left by chunks < i:
 *
 *     out_i = f_W(q_i),   f_W(x) = W2 (silu(W1 x) * (W3 x))
 *     W    <- W - grad_W sum_{t in i} eta_t l_t(W)
 *     l_t   = -<f_W(k_t), v_t>          loss = TTT_LOSS_DOT
 *     l_t   = 1/2 ||f_W(k_t) - v_t||^2  loss = TTT_LOSS_MSE
 *
 *   q, k [B, H, L, dk], v, out [B, H, L, dv]: bf16, contiguous.
 *   eta [B, H, L] fp32 per-token step sizes, or NULL: eta_scalar for all.
 *   W1, W3 [B, H, m, dk] and W2 [B, H, dv, m]: fp32, contiguous, row =
 *   output feature; read as the initial weights and OVERWRITTEN with the
 *   weights after the last chunk.
 *   Arithmetic: bf16 MFMA operands (activations and a bf16 copy of the
 *   weights, refreshed after every chunk), fp32 accumulation, fp32 weights.
 *   workspace: ttt_swiglu_workspace_size bytes of device memory,
 *   caller-owned, no initial contents needed (bf16 weight copies and one
 *   chunk's activations).
 * Supported (else TTT_ERR_UNSUPPORTED): dk, dv, m and chunk multiples of
 * 128, and chunk * max(dk, dv, 2 m) below 2^31.  A chunk longer than the
 * sequence acts as one chunk of the whole sequence.
 * Errors (before anything is enqueued): TTT_ERR_NULL, TTT_ERR_SHAPE,
 * TTT_ERR_VALUE (loss), TTT_ERR_ALIGN (16 bytes), TTT_ERR_UNSUPPORTED,
 * TTT_ERR_WORKSPACE, TTT_ERR_ALIAS (out, a weight or the workspace overlaps
 * another buffer); TTT_ERR_HIP if a launch fails.
 */
typedef enum { TTT_LOSS_DOT = 0, TTT_LOSS_MSE = 1 } ttt_loss_t;
ttt_status_t ttt_swiglu_workspace_size(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t m,
                                       int32_t chunk, size_t* bytes);
ttt_status_t ttt_swiglu_fwd_chunked(int32_t B, int32_t H, int32_t L, int32_t dk, int32_t dv, int32_t m,
                                    int32_t chunk, int32_t loss, const void* q, const void* k, const void* v,
                                    const float* eta, float eta_scalar, float* W1, float* W3, float* W2,
                                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* ttt_status_string(ttt_status_t status);

/* sizeof(ttt_fwd_args) as compiled into the library (ABI check for bindings). */
size_t ttt_fwd_args_size(void);

#ifdef __cplusplus
}
#endif
#endif /* TTT_MI355X_H */
