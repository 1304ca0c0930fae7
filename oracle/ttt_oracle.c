/*
 * ttt_oracle.c -- fp64 CPU oracle for the chunked TTT fast-weight forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the HIP library and includes nothing of
 * it.
 *
 * Every routine walks tokens one at a time in plain loops, in double
 * precision, exactly in the order the definitions state.  No blocking, no
 * reordering, no fused kernels.  OpenMP only spreads independent (batch,
 * head) pairs over host threads; the arithmetic inside a pair is sequential.
 *
 * Sources (pages, cited by title and paragraph/section):
 *  [P1] "KV 바인딩 기반 테스트 시간 학습은 사실상 선형 어텐션이다"
 *       (aitrends.kr/articles/4698): inner-loop update of TTT with KV binding
 *       is a linear-attention state update; one gradient step of a bias-free
 *       linear last layer gives o = q(S0 + k^T v); momentum SGD is a weighted
 *       linear attention; per-token learning rates fold into the values.
 *  [P4] "RNN의 기억을 작은 모델로 바꾼다면: Test-Time Training 읽기"
 *       (ariser.io), section "읽는 동안 문제를 하나 더 푼다": the state is the
 *       weight of a small model, updated by W_t = W_{t-1} - eta*grad l(W_{t-1}; x_t)
 *       and the output is read from the updated model; section "gradient를
 *       효율적인 layer로 만드는 작업": mini-batch TTT and its dual form.
 *
 * Layout: every array is contiguous, q/k [B,H,L,dk], v/out [B,H,L,dv],
 * states [B,H,dk,dv], per-token eta [B,H,L].
 */
#include <stdlib.h>
#include <string.h>

/*
 * Token-causal fast-weight recurrence, with optional momentum ([P1], the
 * paragraphs on the state-matrix update and on momentum SGD; [P4] update
 * rule W_t = W_{t-1} - eta*grad l).  With the binding loss l_t = -eta_t<k_t W, v_t>
 * the gradient step adds g_t = eta_t k_t^T v_t ("gradient ascent" on the
 * binding, [P1] paragraph on LaCT-LLM / ViTTT).  Per token t = 0..L-1:
 *
 *     g_t = eta_t * k_t^T v_t
 *     m_t = beta * m_{t-1} + g_t            (m_{-1} = M0, zero if NULL)
 *     S_t = S_{t-1} + m_t                   (S_{-1} = S0, zero if NULL)
 *     o_t = q_t S_t                         (read after the update: inclusive)
 *
 * beta = 0 gives plain linear attention S_t = S_{t-1} + g_t.  eta may be NULL,
 * then eta_scalar is used for every token.  S_final / M_final may be NULL.
 */
void ttt_oracle_token_causal(int B, int H, int L, int dk, int dv,
                             const double* q, const double* k, const double* v,
                             const double* eta, double eta_scalar, double beta,
                             const double* S0, const double* M0,
                             double* out, double* S_final, double* M_final)
{
    const long nbh = (long)B * H;
    const long sz = (long)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* S = (double*)malloc(sizeof(double) * sz);
        double* m = (double*)malloc(sizeof(double) * sz);
        for (long e = 0; e < sz; ++e) {
            S[e] = S0 ? S0[bh * sz + e] : 0.0;
            m[e] = M0 ? M0[bh * sz + e] : 0.0;
        }
        for (int t = 0; t < L; ++t) {
            const double* qt = q + (bh * L + t) * dk;
            const double* kt = k + (bh * L + t) * dk;
            const double* vt = v + (bh * L + t) * dv;
            const double et = eta ? eta[bh * L + t] : eta_scalar;
            for (int i = 0; i < dk; ++i) {
                for (int j = 0; j < dv; ++j) {
                    const double g = et * kt[i] * vt[j];
                    m[(long)i * dv + j] = beta * m[(long)i * dv + j] + g;
                    S[(long)i * dv + j] += m[(long)i * dv + j];
                }
            }
            double* ot = out + (bh * L + t) * dv;
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qt[i] * S[(long)i * dv + j];
                ot[j] = acc;
            }
        }
        if (S_final) memcpy(S_final + bh * sz, S, sizeof(double) * sz);
        if (M_final) memcpy(M_final + bh * sz, m, sizeof(double) * sz);
        free(S);
        free(m);
    }
}

/*
 * TTT-Linear mini-batch update in primal form ([P4], section on turning the
 * gradient into an efficient layer: tokens are grouped into mini-batches,
 * every gradient inside a mini-batch is taken at the weights the mini-batch
 * started from, and the dual form is only another way to compute exactly this
 * mini-batch update -- it is not per-token SGD).  Inner model f(k) = k W,
 * loss l_s(W) = 1/2 ||k_s W - v_s||^2, gradient k_s^T (k_s W - v_s).
 * For mini-batch n starting at W_n and each token t in it, in order:
 *
 *     G_t     = sum_{s in n, s <= t} k_s^T (k_s W_n - v_s)
 *     o_t     = q_t (W_n - eta * G_t)
 *     W_{n+1} = W_n - eta * G_last
 *
 * The last mini-batch may be shorter (L not a multiple of b).
 * q/k [B,H,L,d], v/out [B,H,L,dv], W0/W_final [B,H,d,dv].
 */
void ttt_oracle_dual_primal(int B, int H, int L, int d, int dv, int minibatch,
                            const double* q, const double* k, const double* v,
                            const double* W0, double eta,
                            double* out, double* W_final)
{
    const long nbh = (long)B * H;
    const long sz = (long)d * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* W = (double*)malloc(sizeof(double) * sz);
        double* G = (double*)malloc(sizeof(double) * sz);
        double* e = (double*)malloc(sizeof(double) * dv);
        memcpy(W, W0 + bh * sz, sizeof(double) * sz);
        for (int n0 = 0; n0 < L; n0 += minibatch) {
            const int n1 = (n0 + minibatch < L) ? n0 + minibatch : L;
            for (long x = 0; x < sz; ++x) G[x] = 0.0;
            for (int t = n0; t < n1; ++t) {
                const double* qt = q + (bh * L + t) * d;
                const double* kt = k + (bh * L + t) * d;
                const double* vt = v + (bh * L + t) * dv;
                /* reconstruction error of token t under W_n */
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i) acc += kt[i] * W[(long)i * dv + j];
                    e[j] = acc - vt[j];
                }
                for (int i = 0; i < d; ++i)
                    for (int j = 0; j < dv; ++j) G[(long)i * dv + j] += kt[i] * e[j];
                double* ot = out + (bh * L + t) * dv;
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += qt[i] * (W[(long)i * dv + j] - eta * G[(long)i * dv + j]);
                    ot[j] = acc;
                }
            }
            for (long x = 0; x < sz; ++x) W[x] -= eta * G[x];
        }
        if (W_final) memcpy(W_final + bh * sz, W, sizeof(double) * sz);
        free(W);
        free(G);
        free(e);
    }
}

/*
 * Sequential scan over chunk states ([P1] paragraph on removing weight
 * normalisation so that state updates become associative and a prefix scan
 * applies; [P2] "In-Place 테스트 시점 학습", paragraph on the associative scan:
 * every chunk's update is computed on its own and a prefix sum applies them,
 * identical to the sequential update).
 *
 * Input: per-chunk aggregates dS_c, dM_c [B,H,N,dk,dv]: the change of (S, m)
 * over chunk c when the chunk starts from S = m = 0.  The chunk transition of
 * the momentum recurrence above, for a chunk of n tokens, is
 *
 *     S_next = S + alpha_n * m + dS_c,   alpha_n = sum_{i=1..n} beta^i
 *     m_next = beta^n * m + dM_c
 *
 * (beta = 0: S_next = S + dS_c).  Chunks hold `chunk` tokens, the last one
 * L - (N-1)*chunk.  Outputs the exclusive prefixes (state at the start of
 * each chunk) and the final state; walked strictly in chunk order.
 */
void ttt_oracle_state_scan(int B, int H, int L, int chunk, int dk, int dv,
                           const double* dS, const double* dM, double beta,
                           const double* S0, const double* M0,
                           double* S_excl, double* M_excl,
                           double* S_final, double* M_final)
{
    const int N = (L + chunk - 1) / chunk;
    const long nbh = (long)B * H;
    const long sz = (long)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* S = (double*)malloc(sizeof(double) * sz);
        double* m = (double*)malloc(sizeof(double) * sz);
        for (long e = 0; e < sz; ++e) {
            S[e] = S0 ? S0[bh * sz + e] : 0.0;
            m[e] = M0 ? M0[bh * sz + e] : 0.0;
        }
        for (int c = 0; c < N; ++c) {
            const int n = (c == N - 1) ? L - c * chunk : chunk;
            double alpha = 0.0, p = 1.0;
            for (int i = 1; i <= n; ++i) {
                p *= beta;
                alpha += p;
            }
            const double gamma = p;
            const long off = (bh * N + c) * sz;
            if (S_excl) memcpy(S_excl + off, S, sizeof(double) * sz);
            if (M_excl) memcpy(M_excl + off, m, sizeof(double) * sz);
            for (long e = 0; e < sz; ++e) {
                S[e] = S[e] + alpha * m[e] + dS[off + e];
                m[e] = gamma * m[e] + (dM ? dM[off + e] : 0.0);
            }
        }
        if (S_final) memcpy(S_final + bh * sz, S, sizeof(double) * sz);
        if (M_final) memcpy(M_final + bh * sz, m, sizeof(double) * sz);
        free(S);
        free(m);
    }
}

/*
 * Backward pass of the token-causal recurrence above: the exact adjoint of
 * ttt_oracle_token_causal, written out from the chain rule.  The pages give
 * the forward rule and state that the fast weights are trained through it
 * ([P4], section on the two kinds of weights: the outer loop learns through
 * the inner updates); the backward pass itself is not printed anywhere, so
 * this is the plain derivative of the recurrence, nothing more.
 *
 * Given dout (dL/do_t) and optional dS_final, dM_final (gradients of the
 * final states), two sweeps per (b, h):
 *   forward sweep (same recurrence as the forward pass):
 *       dq_t = do_t S_t^T                         (o_t = q_t S_t)
 *   reverse sweep, t = L-1 .. 0, adjoints Sa (of S_t) and ma (of m_t):
 *       Sa  += q_t^T do_t                         (o_t reads S_t)
 *       ma  += Sa                                 (S_t = S_{t-1} + m_t)
 *       dv_t   = eta_t k_t ma,  dk_t = eta_t ma v_t^T,
 *       deta_t = k_t ma v_t^T                      (m_t = beta m_{t-1} + g_t)
 *       ma   = beta ma                            (adjoint of m_{t-1})
 *   with Sa = dS_final, ma = dM_final at the start (zero if NULL), and
 *   dS0 = Sa, dM0 = ma at the end.
 * deta is per token even when the forward used a scalar eta (its gradient
 * is then the sum over tokens).  Any output pointer may be NULL.
 */
void ttt_oracle_token_causal_bwd(int B, int H, int L, int dk, int dv,
                                 const double* q, const double* k, const double* v,
                                 const double* eta, double eta_scalar, double beta,
                                 const double* S0, const double* M0,
                                 const double* dout, const double* dS_final, const double* dM_final,
                                 double* dq, double* dkk, double* dvv, double* deta,
                                 double* dS0, double* dM0)
{
    const long nbh = (long)B * H;
    const long sz = (long)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* S = (double*)malloc(sizeof(double) * sz);
        double* m = (double*)malloc(sizeof(double) * sz);
        double* Sa = (double*)malloc(sizeof(double) * sz);
        double* ma = (double*)malloc(sizeof(double) * sz);
        double* kr = (double*)malloc(sizeof(double) * dv);
        /* forward sweep: S_t, then dq_t = do_t S_t^T */
        for (long e = 0; e < sz; ++e) {
            S[e] = S0 ? S0[bh * sz + e] : 0.0;
            m[e] = M0 ? M0[bh * sz + e] : 0.0;
        }
        for (int t = 0; t < L; ++t) {
            const double* kt = k + (bh * L + t) * dk;
            const double* vt = v + (bh * L + t) * dv;
            const double* dot = dout + (bh * L + t) * dv;
            const double et = eta ? eta[bh * L + t] : eta_scalar;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    m[(long)i * dv + j] = beta * m[(long)i * dv + j] + et * kt[i] * vt[j];
                    S[(long)i * dv + j] += m[(long)i * dv + j];
                }
            if (dq) {
                double* dqt = dq + (bh * L + t) * dk;
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += dot[j] * S[(long)i * dv + j];
                    dqt[i] = acc;
                }
            }
        }
        /* reverse sweep */
        for (long e = 0; e < sz; ++e) {
            Sa[e] = dS_final ? dS_final[bh * sz + e] : 0.0;
            ma[e] = dM_final ? dM_final[bh * sz + e] : 0.0;
        }
        for (int t = L - 1; t >= 0; --t) {
            const double* qt = q + (bh * L + t) * dk;
            const double* kt = k + (bh * L + t) * dk;
            const double* vt = v + (bh * L + t) * dv;
            const double* dot = dout + (bh * L + t) * dv;
            const double et = eta ? eta[bh * L + t] : eta_scalar;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    Sa[(long)i * dv + j] += qt[i] * dot[j];
                    ma[(long)i * dv + j] += Sa[(long)i * dv + j];
                }
            /* kr = k_t ma (a row of length dv) */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += kt[i] * ma[(long)i * dv + j];
                kr[j] = acc;
            }
            if (dvv) {
                double* dvt = dvv + (bh * L + t) * dv;
                for (int j = 0; j < dv; ++j) dvt[j] = et * kr[j];
            }
            if (deta) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += kr[j] * vt[j];
                deta[bh * L + t] = acc;
            }
            if (dkk) {
                double* dkt = dkk + (bh * L + t) * dk;
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += ma[(long)i * dv + j] * vt[j];
                    dkt[i] = et * acc;
                }
            }
            for (long e = 0; e < sz; ++e) ma[e] *= beta;
        }
        if (dS0) memcpy(dS0 + bh * sz, Sa, sizeof(double) * sz);
        if (dM0) memcpy(dM0 + bh * sz, ma, sizeof(double) * sz);
        free(S);
        free(m);
        free(Sa);
        free(ma);
        free(kr);
    }
}

/*
 * Derivative of the token-causal forward with respect to the momentum
 * coefficient beta, taken in forward mode: every line of the recurrence of
 * ttt_oracle_token_causal is differentiated with respect to beta.  [P1]
 * (paragraph on momentum) makes beta part of the update; [P4] (section on the
 * two kinds of weights) trains such parameters through the inner updates,
 * which needs dL/dbeta.  The pages print no backward pass; this is the plain
 * derivative.  With g_t = eta_t k_t^T v_t:
 *     m_t  = beta m_{t-1} + g_t            m'_t = beta m'_{t-1} + m_{t-1}
 *     S_t  = S_{t-1} + m_t                 S'_t = S'_{t-1} + m'_t
 *     o_t  = q_t S_t                       o'_t = q_t S'_t
 * from m_{-1} = M0, m'_{-1} = S'_{-1} = 0 (S0 does not depend on beta), and
 *     dbeta = sum_t <dout_t, o'_t> + <dS_final, S'_{L-1}> + <dM_final, m'_{L-1}>
 * (dS_final, dM_final NULL: zero).  dbeta is [B,H].
 */
void ttt_oracle_token_causal_dbeta(int B, int H, int L, int dk, int dv,
                                   const double* q, const double* k, const double* v,
                                   const double* eta, double eta_scalar, double beta,
                                   const double* M0, const double* dout,
                                   const double* dS_final, const double* dM_final, double* dbeta)
{
    const long nbh = (long)B * H;
    const long sz = (long)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        double* m = (double*)malloc(sizeof(double) * sz);
        double* mt = (double*)malloc(sizeof(double) * sz);   /* m' */
        double* St = (double*)malloc(sizeof(double) * sz);   /* S' */
        for (long e = 0; e < sz; ++e) {
            m[e] = M0 ? M0[bh * sz + e] : 0.0;
            mt[e] = 0.0;
            St[e] = 0.0;
        }
        double acc = 0.0;
        for (int t = 0; t < L; ++t) {
            const double* qt = q + (bh * L + t) * dk;
            const double* kt = k + (bh * L + t) * dk;
            const double* vt = v + (bh * L + t) * dv;
            const double* dot = dout + (bh * L + t) * dv;
            const double et = eta ? eta[bh * L + t] : eta_scalar;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    const long e = (long)i * dv + j;
                    mt[e] = beta * mt[e] + m[e];          /* uses m_{t-1} */
                    m[e] = beta * m[e] + et * kt[i] * vt[j];
                    St[e] += mt[e];
                }
            /* <dout_t, q_t S'_t> */
            for (int j = 0; j < dv; ++j) {
                double o = 0.0;
                for (int i = 0; i < dk; ++i) o += qt[i] * St[(long)i * dv + j];
                acc += dot[j] * o;
            }
        }
        for (long e = 0; e < sz; ++e) {
            if (dS_final) acc += dS_final[bh * sz + e] * St[e];
            if (dM_final) acc += dM_final[bh * sz + e] * mt[e];
        }
        dbeta[bh] = acc;
        free(m);
        free(mt);
        free(St);
    }
}

/* Number of host threads the OpenMP loops above use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
#endif
int ttt_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
