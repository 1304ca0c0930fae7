/* oracle_driver.c -- the C oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only, test code).
 *
 * Calls every routine of oracle/ttt_oracle.c on small inputs that reach its
 * edge cases (one token, ragged last chunk and mini-batch, NULL optional
 * inputs and outputs, beta = 0 and beta > 0) and checks a few identities
 * that hold exactly for these inputs, so that a sanitizer report cannot hide
 * behind a wrong but quiet result:
 *   - the scan with beta = 0 gives exclusive prefix sums of the deltas;
 *   - the token-causal output of a one-token sequence is q (S0 + eta k^T v);
 *   - the dual form with eta = 0 reads q W0.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void ttt_oracle_token_causal(int B, int H, int L, int dk, int dv, const double* q, const double* k, const double* v,
                             const double* eta, double eta_scalar, double beta, const double* S0, const double* M0,
                             double* out, double* S_final, double* M_final);
void ttt_oracle_dual_primal(int B, int H, int L, int d, int dv, int minibatch, const double* q, const double* k,
                            const double* v, const double* W0, double eta, double* out, double* W_final);
void ttt_oracle_state_scan(int B, int H, int L, int chunk, int dk, int dv, const double* dS, const double* dM,
                           double beta, const double* S0, const double* M0, double* S_excl, double* M_excl,
                           double* S_final, double* M_final);
void ttt_oracle_token_causal_bwd(int B, int H, int L, int dk, int dv, const double* q, const double* k,
                                 const double* v, const double* eta, double eta_scalar, double beta,
                                 const double* S0, const double* M0, const double* dout, const double* dS_final,
                                 const double* dM_final, double* dq, double* dkk, double* dvv, double* deta,
                                 double* dS0, double* dM0);

static unsigned seed = 12345u;
static double rnd(void) {
    seed = seed * 1103515245u + 12345u;
    return (double)((seed >> 8) & 0xffff) / 32768.0 - 1.0;
}
static double* arr(long n) {
    double* a = (double*)malloc(sizeof(double) * (size_t)n);
    for (long i = 0; i < n; ++i) a[i] = rnd();
    return a;
}

static int fails = 0;
static void expect(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "oracle driver: %s\n", what);
        ++fails;
    }
}

int main(void) {
    const int shapes[][5] = {{1, 1, 1, 3, 2}, {2, 3, 37, 5, 7}, {1, 2, 64, 8, 8}, {2, 1, 17, 4, 6}};
    const double betas[] = {0.0, 0.9, 1e-30};
    for (int si = 0; si < 4; ++si)
        for (int bi = 0; bi < 3; ++bi) {
            const int B = shapes[si][0], H = shapes[si][1], L = shapes[si][2], dk = shapes[si][3], dv = shapes[si][4];
            const double beta = betas[bi];
            const long T = (long)B * H * L, st = (long)B * H * dk * dv;
            double *q = arr(T * dk), *k = arr(T * dk), *v = arr(T * dv), *eta = arr(T), *S0 = arr(st), *M0 = arr(st);
            double *out = arr(T * dv), *Sf = arr(st), *Mf = arr(st), *dout = arr(T * dv), *dSf = arr(st),
                   *dMf = arr(st);
            double *dq = arr(T * dk), *dkk = arr(T * dk), *dvv = arr(T * dv), *deta = arr(T), *dS0 = arr(st),
                   *dM0 = arr(st);
            ttt_oracle_token_causal(B, H, L, dk, dv, q, k, v, eta, 0.0, beta, S0, M0, out, Sf, Mf);
            ttt_oracle_token_causal(B, H, L, dk, dv, q, k, v, NULL, 0.1, beta, NULL, NULL, out, NULL, NULL);
            ttt_oracle_token_causal_bwd(B, H, L, dk, dv, q, k, v, eta, 0.0, beta, S0, M0, dout, dSf, dMf, dq, dkk,
                                        dvv, deta, dS0, dM0);
            ttt_oracle_token_causal_bwd(B, H, L, dk, dv, q, k, v, NULL, 0.2, beta, NULL, NULL, dout, NULL, NULL,
                                        dq, NULL, NULL, NULL, NULL, NULL);
            if (L == 1) {   /* o = q (S0 + eta k^T v) with beta M0 added to the step */
                for (int j = 0; j < dv; ++j) {
                    double o = 0.0;
                    for (int i = 0; i < dk; ++i)
                        o += q[i] * (S0[i * dv + j] + beta * M0[i * dv + j] + eta[0] * k[i] * v[j]);
                    ttt_oracle_token_causal(1, 1, 1, dk, dv, q, k, v, eta, 0.0, beta, S0, M0, out, NULL, NULL);
                    expect(fabs(out[j] - o) <= 1e-12 * (1.0 + fabs(o)), "one-token identity");
                }
            }
            /* scan: N chunks with a ragged last one */
            const int chunk = 5, N = (L + chunk - 1) / chunk;
            const long ns = (long)B * H * N * dk * dv;
            double *dS = arr(ns), *dM = arr(ns), *Se = arr(ns), *Me = arr(ns);
            ttt_oracle_state_scan(B, H, L, chunk, dk, dv, dS, dM, beta, S0, M0, Se, Me, Sf, Mf);
            ttt_oracle_state_scan(B, H, L, chunk, dk, dv, dS, NULL, 0.0, NULL, NULL, Se, NULL, Sf, NULL);
            for (long bh = 0; bh < (long)B * H; ++bh)
                for (long e = 0; e < (long)dk * dv; ++e) {
                    double acc = 0.0;
                    for (int c = 0; c < N; ++c) {
                        const long off = (bh * N + c) * dk * dv + e;
                        expect(Se[off] == acc, "scan is the exclusive prefix sum (beta = 0)");
                        acc += dS[off];
                    }
                    expect(Sf[bh * dk * dv + e] == acc, "scan final state (beta = 0)");
                }
            /* dual form, d x dv state, ragged last mini-batch */
            double* W0 = arr((long)B * H * dk * dv);
            ttt_oracle_dual_primal(B, H, L, dk, dv, 4, q, k, v, W0, 0.05, out, Sf);
            ttt_oracle_dual_primal(B, H, L, dk, dv, 3, q, k, v, W0, 0.0, out, NULL);
            for (long t = 0; t < T; ++t) {
                const long bh = t / L;
                for (int j = 0; j < dv; ++j) {
                    double o = 0.0;
                    for (int i = 0; i < dk; ++i) o += q[t * dk + i] * W0[(bh * dk + i) * dv + j];
                    expect(fabs(out[t * dv + j] - o) <= 1e-12 * (1.0 + fabs(o)), "dual form at eta = 0");
                }
            }
            free(q); free(k); free(v); free(eta); free(S0); free(M0); free(out); free(Sf); free(Mf); free(dout);
            free(dSf); free(dMf); free(dq); free(dkk); free(dvv); free(deta); free(dS0); free(dM0);
            free(dS); free(dM); free(Se); free(Me); free(W0);
        }
    printf("oracle driver: %d failures\n", fails);
    return fails ? 1 : 0;
}
