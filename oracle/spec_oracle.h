/*
 * spec_oracle.h -- fp64 CPU oracle of the draft-verification sampler.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
 *
 * Logits are row-major [requests][rows][V], read as the exact stored values
 * (fp32, or bf16 bit patterns widened exactly).  Outputs are per request;
 * entries past the emitted length are -1 (tokens) and 0 (log-probs).
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H
#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#ifdef __cplusplus
extern "C" {
#endif

void oracle_set_threads(int n);
int oracle_max_threads(void);

/* M[r], g[r] (lowest index of the max), S[r] = sum exp(l - M) for each row */
void oracle_row_stats(const void *x, int dtype, long rows, int V, double *M, int64_t *g, double *S);

/* T [B][K+1][V]; x [B][K]; outputs tok/tlp/blp [B][K+1], len/status/decisions [B] */
void oracle_greedy(const void *T, int dt, const int32_t *x, int B, int K, int V,
                   int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                   int32_t *out_status, int32_t *out_decisions);

/* T [B][K+1][V]; D [B][K][V]; u [B][K+1]; flag[b] = first position decided
 * by a near-tie or -1 */
void oracle_exact(const void *T, const void *D, int dt, const int32_t *x, const float *u,
                  int B, int K, int V, double eps_accept, double eps_sample,
                  int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                  int32_t *out_status, int32_t *out_flag, int32_t *out_decisions);

void oracle_relaxed(const void *T, int dt, const int32_t *x, const float *u, int B, int K, int V,
                    double tau, int top_k, double eps_accept, double eps_sample,
                    int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                    int32_t *out_status, int32_t *out_flag, int32_t *out_decisions);

/* T [B][N][V]; node_tok, parents [B][N]; num_nodes [B] or NULL;
 * out_path, out_tok, out_tlp, out_blp [B][N]; out_len, out_status [B] */
void oracle_tree(const void *T, int dt, const int32_t *node_tok, const int32_t *parents,
                 const int32_t *num_nodes, int B, int N, int V,
                 int32_t *out_path, int32_t *out_tok, int32_t *out_len, double *out_tlp,
                 double *out_blp, int32_t *out_status);

/* power rule: as oracle_exact's shapes, accept iff u_j < min(1, p/q)^alpha;
 * after a rejection n the sample is y ~ p_n */
void oracle_power(const void *T, const void *D, int dt, const int32_t *x, const float *u,
                  int B, int K, int V, double alpha, double eps_accept, double eps_sample,
                  int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                  int32_t *out_status, int32_t *out_flag, int32_t *out_decisions);

/* X [rows][V]; u [rows]; out_tok, out_logq, out_flag [rows]: one inverse-CDF
 * draw per row and its log-prob; flag 1 when u*Z lies within eps_sample*Z
 * of a CDF boundary */
void oracle_sample(const void *X, int dt, const float *u, long rows, int V, double eps_sample,
                   int32_t *out_tok, double *out_logq, int32_t *out_flag);

/* the weights w [B][V] and their sum Z [B] that a rule's terminal draw
 * inverts at first-rejection position n[b]: rule 0 exact (out_residual[b] = 1
 * when w = relu(p_n - q_n)), 1 target row n (relaxed, power), 2 the draft
 * sampler's row b of T */
void oracle_terminal_weights(int rule, const void *T, const void *D, int dt, const int32_t *n,
                             int B, int K, int V, double *out_w, double *out_Z,
                             int32_t *out_residual);

#ifdef __cplusplus
}
#endif
#endif
