/*
 * dspark_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 *
 * Every array is host memory owned by the caller, row-major and contiguous.
 * Logits and Markov factors are passed widened to float (bf16 values widen
 * exactly); all internal arithmetic is double unless stated.
 * Return codes: ORC_OK (0) or a negative ORC_ERR_* value.
 */
#ifndef DSPARK_ORACLE_H
#define DSPARK_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_ALLOC -2
#define ORC_ERR_NOT_PREFIX -3

typedef struct {
    int32_t tok;        /* sampled token */
    int32_t degenerate; /* 1 when a residual had zero mass and p_t was used */
    double p;           /* weight of tok divided by the total weight */
    double lse;         /* log-normaliser of the row (draft: of f; final: of the target row) */
    double mass;        /* total weight S of the distribution sampled */
    double cdf_before;  /* C_{q-1}/S for the query token q, or -1 */
    double cdf_through; /* C_q/S for the query token q, or -1 */
    float u;            /* the uniform used */
} orc_row_out;

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float orc_uniform(uint64_t seed, uint32_t b, uint32_t k, uint32_t d);
void orc_uniform_batch(uint64_t seed, const uint32_t* b, const uint32_t* k, const uint32_t* d, int n, float* u);

int orc_inverse_cdf(const double* w, int n, float u, double* mass);
void orc_inverse_cdf_batch(const double* w, int n, const float* u, int m, int32_t* out);

double orc_logsumexp(const float* row, int V);
void orc_markov_logits(const float* L_row, const float* A, const float* Bm, int V, int r, int prev, double* f);
int orc_draft_row(const float* L_row, const float* A, const float* Bm, int V, int r, int prev, float u, int q,
                  orc_row_out* out);
int orc_markov_draft(const float* L, const float* A, const float* Bm, const int32_t* x0, int B, int gamma, int V,
                     int r, uint64_t seed, int32_t* tok, float* p, double* lse);

void orc_survival(const float* z, const float* T, int B, int gamma, float* theta);
void orc_rnn_state(const float* Wt, const float* h_prev, const float* a, int r, double* out);
int orc_markov_confidence(const float* A, const float* wc, const int32_t* x0, const int32_t* tok, const float* z0,
                          int B, int gamma, int V, int r, float* z);
int orc_select(const float* theta, int B, int gamma, int64_t budget, int32_t* len);
int orc_select_objective(const float* theta, int B, int gamma, const float* step_time, int n_time,
                         int64_t max_admit, int32_t* len, int64_t* admitted);
void orc_select_threshold(const float* theta, int B, int gamma, float tau, int32_t* len);

int orc_accept_scan(const float* T_b, const int32_t* tok_b, const float* pd_b, int ell, int V, uint64_t seed, int b,
                    double* pt, double* ratio, float* us);
int orc_final_token(const float* T_b, const float* L_b, const float* A, const float* Bm, int32_t x0_b,
                    const int32_t* tok_b, int ell, int a, int V, int r, uint64_t seed, int b, int q,
                    orc_row_out* out);
int orc_verify(const float* T, const float* L, const float* A, const float* Bm, const int32_t* x0,
               const int32_t* tok, const float* pd, const int32_t* len, int B, int gamma, int V, int r, uint64_t seed,
               int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p);

/* orc_markov_draft / orc_verify with the requests split over nthreads POSIX
 * threads; results identical to the one-thread calls. */
int orc_markov_draft_mt(const float* L, const float* A, const float* Bm, const int32_t* x0, int B, int gamma, int V,
                        int r, uint64_t seed, int32_t* tok, float* p, double* lse, int nthreads);
int orc_verify_mt(const float* T, const float* L, const float* A, const float* Bm, const int32_t* x0,
                  const int32_t* tok, const float* pd, const int32_t* len, int B, int gamma, int V, int r,
                  uint64_t seed, int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
