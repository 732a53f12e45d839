/*
 * dspark_oracle.c -- plain CPU oracle of the DSpark per-step token path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never includes, links or calls it, and it shares no source with the GPU
 * library (not even the random-number generator).
 *
 * It is deliberately plain: sequential loops, double precision for every
 * floating-point quantity except where a single-precision result is part of
 * the definition (the survival product, the fp32 outputs), no SIMD, no
 * blocking, no fusion.  Each function names the passage it follows.
 *
 * Sources.  The method is arXiv 2607.05147, "DSpark: Confidence-Scheduled
 * Speculative Decoding with Semi-Autoregressive Generation".  The pages are
 * cited by their short names:
 *   [PL]  paperlayer.ai summary of 2607.05147 (Korean): section 2
 *         (background), 3.1 (semi-autoregressive generation), 3.2
 *         (confidence-scheduled verification), Appendix A (counterexample).
 *   [MF]  menfem.com knowledge-base note on DSpark: "Key Contributions"
 *         and "Methodology" (the acceptance rule, rank-256 Markov head).
 *   [WK]  llm-wiki.hwlabs.dev explainer no. 116: the Markov-head diagram and
 *         the definition of the prefix survival probability.
 * Philox-4x32-10 is the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), written here
 * from that paper's description of the S-box and key schedule.
 *
 * Readings of the pages that this file relies on (each also listed in the
 * design notes of the repository):
 *   - positions are 1-based, k = 1..gamma, as in [PL] Appendix A (x_1, c_2,
 *     Theta_0 = 1);
 *   - the Markov bias is exactly Delta = A[x_{k-1}] . Bm (rank-r factors),
 *     with x_0 the last committed token ([PL] 3.1, [MF] Methodology, [WK]);
 *   - sampling is at temperature 1 with no truncation, by inverse CDF over
 *     vocabulary index order with one uniform per event;
 *   - the CDF rule is strict: token = min{ j : C_j > u*S }, with a fallback to
 *     the last index of positive weight if rounding leaves no such j;
 *   - uniforms: key = (lo32 seed, hi32 seed), counter = (k, b, d, 0), output
 *     word 0, u = (w0 >> 8) * 2^-24; draws d = 0 draft, 1 accept,
 *     2 residual, 3 bonus;
 *   - the accept decision is taken in single precision: u < fl32(ratio),
 *     with ratio computed in double;
 *   - a degenerate residual (all max(0, p_t - p_d) == 0) falls back to p_t.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "dspark_oracle.h"

/* ------------------------------------------------------------------------ */
/* Philox-4x32-10 (SC'11).  Each round multiplies words 0 and 2 by the two   */
/* round constants, keeps the high and low halves, and mixes the high halves */
/* with the other two words and the round key; the key is advanced by the    */
/* two Weyl constants between rounds.                                        */
/* ------------------------------------------------------------------------ */
#define ORC_PHILOX_M0 0xD2511F53u
#define ORC_PHILOX_M1 0xCD9E8D57u
#define ORC_PHILOX_W0 0x9E3779B9u
#define ORC_PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += ORC_PHILOX_W0;
            k1 += ORC_PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)ORC_PHILOX_M0 * (uint64_t)x0;
        uint64_t p1 = (uint64_t)ORC_PHILOX_M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

float orc_uniform(uint64_t seed, uint32_t b, uint32_t k, uint32_t d)
{
    uint32_t ctr[4] = { k, b, d, 0u };
    uint32_t key[2] = { (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32) };
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    /* 24 high bits of word 0 scaled by 2^-24: exact in single precision. */
    return (float)(out[0] >> 8) * (1.0f / 16777216.0f);
}

void orc_uniform_batch(uint64_t seed, const uint32_t* b, const uint32_t* k, const uint32_t* d, int n, float* u)
{
    for (int i = 0; i < n; ++i) u[i] = orc_uniform(seed, b[i], k[i], d[i]);
}

/* ------------------------------------------------------------------------ */
/* Inverse-CDF sampling over index order.                                    */
/* ------------------------------------------------------------------------ */
static double orc_total(const double* w, int n)
{
    double s = 0.0;
    for (int j = 0; j < n; ++j) s += w[j];
    return s;
}

int orc_inverse_cdf(const double* w, int n, float u, double* mass)
{
    double S = orc_total(w, n);
    double tau = (double)u * S;
    double c = 0.0;
    int last_pos = -1;
    int pick = -1;
    for (int j = 0; j < n; ++j) {
        if (w[j] > 0.0) last_pos = j;
        c += w[j];
        if (pick < 0 && c > tau) pick = j;
    }
    if (pick < 0) pick = last_pos;
    if (mass) *mass = S;
    return pick;
}

void orc_inverse_cdf_batch(const double* w, int n, const float* u, int m, int32_t* out)
{
    for (int i = 0; i < m; ++i) out[i] = orc_inverse_cdf(w, n, u[i], NULL);
}

/* C_{q-1}/S and C_q/S for token q (left-to-right double sums). */
static void orc_bracket(const double* w, int n, int q, double S, double* before, double* through)
{
    double c = 0.0, cb = 0.0;
    for (int j = 0; j < n && j <= q; ++j) {
        cb = c;
        c += w[j];
    }
    *before = cb / S;
    *through = c / S;
}

/* ------------------------------------------------------------------------ */
/* Softmax pieces.                                                           */
/* ------------------------------------------------------------------------ */
static double orc_max(const double* f, int n)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (f[j] > m) m = f[j];
    return m;
}

double orc_logsumexp(const float* row, int V)
{
    double m = -INFINITY;
    for (int j = 0; j < V; ++j)
        if ((double)row[j] > m) m = (double)row[j];
    double s = 0.0;
    for (int j = 0; j < V; ++j) s += exp((double)row[j] - m);
    return m + log(s);
}

/* ------------------------------------------------------------------------ */
/* Markov head: f_j = L_j + sum_i A[prev][i] * Bm[i][j]  ([PL] 3.1: the       */
/* sequential module adds a transition bias chosen by the previously sampled  */
/* token to the backbone logits; [MF]: the transition is a rank-256           */
/* factorisation; [WK] diagram: final logits are L[i] + Delta[i]).            */
/* ------------------------------------------------------------------------ */
void orc_markov_logits(const float* L_row, const float* A, const float* Bm, int V, int r, int prev, double* f)
{
    for (int j = 0; j < V; ++j) f[j] = 0.0;
    const float* a = A + (size_t)prev * (size_t)r;
    for (int i = 0; i < r; ++i) {
        double ai = (double)a[i];
        const float* brow = Bm + (size_t)i * (size_t)V;
        for (int j = 0; j < V; ++j) f[j] += ai * (double)brow[j];
    }
    for (int j = 0; j < V; ++j) f[j] = (double)L_row[j] + f[j];
}

/* One draft position, conditioned on the token prev ([PL] 3.1; [WK]).       */
int orc_draft_row(const float* L_row, const float* A, const float* Bm, int V, int r, int prev, float u,
                  int q, orc_row_out* out)
{
    if (V <= 0 || r < 0 || prev < 0 || prev >= V) return ORC_ERR_ARG;
    double* f = (double*)malloc(sizeof(double) * (size_t)V);
    if (!f) return ORC_ERR_ALLOC;
    orc_markov_logits(L_row, A, Bm, V, r, prev, f);
    double m = orc_max(f, V);
    for (int j = 0; j < V; ++j) f[j] = exp(f[j] - m); /* f now holds the weights w_j */
    double S = 0.0;
    int tok = orc_inverse_cdf(f, V, u, &S);
    out->tok = tok;
    out->p = f[tok] / S;
    out->lse = m + log(S);
    out->mass = S;
    out->u = u;
    out->degenerate = 0;
    if (q >= 0 && q < V) orc_bracket(f, V, q, S, &out->cdf_before, &out->cdf_through);
    else out->cdf_before = out->cdf_through = -1.0;
    free(f);
    return ORC_OK;
}

/* gamma sequential draft steps for requests b0..b1-1 ([PL] 3.1: the        */
/* sequential stage samples left to right, each position conditioned on the */
/* token just sampled; x_0 is the last committed token).  Arrays are the    */
/* whole batch; b is the request index of the random-number counter.         */
static int orc_markov_draft_range(const float* L, const float* A, const float* Bm, const int32_t* x0, int b0, int b1,
                                  int gamma, int V, int r, uint64_t seed, int32_t* tok, float* p, double* lse)
{
    for (int b = b0; b < b1; ++b) {
        int prev = x0[b];
        for (int k = 1; k <= gamma; ++k) {
            orc_row_out o;
            const float* Lrow = L + ((size_t)b * (size_t)gamma + (size_t)(k - 1)) * (size_t)V;
            float u = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
            int rc = orc_draft_row(Lrow, A, Bm, V, r, prev, u, -1, &o);
            if (rc != ORC_OK) return rc;
            tok[b * gamma + (k - 1)] = o.tok;
            p[b * gamma + (k - 1)] = (float)o.p;
            lse[b * gamma + (k - 1)] = o.lse;
            prev = o.tok;
        }
    }
    return ORC_OK;
}

int orc_markov_draft(const float* L, const float* A, const float* Bm, const int32_t* x0, int B, int gamma, int V,
                     int r, uint64_t seed, int32_t* tok, float* p, double* lse)
{
    return orc_markov_draft_range(L, A, Bm, x0, 0, B, gamma, V, r, seed, tok, p, lse);
}

/* ------------------------------------------------------------------------ */
/* Survival ([PL] 3.2: the confidence head gives a per-position conditional  */
/* survival; sequential temperature scaling calibrates it position by        */
/* position; [WK]: the prefix survival is the probability that positions     */
/* 1..i are all accepted, i.e. the running product).  Single precision by    */
/* definition of the path: c = 1/(1+expf(-z/T_k)), Theta_k = Theta_{k-1}*c.  */
/* ------------------------------------------------------------------------ */
void orc_survival(const float* z, const float* T, int B, int gamma, float* theta)
{
    for (int b = 0; b < B; ++b) {
        float th = 1.0f;
        for (int k = 0; k < gamma; ++k) {
            float t = z[b * gamma + k] / T[k];
            float e = expf(-t);
            float c = 1.0f / (1.0f + e);
            th = th * c;
            theta[b * gamma + k] = th;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* RNN sequential head (menfem.com note, Key Contributions: the second head    */
/* variant keeps the whole in-block prefix in a recurrent state instead of    */
/* the first-order Markov dependency).  Reading taken here: a state          */
/* h_k = tanh(W h_{k-1} + A[x_{k-1}]), h_0 = 0, replaces A[x_{k-1}] in the    */
/* bias, Delta_k = h_k . Bm.  Wt is W transposed: Wt[j][i] multiplies         */
/* h_{k-1}[j] into output i.  This computes one update in double:            */
/* out[i] = tanh(sum_j Wt[j][i] h_prev[j] + a[i]).                           */
/* ------------------------------------------------------------------------ */
void orc_rnn_state(const float* Wt, const float* h_prev, const float* a, int r, double* out)
{
    for (int i = 0; i < r; ++i) {
        double s = a[i];
        for (int j = 0; j < r; ++j) s += (double)Wt[(size_t)j * r + i] * (double)h_prev[j];
        out[i] = tanh(s);
    }
}

/* ------------------------------------------------------------------------ */
/* Markov-conditioned confidence logit (paperlayer.ai summary, Appendix A: the */
/* Markov confidence head sees the previously sampled token, so c_2 depends on */
/* x_1; menfem.com note: the confidence head is linear).  Reading taken here:  */
/* z[b][k] = z0[b][k] + <A[x_{k-1}], wc>, the backbone part z0 an input and    */
/* the token part the dot product of the token's Markov code A[x] (the same    */
/* rows the Markov head uses) with a weight vector wc[r]; x_0 = x0[b],         */
/* x_{k-1} = tok[b][k-2].  Summed in double, rounded once to float.           */
/* ------------------------------------------------------------------------ */
int orc_markov_confidence(const float* A, const float* wc, const int32_t* x0, const int32_t* tok, const float* z0,
                          int B, int gamma, int V, int r, float* z)
{
    for (int b = 0; b < B; ++b)
        for (int k = 1; k <= gamma; ++k) {
            int x = k == 1 ? x0[b] : tok[b * gamma + (k - 2)];
            if (x < 0 || x >= V) return ORC_ERR_ARG;
            double s = z0[b * gamma + (k - 1)];
            for (int j = 0; j < r; ++j) s += (double)A[(size_t)x * r + j] * (double)wc[j];
            z[b * gamma + (k - 1)] = (float)s;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Selection ([MF] "Hardware-aware prefix scheduler": candidates are sorted  */
/* globally by cumulative survival and admitted greedily; here the budget   */
/* form: admit the first min(budget, B*gamma) of the order (Theta desc,     */
/* request asc, position asc)).                                             */
/* ------------------------------------------------------------------------ */
typedef struct {
    float theta;
    int b;
    int k;
} orc_cand;

static int orc_cand_cmp(const void* pa, const void* pb)
{
    const orc_cand* x = (const orc_cand*)pa;
    const orc_cand* y = (const orc_cand*)pb;
    if (x->theta > y->theta) return -1;
    if (x->theta < y->theta) return 1;
    if (x->b != y->b) return x->b < y->b ? -1 : 1;
    if (x->k != y->k) return x->k < y->k ? -1 : 1;
    return 0;
}

int orc_select(const float* theta, int B, int gamma, int64_t budget, int32_t* len)
{
    if (B < 0 || gamma <= 0 || budget < 0) return ORC_ERR_ARG;
    int64_t n = (int64_t)B * gamma;
    int64_t admit = budget < n ? budget : n;
    for (int b = 0; b < B; ++b) len[b] = 0;
    if (n == 0) return ORC_OK;
    orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)n);
    if (!c) return ORC_ERR_ALLOC;
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < gamma; ++k) {
            float t = theta[b * gamma + k];
            if (isnan(t)) {
                free(c);
                return ORC_ERR_ARG;
            }
            c[b * gamma + k].theta = t;
            c[b * gamma + k].b = b;
            c[b * gamma + k].k = k;
        }
    qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
    /* admitted flags, to check that each admitted set is a per-request prefix */
    unsigned char* adm = (unsigned char*)calloc((size_t)n, 1);
    if (!adm) {
        free(c);
        return ORC_ERR_ALLOC;
    }
    for (int64_t i = 0; i < admit; ++i) adm[c[i].b * gamma + c[i].k] = 1;
    int rc = ORC_OK;
    for (int b = 0; b < B; ++b) {
        int l = 0;
        while (l < gamma && adm[b * gamma + l]) ++l;
        for (int k = l; k < gamma; ++k)
            if (adm[b * gamma + k]) rc = ORC_ERR_NOT_PREFIX;
        len[b] = l;
    }
    free(adm);
    free(c);
    return rc;
}

/* Objective-based admission: the scheduler's greedy global order (the same
 * order as orc_select) with incremental admission and early stopping
 * (menfem.com note, Key Contributions, hardware-aware prefix scheduler;
 * paperlayer.ai summary, section 5.2 and Appendix A).  Reading taken here:
 * the objective after m admissions is the expected number of emitted tokens
 * per unit of verification time,
 *     J(m) = E(m) / t[B + m],   E(m) = B + sum of the m first Theta,
 * (every request emits one token whatever happens, Theta_0 = 1; the batch
 * verifies the admitted drafts plus one position per request), where t[n]
 * is the engine's time for a verification batch of n tokens.  Candidates
 * are admitted in order while J does not drop; the first candidate whose
 * admission would make J strictly smaller stops the scan (early stopping),
 * and at most max_admit are admitted.
 * Arithmetic fixed here so that two implementations take the same decisions:
 * Theta is clamped into [0, 1] (NaN counts as 0) and E is kept in integer
 * units of 2^-36 (each term floor(Theta * 2^36), exact below 2^53); the test
 * J(m+1) < J(m) is E(m+1) * t[B+m] < E(m) * t[B+m+1], both products in
 * double from the exact E and the float t.  Requires n_time > B + min(max_admit, B*gamma).
 * *admitted receives the number admitted; len[b] the leading run of admitted
 * positions of row b (ORC_ERR_NOT_PREFIX if an admitted set is not a prefix). */
int orc_select_objective(const float* theta, int B, int gamma, const float* step_time, int n_time,
                         int64_t max_admit, int32_t* len, int64_t* admitted)
{
    if (B < 0 || gamma <= 0 || max_admit < 0) return ORC_ERR_ARG;
    int64_t n = (int64_t)B * gamma;
    int64_t cap = max_admit < n ? max_admit : n;
    if ((int64_t)n_time <= (int64_t)B + cap) return ORC_ERR_ARG;
    for (int b = 0; b < B; ++b) len[b] = 0;
    *admitted = 0;
    if (n == 0) return ORC_OK;
    orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)n);
    if (!c) return ORC_ERR_ALLOC;
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < gamma; ++k) {
            float t = theta[b * gamma + k];
            if (isnan(t)) {
                free(c);
                return ORC_ERR_ARG;
            }
            c[b * gamma + k].theta = t;
            c[b * gamma + k].b = b;
            c[b * gamma + k].k = k;
        }
    qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
    const double unit = 68719476736.0; /* 2^36 */
    int64_t E = (int64_t)B * (int64_t)68719476736LL;
    int64_t m = 0;
    while (m < cap) {
        float th = c[m].theta;
        if (!(th > 0.0f)) th = 0.0f;
        if (th > 1.0f) th = 1.0f;
        int64_t q = (int64_t)floor((double)th * unit);
        int64_t E1 = E + q;
        double keep_new = (double)E1 * (double)step_time[B + m];
        double keep_old = (double)E * (double)step_time[B + m + 1];
        if (keep_new < keep_old) break; /* J(m+1) < J(m): stop */
        E = E1;
        ++m;
    }
    *admitted = m;
    unsigned char* adm = (unsigned char*)calloc((size_t)n, 1);
    if (!adm) {
        free(c);
        return ORC_ERR_ALLOC;
    }
    for (int64_t i = 0; i < m; ++i) adm[c[i].b * gamma + c[i].k] = 1;
    int rc = ORC_OK;
    for (int b = 0; b < B; ++b) {
        int l = 0;
        while (l < gamma && adm[b * gamma + l]) ++l;
        for (int k = l; k < gamma; ++k)
            if (adm[b * gamma + k]) rc = ORC_ERR_NOT_PREFIX;
        len[b] = l;
    }
    free(adm);
    free(c);
    return rc;
}

/* Static-threshold admission (paperlayer.ai summary, section 4.3): a
 * position is verified when its prefix survival is at least tau; len[b] is
 * the leading run of positions with Theta >= tau (NaN stops the run). */
void orc_select_threshold(const float* theta, int B, int gamma, float tau, int32_t* len)
{
    for (int b = 0; b < B; ++b) {
        int l = 0;
        while (l < gamma && theta[b * gamma + l] >= tau) ++l;
        len[b] = l;
    }
}

/* ------------------------------------------------------------------------ */
/* Verification ([MF] Methodology: the k-th drafted token is kept with       */
/* probability min(1, p_t(x_k)/p_d(x_k)) and the first rejection drops every */
/* later token; [PL] 2: left-to-right verification in one target pass).      */
/* ------------------------------------------------------------------------ */
int orc_accept_scan(const float* T_b, const int32_t* tok_b, const float* pd_b, int ell, int V, uint64_t seed, int b,
                    double* pt, double* ratio, float* us)
{
    int a = -1;
    for (int k = 1; k <= ell; ++k) {
        const float* row = T_b + (size_t)(k - 1) * (size_t)V;
        int x = tok_b[k - 1];
        if (x < 0 || x >= V) return ORC_ERR_ARG;
        double lse = orc_logsumexp(row, V);
        double ptk = exp((double)row[x] - lse);
        double rk = ptk / (double)pd_b[k - 1];
        float u = orc_uniform(seed, (uint32_t)b, (uint32_t)k, 1u);
        if (pt) pt[k - 1] = ptk;
        if (ratio) ratio[k - 1] = rk;
        if (us) us[k - 1] = u;
        int accept = u < (float)rk;
        if (!accept && a < 0) a = k - 1;
    }
    if (a < 0) a = ell;
    return a;
}

/* The token emitted after the a accepted ones: the residual at the first    */
/* rejected position k* = a+1, normalise(max(0, p_t - p_d)) with the draft   */
/* row recomputed from its conditioning token; or, when all ell verified     */
/* tokens were accepted (including ell = 0, [PL] Appendix A: the target      */
/* then produces a fresh token), a sample of p_t at position ell+1.          */
int orc_final_token(const float* T_b, const float* L_b, const float* A, const float* Bm, int32_t x0_b,
                    const int32_t* tok_b, int ell, int a, int V, int r, uint64_t seed, int b, int q,
                    orc_row_out* out)
{
    if (a < 0 || a > ell) return ORC_ERR_ARG;
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!w) return ORC_ERR_ALLOC;
    int rc = ORC_OK;
    out->degenerate = 0;
    if (a < ell) {
        int ks = a + 1; /* first rejected position, 1-based */
        int prev = ks == 1 ? x0_b : tok_b[ks - 2];
        if (prev < 0 || prev >= V) {
            free(w);
            return ORC_ERR_ARG;
        }
        const float* trow = T_b + (size_t)(ks - 1) * (size_t)V;
        const float* lrow = L_b + (size_t)(ks - 1) * (size_t)V;
        double* f = (double*)malloc(sizeof(double) * (size_t)V);
        if (!f) {
            free(w);
            return ORC_ERR_ALLOC;
        }
        orc_markov_logits(lrow, A, Bm, V, r, prev, f);
        double md = orc_max(f, V);
        double sd = 0.0;
        for (int j = 0; j < V; ++j) sd += exp(f[j] - md);
        double lse_d = md + log(sd);
        double lse_t = orc_logsumexp(trow, V);
        for (int j = 0; j < V; ++j) {
            double ptj = exp((double)trow[j] - lse_t);
            double pdj = exp(f[j] - lse_d);
            double d = ptj - pdj;
            w[j] = d > 0.0 ? d : 0.0;
        }
        free(f);
        if (orc_total(w, V) == 0.0) {
            out->degenerate = 1;
            double mt = -INFINITY;
            for (int j = 0; j < V; ++j)
                if ((double)trow[j] > mt) mt = (double)trow[j];
            for (int j = 0; j < V; ++j) w[j] = exp((double)trow[j] - mt);
        }
        out->u = orc_uniform(seed, (uint32_t)b, (uint32_t)ks, 2u);
        out->lse = lse_t;
    } else {
        int kb = ell + 1; /* bonus position, 1-based; target row index ell */
        const float* trow = T_b + (size_t)ell * (size_t)V;
        double mt = -INFINITY;
        for (int j = 0; j < V; ++j)
            if ((double)trow[j] > mt) mt = (double)trow[j];
        for (int j = 0; j < V; ++j) w[j] = exp((double)trow[j] - mt);
        out->u = orc_uniform(seed, (uint32_t)b, (uint32_t)kb, 3u);
        out->lse = mt + log(orc_total(w, V));
    }
    double S = 0.0;
    int tok = orc_inverse_cdf(w, V, out->u, &S);
    out->tok = tok;
    out->mass = S;
    out->p = w[tok] / S;
    if (q >= 0 && q < V) orc_bracket(w, V, q, S, &out->cdf_before, &out->cdf_through);
    else out->cdf_before = out->cdf_through = -1.0;
    free(w);
    return rc;
}

/* Verification of requests b0..b1-1 (whole-batch arrays). */
static int orc_verify_range(const float* T, const float* L, const float* A, const float* Bm, const int32_t* x0,
                            const int32_t* tok, const float* pd, const int32_t* len, int b0, int b1, int gamma, int V,
                            int r, uint64_t seed, int32_t* accepted, int32_t* out_tok, int32_t* n_out,
                            float* target_p)
{
    double* pt = (double*)malloc(sizeof(double) * (size_t)(gamma > 0 ? gamma : 1));
    if (!pt) return ORC_ERR_ALLOC;
    for (int b = b0; b < b1; ++b) {
        int ell = len[b];
        if (ell < 0 || ell > gamma) {
            free(pt);
            return ORC_ERR_ARG;
        }
        const float* T_b = T + (size_t)b * (size_t)(gamma + 1) * (size_t)V;
        const float* L_b = L + (size_t)b * (size_t)gamma * (size_t)V;
        const int32_t* tok_b = tok + (size_t)b * (size_t)gamma;
        int a = orc_accept_scan(T_b, tok_b, pd + (size_t)b * gamma, ell, V, seed, b, pt, NULL, NULL);
        if (a < 0) {
            free(pt);
            return a;
        }
        orc_row_out o;
        int rc = orc_final_token(T_b, L_b, A, Bm, x0[b], tok_b, ell, a, V, r, seed, b, -1, &o);
        if (rc != ORC_OK) {
            free(pt);
            return rc;
        }
        for (int k = 0; k <= gamma; ++k) out_tok[b * (gamma + 1) + k] = -1;
        for (int k = 0; k < a; ++k) out_tok[b * (gamma + 1) + k] = tok_b[k];
        out_tok[b * (gamma + 1) + a] = o.tok;
        accepted[b] = a;
        n_out[b] = a + 1;
        if (target_p)
            for (int k = 0; k < gamma; ++k) target_p[b * gamma + k] = k < ell ? (float)pt[k] : 0.0f;
    }
    free(pt);
    return ORC_OK;
}

int orc_verify(const float* T, const float* L, const float* A, const float* Bm, const int32_t* x0,
               const int32_t* tok, const float* pd, const int32_t* len, int B, int gamma, int V, int r, uint64_t seed,
               int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p)
{
    return orc_verify_range(T, L, A, Bm, x0, tok, pd, len, 0, B, gamma, V, r, seed, accepted, out_tok, n_out,
                            target_p);
}

/* ------------------------------------------------------------------------ */
/* The same two calls with the requests split into contiguous ranges over   */
/* POSIX threads (requests are independent in the draft and the verify;     */
/* only the selection couples them).  Each thread runs the sequential code  */
/* above on its own range, so the results are those of the one-thread call */
/* bit for bit.  nthreads < 1 means 1.                                      */
/* ------------------------------------------------------------------------ */
typedef struct {
    const float *T, *L, *A, *Bm, *pd;
    const int32_t *x0, *tok, *len;
    int b0, b1, gamma, V, r;
    uint64_t seed;
    int32_t *tok_out, *accepted, *out_tok, *n_out;
    float *p, *target_p;
    double* lse;
    int rc;
} orc_job;

static void* orc_draft_job(void* arg)
{
    orc_job* j = (orc_job*)arg;
    j->rc = orc_markov_draft_range(j->L, j->A, j->Bm, j->x0, j->b0, j->b1, j->gamma, j->V, j->r, j->seed, j->tok_out,
                                   j->p, j->lse);
    return NULL;
}

static void* orc_verify_job(void* arg)
{
    orc_job* j = (orc_job*)arg;
    j->rc = orc_verify_range(j->T, j->L, j->A, j->Bm, j->x0, j->tok, j->pd, j->len, j->b0, j->b1, j->gamma, j->V,
                             j->r, j->seed, j->accepted, j->out_tok, j->n_out, j->target_p);
    return NULL;
}

static int orc_run_jobs(orc_job* proto, int B, int nthreads, void* (*fn)(void*))
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = B > 0 ? B : 1;
    orc_job* jobs = (orc_job*)malloc(sizeof(orc_job) * (size_t)nthreads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    unsigned char* running = (unsigned char*)calloc((size_t)nthreads, 1);
    if (!jobs || !th || !running) {
        free(jobs);
        free(th);
        free(running);
        return ORC_ERR_ALLOC;
    }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *proto;
        jobs[i].b0 = (int)((int64_t)B * i / nthreads);
        jobs[i].b1 = (int)((int64_t)B * (i + 1) / nthreads);
        jobs[i].rc = ORC_OK;
        /* the last range runs on the calling thread, as does any whose thread fails to start */
        if (i + 1 < nthreads && pthread_create(&th[i], NULL, fn, &jobs[i]) == 0) running[i] = 1;
        else fn(&jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        if (running[i]) pthread_join(th[i], NULL);
    int rc = ORC_OK;
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].rc != ORC_OK && rc == ORC_OK) rc = jobs[i].rc;
    free(jobs);
    free(th);
    free(running);
    return rc;
}

int orc_markov_draft_mt(const float* L, const float* A, const float* Bm, const int32_t* x0, int B, int gamma, int V,
                        int r, uint64_t seed, int32_t* tok, float* p, double* lse, int nthreads)
{
    orc_job j;
    memset(&j, 0, sizeof(j));
    j.L = L; j.A = A; j.Bm = Bm; j.x0 = x0; j.gamma = gamma; j.V = V; j.r = r; j.seed = seed;
    j.tok_out = tok; j.p = p; j.lse = lse;
    return orc_run_jobs(&j, B, nthreads, orc_draft_job);
}

int orc_verify_mt(const float* T, const float* L, const float* A, const float* Bm, const int32_t* x0,
                  const int32_t* tok, const float* pd, const int32_t* len, int B, int gamma, int V, int r,
                  uint64_t seed, int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p, int nthreads)
{
    orc_job j;
    memset(&j, 0, sizeof(j));
    j.T = T; j.L = L; j.A = A; j.Bm = Bm; j.x0 = x0; j.tok = tok; j.pd = pd; j.len = len; j.gamma = gamma; j.V = V;
    j.r = r; j.seed = seed; j.accepted = accepted; j.out_tok = out_tok; j.n_out = n_out; j.target_p = target_p;
    return orc_run_jobs(&j, B, nthreads, orc_verify_job);
}
