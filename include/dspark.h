/*
 * dspark.h -- C ABI of libdspark, the MI355X (gfx950) implementation of the
 * DSpark per-step token path: semi-autoregressive Markov draft, confidence
 * scheduling, and exact rejection-sampling verification.
 *
 * Method: arXiv 2607.05147, "DSpark: Confidence-Scheduled Speculative
 * Decoding with Semi-Autoregressive Generation".  Pages cited below:
 *   paperlayer.ai summary (Korean) of 2607.05147 -- sections 2, 3.1, 3.2 and
 *     Appendix A;
 *   menfem.com knowledge-base note on DSpark -- "Key Contributions" and
 *     "Methodology";
 *   llm-wiki.hwlabs.dev explainer no. 116 -- the Markov-head diagram and the
 *     prefix-survival definition.
 *
 * Conventions shared by every call
 *   - Every pointer except `stream` is DEVICE memory owned by the caller,
 *     row-major and contiguous.  The library allocates nothing, keeps no state
 *     between calls (the measurement-only timing hook at the end aside) and
 *     never synchronises the host; a call only validates its arguments and
 *     enqueues fixed-shape kernels on `stream` (a hipStream_t; NULL = the null
 *     stream), so a sequence of calls can be captured in a HIP graph (see
 *     seed_dev below for fresh random draws on each replay).  Inputs must stay alive until the stream has
 *     passed the work.
 *   - Positions are 1-based, k = 1..gamma; array index k-1.
 *   - dtype: DSPARK_BF16 (bfloat16 logits and Markov factors) or DSPARK_F32;
 *     logits L, target logits Tgt, A and Bm share it.  All arithmetic is at
 *     least fp32: the rank-r product accumulates in fp32, exponentials are
 *     fp32, sums within a 64-column (bf16) or 128-column (fp32) tile or a
 *     16-byte vector are fp32, and sums across tiles, chunks and vectors are
 *     fp64.
 *   - Limits: 1 <= gamma <= 16; B*gamma <= 16384; V a multiple of 8 in
 *     [8, 2^24]; r a multiple of 8 in [8, 256].  L, Tgt, A and Bm must be
 *     16-byte aligned.  B == 0 is a no-op that returns DSPARK_OK.
 *   - Randomness: every uniform is U(seed, b, k, d) = top 24 bits of word 0 of
 *     Philox-4x32-10 (Salmon et al., SC'11) with key (lo32 seed, hi32 seed)
 *     and counter (k, b, d, 0), times 2^-24.  Draw d = 0 draft sample,
 *     1 accept test, 2 residual sample, 3 bonus sample.  A step is therefore a
 *     pure function of its inputs and the seed.
 *   - Seed: the calls that draw uniforms take `uint64_t seed` and
 *     `const uint64_t* seed_dev`.  With seed_dev == NULL the seed is `seed`,
 *     fixed at enqueue time (and therefore fixed inside a captured graph:
 *     every replay would draw the same uniforms).  With seed_dev set (device
 *     memory, 8-byte aligned) `seed` is ignored and each kernel reads the seed
 *     from *seed_dev when it runs, so a graph replayed after the caller has
 *     written a new value there (e.g. one per decoding step) draws new
 *     uniforms.  The value must not change while the call's kernels run.
 *   - Sampling is at temperature 1 by inverse CDF over vocabulary index
 *     order: token = min{ j : w_0 + ... + w_j > u * S }.
 *   - Errors: a negative return means nothing was enqueued;
 *     dspark_last_error() gives a message (thread-local).  Token ids given by
 *     the caller (x0, draft_tok) must lie in [0, V); out-of-range ids are
 *     clamped for memory safety, with undefined sampling results.  A launch
 *     failure returns DSPARK_ERR_HIP; faults during execution surface at the
 *     caller's next synchronisation.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 };

enum {
    DSPARK_OK = 0,
    DSPARK_ERR_INVALID_ARG = -1, /* null pointer, negative size or budget, misalignment */
    DSPARK_ERR_UNSUPPORTED = -2, /* dtype or a size outside the limits above */
    DSPARK_ERR_WORKSPACE = -3,   /* ws_bytes < dspark_workspace_size(...) */
    DSPARK_ERR_HIP = -4          /* a HIP launch or event call failed */
};

/* Library version string (static storage). */
const char* dspark_version(void);

/* Message for the last non-OK return on this thread ("" if none). */
const char* dspark_last_error(void);

/*
 * Bytes of device workspace that dspark_markov_draft and dspark_verify need
 * for these sizes (the larger of the two; one buffer serves both).  Returns 0
 * for invalid sizes.  The workspace holds per-tile softmax partials and the
 * verifier's bookkeeping; its contents need no initialisation and are
 * meaningless between calls.  Calls on different streams need different
 * workspaces.
 */
size_t dspark_workspace_size(int B, int gamma, int V, int r);

/*
 * dspark_markov_draft -- gamma sequential draft steps (paperlayer.ai summary,
 * section 3.1: the parallel backbone gives all logits, the sequential module
 * samples left to right conditioning each position on the token just sampled;
 * menfem.com note: Markov head with a rank-256 low-rank transition;
 * llm-wiki.hwlabs.dev diagram: final logits are L[i] + Delta[i]).
 *
 * For every request b and k = 1..gamma:
 *     f   = L[b][k-1][:] + A[x_{k-1}][:] . Bm        (x_0 = x0[b])
 *     x_k = inverse-CDF sample of softmax(f) with u = U(seed, b, k, 0)
 *
 *   L          [B][gamma][V]  backbone draft logits (dtype)
 *   A          [V][r]         Markov factor, row x is the conditioning code of token x
 *   Bm         [r][V]         Markov factor
 *   x0         [B] int32      last committed token of each request
 *   draft_tok  [B][gamma] int32   out: x_1..x_gamma
 *   draft_p    [B][gamma] f32     out: p_d(x_k), the exact softmax probability
 *                                 of the drawn token (required by the
 *                                 verifier: paperlayer.ai summary, section 6)
 *   draft_lse  [B][gamma] f64     out: log sum_j exp(f_j); kept in double so the
 *                                 verifier can rebuild p_d over the vocabulary
 *   seed, seed_dev  the Philox seed (see the conventions above)
 *   ws         workspace of at least dspark_workspace_size(B, gamma, V, r) bytes
 */
int dspark_markov_draft(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B, int gamma,
                        int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok, float* draft_p,
                        double* draft_lse, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_markov_draft_noalloc -- dspark_markov_draft for callers that cannot
 * allocate or pass device memory for a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, outputs, limits and errors as dspark_markov_draft, without
 * ws/ws_bytes: the draft's per-tile softmax partials, its A-row hand-over
 * and (B > 256) the partials' per-slot aggregates live in a static device
 * array of the library (32 MiB per device, held until the process ends),
 * enough for B * ceil(V/64) * 8 + ceil(B/16) * 8192 (+ B * 2048 when
 * B > 256) bytes (e.g. B = 256 at V up to ~1M, B = 1024 at V = 129280).  Larger sizes return
 * DSPARK_ERR_WORKSPACE with nothing enqueued.  The call allocates nothing
 * (no hipMalloc/hipFree, no allocating library call); its first call on a
 * device looks up that device's copy of the array.  All calls on one device
 * share the array, whose contents need no initialisation: calls that overlap
 * in time on one device (different streams, or different threads without
 * ordering) race and give undefined results.
 */
int dspark_markov_draft_noalloc(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                                int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok,
                                float* draft_p, double* draft_lse, void* stream);

/*
 * dspark_markov_draft_conf -- dspark_markov_draft plus the Markov-conditioned
 * confidence logits, fused into the draft steps (paperlayer.ai summary,
 * Appendix A: the Markov confidence head sees the previously sampled token,
 * so the survival of position 2 depends on x_1; menfem.com note: the
 * confidence head is linear).  Draft outputs are exactly those of
 * dspark_markov_draft; in addition, for k = 1..gamma,
 *     z_out[b][k-1] = z0[b][k-1] + sum_j A[x_{k-1}][j] * wc[j]   (fp32)
 * (x_0 = x0[b]), the token part being the conditioning code of the token the
 * step conditions on (the same rows of A the Markov head uses) dotted with
 * the head's weight vector.  z_out feeds dspark_schedule* as z.
 *
 *   z0     [B][gamma] f32   backbone part of the confidence logit (input)
 *   wc     [r] (dtype)      confidence weights on the Markov code
 *   z_out  [B][gamma] f32   out
 * Other arguments, limits and errors as dspark_markov_draft (z0, wc, z_out
 * must be non-null when B > 0).
 */
int dspark_markov_draft_conf(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, const float* z0,
                             const void* wc, int32_t* draft_tok, float* draft_p, double* draft_lse, float* z_out,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_markov_draft_sched -- dspark_markov_draft followed by
 * dspark_schedule(z, temps, B, gamma, budget, survival, verify_len), in one
 * call.  Given z as an input (not the Markov-conditioned z of
 * dspark_markov_draft_conf, which depends on the sampled tokens: paperlayer.ai
 * summary, Appendix A), the budget schedule needs nothing the draft steps
 * produce, and it runs beside them, as the production scheduler runs
 * asynchronously to drafting (paperlayer.ai summary, section 5.2): with bf16
 * logits and B*gamma <= 7680 it runs as one extra workgroup of a draft
 * launch -- of the first tile launch when B <= 256 and the tiles spread over
 * one workgroup fewer need no more tiles per workgroup, else of the last
 * step's locate launch when V <= 262144 (at most 4096 tiles of 64 columns);
 * otherwise it is launched after the draft steps.  Outputs
 * are bit-identical to the two separate calls in either case.
 *
 *   z, temps, budget, survival, verify_len  as in dspark_schedule, except that
 *              z and temps must be non-null (no given-survival form)
 * Other arguments, limits and errors as dspark_markov_draft and
 * dspark_schedule; on an argument error nothing is enqueued.
 */
int dspark_markov_draft_sched(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                              int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, const float* z,
                              const float* temps, int64_t budget, int32_t* draft_tok, float* draft_p,
                              double* draft_lse, float* survival, int32_t* verify_len, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * dspark_rnn_draft -- the draft steps with the RNN sequential head instead of
 * the Markov head (menfem.com note, Key Contributions: the head variant that
 * keeps the whole in-block prefix history in a recurrent state).  Before
 * draft step k the state
 *     h_k = tanh(W h_{k-1} + A[x_{k-1}]),  h_0 = 0  (fp32, then rounded to dtype)
 * is written to H[b][k-1][:], and it replaces A[x_{k-1}] in the bias:
 *     f = L[b][k-1][:] + h_k . Bm,   x_k = inverse-CDF sample of softmax(f).
 * Everything else (sampling, p_d, lse_d, limits, errors) as
 * dspark_markov_draft.
 *
 *   Wt  [r][r] (dtype)        W transposed: Wt[j][i] multiplies h_{k-1}[j]
 *                             into output i; 16-byte aligned
 *   H   [B][gamma][r] (dtype) out: the states, 16-byte aligned; the verifier
 *                             needs them (dspark_rnn_verify)
 */
int dspark_rnn_draft(int dtype, const void* L, const void* A, const void* Bm, const void* Wt, const int32_t* x0, int B,
                     int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok,
                     float* draft_p, double* draft_lse, void* H, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_schedule -- confidence-scheduled verify lengths (paperlayer.ai
 * summary, section 3.2; menfem.com note, "Hardware-aware prefix scheduler";
 * llm-wiki.hwlabs.dev: prefix survival = probability that positions 1..i are
 * all accepted).
 *
 *   c[b][k]     = 1 / (1 + exp(-z[b][k-1] / temps[k-1]))   (fp32; sequential
 *                 temperature scaling, one temperature per position)
 *   Theta[b][k] = Theta[b][k-1] * c[b][k], Theta[b][0] = 1 (fp32, left to right)
 *   Admit the first min(budget, B*gamma) candidates of the order
 *   (Theta desc, b asc, k asc); verify_len[b] = number admitted in row b.
 * Because Theta is non-increasing along a row, the admitted positions of a
 * request are always a prefix 1..verify_len[b], and whether (b, k) is admitted
 * never depends on the survival of later positions (non-anticipation,
 * paperlayer.ai summary, Appendix A).
 *
 *   z          [B][gamma] f32 confidence logits, or NULL: then `survival` is
 *              read as the input Theta (must be in [0, 1], non-increasing
 *              along each row, no NaN)
 *   temps      [gamma] f32 STS temperatures (> 0); ignored when z is NULL
 *   budget     number of draft tokens that may be verified (>= 0; values
 *              above B*gamma are clamped)
 *   survival   [B][gamma] f32: out Theta (or in, see z)
 *   verify_len [B] int32 out, in [0, gamma]
 */
int dspark_schedule(const float* z, const float* temps, int B, int gamma, int64_t budget, float* survival,
                    int32_t* verify_len, void* stream);

/*
 * dspark_schedule_objective -- objective-based admission: the scheduler's
 * greedy global order with incremental batch admission and early stopping
 * (menfem.com note, "Hardware-aware prefix scheduler"; paperlayer.ai summary,
 * section 5.2: verification budget routed by an engine throughput profile,
 * and Appendix A: early stopping keeps admission non-anticipating).
 *
 * Survivals as in dspark_schedule.  Candidates are taken in the order
 * (Theta desc, b asc, k asc); with m admitted the objective is the expected
 * number of emitted tokens per unit of verification time
 *     J(m) = E(m) / step_time[B + m],   E(m) = B + sum of the m first Theta
 * (each request emits one token in any case; the verification batch holds
 * the admitted drafts plus one position per request).  Candidates are
 * admitted while J does not drop; the first one whose admission would make
 * J strictly smaller ends the scan, and at most max_admit are admitted.
 * Reproducible arithmetic: Theta clamped into [0, 1]; E in integer units of
 * 2^-36 (each term floor(Theta * 2^36)); the test J(m+1) < J(m) is
 * E(m+1) * step_time[B+m] < E(m) * step_time[B+m+1] in double.
 *
 *   step_time  [n_time] f32 device array: time of a verification batch of n
 *              tokens (any unit, > 0, finite); n_time must exceed
 *              B + min(max_admit, B*gamma), else DSPARK_ERR_INVALID_ARG
 *   max_admit  upper bound on admitted drafts (>= 0)
 *   survival, verify_len, z, temps: as in dspark_schedule (given survivals
 *              must not be NaN)
 * One workgroup; B*gamma <= 16384.  Enqueues one kernel on `stream`.
 */
int dspark_schedule_objective(const float* z, const float* temps, int B, int gamma, const float* step_time,
                              int n_time, int64_t max_admit, float* survival, int32_t* verify_len, void* stream);

/*
 * dspark_schedule_threshold -- static confidence threshold (paperlayer.ai
 * summary, section 4.3: positions whose prefix survival falls below a fixed
 * threshold are not verified).  verify_len[b] = the number of leading
 * positions k = 1, 2, ... with Theta[b][k] >= tau (a NaN ends the run).
 * Survivals as in dspark_schedule.  One thread per request.
 */
int dspark_schedule_threshold(const float* z, const float* temps, int B, int gamma, float tau, float* survival,
                              int32_t* verify_len, void* stream);

/*
 * dspark_verify -- exact rejection sampling (menfem.com note, Methodology:
 * token x_k is kept with probability min(1, p_t(x_k)/p_d(x_k)) and the first
 * rejection drops all later tokens; paperlayer.ai summary, section 2).
 *
 * For request b with ell = verify_len[b], for k = 1..ell in order:
 *     p_t(x_k) = softmax(Tgt[b][k-1][:])[x_k];  accept iff
 *     U(seed, b, k, 1) < fl32(p_t(x_k) / draft_p[b][k-1]); stop at the first
 *     rejection k*.
 * accepted[b] = a = k* - 1 (or ell).  Then one more token:
 *   - rejection at k*: sample normalise(max(0, p_t - p_d)) at position k*, the
 *     draft row rebuilt as L[b][k*-1] + A[x_{k*-1}] Bm with draft_lse
 *     (falls back to p_t if every difference is zero), u = U(seed, b, k*, 2);
 *   - no rejection (also ell = 0, paperlayer.ai Appendix A: the target then
 *     produces a fresh token): sample p_t of row Tgt[b][ell], u = U(seed, b, ell+1, 3).
 * out_tok[b] = x_1..x_a, then that token, then -1; n_out[b] = a + 1.
 *
 *   Tgt        [B][gamma+1][V] target logits; row k-1 scores position k, row
 *              ell supplies the bonus token (dtype)
 *   L, A, Bm, x0    as given to dspark_markov_draft
 *   draft_tok, draft_p, draft_lse   outputs of dspark_markov_draft
 *   verify_len [B] int32 in [0, gamma] (from dspark_schedule)
 *   accepted   [B] int32 out
 *   out_tok    [B][gamma+1] int32 out
 *   n_out      [B] int32 out
 *   target_p   [B][gamma] f32 out p_t(x_k) for k <= ell, 0 beyond; may be NULL
 *   seed, seed_dev  the Philox seed; the same value as the draft's
 */
int dspark_verify(int dtype, const void* Tgt, const void* L, const void* A, const void* Bm, const int32_t* x0,
                  const int32_t* draft_tok, const float* draft_p, const double* draft_lse, const int32_t* verify_len,
                  int B, int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* accepted,
                  int32_t* out_tok, int32_t* n_out, float* target_p, void* ws, size_t ws_bytes, void* stream);

/*
 * dspark_rnn_verify -- dspark_verify for a draft made by dspark_rnn_draft:
 * the residual at a rejected position k rebuilds the draft logits from the
 * state H[b][k-1] (f = L[b][k-1] + h_k . Bm) instead of A[x_{k-1}]; there is
 * no x0.  Everything else as dspark_verify.
 */
int dspark_rnn_verify(int dtype, const void* Tgt, const void* L, const void* H, const void* Bm,
                      const int32_t* draft_tok, const float* draft_p, const double* draft_lse,
                      const int32_t* verify_len, int B, int gamma, int V, int r, uint64_t seed,
                      const uint64_t* seed_dev, int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Opt-in kernel timing, for measurement tools only (benchmarks, profiling
 * scripts; not for production paths and not for use under graph capture).
 * Its state is process-wide (shared by all threads and devices, guarded by a
 * lock); while it is off (the default) no call above touches it.
 * dspark_profile_start creates up to 2*max_launches hipEvents and from then
 * on binds an event pair to every launch of the kernels whose bit is set in
 * kernel_mask (bit i = kernel id i below), through hipExtLaunchKernelGGL, so
 * a pair's interval is that kernel's own execution.
 * dspark_profile_query waits for the recorded events and returns the summed
 * duration in ms and the launch count of one kernel:
 *   0 draft tiles, 1 draft locate, 2 schedule, 3 target partials, 4 accept,
 *   5 residual tiles, 6 bonus partials, 7 final.
 */
int dspark_profile_start(int max_launches, unsigned kernel_mask);
int dspark_profile_stop(void);
int dspark_profile_query(int kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif
