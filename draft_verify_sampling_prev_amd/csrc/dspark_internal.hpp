// dspark_internal.hpp -- host-side pieces shared by the C-ABI layer and the
// kernel launchers: workspace layout, launcher declarations, kernel timing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

constexpr int kMaxGamma = 16;
constexpr int kMaxRank = 256;
constexpr int kMaxCandidates = 16384;  // B * gamma handled by the one-workgroup selection
constexpr int kChunkElems = 8192;       // vocabulary elements per workgroup in the row passes
// Vocabulary columns per Markov tile (the granularity of the draft and
// residual softmax partials): 64 for bf16, 128 for fp32.
inline int tile_cols(int dtype) { return dtype == 1 ? 64 : 128; }
inline int n_tiles(int dtype, int V) { return (V + tile_cols(dtype) - 1) / tile_cols(dtype); }
inline int n_chunks(int V) { return (V + kChunkElems - 1) / kChunkElems; }

// Rank of the Markov factors whose draft steps hand the next step its A rows
// in MFMA order (the "ag" workspace region, see dspark_tile.hpp).
constexpr int kAgRank = 256;

// Slot aggregates of the draft tile partials: a bf16 draft tile launch of at
// most this many slots also writes, per row and slot, the max and sum of exp
// of the slot's contiguous tile range, and the locate reads those first.
// Every workspace layout puts them right after the A-row hand-over, at
// ag + slot_agg_offset(B) (so the locate finds them without an argument).
constexpr int kSlotAggMax = 256;
__host__ __device__ inline size_t ag_bytes(int B) { return ((size_t)(B > 0 ? B : 0) + 15) / 16 * 16 * kAgRank * 2; }
__host__ __device__ inline size_t slot_agg_offset(int B) { return (ag_bytes(B) + 255) & ~(size_t)255; }
// Their size: only batches above one row block (kTileRows) use them (there
// the locate workgroups share CUs); smaller batches keep the workspace as it
// is without them.
inline size_t slot_agg_bytes(int B) { return B > 256 ? (size_t)B * kSlotAggMax * 8 : 0; }

// Byte offsets into the caller's workspace (each 256-byte aligned).
struct WsLayout {
    size_t draft_part;            // [B][nT] float2 : draft tile max and sum of exp(f - max)
    size_t slot_agg;              // [B][kSlotAggMax] float2 : the same per tile slot (contiguous tile range)
    size_t tgt_m, tgt_s;          // [B*gamma][nC] f32 / f64 : target chunk max and sum of exp
    size_t lse_t;                 // [B][gamma] f64 : target log-normalisers of verified rows
    size_t resid_list;            // [B] int4 : (request, first rejected position, its conditioning token), in no fixed order
    size_t resid_count;           // [1] i32
    size_t res_part;              // [B][nT] float2 : per tile sum of max(0, p_t - p_d) and of p_t, row b for request b
    size_t bon_m, bon_s;          // [B][nC] f32 / f64 : bonus-row chunk max and sum of exp
    size_t ag;                    // [ceil(B/16)*16][256] bf16 : the next draft step's A rows, MFMA order (rank 256)
    size_t total;
};

WsLayout ws_layout(int B, int gamma, int V);

// The Philox seed of a call as the kernels receive it: the by-value seed, or,
// when `dev` is set, the 64-bit value at that device address, read by each
// kernel when it runs (so a captured graph replayed after the caller has
// written a new value there draws new uniforms).
struct SeedArg {
    uint64_t value;
    const uint64_t* dev;
};

__device__ __forceinline__ uint64_t seed_of(const SeedArg& s) { return s.dev ? *s.dev : s.value; }

// Kernel timing (opt-in; event pairs attached to the timed kernels' own
// dispatches, so an interval is one kernel's execution).
enum KernelId {
    K_DRAFT_TILES = 0,
    K_DRAFT_LOCATE,
    K_SCHEDULE,
    K_TARGET_PARTIALS,
    K_ACCEPT,
    K_RESID_TILES,
    K_BONUS_PARTIALS,
    K_FINAL,
    K_COUNT
};
// Persistent slots per row block of a tile pass over nT tiles with nM row
// blocks (one workgroup per compute unit at a time): the fewest slots that
// keep every slot within max_tiles tiles (its partial staging) and make the
// grid S * nM a whole number of rounds over the compute units, so that no
// round runs on a fraction of the chip.
inline int tile_slots(int nT, int nM, int cus, int max_tiles)
{
    const int per_round = cus / nM > 0 ? cus / nM : 1;
    const int need = (nT + max_tiles - 1) / max_tiles;
    const int rounds = (need + per_round - 1) / per_round;
    return nT < per_round * rounds ? nT : per_round * rounds;
}

// Compute units of the current device (cached per device).
int cu_count();

// A free pair of timing events for one launch of kernel `id`, or {null, null}
// when timing is off for it (or the event pool is exhausted).
struct ProfPair {
    hipEvent_t start, stop;
};
ProfPair prof_pair(int id);

// Launch `kernel` on `s`; when kernel `id` is being timed, through
// hipExtLaunchKernelGGL with the pair's events bound to this dispatch.
template <typename F, typename... Args>
inline void launch_timed(int id, F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args)
{
    const ProfPair e = prof_pair(id);
    if (e.start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0u, s, e.start, e.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Launchers (return hipGetLastError()).
// z0/wc/z_out (all null, or all set): the Markov-conditioned confidence
// logit z_out[b][k-1] = z0[b][k-1] + <A[x_{k-1}], wc>, computed by the locate.
// Wt/H (both null, or both set): the RNN head -- the step first writes the
// state h_k = tanh(W h_{k-1} + A[x_{k-1}]) into row (b, k-1) of H, which
// then replaces A[x_{k-1}] as the operand.
// sched (given at k = 1 and k = gamma, only when draft_step_can_schedule):
// the budget schedule of dspark_schedule runs as one extra workgroup of the
// first tile launch (schedule_in_first_tiles) or else of the last locate
// launch.
struct SchedArg {
    const float* z;      // [B][gamma] confidence logits
    const float* temps;  // [gamma]
    long long admit;     // min(budget, B*gamma)
    float* surv;         // [B][gamma] out
    int32_t* len;        // [B] out
};
hipError_t launch_draft_step(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0,
                             int B, int gamma, int V, int r, int k, SeedArg seed, int32_t* tok, float* p,
                             double* lse, const float* z0, const void* wc, float* z_out, const void* Wt, void* H,
                             void* ws, const WsLayout& lay, hipStream_t s, const SchedArg* sched = nullptr);
// Whether a draft launch can carry the budget schedule (bf16, Markov head,
// B*gamma keys within a 32 KB LDS buffer): the first tile launch, when one
// slot fewer leaves every slot's tile count unchanged (B <= 256), or the
// last step's one-wave locate launch.
bool schedule_in_first_tiles(int dtype, int B, int gamma, int V);
// Persistent slots of the bf16 draft tile launch for B rows and nT tiles:
// tile_slots with at most 12 tiles per slot, or 36 for full-batch launches
// (B a multiple of 256), which write their staged partials out every 12.
int draft_tile_slots(int B, int nT);
bool draft_step_can_schedule(int dtype, int B, int gamma, int V);

hipError_t launch_schedule(const float* z, const float* temps, int B, int gamma, int64_t admit, float* survival,
                           int32_t* len, hipStream_t s);
hipError_t launch_schedule_objective(const float* z, const float* temps, int B, int gamma, const float* step_time,
                                     int64_t cap, float* survival, int32_t* len, hipStream_t s);
hipError_t launch_schedule_threshold(const float* z, const float* temps, int B, int gamma, float tau,
                                     float* survival, int32_t* len, hipStream_t s);

hipError_t launch_verify(int dtype, const void* Tg, const void* L, const void* A, const void* Bm, const int32_t* x0,
                         const int32_t* tok, const float* pd, const double* lse_d, const int32_t* len, int B,
                         int gamma, int V, int r, SeedArg seed, int32_t* accepted, int32_t* out_tok,
                         int32_t* n_out, float* target_p, const void* H, void* ws, const WsLayout& lay, hipStream_t s);

}  // namespace dspark
