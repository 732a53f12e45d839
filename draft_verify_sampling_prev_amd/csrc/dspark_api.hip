// dspark_api.hip -- the C ABI of libdspark: argument validation, workspace
// layout, launch sequencing on the caller's stream, error reporting and
// opt-in kernel timing.  No allocation happens inside the three calls.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "dspark.h"
#include "dspark_internal.hpp"

namespace dspark {

static thread_local char g_err[512] = "";

static int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int B, int gamma, int V)
{
    WsLayout l;
    const size_t nT = (size_t)n_tiles(1, V), nC = (size_t)n_chunks(V);  // the larger tile count
    const size_t Bz = (size_t)(B > 0 ? B : 0), G = (size_t)gamma;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    l.draft_part = take(Bz * nT * 8);
    l.tgt_m = take(Bz * G * nC * 4);
    l.tgt_s = take(Bz * G * nC * 8);
    l.lse_t = take(Bz * G * 8);
    l.resid_list = take(Bz * 16);
    l.resid_count = take(4);
    l.res_part = take(Bz * nT * 8);
    l.bon_m = take(Bz * nC * 4);
    l.bon_s = take(Bz * nC * 8);
    l.ag = take(ag_bytes(B));
    l.slot_agg = take(slot_agg_bytes(B));  // = ag + slot_agg_offset(B)
    l.total = o;
    return l;
}

static int g_cu_count[64];

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cu_count[dev] = n;
    }
    return g_cu_count[dev];
}

// ---------------------------------------------------------------------------
// Static scratch for the allocation-free draft entry point: the draft's tile
// partials and A-row hand-over, in a file-scope device array.  Each device
// that runs the library holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is taken once per device with hipGetSymbolAddress (the
// device current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static void* g_scratch_ptr[64];
static std::mutex g_scratch_mu;

// Device address of this device's scratch array (nullptr and *err set on failure).
static void* scratch_address(hipError_t* err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// The draft's share of a workspace (the tile partials, the A rows in MFMA
// order, then the tile partials' slot aggregates); the other offsets are
// unused by the draft kernels.
static WsLayout draft_layout(int B, int V)
{
    WsLayout l = {};
    const size_t Bz = (size_t)(B > 0 ? B : 0);
    l.draft_part = 0;
    l.ag = align256(Bz * (size_t)n_tiles(1, V) * 8);
    l.slot_agg = l.ag + slot_agg_offset(B);
    l.total = align256(l.slot_agg + slot_agg_bytes(B));
    return l;
}

// ---------------------------------------------------------------------------
// Kernel timing (measurement only; off unless dspark_profile_start was
// called).  The state is process-wide and guarded by a mutex; the events of
// a pair are bound to one kernel dispatch (hipExtLaunchKernelGGL), so an
// interval is that kernel's execution, not the gap before it.
// ---------------------------------------------------------------------------
struct ProfState {
    bool on = false;
    unsigned mask = 0u;                // bit i set: time kernel i
    int capacity = 0;                  // events available (two per launch)
    std::vector<hipEvent_t> pool;
    int used = 0;
    std::vector<int> ids;              // kernel id of each recorded pair
    std::vector<int> starts;           // index into pool of each pair's start (stop = start + 1)
    bool overflow = false;
};
static ProfState g_prof;
static std::mutex g_prof_mu;

ProfPair prof_pair(int id)
{
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof.on || !(g_prof.mask & (1u << id))) return ProfPair{ nullptr, nullptr };
    if (g_prof.used + 2 > g_prof.capacity) {
        g_prof.overflow = true;
        return ProfPair{ nullptr, nullptr };
    }
    const int e = g_prof.used;
    g_prof.used += 2;
    g_prof.ids.push_back(id);
    g_prof.starts.push_back(e);
    return ProfPair{ g_prof.pool[e], g_prof.pool[e + 1] };
}

static int check_common(int B, int gamma, int V, int r)
{
    if (B < 0) return fail(DSPARK_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (gamma < 1 || gamma > kMaxGamma) return fail(DSPARK_ERR_UNSUPPORTED, "gamma must be in [1, %d] (got %d)", kMaxGamma, gamma);
    if (V < 8 || V % 8 != 0 || V > (1 << 24))
        return fail(DSPARK_ERR_UNSUPPORTED, "V must be a multiple of 8 in [8, 2^24] (got %d)", V);
    if (r < 8 || r > kMaxRank || r % 8 != 0)
        return fail(DSPARK_ERR_UNSUPPORTED, "r must be a multiple of 8 in [8, %d] (got %d)", kMaxRank, r);
    if ((long long)B * gamma > kMaxCandidates)
        return fail(DSPARK_ERR_UNSUPPORTED, "B*gamma must be <= %d (got %lld)", kMaxCandidates, (long long)B * gamma);
    return DSPARK_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(DSPARK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return DSPARK_OK;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

const char* dspark_version(void) { return "dspark-mi355x 0.1.0 (gfx950)"; }

const char* dspark_last_error(void) { return g_err; }

size_t dspark_workspace_size(int B, int gamma, int V, int r)
{
    (void)r;
    if (B < 0 || gamma < 1 || V < 1) return 0;
    return ws_layout(B, gamma, V).total;
}

static int markov_draft_impl(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, SeedArg seed, const float* z0, const void* wc,
                             int32_t* draft_tok, float* draft_p, double* draft_lse, float* z_out, const void* Wt,
                             void* H, void* ws, size_t ws_bytes, void* stream, const WsLayout* layout = nullptr,
                             const SchedArg* sched = nullptr)
{
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    int rc = check_common(B, gamma, V, r);
    if (rc) return rc;
    if (B == 0) return DSPARK_OK;
    if (!L || !A || !Bm || !x0 || !draft_tok || !draft_p || !draft_lse || !ws)
        return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(L) || !aligned16(A) || !aligned16(Bm))
        return fail(DSPARK_ERR_INVALID_ARG, "L, A and Bm must be 16-byte aligned");
    const WsLayout lay = layout ? *layout : ws_layout(B, gamma, V);
    if (ws_bytes < lay.total)
        return fail(DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, lay.total);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int k = 1; k <= gamma; ++k) {
        hipError_t e = launch_draft_step(dtype, L, A, Bm, x0, B, gamma, V, r, k, seed, draft_tok, draft_p, draft_lse,
                                         z0, wc, z_out, Wt, H, ws, lay, s, k == 1 || k == gamma ? sched : nullptr);
        if (e != hipSuccess) return hip_status(e, "draft launch");
    }
    return DSPARK_OK;
}

int dspark_markov_draft(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B, int gamma,
                        int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok, float* draft_p,
                        double* draft_lse, void* ws, size_t ws_bytes, void* stream)
{
    g_err[0] = 0;
    return markov_draft_impl(dtype, L, A, Bm, x0, B, gamma, V, r, SeedArg{ seed, seed_dev }, nullptr, nullptr, draft_tok, draft_p,
                             draft_lse, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

int dspark_markov_draft_sched(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                              int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, const float* z,
                              const float* temps, int64_t budget, int32_t* draft_tok, float* draft_p,
                              double* draft_lse, float* survival, int32_t* verify_len, void* ws, size_t ws_bytes,
                              void* stream)
{
    g_err[0] = 0;
    if (budget < 0) return fail(DSPARK_ERR_INVALID_ARG, "budget must be >= 0 (got %lld)", (long long)budget);
    if (B > 0 && (!z || !temps || !survival || !verify_len)) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    const int64_t n = (int64_t)B * gamma;
    const SchedArg sa{ z, temps, (long long)(budget < n ? budget : n), survival, verify_len };
    // The schedule rides in a draft launch where one can carry it (the first
    // tile launch or the last locate launch); otherwise it is launched after
    // the draft.
    const bool fused = draft_step_can_schedule(dtype, B, gamma, V);
    const int rc = markov_draft_impl(dtype, L, A, Bm, x0, B, gamma, V, r, SeedArg{ seed, seed_dev }, nullptr, nullptr,
                                     draft_tok, draft_p, draft_lse, nullptr, nullptr, nullptr, ws, ws_bytes, stream,
                                     nullptr, fused ? &sa : nullptr);
    if (rc || B == 0 || fused) return rc;
    return hip_status(launch_schedule(z, temps, B, gamma, sa.admit, survival, verify_len,
                                      static_cast<hipStream_t>(stream)),
                      "schedule launch");
}

int dspark_markov_draft_noalloc(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                                int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok,
                                float* draft_p, double* draft_lse, void* stream)
{
    g_err[0] = 0;
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    int rc = check_common(B, gamma, V, r);
    if (rc) return rc;
    if (B == 0) return DSPARK_OK;
    const WsLayout lay = draft_layout(B, V);
    if (lay.total > kScratchBytes)
        return fail(DSPARK_ERR_WORKSPACE, "the draft needs %zu bytes of scratch; the static scratch holds %zu", lay.total,
                    kScratchBytes);
    if (!L || !A || !Bm || !x0 || !draft_tok || !draft_p || !draft_lse)
        return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    hipError_t e = hipSuccess;
    void* ws = scratch_address(&e);
    if (!ws) return hip_status(e, "hipGetSymbolAddress(scratch)");
    return markov_draft_impl(dtype, L, A, Bm, x0, B, gamma, V, r, SeedArg{ seed, seed_dev }, nullptr, nullptr, draft_tok,
                             draft_p, draft_lse, nullptr, nullptr, nullptr, ws, lay.total, stream, &lay);
}

int dspark_markov_draft_conf(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, const float* z0,
                             const void* wc, int32_t* draft_tok, float* draft_p, double* draft_lse, float* z_out,
                             void* ws, size_t ws_bytes, void* stream)
{
    g_err[0] = 0;
    if (B > 0 && (!z0 || !wc || !z_out)) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    return markov_draft_impl(dtype, L, A, Bm, x0, B, gamma, V, r, SeedArg{ seed, seed_dev }, z0, wc, draft_tok, draft_p, draft_lse, z_out,
                             nullptr, nullptr, ws, ws_bytes, stream);
}

int dspark_rnn_draft(int dtype, const void* L, const void* A, const void* Bm, const void* Wt, const int32_t* x0, int B,
                     int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* draft_tok,
                     float* draft_p, double* draft_lse, void* H, void* ws, size_t ws_bytes, void* stream)
{
    g_err[0] = 0;
    if (B > 0 && (!Wt || !H)) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (B > 0 && (!aligned16(H) || !aligned16(Wt))) return fail(DSPARK_ERR_INVALID_ARG, "H and Wt must be 16-byte aligned");
    return markov_draft_impl(dtype, L, A, Bm, x0, B, gamma, V, r, SeedArg{ seed, seed_dev }, nullptr, nullptr,
                             draft_tok, draft_p, draft_lse, nullptr, Wt, H, ws, ws_bytes, stream);
}

int dspark_schedule(const float* z, const float* temps, int B, int gamma, int64_t budget, float* survival,
                    int32_t* verify_len, void* stream)
{
    g_err[0] = 0;
    if (B < 0) return fail(DSPARK_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (gamma < 1 || gamma > kMaxGamma) return fail(DSPARK_ERR_UNSUPPORTED, "gamma must be in [1, %d] (got %d)", kMaxGamma, gamma);
    if ((long long)B * gamma > kMaxCandidates)
        return fail(DSPARK_ERR_UNSUPPORTED, "B*gamma must be <= %d", kMaxCandidates);
    if (budget < 0) return fail(DSPARK_ERR_INVALID_ARG, "budget must be >= 0 (got %lld)", (long long)budget);
    if (B == 0) return DSPARK_OK;
    if (!survival || !verify_len) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (z && !temps) return fail(DSPARK_ERR_INVALID_ARG, "temps must be given with z");
    const int64_t n = (int64_t)B * gamma;
    const int64_t admit = budget < n ? budget : n;
    return hip_status(launch_schedule(z, temps, B, gamma, admit, survival, verify_len, static_cast<hipStream_t>(stream)),
                      "schedule launch");
}

int dspark_schedule_objective(const float* z, const float* temps, int B, int gamma, const float* step_time,
                              int n_time, int64_t max_admit, float* survival, int32_t* verify_len, void* stream)
{
    g_err[0] = 0;
    if (B < 0) return fail(DSPARK_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (gamma < 1 || gamma > kMaxGamma) return fail(DSPARK_ERR_UNSUPPORTED, "gamma must be in [1, %d] (got %d)", kMaxGamma, gamma);
    if ((long long)B * gamma > kMaxCandidates)
        return fail(DSPARK_ERR_UNSUPPORTED, "B*gamma must be <= %d", kMaxCandidates);
    if (max_admit < 0) return fail(DSPARK_ERR_INVALID_ARG, "max_admit must be >= 0 (got %lld)", (long long)max_admit);
    if (B == 0) return DSPARK_OK;
    if (!survival || !verify_len || !step_time) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (z && !temps) return fail(DSPARK_ERR_INVALID_ARG, "temps must be given with z");
    const int64_t n = (int64_t)B * gamma;
    const int64_t cap = max_admit < n ? max_admit : n;
    if ((int64_t)n_time <= (int64_t)B + cap)
        return fail(DSPARK_ERR_INVALID_ARG, "step_time needs B + min(max_admit, B*gamma) + 1 = %lld entries (got %d)",
                    (long long)(B + cap + 1), n_time);
    return hip_status(launch_schedule_objective(z, temps, B, gamma, step_time, cap, survival, verify_len,
                                                static_cast<hipStream_t>(stream)),
                      "schedule_objective launch");
}

int dspark_schedule_threshold(const float* z, const float* temps, int B, int gamma, float tau, float* survival,
                              int32_t* verify_len, void* stream)
{
    g_err[0] = 0;
    if (B < 0) return fail(DSPARK_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (gamma < 1 || gamma > kMaxGamma) return fail(DSPARK_ERR_UNSUPPORTED, "gamma must be in [1, %d] (got %d)", kMaxGamma, gamma);
    if (B == 0) return DSPARK_OK;
    if (!survival || !verify_len) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (z && !temps) return fail(DSPARK_ERR_INVALID_ARG, "temps must be given with z");
    return hip_status(launch_schedule_threshold(z, temps, B, gamma, tau, survival, verify_len,
                                                static_cast<hipStream_t>(stream)),
                      "schedule_threshold launch");
}

static int verify_impl(int dtype, const void* Tgt, const void* L, const void* A, const void* Bm, const int32_t* x0,
                       const int32_t* draft_tok, const float* draft_p, const double* draft_lse,
                       const int32_t* verify_len, int B, int gamma, int V, int r, SeedArg seed, int32_t* accepted,
                       int32_t* out_tok, int32_t* n_out, float* target_p, const void* H, void* ws, size_t ws_bytes,
                       void* stream)
{
    if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return fail(DSPARK_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
    int rc = check_common(B, gamma, V, r);
    if (rc) return rc;
    if (B == 0) return DSPARK_OK;
    if (!Tgt || !L || !A || !Bm || (!x0 && !H) || !draft_tok || !draft_p || !draft_lse || !verify_len || !accepted ||
        !out_tok || !n_out || !ws)
        return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(Tgt) || !aligned16(L) || !aligned16(A) || !aligned16(Bm))
        return fail(DSPARK_ERR_INVALID_ARG, "Tgt, L, A (or H) and Bm must be 16-byte aligned");
    const WsLayout lay = ws_layout(B, gamma, V);
    if (ws_bytes < lay.total)
        return fail(DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, lay.total);
    return hip_status(launch_verify(dtype, Tgt, L, A, Bm, x0, draft_tok, draft_p, draft_lse, verify_len, B, gamma, V, r,
                                    seed, accepted, out_tok, n_out, target_p, H, ws, lay,
                                    static_cast<hipStream_t>(stream)),
                      "verify launch");
}

int dspark_verify(int dtype, const void* Tgt, const void* L, const void* A, const void* Bm, const int32_t* x0,
                  const int32_t* draft_tok, const float* draft_p, const double* draft_lse, const int32_t* verify_len,
                  int B, int gamma, int V, int r, uint64_t seed, const uint64_t* seed_dev, int32_t* accepted,
                  int32_t* out_tok, int32_t* n_out, float* target_p, void* ws, size_t ws_bytes, void* stream)
{
    g_err[0] = 0;
    return verify_impl(dtype, Tgt, L, A, Bm, x0, draft_tok, draft_p, draft_lse, verify_len, B, gamma, V, r,
                       SeedArg{ seed, seed_dev },
                       accepted, out_tok, n_out, target_p, nullptr, ws, ws_bytes, stream);
}

int dspark_rnn_verify(int dtype, const void* Tgt, const void* L, const void* H, const void* Bm,
                      const int32_t* draft_tok, const float* draft_p, const double* draft_lse,
                      const int32_t* verify_len, int B, int gamma, int V, int r, uint64_t seed,
                      const uint64_t* seed_dev, int32_t* accepted, int32_t* out_tok, int32_t* n_out, float* target_p,
                      void* ws, size_t ws_bytes, void* stream)
{
    g_err[0] = 0;
    if (B > 0 && !H) return fail(DSPARK_ERR_INVALID_ARG, "null pointer argument");
    return verify_impl(dtype, Tgt, L, H, Bm, nullptr, draft_tok, draft_p, draft_lse, verify_len, B, gamma, V, r,
                       SeedArg{ seed, seed_dev },
                       accepted, out_tok, n_out, target_p, H, ws, ws_bytes, stream);
}

int dspark_profile_start(int max_launches, unsigned kernel_mask)
{
    g_err[0] = 0;
    if (max_launches < 1) return fail(DSPARK_ERR_INVALID_ARG, "max_launches must be >= 1");
    std::lock_guard<std::mutex> lock(g_prof_mu);
    const int need = 2 * max_launches;
    while ((int)g_prof.pool.size() < need) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return hip_status(err, "hipEventCreate");
        g_prof.pool.push_back(e);
    }
    g_prof.mask = kernel_mask;
    g_prof.capacity = need;
    g_prof.used = 0;
    g_prof.ids.clear();
    g_prof.starts.clear();
    g_prof.overflow = false;
    g_prof.on = true;
    return DSPARK_OK;
}

int dspark_profile_stop(void)
{
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof.on = false;
    return DSPARK_OK;
}

int dspark_profile_query(int kernel, double* total_ms, int* launches)
{
    g_err[0] = 0;
    if (kernel < 0 || kernel >= K_COUNT || !total_ms || !launches)
        return fail(DSPARK_ERR_INVALID_ARG, "bad profile query");
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (g_prof.overflow) return fail(DSPARK_ERR_INVALID_ARG, "profile event capacity exceeded");
    double tot = 0.0;
    int n = 0;
    for (size_t i = 0; i < g_prof.ids.size(); ++i) {
        if (g_prof.ids[i] != kernel) continue;
        hipEvent_t e0 = g_prof.pool[g_prof.starts[i]], e1 = g_prof.pool[g_prof.starts[i] + 1];
        hipError_t e = hipEventSynchronize(e1);
        if (e != hipSuccess) return hip_status(e, "hipEventSynchronize");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, e0, e1);
        if (e != hipSuccess) return hip_status(e, "hipEventElapsedTime");
        tot += ms;
        ++n;
    }
    *total_ms = tot;
    *launches = n;
    return DSPARK_OK;
}

}  // extern "C"
