// dspark_schedule.hip -- confidence scheduling on gfx950: survival product and
// budget selection (dspark_select.hpp), objective-based admission and the
// static threshold, each in one workgroup of 1024 threads.
#include <limits.h>

#include <algorithm>

#include "dspark_device.hpp"
#include "dspark_internal.hpp"
#include "dspark_select.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;

__global__ __launch_bounds__(kSchedThreads) void k_schedule(const float* __restrict__ z,
                                                            const float* __restrict__ temps, int B, int gamma,
                                                            long long admit, float* surv, int32_t* __restrict__ len)
{
    __shared__ uint32_t keys[kMaxCandidates];
    __shared__ SelectScratch<kSchedThreads> sc;
    budget_select<kSchedThreads>(z, temps, B, gamma, admit, surv, len, keys, sc);
}

// ---------------------------------------------------------------------------
// Objective-based admission: the same greedy order, admitted one candidate
// at a time while the expected number of emitted tokens per unit of
// verification time does not drop, stopping at the first candidate that
// would lower it (menfem.com note, hardware-aware prefix scheduler:
// incremental batch admission with early stopping; paperlayer.ai summary,
// section 5.2 (engine throughput profile) and Appendix A (early stopping)).
//   J(m) = E(m) / t[B + m],  E(m) = B + (sum of the m first Theta),
// t[n] the time of a verification batch of n tokens.  Arithmetic fixed so
// the decision is reproducible: Theta clamped into [0, 1] (NaN -> 0), E in
// integer units of 2^-36 (terms floor(Theta * 2^36), sums exact), and
// "J(m+1) < J(m)" evaluated as E(m+1) * t[B+m] < E(m) * t[B+m+1] with both
// products in double.
//
// One workgroup: the N keys ((order key of Theta) complemented, index) are
// bitonic-sorted ascending (Theta desc, then index = request-major order
// asc) in registers, with shuffles inside a wave and LDS only across waves;
// then each thread takes a contiguous run of ranks, the per-rank
// terms are scanned across the workgroup (int64), every rank evaluates its
// own stop test, and the first failing rank (capped at `cap`) is the number
// admitted.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float key_to_float(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

constexpr double kThetaUnit = 68719476736.0;  // 2^36

// Bitonic sort of P keys held in registers: thread t keeps E = P / 1024 keys
// (at least one; threads past P / E hold none) at indices
// (t / 64) * 64E + (t % 64) + 64e (e < E), so a compare partner at distance
// j < 64 is another lane of the same wave (a shuffle), at 64 <= j < 64E it
// is in the same thread, and only j >= 64E crosses waves (through LDS,
// between two barriers).  (Measured on MI355X at 1280 keys: 29 us for the
// whole kernel, against 34 us with every stage through LDS and 40 us with the
// sort on four waves with DPP lane moves.)
template <int E>
__device__ __forceinline__ int bitonic_index(int t, int e)
{
    return (t >> 6) * 64 * E + (t & 63) + 64 * e;
}

__device__ __forceinline__ unsigned long long keep(unsigned long long a, unsigned long long b, bool take_min)
{
    return take_min ? (a < b ? a : b) : (a < b ? b : a);
}

template <int E>
__device__ void bitonic_sort_regs(unsigned long long (&v)[E], int P, unsigned long long* lds)
{
    const int t = threadIdx.x;
    const bool holds = t < P / E;
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 64 * E) {  // partner in another wave
                if (holds) {
#pragma unroll
                    for (int e = 0; e < E; ++e) lds[bitonic_index<E>(t, e)] = v[e];
                }
                __syncthreads();
                if (holds) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int i = bitonic_index<E>(t, e), pi = i ^ j;
                        v[e] = keep(v[e], lds[pi], ((i & k) == 0) == (i < pi));
                    }
                }
                __syncthreads();
            } else if (j >= 64) {  // partner in this thread: slot e ^ (j / 64)
                if (holds) {
                    const int d = j >> 6;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if ((e & d) == 0) {
                            const int i = bitonic_index<E>(t, e);
                            const bool asc = (i & k) == 0;  // i is the lower index of the pair
#pragma unroll
                            for (int f = 0; f < E; ++f) {
                                if (f == (e | d)) {
                                    const unsigned long long x = v[e], y = v[f];
                                    v[e] = keep(x, y, asc);
                                    v[f] = keep(x, y, !asc);
                                }
                            }
                        }
                    }
                }
            } else {  // partner lane ^ j of the same wave
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = bitonic_index<E>(t, e), pi = i ^ j;
                    const unsigned long long o = __shfl_xor(v[e], j, 64);
                    if (holds) v[e] = keep(v[e], o, ((i & k) == 0) == (i < pi));
                }
            }
        }
    }
}

template <int E>
__global__ __launch_bounds__(kSchedThreads) void k_schedule_objective(const float* __restrict__ z,
                                                                      const float* __restrict__ temps, int B,
                                                                      int gamma, const float* __restrict__ step_time,
                                                                      long long cap, float* surv,
                                                                      int32_t* __restrict__ len)
{
    __shared__ unsigned long long skey[kMaxCandidates];  // 128 KB
    __shared__ unsigned char adm[kMaxCandidates];
    __shared__ long long wsum[kSchedThreads / 64];
    __shared__ float tsh[kMaxGamma];
    __shared__ int sh_stop;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int N = B * gamma;
    int P = 64;
    while (P < N) P <<= 1;  // host picks E (see bitonic_sort_regs)
    // Survivals into the upper half of skey (as 32-bit words); sort keys
    // ((order key of Theta) complemented, index) into registers.
    uint32_t* vals = reinterpret_cast<uint32_t*>(skey) + kMaxCandidates;
    survival_lds<kSchedThreads>(z, temps, B, gamma, surv, vals, tsh);
    unsigned long long v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = bitonic_index<E>(t, e);
        v[e] = (t < P / E && i < N)
                   ? ((unsigned long long)~order_key(__uint_as_float(vals[i])) << 32) | (uint32_t)i
                   : ~0ull;
    }
    for (int i = t; i < N; i += kSchedThreads) adm[i] = 0;
    if (t == 0) sh_stop = (int)min(cap, (long long)N);
    __syncthreads();
    bitonic_sort_regs<E>(v, P, skey);
    if (t < P / E) {
#pragma unroll
        for (int e = 0; e < E; ++e) skey[bitonic_index<E>(t, e)] = v[e];
    }
    __syncthreads();

    // Ranks [r0, r1) of this thread: terms, their sum, the exclusive scan.
    const int per = (N + kSchedThreads - 1) / kSchedThreads;
    const int r0 = min(t * per, N), r1 = min(r0 + per, N);
    long long local = 0;
    for (int m = r0; m < r1; ++m) {
        float th = key_to_float(~(uint32_t)(skey[m] >> 32));
        th = fminf(fmaxf(th, 0.0f), 1.0f);  // NaN -> 0
        local += (long long)floor((double)th * kThetaUnit);
    }
    long long inc = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long n = __shfl_up(inc, o, 64);
        if (lane >= o) inc += n;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    long long excl = inc - local;
    for (int i = 0; i < w; ++i) excl += wsum[i];

    // Stop test of each rank m < cap: admitting rank m moves E(m) -> E(m+1).
    const long long mcap = min(cap, (long long)N);
    long long Em = (long long)B * (long long)kThetaUnit + excl;
    int first = INT_MAX;
    for (int m = r0; m < r1 && m < mcap; ++m) {
        float th = key_to_float(~(uint32_t)(skey[m] >> 32));
        th = fminf(fmaxf(th, 0.0f), 1.0f);
        const long long E1 = Em + (long long)floor((double)th * kThetaUnit);
        const double keep_new = (double)E1 * (double)step_time[B + m];
        const double keep_old = (double)Em * (double)step_time[B + m + 1];
        if (keep_new < keep_old) {
            first = m;
            break;
        }
        Em = E1;
    }
    if (first != INT_MAX) atomicMin(&sh_stop, first);
    __syncthreads();
    const int admit = sh_stop;
    for (int m = t; m < admit; m += kSchedThreads) adm[(uint32_t)skey[m]] = 1;
    __syncthreads();
    for (int b = t; b < B; b += kSchedThreads) {
        int l = 0;
        while (l < gamma && adm[b * gamma + l]) ++l;
        len[b] = l;
    }
}

// Static threshold: verify_len[b] is the leading run of positions whose
// survival is at least tau (paperlayer.ai summary, section 4.3).  One thread
// per request; the survival product is the one of survival_lds.
__global__ __launch_bounds__(256) void k_schedule_threshold(const float* __restrict__ z,
                                                            const float* __restrict__ temps, int B, int gamma,
                                                            float tau, float* surv, int32_t* __restrict__ len)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    float th = 1.0f;
    int l = 0;
    bool run = true;
    for (int kk = 0; kk < gamma; ++kk) {
        float v;
        if (z) {
            const float q = z[b * gamma + kk] / temps[kk];
            const float c = 1.0f / (1.0f + expf(-q));
            th = th * c;
            v = th;
            surv[b * gamma + kk] = v;
        } else {
            v = surv[b * gamma + kk];
        }
        run = run && v >= tau;
        l += run ? 1 : 0;
    }
    len[b] = l;
}

hipError_t launch_schedule_objective(const float* z, const float* temps, int B, int gamma, const float* step_time,
                                     int64_t cap, float* survival, int32_t* len, hipStream_t s)
{
    int P = 64;
    while (P < B * gamma) P <<= 1;
    const int E = std::max(1, P / kSchedThreads);
    auto kern = E == 1 ? k_schedule_objective<1>
              : E == 2 ? k_schedule_objective<2>
              : E == 4 ? k_schedule_objective<4>
              : E == 8 ? k_schedule_objective<8>
                       : k_schedule_objective<16>;
    launch_timed(K_SCHEDULE, kern, dim3(1), dim3(kSchedThreads), s, z, temps, B, gamma, step_time, (long long)cap,
                       survival, len);
    return hipGetLastError();
}

hipError_t launch_schedule_threshold(const float* z, const float* temps, int B, int gamma, float tau,
                                     float* survival, int32_t* len, hipStream_t s)
{
    launch_timed(K_SCHEDULE, k_schedule_threshold, dim3((B + 255) / 256), dim3(256), s, z, temps, B, gamma, tau,
                       survival, len);
    return hipGetLastError();
}

hipError_t launch_schedule(const float* z, const float* temps, int B, int gamma, int64_t admit, float* survival,
                           int32_t* len, hipStream_t s)
{
    launch_timed(K_SCHEDULE, k_schedule, dim3(1), dim3(kSchedThreads), s, z, temps, B, gamma, (long long)admit,
                       survival, len);
    return hipGetLastError();
}

}  // namespace dspark
