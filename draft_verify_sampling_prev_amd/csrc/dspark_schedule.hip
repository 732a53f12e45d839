// dspark_schedule.hip -- confidence scheduling on gfx950: survival product and
// budget selection, one workgroup of 1024 threads.
//
// Survival: the confidence head's per-position conditional survival is
// calibrated by one temperature per position, c = sigmoid(z / T_k)
// (sequential temperature scaling, paperlayer.ai summary of arXiv 2607.05147,
// section 3.2; menfem.com note, Key Contributions), and the prefix survival
// is the running product Theta_k = Theta_{k-1} * c_k with Theta_0 = 1
// (llm-wiki.hwlabs.dev explainer, prefix-survival definition), in fp32.
//
// Selection: the scheduler orders all B*gamma candidates by cumulative
// survival and admits greedily (menfem.com note, hardware-aware prefix
// scheduler); here the first `admit` of the order (Theta desc, request asc,
// position asc).  Instead of sorting, an 8-bit LDS radix select finds the
// admit-th largest key in four passes over the fp32 bit patterns; keys above
// it are admitted, and among keys equal to it the first ones in (request,
// position) order.  Because each row's Theta is non-increasing, the admitted
// set of a row is a prefix and its verify length is its admitted count.
#include "dspark_device.hpp"
#include "dspark_internal.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;

// Order-preserving map of a float onto uint32 (-0 and +0 both map to the key of +0).
__device__ __forceinline__ uint32_t order_key(float v)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int block_excl_scan_int(int v, int* wsum, int* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(inc, o, 64);
        if (lane >= o) inc += n;
    }
    __syncthreads();
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    int off = 0, tot = 0;
    for (int i = 0; i < kSchedThreads / 64; ++i) {
        if (i < w) off += wsum[i];
        tot += wsum[i];
    }
    *total = tot;
    return off + inc - v;
}

__global__ __launch_bounds__(kSchedThreads) void k_schedule(const float* __restrict__ z,
                                                            const float* __restrict__ temps, int B, int gamma,
                                                            long long admit, float* surv, int32_t* __restrict__ len)
{
    __shared__ uint32_t keys[kMaxCandidates];
    __shared__ uint32_t hist[256];
    __shared__ int wsum[kSchedThreads / 64];
    __shared__ uint32_t sh_prefix;
    __shared__ long long sh_rem;

    const int t = threadIdx.x;
    const int N = B * gamma;

    // Inputs (z, or the given survivals) into LDS with coalesced loads, and
    // the temperatures; then one thread per row runs the product.
    __shared__ float tsh[kMaxGamma];
    const float* src = z ? z : surv;
    for (int i = t; i < N; i += kSchedThreads) keys[i] = __float_as_uint(src[i]);
    if (z && t < gamma) tsh[t] = temps[t];
    __syncthreads();
    if (z) {
        for (int b = t; b < B; b += kSchedThreads) {
            float th = 1.0f;
            for (int kk = 0; kk < gamma; ++kk) {
                const float q = __uint_as_float(keys[b * gamma + kk]) / tsh[kk];
                const float c = 1.0f / (1.0f + expf(-q));
                th = th * c;
                keys[b * gamma + kk] = __float_as_uint(th);  // the row's own slots only
            }
        }
        __syncthreads();
    }
    for (int i = t; i < N; i += kSchedThreads) {
        const float v = __uint_as_float(keys[i]);
        if (z) surv[i] = v;
        keys[i] = order_key(v);
    }
    __syncthreads();

    if (admit <= 0 || admit >= N) {
        const int l = admit <= 0 ? 0 : gamma;
        for (int b = t; b < B; b += kSchedThreads) len[b] = l;
        return;
    }

    // Radix select of the admit-th largest key, most significant digit first.
    // Per pass: histogram of the current digit among keys matching the prefix
    // so far, then threads 0..255 scan the bins from the top digit down
    // (thread t holds digit 255 - t) and the one whose running count first
    // reaches the remaining rank selects its digit.
    if (t == 0) {
        sh_prefix = 0u;
        sh_rem = admit;
    }
    uint32_t mask = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = t; i < 256; i += kSchedThreads) hist[i] = 0u;
        __syncthreads();
        const uint32_t prefix = sh_prefix;
        const long long rem = sh_rem;
        for (int i = t; i < N; i += kSchedThreads) {
            const uint32_t key = keys[i];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        int cnt = 0, inc = 0;
        if (t < 256) {
            cnt = (int)hist[255 - t];
            inc = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int n = __shfl_up(inc, o, 64);
                if ((t & 63) >= o) inc += n;
            }
            if ((t & 63) == 63) wsum[t >> 6] = inc;
        }
        __syncthreads();
        if (t < 256) {
            int off = 0;
            for (int i = 0; i < (t >> 6); ++i) off += wsum[i];
            const long long upto = (long long)(off + inc);  // keys with digit >= 255 - t
            const long long above = upto - cnt;              // keys with digit >  255 - t
            if (above < rem && rem <= upto) {
                sh_rem = rem - above;
                sh_prefix = prefix | ((uint32_t)(255 - t) << shift);
            }
        }
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t kth = sh_prefix;      // key of the admit-th largest candidate
    const long long need_eq = sh_rem;    // how many candidates equal to it are admitted

    // Rank of each equal key in index order: contiguous segments per thread.
    const int per = (N + kSchedThreads - 1) / kSchedThreads;
    const int i0 = min(t * per, N), i1 = min(i0 + per, N);
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += keys[i] == kth;
    int tot = 0;
    int rank = block_excl_scan_int(eq, wsum, &tot);
    for (int i = i0; i < i1; ++i) {
        const uint32_t key = keys[i];
        uint32_t adm = key > kth ? 1u : 0u;
        if (key == kth) {
            adm = (long long)rank < need_eq ? 1u : 0u;
            ++rank;
        }
        keys[i] = adm;  // each thread rewrites only its own segment
    }
    __syncthreads();
    for (int b = t; b < B; b += kSchedThreads) {
        int l = 0;
        for (int kk = 0; kk < gamma; ++kk) l += (int)keys[b * gamma + kk];
        len[b] = l;
    }
}

hipError_t launch_schedule(const float* z, const float* temps, int B, int gamma, int64_t admit, float* survival,
                           int32_t* len, hipStream_t s)
{
    prof_begin(K_SCHEDULE, s);
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, s, z, temps, B, gamma, (long long)admit,
                       survival, len);
    prof_end(K_SCHEDULE, s);
    return hipGetLastError();
}

}  // namespace dspark
