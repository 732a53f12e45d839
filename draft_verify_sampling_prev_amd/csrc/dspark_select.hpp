// dspark_select.hpp -- the budget schedule's device code, for a workgroup of
// NT threads (NT a multiple of 256, at most 1024): prefix survivals and the
// radix selection of the admitted candidates.  k_schedule runs it with 1024
// threads; the draft's last locate launch can run it with 256 threads in one
// extra workgroup.  The arithmetic does not depend on NT: the survivals are
// the same fp32 expressions in the same order, and the selection is exact
// integer work, so both give the same bits.
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
#pragma once

#include <stdint.h>

#include "dspark_internal.hpp"

namespace dspark {

// Order-preserving map of a float onto uint32 (-0 and +0 both map to the key of +0).
__device__ __forceinline__ uint32_t order_key(float v)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over the NT threads (wsum: NT/64 ints
// of LDS); *total receives the sum.
template <int NT>
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
    for (int i = 0; i < NT / 64; ++i) {
        if (i < w) off += wsum[i];
        tot += wsum[i];
    }
    *total = tot;
    return off + inc - v;
}

// Prefix survivals of all N = B*gamma candidates into vals[] (LDS, fp32 bit
// patterns, index b*gamma + k-1): the inputs (z, or the given survivals) are
// read with coalesced loads, then one thread per row runs the product, and
// with z the results go out to surv with coalesced stores.  Ends with a
// barrier.
template <int NT>
__device__ __forceinline__ void survival_lds(const float* __restrict__ z, const float* __restrict__ temps, int B,
                                             int gamma, float* surv, uint32_t* vals, float* tsh)
{
    const int t = threadIdx.x, N = B * gamma;
    const float* src = z ? z : surv;
    for (int i = t; i < N; i += NT) vals[i] = __float_as_uint(src[i]);
    if (z && t < gamma) tsh[t] = temps[t];
    __syncthreads();
    if (z) {
        for (int b = t; b < B; b += NT) {
            float th = 1.0f;
            for (int kk = 0; kk < gamma; ++kk) {
                const float q = __uint_as_float(vals[b * gamma + kk]) / tsh[kk];
                const float c = 1.0f / (1.0f + expf(-q));
                th = th * c;
                vals[b * gamma + kk] = __float_as_uint(th);  // the row's own slots only
            }
        }
        __syncthreads();
        for (int i = t; i < N; i += NT) surv[i] = __uint_as_float(vals[i]);
    }
    __syncthreads();
}

// LDS of budget_select besides the N keys.
template <int NT>
struct SelectScratch {
    uint32_t hist[256];
    int wsum[NT / 64];
    float tsh[kMaxGamma];
    uint32_t prefix;
    long long rem;
};

// The budget schedule of one workgroup of NT threads: survivals to surv (or
// read from it when z is null), then the first `admit` candidates of the
// order (Theta desc, b asc, k asc) admitted and len[b] = admitted count of
// row b.  keys: LDS for N = B*gamma words.
template <int NT>
__device__ void budget_select(const float* __restrict__ z, const float* __restrict__ temps, int B, int gamma,
                              long long admit, float* surv, int32_t* __restrict__ len, uint32_t* keys,
                              SelectScratch<NT>& sc)
{
    static_assert(NT % 256 == 0 && NT <= 1024, "one digit per thread in the bin scan");
    const int t = threadIdx.x;
    const int N = B * gamma;

    survival_lds<NT>(z, temps, B, gamma, surv, keys, sc.tsh);
    for (int i = t; i < N; i += NT) keys[i] = order_key(__uint_as_float(keys[i]));
    __syncthreads();

    if (admit <= 0 || admit >= N) {
        const int l = admit <= 0 ? 0 : gamma;
        for (int b = t; b < B; b += NT) len[b] = l;
        return;
    }

    // Radix select of the admit-th largest key, most significant digit first.
    // Per pass: histogram of the current digit among keys matching the prefix
    // so far, then threads 0..255 scan the bins from the top digit down
    // (thread t holds digit 255 - t) and the one whose running count first
    // reaches the remaining rank selects its digit.
    if (t == 0) {
        sc.prefix = 0u;
        sc.rem = admit;
    }
    uint32_t mask = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = t; i < 256; i += NT) sc.hist[i] = 0u;
        __syncthreads();
        const uint32_t prefix = sc.prefix;
        const long long rem = sc.rem;
        for (int i = t; i < N; i += NT) {
            const uint32_t key = keys[i];
            if ((key & mask) == prefix) atomicAdd(&sc.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        int cnt = 0, inc = 0;
        if (t < 256) {
            cnt = (int)sc.hist[255 - t];
            inc = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int n = __shfl_up(inc, o, 64);
                if ((t & 63) >= o) inc += n;
            }
            if ((t & 63) == 63) sc.wsum[t >> 6] = inc;
        }
        __syncthreads();
        if (t < 256) {
            int off = 0;
            for (int i = 0; i < (t >> 6); ++i) off += sc.wsum[i];
            const long long upto = (long long)(off + inc);  // keys with digit >= 255 - t
            const long long above = upto - cnt;              // keys with digit >  255 - t
            if (above < rem && rem <= upto) {
                sc.rem = rem - above;
                sc.prefix = prefix | ((uint32_t)(255 - t) << shift);
            }
        }
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t kth = sc.prefix;      // key of the admit-th largest candidate
    const long long need_eq = sc.rem;    // how many candidates equal to it are admitted

    // Rank of each equal key in index order: contiguous segments per thread.
    const int per = (N + NT - 1) / NT;
    const int i0 = min(t * per, N), i1 = min(i0 + per, N);
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += keys[i] == kth;
    int tot = 0;
    int rank = block_excl_scan_int<NT>(eq, sc.wsum, &tot);
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
    for (int b = t; b < B; b += NT) {
        int l = 0;
        for (int kk = 0; kk < gamma; ++kk) l += (int)keys[b * gamma + kk];
        len[b] = l;
    }
}

}  // namespace dspark
