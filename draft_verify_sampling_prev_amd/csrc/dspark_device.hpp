// dspark_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// element traits, 128-bit loads, Philox-4x32-10 uniforms, exponentials and
// wavefront / workgroup reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dspark {

constexpr int kThreads = 256;  // every kernel except the schedule uses 4 wave64s
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLog2eD = 1.4426950408889634074;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element traits.  Logits, A and Bm share one element type per call.
// ---------------------------------------------------------------------------
struct Bf16 {
    typedef uint16_t T;            // raw bfloat16 bits
    static constexpr int kPerVec = 8;   // elements per 16-byte vector
    __device__ static __forceinline__ float to_f32(T h) { return __uint_as_float((uint32_t)h << 16); }
    // element j of a 16-byte vector
    __device__ static __forceinline__ float get(const uint4& v, int j)
    {
        uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
        return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};

struct F32 {
    typedef float T;
    static constexpr int kPerVec = 4;
    __device__ static __forceinline__ float to_f32(T h) { return h; }
    __device__ static __forceinline__ float get(const uint4& v, int j)
    {
        uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
        return __uint_as_float(w);
    }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Markov-conditioned confidence logit of one draft position (the linear
// confidence head's token part; paperlayer.ai summary, Appendix A: the Markov
// confidence head sees the previously sampled token):
//     z[i] = z0[i] + <A[x], wc>.
// One wave: lane l multiplies elements 4l .. 4l+3 (r <= 256, a multiple of 8)
// in order with fused multiply-adds, the lane sums are added by the xor
// butterflies 32, 16, ..., 1, and lane 0 stores.  z == nullptr: nothing.
struct ConfOut {
    const float* z0;
    const void* wc;
    float* z;
};

template <class DT>
__device__ __forceinline__ void markov_confidence(const typename DT::T* __restrict__ A, const ConfOut& co, int x,
                                                  int r, int i)
{
    const int lane = threadIdx.x & 63;
    const auto* wc = static_cast<const typename DT::T*>(co.wc);
    float s = 0.0f;
    if (4 * lane < r) {
        const typename DT::T* a = A + (size_t)x * r + 4 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) s = __builtin_fmaf(DT::to_f32(a[j]), DT::to_f32(wc[4 * lane + j]), s);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) co.z[i] = co.z0[i] + s;
}

// ---------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// 4-word S-box with multipliers 0xD2511F53 / 0xCD9E8D57 and a key advanced by
// the Weyl increments 0x9E3779B9 / 0xBB67AE85 after each round.  Counter
// (k, b, draw, 0), key (lo32 seed, hi32 seed); the uniform is the top 24 bits
// of output word 0 times 2^-24.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t b, uint32_t k, uint32_t draw)
{
    uint32_t w0 = k, w1 = b, w2 = draw, w3 = 0u;
    uint32_t key_lo = (uint32_t)seed, key_hi = (uint32_t)(seed >> 32);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t a0 = w0, a2 = w2;
        const uint32_t lo_a = 0xD2511F53u * a0, hi_a = __umulhi(0xD2511F53u, a0);
        const uint32_t lo_c = 0xCD9E8D57u * a2, hi_c = __umulhi(0xCD9E8D57u, a2);
        w0 = hi_c ^ w1 ^ key_lo;
        w2 = hi_a ^ w3 ^ key_hi;
        w1 = lo_c;
        w3 = lo_a;
        key_lo += 0x9E3779B9u;
        key_hi += 0xBB67AE85u;
    }
    return (float)(w0 >> 8) * 0x1p-24f;
}

// ---------------------------------------------------------------------------
// Exponentials.
//   exp_fast(x): e^x = 2^(x log2 e) with the hardware base-2 exponential;
//     used for the un-normalised softmax weights exp(x - m) inside the vocab
//     passes, where every weight is then summed in double.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Softmax weight exp(x - m) as 2^(x log2 e - mlog2) with one FMA, where
// mlog2 = m * log2 e rounded to float (m finite).  Every pass that sums the
// weights of a row segment and every pass that rescans that segment uses this
// expression with the same m, so they see the same weights bit for bit.
// x = -inf gives 0.
__device__ __forceinline__ float softmax_w(float x, float mlog2)
{
    return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mlog2));
}

// Reference exponent of a row segment with max m for softmax_w: m log2 e, or
// 0 when the segment has no finite value (every weight is then exp2(-inf) = 0).
__device__ __forceinline__ float row_mlog2(float m) { return m == -INFINITY ? 0.0f : m * kLog2e; }


// ---------------------------------------------------------------------------
// Reductions.  Within a 16-lane row (one MFMA output row group) they use DPP
// lane moves, which run on the VALU: a butterfly of quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror and row_mirror leaves the full
// reduction in every lane of the row; an inclusive scan uses row_shr by
// 1, 2, 4, 8 with zero fill.  Wave-wide reductions use xor-shuffles.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;

template <int CTRL> __device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ double dpp_d(double v)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFFll), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ float max16(float v)
{
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float sum16f(float v)
{
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ double sum16(double v)
{
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    return v;
}

// Inclusive prefix sum over the 16 lanes of each row, in lane order.
__device__ __forceinline__ double scan16(double v)
{
    v += dpp_d<kDppShr1>(v);
    v += dpp_d<kDppShr2>(v);
    v += dpp_d<kDppShr4>(v);
    v += dpp_d<kDppShr8>(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ int wave_min_int(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_max_int(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// DPP move restricted to the rows in ROWS (others read 0).
template <int CTRL, int ROWS> __device__ __forceinline__ double dpp_d_rows(double v)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xFFFFFFFFll), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Inclusive scan across the 64 lanes in lane order (fixed order,
// deterministic): row scans, then rows 1 and 3 add the last lane of rows 0
// and 2, then rows 2 and 3 add lane 31.
__device__ __forceinline__ double wave_incl_scan(double v)
{
    v = scan16(v);
    v += dpp_d_rows<kDppRowBcast15, 0xA>(v);
    v += dpp_d_rows<kDppRowBcast31, 0xC>(v);
    return v;
}

constexpr int kDppWaveShr1 = 0x138;  // lane i <- lane i-1 across the wave (lane 0 reads 0)

// Exclusive prefix from an inclusive scan: the inclusive value of the previous lane (0 in lane 0).
__device__ __forceinline__ double wave_excl_from_incl(double inc) { return dpp_d<kDppWaveShr1>(inc); }

// Value of lane 63 in every lane.
__device__ __forceinline__ double wave_last(double v)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), 63);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Workgroup (256 threads) reductions through a small LDS scratch.
struct BlockScratch {
    float f[kThreads / 64];
    double d[kThreads / 64];
    int i[kThreads / 64];
};

__device__ __forceinline__ float block_max(float v, BlockScratch& s)
{
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.f[w] = v;
    __syncthreads();
    float r = s.f[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, s.f[i]);
    return r;
}

// Sum in a fixed order: lanes by xor tree, then waves 0..3 in order.
__device__ __forceinline__ double block_sum(double v, BlockScratch& s)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.d[w] = v;
    __syncthreads();
    double r = s.d[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r += s.d[i];
    return r;
}

__device__ __forceinline__ int block_min_int(int v, BlockScratch& s)
{
    v = wave_min_int(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.i[w] = v;
    __syncthreads();
    int r = s.i[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = min(r, s.i[i]);
    return r;
}

__device__ __forceinline__ int block_max_int(int v, BlockScratch& s)
{
    v = wave_max_int(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.i[w] = v;
    __syncthreads();
    int r = s.i[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, s.i[i]);
    return r;
}

// Exclusive scan of one double per thread over the workgroup, in thread order.
// Returns the exclusive prefix; *total receives the sum of all threads.
__device__ __forceinline__ double block_excl_scan(double v, BlockScratch& s, double* total)
{
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    double inc = wave_incl_scan(v);
    double exc = __shfl_up(inc, 1, 64);
    if (lane == 0) exc = 0.0;
    __syncthreads();
    if (lane == 63) s.d[w] = inc;
    __syncthreads();
    double off = 0.0;
    for (int i = 0; i < w; ++i) off += s.d[i];
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) tot += s.d[i];
    *total = tot;
    return off + exc;
}

// Map a linear workgroup id to a logical id so that workgroups that run on
// the same XCD (hardware dispatches ids round-robin over the 8 XCDs) receive
// consecutive logical ids.  Ids past the last multiple of 8 keep their value.
__device__ __forceinline__ int xcd_logical_id(int id, int count)
{
    const int full = (count / 8) * 8;
    if (id >= full) return id;
    return (id % 8) * (count / 8) + id / 8;
}

}  // namespace dspark
