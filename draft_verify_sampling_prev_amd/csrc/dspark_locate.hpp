// dspark_locate.hpp -- inverse-CDF location over per-tile partial masses and
// bit-identical recomputation of one row of one Markov tile.
//
// Sampling rule: token = min{ j : C_j > u*S } with C_j the running mass in
// vocabulary order (fallback: last index of positive weight).  The running
// mass is split into tile masses (combined per thread in tile order, then
// across threads by a fixed-order exclusive scan) and the weights inside the
// chosen tile (recomputed by the same instruction sequence that produced the
// tile's partial, then scanned in index order).  All sums are fp64.
#pragma once

#include <limits.h>

#include "dspark_device.hpp"
#include "dspark_markov.hpp"
#include "dspark_tile.hpp"

namespace dspark {

// Mass of a (max m, sum of exp(x - m) = s) partial relative to the row max M;
// partials without a finite value weigh 0.
__device__ __forceinline__ double tile_mass(float m, double s, float M)
{
    return m == -INFINITY ? 0.0 : s * exp_to_double((double)m - (double)M);
}

struct Located {
    double S;      // total mass
    double tau;    // u * S
    int idx;       // chosen tile / chunk
    double cprev;  // running mass before it
};

// All threads.  mass(i) >= 0 for i in [0, n).
template <class MassFn>
__device__ __forceinline__ Located locate(int n, MassFn mass, float u, BlockScratch& bs, double* sh_cprev)
{
    const int t = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int i0 = min(t * per, n), i1 = min(i0 + per, n);
    Located L;
    double sloc = 0.0;
    for (int i = i0; i < i1; ++i) sloc += mass(i);
    const double off = block_excl_scan(sloc, bs, &L.S);
    L.tau = (double)u * L.S;
    int hit = INT_MAX, lastpos = -1;
    double c = off, cph = 0.0, cpl = 0.0;
    for (int i = i0; i < i1; ++i) {
        const double mi = mass(i);
        const double cb = c;
        c += mi;
        if (hit == INT_MAX && c > L.tau) {
            hit = i;
            cph = cb;
        }
        if (mi > 0.0) {
            lastpos = i;
            cpl = cb;
        }
    }
    if (t == 0) *sh_cprev = 0.0;
    const int th = block_min_int(hit, bs);
    const int tl = block_max_int(lastpos, bs);
    const bool use_hit = th != INT_MAX;
    L.idx = use_hit ? th : max(tl, 0);
    if (use_hit ? (hit == L.idx) : (tl >= 0 && lastpos == L.idx)) *sh_cprev = use_hit ? cph : cpl;
    __syncthreads();
    L.cprev = *sh_cprev;
    return L;
}

// Wave 0, lanes 0..15: w[nb] is the weight of column 16*nb + lane of the
// chosen tile (NB blocks of 16 columns).  Returns the column where
// cprev + scale * (running weight) first exceeds tau, or the last column of
// positive weight; *w_sel receives that column's weight.
template <int NB>
__device__ __forceinline__ int scan_tile_weights(const double (&w)[NB], double scale, double cprev, double tau,
                                                 double* w_sel)
{
    const int lane = threadIdx.x & 63, l16 = lane & 15;
    double carry = 0.0;
    int jhit = -1, jlast = -1;
    double whit = 0.0, wlast = 0.0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const double cum = carry + scan16(w[nb]);
        carry = __shfl(cum, 15, 16);
        const uint64_t mc = __ballot(cprev + scale * cum > tau) & 0xFFFFull;
        const uint64_t mp = __ballot(w[nb] > 0.0) & 0xFFFFull;
        if (jhit < 0 && mc) {
            const int ls = __builtin_ctzll(mc);
            jhit = 16 * nb + ls;
            whit = __shfl(w[nb], ls, 64);
        }
        if (mp) {
            const int ls = 63 - __builtin_clzll(mp);
            jlast = 16 * nb + ls;
            wlast = __shfl(w[nb], ls, 64);
        }
    }
    *w_sel = jhit >= 0 ? whit : wlast;
    return jhit >= 0 ? jhit : max(jlast, 0);
}

// Per-dtype tile geometry of the Markov pass: columns per tile (the
// granularity of the softmax partials) and the LDS the recompute needs.
template <class DT> struct TileTraits;
template <> struct TileTraits<F32> {
    static constexpr int kCols = kTileN;  // 128
    static constexpr int kNB = kCols / 16;
    static constexpr int kLdsBytes = markov_lds_bytes<F32>();
};
template <> struct TileTraits<Bf16> {
    static constexpr int kCols = kTcols;  // 64
    static constexpr int kNB = kCols / 16;
    static constexpr int kLdsBytes = kBmTileBytes;
};

// Biased logits f = L_row + A[prev] . Bm of the tile starting at column n0,
// bit-identical to the tile kernel of the same dtype.  All threads of the
// 4-wave workgroup call; wave 0, lane l receives column 16*nb + (l & 15) in f[nb].
__device__ __forceinline__ void row_tile_f(const float* L_row, const float* A, const float* Bm, int prev, int V, int r,
                                           int n0, char* lds, float (&f)[TileTraits<F32>::kNB])
{
    const int lane = threadIdx.x & 63;
    const float* arow[1] = { A + (size_t)prev * r };
    floatx4 acc[1][8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int col = n0 + 16 * nb + (lane & 15);
        const float v = col < V ? L_row[col] : 0.0f;
        acc[0][nb] = floatx4{ v, v, v, v };
    }
    markov_tile<F32, 1>(Bm, V, r, n0, arow, (threadIdx.x >> 6) == 0, lds, acc);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) f[nb] = acc[0][nb][0];
}

__device__ __forceinline__ void row_tile_f(const uint16_t* L_row, const uint16_t* A, const uint16_t* Bm, int prev,
                                           int V, int r, int n0, char* lds, float (&f)[TileTraits<Bf16>::kNB])
{
    const int lane = threadIdx.x & 63;
    const bool w0 = (threadIdx.x >> 6) == 0;
    const int nks = (r + 31) / 32;
    dma_bm_tile<kThreads / 64>(Bm, V, r, n0, 32 * nks, lds);
    uint4 a[1][8];
    float lv[4];
    if (w0) {
        const uint16_t* arow[1] = { A + (size_t)prev * r };
        load_a_frags<1>(arow, r, a);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int col = n0 + 16 * nb + (lane & 15);
            lv[nb] = col < V ? Bf16::to_f32(L_row[col]) : 0.0f;
        }
    }
    wait_all_mem();
    __syncthreads();
    if (w0) {
        floatx4 acc[1][4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[0][nb] = floatx4{ 0.f, 0.f, 0.f, 0.f };
        if (nks == 8) tile_mma64<1, 8>(a, lds, nks, acc);
        else tile_mma64<1, 0>(a, lds, nks, acc);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) f[nb] = acc[0][nb][0] + lv[nb];
    }
    __syncthreads();  // LDS may be reused after this point
}

}  // namespace dspark
