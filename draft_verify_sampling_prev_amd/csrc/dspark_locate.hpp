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

// Mass of a (max m, sum of exp(x - m) = s) partial relative to the row max
// M >= m: s * 2^((m - M) log2 e) with the single-precision exponential.  The
// relative error is about 1e-7 * (1 + |m - M|), i.e. below 3e-6 for every
// partial within 30 of the max; farther ones weigh less than e^-30 of the
// row.  Partials without a finite value weigh 0.
__device__ __forceinline__ double tile_mass(float m, double s, float M)
{
    return m == -INFINITY ? 0.0 : s * (double)__builtin_amdgcn_exp2f((m - M) * kLog2e);
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
    static constexpr int kLdsBytes = kBmTileBytes;
};

// fp32: biased logits f = L_row + A[prev] . Bm of the tile starting at column
// n0, bit-identical to the fp32 tile kernel.  All threads of the 4-wave
// workgroup call; wave 0, lane l receives column 16*nb + (l & 15) in f[nb].
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

// bf16: biased logits of one row over the tile starting at column n0, in the
// vocabulary-major layout of the bf16 tile kernels (dspark_tile.hpp) and
// bit-identical to them: every batch column of the MFMA carries the row's A
// operand, and wave 0, lane (G, c) receives in f[vb][i] column
// n0 + vm_col(G, vb) + i.  All threads of the 4-wave workgroup call.
__device__ __forceinline__ void row_tile_vm(const uint16_t* L_row, const uint16_t* A, const uint16_t* Bm, int prev,
                                            int V, int r, int n0, char* lds, floatx4 (&f)[4])
{
    const bool w0 = (threadIdx.x >> 6) == 0;
    const int nks = (r + 31) / 32;
    dma_bm_tile<kThreads / 64>(Bm, V, r, n0, false, lds);
    uint4 a[1][8];
    uint4 lv[2];
    if (w0) {
        const uint16_t* arow[1] = { A + (size_t)prev * r };
        load_a_frags<1>(arow, r, a);
        load_row16(L_row, n0, V, false, lv);
    }
    wait_all_mem();
    __syncthreads();
    if (w0) {
        floatx4 acc[4][1];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) acc[vb][0] = bf16x4_to_f32(row16_block(lv, vb));
        if (nks == 8) tile_mma_vm<1, 8>(a, lds, nks, acc);
        else tile_mma_vm<1, 0>(a, lds, nks, acc);
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) f[vb] = acc[vb][0];
    }
    __syncthreads();  // LDS may be reused after this point
}

// One-wave form of row_tile_vm for kernels that run one wave per row: the
// wave stages the Bm tile in its own LDS buffer and waits only for its own
// loads (no barrier).  The A operand (a, k steps < nks) is loaded by the
// caller ahead of time.
template <int KS>
__device__ __forceinline__ void row_tile_vm_wave(const uint16_t* L_row, const uint4 (&a)[1][8], const uint16_t* Bm,
                                                 int V, int r, int n0, char* lds, floatx4 (&f)[4])
{
    dma_bm_tile<1>(Bm, V, r, n0, false, lds);
    uint4 lv[2];
    load_row16(L_row, n0, V, false, lv);
    wait_all_mem();
    floatx4 acc[4][1];
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) acc[vb][0] = bf16x4_to_f32(row16_block(lv, vb));
    tile_mma_vm<1, KS>(a, lds, (r + 31) / 32, acc);
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) f[vb] = acc[vb][0];
}

// One wave, masses held in registers: lane l owns the contiguous slice
// [i0, i0 + PER) (i0 = l * per, per <= PER <= 64; slots past the slice or
// past n must have mass 0) and mass(j) gives the mass of its slot j.  Same
// rule as locate(): the first index whose running mass exceeds u*S, else the
// last index of positive mass, else 0.
//
// Slice sums are combined by a wave scan in lane order.  The slice holding
// the crossing is the first lane whose inclusive sum exceeds tau; that
// lane's PER masses are then spread over lanes 0..PER-1 (through `scratch`,
// LDS with room for PER doubles) and scanned by a second wave scan from the
// slice's exclusive prefix, so no lane walks its slots one by one.  If
// rounding leaves every running sum in that slice at or below tau, its last
// slot of positive mass is taken.  With no crossing at all the last slice
// with positive mass is treated the same way.  The chosen slot always has
// positive mass (a crossing slot must, too).
template <int PER, class MassFn>
__device__ __forceinline__ Located wave_locate_slices(int i0, MassFn mass, float u, double* scratch)
{
    static_assert(PER <= 64, "one slot per lane in the second scan");
    const int lane = threadIdx.x & 63;
    Located L;
    double sl = 0.0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sl += mass(j);
    const double inc = wave_incl_scan(sl);
    const double off = wave_excl_from_incl(inc);
    L.S = wave_last(inc);
    L.tau = (double)u * L.S;
    // (A slice needs positive mass to hold the crossing: the two scans round
    // differently, so a slice of zero mass can sit just past tau.)
    const uint64_t mh = __ballot(inc > L.tau && sl > 0.0), mp = __ballot(sl > 0.0);
    if (!mh && !mp) {  // no mass at all
        L.idx = 0;
        L.cprev = 0.0;
        return L;
    }
    const int src = mh ? __builtin_ctzll(mh) : 63 - __builtin_clzll(mp);
    if (lane == src) {
#pragma unroll
        for (int j = 0; j < PER; ++j) scratch[j] = mass(j);
    }
    __builtin_amdgcn_wave_barrier();  // one wave: its LDS accesses complete in order
    const double mj = lane < PER ? scratch[lane] : 0.0;
    __builtin_amdgcn_wave_barrier();
    const double base = __shfl(off, src, 64);
    const int s0 = __shfl(i0, src, 64);
    const double ej = wave_incl_scan(mj);
    const double cj = base + ej, cb = base + wave_excl_from_incl(ej);
    const uint64_t hj = mh ? __ballot(lane < PER && mj > 0.0 && cj > L.tau) : 0ull;
    const uint64_t pj = __ballot(lane < PER && mj > 0.0);
    const int j = hj ? __builtin_ctzll(hj) : 63 - __builtin_clzll(pj);
    L.idx = s0 + j;
    L.cprev = __shfl(cb, j, 64);
    return L;
}

// Lane l's slice [l*per, l*per + PER) of a row of n float2 entries, loaded
// with every load in flight at once (clamped addresses); slots past the
// slice or past n get `pad`.
template <int PER>
__device__ __forceinline__ void load_slices(const float2* __restrict__ row, int n, float2 pad, float2 (&q)[PER],
                                            int* i0_out)
{
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) / 64;
    const int i0 = lane * per;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const float2 v = row[min(i0 + j, n - 1)];
        q[j] = (j < per && i0 + j < n) ? v : pad;
    }
    *i0_out = i0;
}

// One-wave kernels whose 16 MFMA batch columns all hold the same row (the A
// operand and the L row are broadcast to every column), with the tile's 64
// values held as row_tile_vm_wave leaves them: lane L takes tile column L,
// which is element L & 3 of stored block ((L >> 2) & 3) ^ ((L >> 4) & 1) in
// its own registers.  wfn(col, pick) returns the weight of column col and
// reads the lane's values through pick(x), x a floatx4[4] array in that
// layout.  Running weights in column order come from one wave scan; the
// result is the first column of positive weight where cprev + scale * run
// exceeds tau, else the last column of positive weight, else 0, and *w_sel
// receives its weight.
// Lanes L whose tile column L is held in stored block vb.
constexpr uint64_t scan_lanes_of_block(int vb)
{
    uint64_t m = 0;
    for (int L = 0; L < 64; ++L)
        if ((((L >> 2) & 3) ^ ((L >> 4) & 1)) == vb) m |= 1ull << L;
    return m;
}

template <class WFn>
__device__ __forceinline__ int scan_row_tile_lanes(int n0, double scale, double cprev, double tau, WFn wfn,
                                                   double* w_sel)
{
    const int lane = threadIdx.x & 63;
    // Lane L needs element L & 3 of block ((L >> 2) & 3) ^ ((L >> 4) & 1):
    // selects with compile-time lane masks.
    auto pick = [&](const floatx4(&x)[4]) {
        floatx4 blk = x[0];
#pragma unroll
        for (int vb = 1; vb < 4; ++vb) {
            const uint64_t m = scan_lanes_of_block(vb);
#pragma unroll
            for (int i = 0; i < 4; ++i) blk[i] = lane_select(blk[i], x[vb][i], m);
        }
        float v = blk[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) v = lane_select(v, blk[i], 0x1111111111111111ull << i);
        return v;
    };
    const double w = wfn(n0 + lane, pick);
    const double run = wave_incl_scan(w);
    const uint64_t mh = __ballot(w > 0.0 && cprev + scale * run > tau);
    const uint64_t mp = __ballot(w > 0.0);
    int col = 0;
    if (mh) col = __builtin_ctzll(mh);
    else if (mp) col = 63 - __builtin_clzll(mp);
    const double ws = __shfl(w, col, 64);
    *w_sel = (mh | mp) ? ws : 0.0;
    return col;
}

// Wave 0: inverse-CDF scan of a 64-column tile held as by row_tile_vm.  The
// row is read from MFMA batch column pos & 15, i.e. lanes 16G + (pos & 15),
// G = 0..3 (every column holds the same row, so any pos gives the same
// bits).  wfn(vb, i, col) gives the
// weight of the lane's element i of block vb, which is column col (the
// function returns 0 for col >= V).  Returns the tile column where
// cprev + scale * (running weight in column order) first exceeds tau, else
// the last column of positive weight, else 0; *w_sel receives its weight.
template <class WFn>
__device__ __forceinline__ int scan_vm_tile(int n0, int pos, double scale, double cprev, double tau, WFn wfn,
                                            double* w_sel)
{
    const int lane = threadIdx.x & 63, G = lane >> 4, c = lane & 15, cp = pos & 15;
    // Weights per stored block (compile-time block index, so the caller's
    // register arrays are indexed statically), then put in column order: the
    // lane's column group q4 is stored in block q4 ^ (G & 1).
    double ws[4][4];
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ws[vb][i] = wfn(vb, i, n0 + vm_col(G, vb) + i);
    const bool odd = (G & 1) != 0;
    double w[16];
    double tot = 0.0;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[4 * q4 + i] = odd ? ws[q4 ^ 1][i] : ws[q4][i];
            tot += w[4 * q4 + i];
        }
    const double t0 = __shfl(tot, cp, 64), t1 = __shfl(tot, 16 + cp, 64), t2 = __shfl(tot, 32 + cp, 64);
    double run = G == 0 ? 0.0 : (G == 1 ? t0 : (G == 2 ? t0 + t1 : (t0 + t1) + t2));
    int hit = -1, last = -1;
    double whit = 0.0, wlast = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        run += w[j];
        if (hit < 0 && cprev + scale * run > tau) {
            hit = 16 * G + j;
            whit = w[j];
        }
        if (w[j] > 0.0) {
            last = 16 * G + j;
            wlast = w[j];
        }
    }
    const uint64_t mh = __ballot(c == cp && hit >= 0);
    const uint64_t mp = __ballot(c == cp && last >= 0);
    int src, col;
    if (mh) {
        src = __builtin_ctzll(mh);
        col = __shfl(hit, src, 64);
        *w_sel = __shfl(whit, src, 64);
    } else if (mp) {
        src = 63 - __builtin_clzll(mp);
        col = __shfl(last, src, 64);
        *w_sel = __shfl(wlast, src, 64);
    } else {
        col = 0;
        *w_sel = 0.0;
    }
    return col;
}

}  // namespace dspark
