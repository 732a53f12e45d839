// dspark_tile.hpp -- bf16 Markov-bias tiles for gfx950, staged by LDS DMA.
//
//   f[m][n] = sum_i A[x_m][i] * Bm[i][n]   (+ L_m[n] added after the MFMAs)
//
// Tile = 64 vocabulary columns.  A workgroup of NW wave64s covers 32*NW rows;
// each wave owns 32 rows (two 16-row MFMA blocks, v_mfma_f32_16x16x32_bf16)
// and the 64 columns (four 16-column blocks).  The wave's A operand (its 32
// gathered A rows, all k <= 256) stays in registers for the whole launch.
//
// Staging: the Bm tile (k rows x 64 columns, 128 bytes per row) and the
// logit tiles (rows x 64 columns) are copied global -> LDS with
// global_load_lds_dwordx4 (no registers involved): each wave instruction
// writes 1 KB = 8 LDS rows, lane l landing at byte 16*l, while its global
// address is free, which is used to XOR-swizzle the eight 16-byte chunks of
// each row.  Kernels double-buffer the staging so the DMA of the next tile
// runs under the MFMAs of the current one.
//
// Operand fetch with ds_read_b64_tr_b16: inside a 16-lane group, source lane
// 4r+q addresses row r, columns 4q..4q+3 of a 4x16 block and lane j receives
// column j of rows 0..3.  Two such reads give the B operand of a lane (8
// consecutive k of one column); one read gives the four logit values a lane
// needs in the MFMA accumulator layout (4 consecutive rows of one column).
// With the swizzles below, every transpose read touches each LDS bank once
// per 32 lanes.
//
// Accumulator layout: acc[mb][nb][i] holds row 16*mb + 4*(lane>>4) + i of the
// wave and tile column 16*nb + (lane&15).  An element depends only on its own
// A row, Bm column and the fixed k-step order, so recomputing one row with
// tile_mma64<1> reproduces it bit for bit.
#pragma once

#include "dspark_device.hpp"

namespace dspark {

constexpr int kTcols = 64;                   // vocabulary columns per tile
constexpr int kTrowBytes = kTcols * 2;       // 128 bytes per LDS row
constexpr int kTileKmax = 256;
constexpr int kBmTileBytes = kTileKmax * kTrowBytes;  // 32 KB

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// Position of 16-byte chunk c inside LDS row k of a Bm tile / row `row` of a logit tile.
__device__ __forceinline__ int swz_k(int k) { return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2); }
__device__ __forceinline__ int swz_row(int row) { return (((row >> 1) & 1) << 1) | (((row >> 2) & 1) << 2); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ void dma16(const void* g, char* lds_wave_dst)
{
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_dst, 16, 0, 0);
}

// DMA rows [0, kr) (kr a multiple of 32) of the Bm tile starting at column n0.
// Rows >= r and chunks past V are fetched from clamped (valid, finite)
// addresses: the A operand is zero for k >= r, and columns >= V are masked.
template <int NW>
__device__ __forceinline__ void dma_bm_tile(const uint16_t* __restrict__ Bm, int V, int r, int n0, int kr, char* buf)
{
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int nblk = kr >> 3;
    for (int blk = w; blk < nblk; blk += NW) {
        const int k = 8 * blk + (lane >> 3);
        const int c = (lane & 7) ^ swz_k(k);
        const int col = min(n0 + 8 * c, V - 8);
        dma16(Bm + (size_t)min(k, r - 1) * V + col, buf + blk * 1024);
    }
}

// DMA a logit tile of 32*NW rows: lane row 8*(w + NW*t) + (lane >> 3) comes
// from global row ridx[t] (row stride V), columns n0..n0+63.
template <int NW>
__device__ __forceinline__ void dma_row_tile(const uint16_t* __restrict__ base, const int (&ridx)[4], int V, int n0,
                                             char* buf)
{
    const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int blk = w + NW * t;
        const int row = 8 * blk + (lane >> 3);
        const int c = (lane & 7) ^ swz_row(row);
        const int col = min(n0 + 8 * c, V - 8);
        dma16(base + (size_t)ridx[t] * V + col, buf + blk * 1024);
    }
}

// Tile row handled by this lane in dma_row_tile for slot t.
template <int NW> __device__ __forceinline__ int dma_row_of(int t)
{
    return 8 * ((int)(threadIdx.x >> 6) + NW * t) + ((int)(threadIdx.x & 63) >> 3);
}

__device__ __forceinline__ v4s tr_read(const char* buf, int off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(buf + off));
}

// B operand of k step ks, column block nb: lane (g = lane>>4, j = lane&15)
// gets k = 32ks + 8g .. +7 of tile column 16nb + j.
__device__ __forceinline__ bf16x8 b_frag(const char* bufB, int ks, int nb)
{
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15, r = j >> 2, q = j & 3;
    const int c = 2 * nb + (q >> 1);
    const int k0 = 32 * ks + 8 * g + r, k1 = k0 + 4;
    const v4s lo = tr_read(bufB, k0 * kTrowBytes + 16 * (c ^ swz_k(k0)) + 8 * (q & 1));
    const v4s hi = tr_read(bufB, k1 * kTrowBytes + 16 * (c ^ swz_k(k1)) + 8 * (q & 1));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s v = { lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3] };
    return __builtin_bit_cast(bf16x8, v);
}

// Logit values in accumulator layout: lane (g, j) gets rows row0 + 4g + 0..3
// of tile column 16nb + j (row0 a multiple of 16), as floats.
__device__ __forceinline__ floatx4 row_vals(const char* bufR, int row0, int nb)
{
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15, r = j >> 2, q = j & 3;
    const int c = 2 * nb + (q >> 1);
    const int row = row0 + 4 * g + r;
    const v4s v = tr_read(bufR, row * kTrowBytes + 16 * (c ^ swz_row(row)) + 8 * (q & 1));
    floatx4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float((uint32_t)(uint16_t)v[i] << 16);
    return o;
}

// A-operand fragments of MB 16-row blocks for all k steps: lane l holds, for
// row (l & 15) of block mb, k = 32*ks + 8*(l>>4) .. +7 (zero beyond r).
template <int MB>
__device__ __forceinline__ void load_a_frags(const uint16_t* const (&arow)[MB], int r, uint4 (&a)[MB][8])
{
    const int kq8 = 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int k = 32 * ks + kq8;
            a[mb][ks] = k < r ? ld16(arow[mb] + k) : make_uint4(0u, 0u, 0u, 0u);
        }
}

// acc[mb][nb] += A block mb x Bm tile over k steps 0..nks-1 (B operand from
// LDS).  KS > 0 fixes the number of k steps at compile time (straight-line
// code, which also keeps the compiler's LDS-DMA alias tracking precise);
// KS == 0 takes nks at run time.
template <int MB, int KS>
__device__ __forceinline__ void tile_mma64(const uint4 (&a)[MB][8], const char* bufB, int nks,
                                           floatx4 (&acc)[MB][4])
{
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (KS > 0 ? ks >= KS : ks >= nks) break;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const bf16x8 b = b_frag(bufB, ks, nb);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[mb][ks]), b,
                                                                      acc[mb][nb], 0, 0, 0);
        }
    }
}

// Wait for this wave's outstanding DMA / memory operations.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Persistent double-buffered tile loop: tiles first, first + S, ... < nT.
// issue(tile, buf) starts the DMA of a tile into a buffer, compute(tile, buf)
// consumes it.  b0 and b1 must be two distinct __shared__ arrays and the loop
// is unrolled by two, so each compute statically reads one array while the
// DMA into the other is in flight; the compiler can then see that they do
// not alias and does not make the LDS reads wait for that DMA.
//
// flush() runs right after each loop-top barrier, before the next DMA is
// issued: kernels use it to store results kept in registers from earlier
// tiles, so those stores drain during a whole iteration instead of being
// waited for at the next loop top.
template <class IssueFn, class ComputeFn, class FlushFn>
__device__ __forceinline__ void persistent_tiles(int first, int nT, int S, char* b0, char* b1, IssueFn issue,
                                                 ComputeFn compute, FlushFn flush)
{
    int tile = first;
    if (tile >= nT) return;
    issue(tile, b0);
    for (;;) {
        wait_all_mem();
        __syncthreads();  // this tile has landed in b0; every wave is done with b1
        flush();
        if (tile + S < nT) issue(tile + S, b1);
        compute(tile, b0);
        tile += S;
        if (tile >= nT) break;
        wait_all_mem();
        __syncthreads();
        flush();
        if (tile + S < nT) issue(tile + S, b0);
        compute(tile, b1);
        tile += S;
        if (tile >= nT) break;
    }
}

}  // namespace dspark
