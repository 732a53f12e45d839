// dspark_tile.hpp -- bf16 Markov-bias tiles for gfx950 in vocabulary-major
// MFMA form.
//
//   f[m][n] = L_m[n] + sum_i A[x_m][i] * Bm[i][n]
//
// is computed as the transposed product D = Bm_tile^T . A_rows^T with
// v_mfma_f32_16x16x32_bf16: the MFMA row axis runs over vocabulary columns
// and its column axis over batch rows.  A tile is 64 vocabulary columns
// (four 16-column blocks vb); a wave covers 16*NBB batch rows (blocks bb).
//
// Operands:
//   B (batch rows)  lane (G = lane>>4, c = lane&15) holds A[x_row][32ks + 8G
//                   .. +7] of batch row c of block bb; all k of a wave's rows
//                   stay in registers for the whole launch.
//   A (Bm^T)        read from an LDS copy of the Bm tile (staged with
//                   global_load_lds_dwordx4) by ds_read_b64_tr_b16.
//   C (initial)     the L values, loaded from global memory straight into
//                   the accumulator layout (8-byte loads).
//
// Column map: element i of accumulator block vb in lane (G, c) is vocabulary
// column n0 + 16G + 4*(vb ^ (G&1)) + i of batch row c.  So each lane holds 16
// consecutive columns of one batch row per batch block, and a row's 64 tile
// columns sit in the four lanes c, c+16, c+32, c+48.  (The XOR with G's low
// bit makes the transpose reads of one instruction use both 8-byte halves of
// the 16-byte LDS chunks; with the row swizzle below, every 32 lanes of a
// transpose read then touch 64 distinct LDS banks.)
//
// Bit-exact recompute: an output element depends only on its initial value,
// its Bm column, its A row and the fixed k-step order, and it occupies the
// same (vocabulary row, batch column) position of the MFMA in the tile pass
// and in the one-row recompute, so both produce the same bits.
#pragma once

#include <type_traits>

#include "dspark_device.hpp"

namespace dspark {

constexpr int kTcols = 64;                   // vocabulary columns per tile
constexpr int kTrowBytes = kTcols * 2;       // 128 bytes per LDS row of a Bm tile
constexpr int kTileKmax = 256;
constexpr int kBmTileBytes = kTileKmax * kTrowBytes;  // 32 KB
constexpr int kTileWaves = 8;                // waves of a tile workgroup (32 rows each)
constexpr int kTileRows = 32 * kTileWaves;   // batch rows of a tile workgroup

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// Position of 16-byte chunk c inside LDS row k of a Bm tile is c ^ swz_k(k).
__device__ __forceinline__ int swz_k(int k) { return ((k >> 3) & 1) | (((k >> 1) & 1) << 1); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Offset (in columns, within the tile) of the 4 columns of accumulator block vb held by lane group G.
__device__ __forceinline__ int vm_col(int G, int vb) { return 16 * G + 4 * (vb ^ (G & 1)); }

// One buffer_load_dwordx4 ... lds per wave: lane i's 16 bytes, at byte
// offset voff from the wave-uniform base, land at lds_wave_dst + 16 i.
//
// Two details keep the compiler's vector-memory waits exact in the tile
// pipelines, whose loads into registers and into LDS are all outstanding at
// once: the MUBUF form is used rather than global_load_lds (a FLAT-encoded
// instruction that writes LDS makes the compiler treat the vector-memory
// counter as unordered and wait for zero), and the LDS address is passed
// through readfirstlane, so the compiler does not track the write against
// later LDS reads (its alias tracking cannot tell the staging buffers of one
// kernel apart and would wait for every outstanding load before each read).
// Every caller orders the DMA and the reads itself: wait_vmem / wait_all_mem
// (this wave's DMA done), then a workgroup barrier.
__device__ __forceinline__ void dma16(const uint16_t* base, uint32_t voff, char* lds_wave_dst)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_wave_dst);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(uintptr_t)a, 16, voff, 0, 0, 0);
}

// DMA the Bm tile starting at column n0 into buf: 32 blocks of 8 LDS rows,
// block w + NW*t issued by wave w (t < 32/NW, so every wave issues the same
// number of DMA instructions; NW == 1: the calling wave issues them all).  Rows >= r and chunks past V come from clamped
// (valid, finite) addresses: the A operand is zero for k >= r and columns >= V
// are masked.  `dummy` (wave-uniform) issues the same instructions with every
// lane reading Bm[0][0..7], for pipelines that keep a fixed number of
// outstanding loads past their last tile.  n0 must be wave-uniform; it is
// re-read from lane 0 so that the buffer descriptor provably is (a descriptor
// the compiler cannot prove uniform costs a loop over the lanes per load).
template <int NW>
__device__ __forceinline__ void dma_bm_tile(const uint16_t* __restrict__ Bm, int V, int r, int n0, bool dummy,
                                            char* buf)
{
    n0 = __builtin_amdgcn_readfirstlane(n0);
    dummy = __builtin_amdgcn_readfirstlane((int)dummy) != 0;
    // With NW == 1 the calling wave issues all 32 blocks, whichever wave of
    // its workgroup it is.
    const int w = NW == 1 ? 0 : wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < 32 / NW; ++t) {
        const int blk = w + NW * t;
        const int kb = min(8 * blk, r - 1);  // wave-uniform base row of the block
        const int k = min(8 * blk + (lane >> 3), r - 1);
        const int c = (lane & 7) ^ swz_k(8 * blk + (lane >> 3));
        const int col = min(n0 + 8 * c, V - 8);
        const uint16_t* base = dummy ? Bm : Bm + (size_t)kb * V + n0;
        const uint32_t voff = dummy ? 0u : (uint32_t)(((k - kb) * V + (col - n0)) * 2);
        dma16(base, voff, buf + blk * 1024);
    }
}

// dma_bm_tile for a pipeline that stages many tiles: the lane-dependent
// part of every DMA offset is computed once (BmDmaLanes) and a tile adds only
// its column clamp.  With c the lane's 16-byte chunk and k, kb its row and the
// wave-uniform base row of block blk,
//   voff = ((k - kb) V + min(n0 + 8c, V - 8) - n0) * 2
//        = 2 (k - kb) V + 2 min(8c, V - 8 - n0),
// the same addresses as dma_bm_tile.
template <int NW>
struct BmDmaLanes {
    uint32_t kv[32 / NW];  // 2 (k - kb) V
    int c8[32 / NW];       // 8c
    long long kbv[32 / NW];  // kb V, wave-uniform
};
template <int NW>
__device__ __forceinline__ BmDmaLanes<NW> bm_dma_lanes(int V, int r)
{
    BmDmaLanes<NW> d;
    const int w = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < 32 / NW; ++t) {
        const int blk = w + NW * t;
        const int kb = min(8 * blk, r - 1);
        const int k = min(8 * blk + (lane >> 3), r - 1);
        d.kv[t] = (uint32_t)((k - kb) * V * 2);
        d.kbv[t] = (long long)kb * V;
        d.c8[t] = 8 * ((lane & 7) ^ swz_k(8 * blk + (lane >> 3)));
    }
    return d;
}
template <int NW>
__device__ __forceinline__ void dma_bm_tile_pre(const uint16_t* __restrict__ Bm, int V, int r, int n0, bool dummy,
                                                char* buf, const BmDmaLanes<NW>& d)
{
    n0 = __builtin_amdgcn_readfirstlane(n0);
    dummy = __builtin_amdgcn_readfirstlane((int)dummy) != 0;
    const int w = wave_id();
    const int lim = V - 8 - n0;
#pragma unroll
    for (int t = 0; t < 32 / NW; ++t) {
        const int blk = w + NW * t;
        // Row kb of the block (wave-uniform), or Bm itself for a dummy: a
        // select, not a branch.
        const uint16_t* base = Bm + (dummy ? 0ll : d.kbv[t] + n0);
        const uint32_t voff = dummy ? 0u : d.kv[t] + 2u * (uint32_t)min(d.c8[t], lim);
        dma16(base, voff, buf + blk * 1024);
    }
}

// Block t (< 32 / NW) of this wave's share of dma_bm_tile_pre, alone: the
// pipelines spread a tile's DMA instructions over the MFMA chain.
template <int NW>
__device__ __forceinline__ void dma_bm_block_pre(const uint16_t* __restrict__ Bm, int V, int n0, bool dummy, char* buf,
                                                 const BmDmaLanes<NW>& d, int t)
{
    n0 = __builtin_amdgcn_readfirstlane(n0);
    dummy = __builtin_amdgcn_readfirstlane((int)dummy) != 0;
    const int blk = wave_id() + NW * t;
    const uint16_t* base = Bm + (dummy ? 0ll : d.kbv[t] + n0);
    const uint32_t voff = dummy ? 0u : d.kv[t] + 2u * (uint32_t)min(d.c8[t], V - 8 - n0);
    dma16(base, voff, buf + blk * 1024);
}

struct NoHook {
    __device__ void operator()(int) const {}
};

__device__ __forceinline__ v4s tr_read(const char* buf, int off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(buf + off));
}

// A operand (Bm^T) of k step ks, vocabulary block vb: lane (G', j) gets
// k = 32ks + 8G' .. +7 of tile column 16(j>>2) + 4(vb ^ ((j>>2)&1)) + (j&3).
// In each 16-lane group, source lane 4r+q addresses LDS row k0 + r at the
// four columns 16q + 4(vb ^ (q&1)) .. +3; rows k0 + 4 + r follow 512 bytes
// later (the swizzle of k0 and k0 + 4 is the same).  Only the lane part of
// the address depends on the lane: bm_lane_offsets computes it per vb, and
// k step ks adds 32 rows (4096 bytes) per step.
__device__ __forceinline__ void bm_lane_offsets(int (&off)[4])
{
    const int lane = threadIdx.x & 63;
    const int Gk = lane >> 4, r = (lane & 15) >> 2, q = lane & 3;
    const int k0 = 8 * Gk + r;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
        const int chunk = 2 * q + (vb >> 1), half = (vb ^ q) & 1;
        off[vb] = k0 * kTrowBytes + 16 * (chunk ^ swz_k(k0)) + 8 * half;
        // Opaque to the optimizer: every LDS read address is then this value
        // plus a constant, a short chain from the buffer.  (The LDS lowering
        // attributes an access to its buffer only through a few address
        // steps; a read it cannot attribute makes the compiler wait for every
        // outstanding LDS DMA before it.)
        asm("" : "+v"(off[vb]));
    }
}

__device__ __forceinline__ bf16x8 bm_frag(const char* bufB, const int (&off)[4], int ks, int vb)
{
    const v4s lo = tr_read(bufB, off[vb] + 32 * ks * kTrowBytes);
    const v4s hi = tr_read(bufB, off[vb] + 32 * ks * kTrowBytes + 4 * kTrowBytes);
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s v = { lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3] };
    return __builtin_bit_cast(bf16x8, v);
}

// B-operand fragments of NBB 16-row batch blocks for all k steps: lane l
// holds, for batch row (l & 15) of block bb, k = 32*ks + 8*(l>>4) .. +7
// (zero beyond r).
template <int NBB>
__device__ __forceinline__ void load_a_frags(const uint16_t* const (&arow)[NBB], int r, uint4 (&a)[NBB][8])
{
    const int kq8 = 8 * ((threadIdx.x & 63) >> 4);
    // A fixed number of loads, in k-step order (the MFMAs of k step ks can
    // start once its loads have landed): k >= r reads a valid address ...
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb) a[bb][ks] = ld16(arow[bb] + min(32 * ks + kq8, r - 8));
    // ... and is replaced by zeros.  Only ranks that are not a multiple of 32
    // have such slots; the (uniform) branch keeps the other ranks from waiting
    // for the loads here, so callers can issue more loads behind them.
    if (r & 31) {
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                if (32 * ks + kq8 >= r) a[bb][ks] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// The conditioning rows' A vectors in MFMA B-operand order ("Ag"), for rank
// 256: row R's 16-byte piece (k step ks, lane group G), A[x_R][32ks + 8G ..
// +7], lives at element ag_offset(R, ks, G), so the wave holding rows
// 16j .. 16j+15 as one batch block reads each k step as 1 KB contiguous
// (the gather from A reads half cache lines of 16 scattered rows instead).
__device__ __forceinline__ size_t ag_offset(int R, int ks, int G)
{
    return ((size_t)((R >> 4) * 8 + ks) * 64 + 16 * G + (R & 15)) * 8;
}

// Four bf16 values (8 bytes) -> floats.
__device__ __forceinline__ floatx4 bf16x4_to_f32(uint2 v)
{
    return floatx4{ __uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                    __uint_as_float(v.y & 0xFFFF0000u) };
}

__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Load the 16 values of one row that lane group G holds in a tile starting
// at column n0: raw[h] = columns n0 + 16G + 8h .. +7 (two 16-byte loads).  A
// load at or past V reads a clamped (valid) address; `dummy` reads the row
// start (fixed load count past the last tile).  The values are used through
// row16_block, after the loads have been waited for: doing the lane-dependent
// rearrangement here would make the compiler wait for the loads at once.
constexpr int kRow16Loads = 2;  // vector-memory loads issued by one load_row16

__device__ __forceinline__ void load_row16(const uint16_t* __restrict__ row, int n0, int V, bool dummy,
                                           uint4 (&raw)[2])
{
    const int G = (threadIdx.x & 63) >> 4;
    const int keep = dummy ? 0 : -1;  // branch-free: a dummy reads the row start
#pragma unroll
    for (int h = 0; h < 2; ++h) raw[h] = ld16(row + (min(n0 + 16 * G + 8 * h, V - 8) & keep));
}

// Per-lane select with a compile-time lane mask: lanes whose bit is set in
// `mask` take b, the others a.  Written as one v_cndmask so the compiler
// cannot turn a chain of lane-dependent selects over a register array into
// an indexed access (which it may place in scratch memory).
__device__ __forceinline__ uint32_t lane_select(uint32_t a, uint32_t b, uint64_t mask)
{
    uint32_t r;
    asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
    return r;
}
__device__ __forceinline__ float lane_select(float a, float b, uint64_t mask)
{
    return __uint_as_float(lane_select(__float_as_uint(a), __float_as_uint(b), mask));
}
// Lanes of odd lane group G = lane >> 4 (16..31, 48..63).
constexpr uint64_t kOddGroupLanes = 0xFFFF0000FFFF0000ull;

// Columns n0 + vm_col(G, vb) .. +3 (accumulator block vb) from load_row16's
// registers: for odd G the two 8-byte halves of each 16-byte load trade places.
__device__ __forceinline__ uint2 row16_block(const uint4 (&raw)[2], int vb)
{
    const uint4 x = raw[vb >> 1];
    const uint64_t high = (vb & 1) ? ~kOddGroupLanes : kOddGroupLanes;  // lanes taking the upper half
    return make_uint2(lane_select(x.x, x.z, high), lane_select(x.y, x.w, high));
}

// hook(ks) runs after the MFMAs of k step ks (KS > 0 only), in program order
// between scheduling fences: the pipelines issue their next tile's DMA there,
// so the address unit's queue, which all waves of a workgroup fill at once
// after each barrier, drains while the matrix unit is busy.
template <int NBB, int KS, class Hook = NoHook>
__device__ __forceinline__ void tile_mma_vm(const uint4 (&a)[NBB][8], const char* bufB, int nks,
                                            floatx4 (&acc)[4][NBB], Hook hook = Hook{})
{
    int off[4];
    bm_lane_offsets(off);
    if constexpr (KS > 0) {
        // The Bm^T fragments of k step ks+2 are read while the MFMAs of step
        // ks run: two steps of MFMAs cover the LDS latency of a workgroup
        // whose eight waves all read at once.
        bf16x8 b[4], b1[4], bn[4];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) b[vb] = bm_frag(bufB, off, 0, vb);
        if (KS > 1) {
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) b1[vb] = bm_frag(bufB, off, 1, vb);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) {
#pragma unroll
                for (int vb = 0; vb < 4; ++vb) bn[vb] = bm_frag(bufB, off, ks + 2, vb);
            }
            // Keep the reads of step ks+2 ahead of the MFMAs of step ks (the
            // scheduler would otherwise sink each read next to its use);
            // VALU, SALU and transcendental work may still move across.
            __builtin_amdgcn_sched_barrier(0x0406);
#pragma unroll
            for (int vb = 0; vb < 4; ++vb)
#pragma unroll
                for (int bb = 0; bb < NBB; ++bb)
                    acc[vb][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        b[vb], __builtin_bit_cast(bf16x8, a[bb][ks]), acc[vb][bb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0x0406);
            if constexpr (!std::is_same<Hook, NoHook>::value) {
                __builtin_amdgcn_sched_barrier(0);
                hook(ks);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                b[vb] = b1[vb];
                b1[vb] = bn[vb];
            }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (ks >= nks) break;
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                const bf16x8 b = bm_frag(bufB, off, ks, vb);
#pragma unroll
                for (int bb = 0; bb < NBB; ++bb)
                    acc[vb][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        b, __builtin_bit_cast(bf16x8, a[bb][ks]), acc[vb][bb], 0, 0, 0);
            }
        }
    }
}

// s_waitcnt encodings (gfx9 family): wait until at most n vector-memory
// operations of this wave are outstanding; LDS/scalar and export counters untouched.
template <int N> __device__ __forceinline__ void wait_vmem()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Stage wait of the tile pipelines, whose prefetch ramps up: the prologue
// issues [rows(0)] [Bm(0)] [NA other loads]; iteration 0 issues, after its
// barrier, [rows(1)] [Bm(1)] [Bm(2)] [Bm(3)]; iteration i >= 1 issues
// [rows(i+1)] [Bm(i+3)].  rows(.) is NL register loads and Bm(.) is ND DMA
// instructions, always issued (dummies past the last tile).  (Asking for only
// the first tile up front lets it arrive before the rest of the launch-wide
// burst of prefetches.)  Before the barrier of iteration i this wave's Bm(i)
// must have landed; the loads issued after it number NA (i = 0), 2ND (i = 1),
// 2ND + NL (i = 2) and 2(NL + ND) (i >= 3).  Vector-memory loads complete in
// order, so waiting until at most that many are outstanding is exact.
template <int NL, int ND, int NA>
__device__ __forceinline__ void wait_stage(int i)
{
    if (i >= 3) wait_vmem<2 * (NL + ND)>();
    else if (i == 2) wait_vmem<2 * ND + NL>();
    else if (i == 1) wait_vmem<2 * ND>();
    else wait_vmem<NA>();
}

// Scheduling fence: the compiler moves no instruction across it.  The tile
// pipelines put one between consecutive groups of loads, so the loads are
// issued in program order -- the order wait_stage's counts assume.
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier without a memory fence.  __syncthreads() also waits for
// every outstanding vector-memory load of the wave (its release fence), which
// would drain a multi-stage load pipeline; the tile pipelines only share LDS
// written by DMA, whose completion each wave establishes with wait_vmem
// before the barrier.
__device__ __forceinline__ void barrier_lds() { __builtin_amdgcn_s_barrier(); }

// Wait for every outstanding memory operation of this wave.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Wait for this wave's LDS operations only (vector-memory count untouched).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// A float pair as one 64-bit word: LDS staging stores it with a single
// ds_write_b64 whose alias information the compiler keeps (two float stores
// merged late lose it, and an LDS store without it waits for every
// outstanding vector-memory load).
__device__ __forceinline__ unsigned long long pack_f2(float x, float y)
{
    return (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
}
__device__ __forceinline__ float2 unpack_f2(unsigned long long v)
{
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Folds the (max, sum of exp relative to it) partials get(0 .. n-1) of
// consecutive tiles into the running pair (*m, *s) of the range before them:
// the range max, then every sum rescaled to it and added in tile order, in
// fp32.  Each factor is 2^((x - max) log2 e), the difference taken first (as
// tile_mass does), so a sum already relative to the max is multiplied by
// exactly 1 (a factor formed as x log2 e - max log2 e would carry the
// rounding of max log2 e, ~1e-6 at logits near 20, with the same sign into
// every rescale).  Partials without a finite value add nothing.
template <class Get>
__device__ __forceinline__ void fold_partials(float* m, float* s, int n, Get get)
{
    float mx = *m;
    for (int j = 0; j < n; ++j) mx = fmaxf(mx, get(j).x);
    float acc = 0.0f;
    if (mx != -INFINITY) {
        if (*m != -INFINITY) acc = *s * __builtin_amdgcn_exp2f((*m - mx) * kLog2e);
        for (int j = 0; j < n; ++j) {
            const float2 p = get(j);
            if (p.x != -INFINITY) acc += p.y * __builtin_amdgcn_exp2f((p.x - mx) * kLog2e);
        }
    }
    *m = mx;
    *s = acc;
}

// Tiles of persistent slot s of S over nT tiles: t0, t0 + ts, ... (cnt of
// them), a contiguous range per slot (ts = 1).  (Measured on MI355X at the
// 129280-column shape, contiguous ranges stream faster than slots
// interleaved tile by tile.)
__device__ __forceinline__ void slot_tiles(int s, int S, int nT, int* t0, int* ts, int* cnt)
{
    const int q = nT / S, rem = nT - q * S;
    *t0 = s * q + min(s, rem);
    *ts = 1;
    *cnt = q + (s < rem ? 1 : 0);
}

// Butterfly steps across 16-lane rows without LDS: the gfx950 permlane swaps
// exchange rows 0<->1 and 2<->3 (xor 16) or the wave halves (xor 32), so
// every lane sees its own value and its partner's.  Both lanes of a pair get
// op(a, b) of the same two values; for max and add the operand order does
// not change the result, so the pair ends with identical bits.
__device__ __forceinline__ void xor16_pair(float x, float* a, float* b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    *a = __uint_as_float(p[0]);
    *b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void xor32_pair(float x, float* a, float* b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    *a = __uint_as_float(p[0]);
    *b = __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor16_32(float s)
{
    float a, b;
    xor16_pair(s, &a, &b);
    xor32_pair(a + b, &a, &b);
    return a + b;
}
// max of two floats as one v_max_f32 (fmaxf would first quiet the operands,
// which the compiler cannot prove canonical after a lane swap; the values
// here are logits or -inf, never NaN).
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float max_xor16_32(float m)
{
    float a, b;
    xor16_pair(m, &a, &b);
    xor32_pair(vmax(a, b), &a, &b);
    return vmax(a, b);
}

// Row-wise max and sum of exp over the 64 columns of a tile held as 16
// values per lane (lanes c, c+16, c+32, c+48 hold one row).  With TAIL,
// values of columns at or past ncol count as absent (without it the code has
// no branch, so the compiler can interleave it with independent MFMAs).  All
// four lanes of the row receive the same bits: the max m (-inf if no finite
// value) and s = sum exp(f - m) (fp32, fixed order: per 4-column block in
// column order, the four block sums pairwise, then the xor-16 and xor-32
// butterflies).  Short dependency chains, and no LDS traffic, so the work
// fills the issue slots between independent MFMAs.
template <bool TAIL>
__device__ __forceinline__ void row64_max_sum(floatx4 (&v)[4], int ncol, float* m_out, float* s_out)
{
    const int G = (threadIdx.x & 63) >> 4;
    if (TAIL) {
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
            if (vm_col(G, vb) >= ncol) v[vb] = floatx4{ -INFINITY, -INFINITY, -INFINITY, -INFINITY };
    }
    // Three-input maxima, depth 3.
    const float t0 = fmaxf(fmaxf(v[0][0], v[0][1]), v[0][2]), t1 = fmaxf(fmaxf(v[0][3], v[1][0]), v[1][1]);
    const float t2 = fmaxf(fmaxf(v[1][2], v[1][3]), v[2][0]), t3 = fmaxf(fmaxf(v[2][1], v[2][2]), v[2][3]);
    const float t4 = fmaxf(fmaxf(v[3][0], v[3][1]), v[3][2]);
    const float mx = max_xor16_32(fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), v[3][3])));
    const float ml = row_mlog2(mx);
    float sb[4];
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
        sb[vb] = softmax_w(v[vb][0], ml);
#pragma unroll
        for (int i = 1; i < 4; ++i) sb[vb] += softmax_w(v[vb][i], ml);
    }
    *m_out = mx;
    *s_out = sum_xor16_32((sb[0] + sb[1]) + (sb[2] + sb[3]));
}

}  // namespace dspark
