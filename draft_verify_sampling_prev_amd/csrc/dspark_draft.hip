// dspark_draft.hip -- one semi-autoregressive draft step on gfx950.
//
// The sequential stage samples the block left to right; position k is drawn
// from softmax(L[b,k,:] + A[x_{k-1}] Bm) where x_{k-1} is the token just
// sampled (x_0 the last committed token) -- paperlayer.ai summary of arXiv
// 2607.05147, section 3.1; llm-wiki.hwlabs.dev explainer, Markov-head
// diagram.  Each step is two launches:
//
//   k_draft_tiles   Markov MFMA tile fused with the vocabulary pass: per
//                   (row, tile) it writes the tile max m_t and
//                   s_t = sum exp(f - m_t) (both fp32, as one float2).  The
//                   biased logits f are never written to memory.  bf16:
//                   persistent kernel of 8-wave workgroups over 256-row x
//                   64-column tiles in vocabulary-major MFMA form
//                   (dspark_tile.hpp), one workgroup per CU, slots
//                   interleaved over the tiles; fp32: one 4-wave workgroup
//                   per 256-row x 128-column tile (dspark_markov.hpp).
//   k_draft_locate  one workgroup per request.  Combines the tile partials in
//                   tile order (fp64), draws u = U(seed, b, k, 0), finds the
//                   tile where the running mass passes u*S, recomputes that
//                   one tile with the same MFMA sequence (bit-identical f) and
//                   scans it in index order.  Inverse-CDF sampling at
//                   temperature 1: token = min{ j : C_j > u*S }.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "dspark_internal.hpp"
#include "dspark_locate.hpp"
#include "dspark_markov.hpp"
#include "dspark_select.hpp"
#include "dspark_tile.hpp"

namespace dspark {

// Conditioning token of request b at draft step k (1-based), clamped into the
// vocabulary so that an out-of-range caller token can never address outside A.
__device__ __forceinline__ int cond_token_raw(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                              int gamma, int k)
{
    return (k == 1) ? x0[b] : tok[b * gamma + (k - 2)];
}
__device__ __forceinline__ int clamp_token(int x, int V) { return min(max(x, 0), V - 1); }
__device__ __forceinline__ int cond_token(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                          int gamma, int k, int V)
{
    return clamp_token(cond_token_raw(x0, tok, b, gamma, k), V);
}

// Tile max m_t and s_t = sum exp(f - m_t) (fp32 within the tile) for the
// rows held in a wave's accumulators: f[mb][nb][i] is row 16mb + 4g + i,
// column 16nb + j of the tile (g = lane >> 4, j = lane & 15).  Columns at or
// beyond ncols count as absent (only when `tail`).  The row results of block
// mb are gathered so that lane (g, j < 4) holds row 4g + j in m[mb], s[mb].
// A row without a finite logit gets m = -inf, s = 0.
template <int MB, int NB>
__device__ __forceinline__ void tile_row_partials(const floatx4 (&f)[MB][NB], bool tail, int ncols, float (&m)[MB],
                                                  float (&s)[MB])
{
    const int j = threadIdx.x & 15;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        float mres = -INFINITY, sres = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float fv[NB];
            float mx = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                fv[nb] = (tail && 16 * nb + j >= ncols) ? -INFINITY : f[mb][nb][i];
                mx = fmaxf(mx, fv[nb]);
            }
            mx = max16(mx);
            const float ml = row_mlog2(mx);
            float sv = 0.0f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sv += softmax_w(fv[nb], ml);
            sv = sum16f(sv);
            mres = j == i ? mx : mres;
            sres = j == i ? sv : sres;
        }
        m[mb] = mres;
        s[mb] = sres;
    }
}

// ---------------------------------------------------------------------------
// fp32: one 4-wave workgroup per (128-column tile, 256-row block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_draft_tiles_f32(const float* __restrict__ L,
                                                              const float* __restrict__ A,
                                                              const float* __restrict__ Bm,
                                                              const int32_t* __restrict__ x0, const int32_t* tok,
                                                              const float* __restrict__ H, int B, int gamma, int V,
                                                              int r, int k, int nT, int nM, float2* __restrict__ part)
{
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<F32>()];
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int tile = lid / nM, mblk = lid % nM;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = tile * kTileN;
    const int mw0 = mblk * 256 + wave * 64;
    const bool compute = mw0 < B;

    const float* arow[4];
    floatx4 acc[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int ra = min(mw0 + 16 * mb + (lane & 15), B - 1);
        arow[mb] = H ? H + ((size_t)ra * gamma + (k - 1)) * r : A + (size_t)cond_token(x0, tok, ra, gamma, k, V) * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const float* lrow = L + ((size_t)min(row, B - 1) * gamma + (k - 1)) * V;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                acc[mb][nb][i] = (compute && row < B && col < V) ? lrow[col] : 0.0f;
            }
        }
    }
    markov_tile<F32, 4>(Bm, V, r, n0, arow, compute, lds, acc);
    if (!compute) return;
    float m[4], sv[4];
    tile_row_partials<4, 8>(acc, n0 + kTileN > V, V - n0, m, sv);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int row = mw0 + 16 * mb + 4 * (lane >> 4) + (lane & 15);
        if ((lane & 15) < 4 && row < B) part[(size_t)row * nT + tile] = make_float2(m[mb], sv[mb]);
    }
}

// ---------------------------------------------------------------------------
// bf16: persistent.  Workgroup `lid` owns row block mblk = lid % nM (256
// rows, 32 per wave) and the tiles of slot lid / nM (slot_tiles).
//
// Pipeline per tile i (one iteration; four LDS buffers s0..s3, the loop body
// unrolled so every copy reads and fills fixed buffers):
//   wait until Bm tile i has landed, barrier;
//   load the L values of tile i+1 into registers, DMA Bm tile i+3;
//   the epilogue (row max and sum of exp) of tile i-1, written to LDS
//   staging, while tile i's L values arrive; then acc = L values of tile i
//   and the MFMAs over Bm tile i.
// Every iteration issues the same number of loads (past the last tile they
// are dummies reading one location), so the wait for Bm tile i is a constant
// count of outstanding loads per wave (wait_stage).
// Staged partials are written out once at the end (coalesced float2 runs per
// row); keeping vector-memory stores out of the loop keeps the compiler's
// waits on the register loads exact.
// ---------------------------------------------------------------------------
constexpr int kPartTiles = 12;  // tiles per slot whose partials fit the LDS staging
// Full-batch launches (B a multiple of 256) may give a slot up to kManyTiles
// tiles: the staging is then written out every kPartTiles tiles (MANY).
constexpr int kManyTiles = 3 * kPartTiles;

// FULL: every row block holds 256 rows of the batch (B a multiple of 256),
// so every wave has rows and the body has no branch.  Otherwise a wave whose
// rows all lie past the batch skips the MFMAs and only issues its share of
// the Bm DMA (the two paths then leave the compiler less exact waits).
// The budget schedule in one workgroup of a draft launch (dspark_markov_draft_sched):
// its scratch first, then the keys, in a 32 KB LDS tile buffer of that launch.
static_assert(kTileRows == 256, "slot_agg_bytes sizes the slot aggregates for batches above one 256-row block");
constexpr int kSchedKeysOffset = 2048;  // bytes
constexpr int kSchedMaxKeys = (kBmTileBytes - kSchedKeysOffset) / 4;
static_assert(sizeof(SelectScratch<64 * kTileWaves>) <= kSchedKeysOffset, "select scratch");

template <int KS, bool FULL, bool MANY = false, bool SLOTS = false>
__global__ __launch_bounds__(64 * kTileWaves) void k_draft_tiles_bf16(
    const uint16_t* __restrict__ L, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, const uint16_t* __restrict__ ag,
    const uint16_t* __restrict__ H, int B, int gamma, int V, int r, int k, int nT, int nM, int S,
    float2* __restrict__ part, float2* __restrict__ sagg, SchedArg sa)
{
    constexpr int NW = kTileWaves, R = kTileRows;
    __shared__ __attribute__((aligned(1024))) char s0[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s1[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s2[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s3[kBmTileBytes];
    __shared__ unsigned long long stage[kPartTiles][R];  // float2 pairs, stored as one 64-bit word each
    // MANY with slot aggregates: row t's running (max, sum) over the tiles
    // already written out, touched by thread t only.
    __shared__ float2 run_agg[MANY && SLOTS ? R : 1];

    // With the schedule (one workgroup more than the S * nM tile workgroups,
    // see launch_draft_step) workgroup 0 runs it: dispatched first, it ends
    // early beside the tile workgroups, which take indices 1 .. S * nM.
    // (Measured on MI355X: 1.0 us per step faster than the last index.)
    const bool sched_wg = (int)gridDim.x > S * nM;  // uniform
    if (sched_wg && blockIdx.x == 0) {
        budget_select<64 * NW>(sa.z, sa.temps, B, gamma, sa.admit, sa.surv, sa.len,
                               reinterpret_cast<uint32_t*>(s0 + kSchedKeysOffset),
                               *reinterpret_cast<SelectScratch<64 * NW>*>(s0));
        return;
    }

    const int lid = xcd_logical_id(blockIdx.x - (sched_wg ? 1 : 0), gridDim.x - (sched_wg ? 1 : 0));
    const int mblk = lid % nM, slot = lid / nM;
    int t0, ts, cnt;
    slot_tiles(slot, S, nT, &t0, &ts, &cnt);
    if (cnt <= 0) return;  // uniform
    if constexpr (MANY && SLOTS) {
        if (threadIdx.x < R) run_agg[threadIdx.x] = make_float2(-INFINITY, 0.0f);
    }
    const int w = wave_id(), lane = threadIdx.x & 63, c = lane & 15;
    const int m0 = mblk * R;
    const int mw = m0 + 32 * w;  // first row of this wave
    const bool active = mw < B;

    uint4 a[2][8];  // B operand: the rows' A vectors (loaded in the prologue)
    const uint16_t* lrow[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) lrow[bb] = L + ((size_t)min(mw + 16 * bb + c, B - 1) * gamma + (k - 1)) * V;
    const int nks = KS > 0 ? KS : (r + 31) / 32;

    auto load_l = [&](int i, uint4 (&lv)[2][2]) {
        const bool dummy = i >= cnt;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) load_row16(lrow[bb], (t0 + i * ts) * kTcols, V, dummy, lv[bb]);
    };
    const BmDmaLanes<NW> dml = bm_dma_lanes<NW>(V, r);
    auto dma = [&](int i, char* buf) { dma_bm_tile_pre<NW>(Bm, V, r, (t0 + i * ts) * kTcols, i >= cnt, buf, dml); };
    auto dma_block = [&](int i, char* buf, int t) {
        dma_bm_block_pre<NW>(Bm, V, (t0 + i * ts) * kTcols, i >= cnt, buf, dml, t);
    };

    floatx4 fprev[4][2];
    int prev = -1;  // local index of the tile held in fprev
    // Row max and sum of exp of the tile held in fprev, written to the LDS
    // staging by every lane of the row (they hold the same bits, so the store
    // needs no lane predicate).  Inside the loop the tile is never the last
    // tile of the vocabulary (that one is each slot's last and is finished
    // after the loop), so that form has no branch at all.
    auto epilogue = [&](auto tail) {
        const int n0 = (t0 + prev * ts) * kTcols;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            floatx4 v[4];
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) v[vb] = fprev[vb][bb];
            float m, sum;
            row64_max_sum<decltype(tail)::value>(v, V - n0, &m, &sum);
            stage[MANY ? prev % kPartTiles : prev][32 * w + 16 * bb + c] = pack_f2(m, sum);
        }
    };
    // MANY (every wave active): the staged partials of tiles base .. base+11
    // are made visible (LDS wait, barrier) and written out; then every memory
    // operation of the wave is waited for, the loads in flight included, so
    // the stage waits that follow see no extra operations in flight (the
    // stores are complete) and keep their counts.  The staging rows are next
    // written after the barrier that opens the following iteration, which
    // every wave reaches only after its reads here.
    auto flush = [&](int base) {
        wait_lds();
        barrier_lds();
        for (int e = threadIdx.x; e < R * kPartTiles; e += 64 * NW) {
            const int row = e / kPartTiles, j = e - row * kPartTiles;
            part[(size_t)(m0 + row) * nT + t0 + (base + j) * ts] = unpack_f2(stage[j][row]);
        }
        if (SLOTS && threadIdx.x < R) {  // fold these tiles into the row's running slot aggregate
            float2 ra = run_agg[threadIdx.x];
            fold_partials(&ra.x, &ra.y, kPartTiles, [&](int j) { return unpack_f2(stage[j][threadIdx.x]); });
            run_agg[threadIdx.x] = ra;
        }
        wait_all_mem();
    };
    // L values of two tiles in flight: the four unrolled bodies alternate
    // between two register sets, so no copy waits on a load just issued.
    uint4 l0[2][2], l1[2][2];
    auto body = [&](auto has_prev, int i, const char* cur, char* nxt, uint4 (&lc)[2][2], uint4 (&ln)[2][2]) {
        if (KS > 0) wait_stage<2 * kRow16Loads, 32 / NW, 16>(i);
        else if (i == 0) wait_all_mem();  // run-time rank: the A-operand load count varies
        else wait_stage<2 * kRow16Loads, 32 / NW, 16>(i);
        barrier_lds();  // Bm tile i has landed in cur; every wave is done with nxt (tile i-1)
        issue_fence();
        load_l(i + 1, ln);
        issue_fence();
        if (i == 0) {  // ramp-up: tiles 1 and 2 (buffers s1, s2) behind tile 3
            dma(1, s1);
            issue_fence();
            dma(2, s2);
            issue_fence();
        }
        // Bm tile i+3: with a compile-time rank its four DMA instructions go
        // between the MFMAs below (after k steps 0, 2, 4, 6), still after this
        // iteration's L loads and before the next iteration's, so the waits
        // keep their counts.
        if constexpr (KS == 0) {
            dma(i + 3, nxt);
            issue_fence();
        }
        if (FULL || active) {
            // The previous tile's epilogue first: it needs no memory, so it
            // runs while this tile's L values are still arriving.  (Measured
            // on MI355X: giving the two waves of a SIMD opposite phase orders
            // was slower.)
            if constexpr (decltype(has_prev)::value) {
                epilogue(std::false_type{});
                issue_fence();
                if constexpr (MANY) {
                    // Tile i-1 filled the staging: write tiles i-12 .. i-1 out.
                    if (i % kPartTiles == 0) flush(i - kPartTiles);
                }
            }
            floatx4 acc[4][2];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int vb = 0; vb < 4; ++vb) acc[vb][bb] = bf16x4_to_f32(row16_block(lc[bb], vb));
            if constexpr (KS > 0) {
                tile_mma_vm<2, KS>(a, cur, nks, acc, [&](int ks) {
                    if ((ks & 1) == 0) dma_block(i + 3, nxt, ks >> 1);
                });
            } else {
                tile_mma_vm<2, KS>(a, cur, nks, acc);
            }
#pragma unroll
            for (int vb = 0; vb < 4; ++vb)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) fprev[vb][bb] = acc[vb][bb];
            prev = i;
        } else if constexpr (KS > 0) {
            for (int t = 0; t < 32 / NW; ++t) dma_block(i + 3, nxt, t);
            issue_fence();
        }
    };

    // Prologue: the conditioning tokens are loaded first (the oldest loads,
    // so waiting for them does not wait for the tile loads behind them), then
    // only the first tile; the tokens are used (clamped) only after that, and
    // then the A-operand gather is issued.  With `ag` (written by the previous
    // step's locate kernel, rank 256) the A operand is read from there instead,
    // 1 KB contiguous per load, and no token is read.
    // (Two separate paths: a token load pending on one side of a join would
    // make the compiler wait for every load at the join.)
    auto first_tile = [&]() {
        issue_fence();
        load_l(0, l0);
        issue_fence();
        dma(0, s0);
        issue_fence();
    };
    if (ag) {
        first_tile();
        const int last_blk = (B - 1) >> 4;  // blocks past the batch read the last one (rows never reported)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
                a[bb][ks] = ld16(ag + ag_offset(16 * min((mw >> 4) + bb, last_blk), ks, 0) + (size_t)lane * 8);
    } else {
        int tk[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) tk[bb] = cond_token_raw(x0, tok, min(mw + 16 * bb + c, B - 1), gamma, k);
        first_tile();
        // The operand rows: A[x] (Markov head) or the rows' RNN states.
        const uint16_t* arow[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            arow[bb] = H ? H + ((size_t)min(mw + 16 * bb + c, B - 1) * gamma + (k - 1)) * r
                         : A + (size_t)clamp_token(tk[bb], V) * r;
        load_a_frags<2>(arow, r, a);
    }
    issue_fence();
    // Tile 0 is peeled off the loop: its MFMAs then wait for the A operand
    // k step by k step as it arrives (loads made before a loop and used in it
    // would otherwise all be waited for before the loop is entered).
    const std::true_type more{};
    body(std::false_type{}, 0, s0, s3, l0, l1);
    // Whole rounds of four tiles, then at most three more.  (A loop with an
    // exit between its bodies joins that exit with its back edge, and the
    // compiler then waits for nearly every load in flight at the top of the
    // loop.)
    int i = 1;
    for (; i + 4 <= cnt; i += 4) {
        body(more, i, s1, s0, l1, l0);
        body(more, i + 1, s2, s1, l0, l1);
        body(more, i + 2, s3, s2, l1, l0);
        body(more, i + 3, s0, s3, l0, l1);
    }
    // The rest as straight-line code per count (a body that may or may not
    // have run before another also makes the compiler wait early).
    const int rest = cnt - i;
    if (rest == 1) {
        body(more, i, s1, s0, l1, l0);
    } else if (rest == 2) {
        body(more, i, s1, s0, l1, l0);
        body(more, i + 1, s2, s1, l0, l1);
    } else if (rest == 3) {
        body(more, i, s1, s0, l1, l0);
        body(more, i + 1, s2, s1, l0, l1);
        body(more, i + 2, s3, s2, l1, l0);
    }
    if (FULL || active) epilogue(std::true_type{});  // the slot's last tile (the vocabulary's tail for the last slot)
    // The staged partials are visible to the workgroup after an LDS wait and
    // a barrier.  The dummy loads past the last tile (DMAs into LDS among
    // them) drain while the partials are written, and are waited for before
    // the waves end.
    wait_lds();
    barrier_lds();
    // Write the staged partials (consecutive threads take consecutive tiles of
    // a row): with MANY, those of the tiles since the last write-out.
    const int base = MANY ? (cnt - 1) / kPartTiles * kPartTiles : 0, left = cnt - base;
    for (int e = threadIdx.x; e < R * left; e += 64 * NW) {
        const int row = e / left, i = e - row * left;
        if (m0 + row < B) part[(size_t)(m0 + row) * nT + t0 + (base + i) * ts] = unpack_f2(stage[i][row]);
    }
    // The slot aggregate of each row: its max and sum of exp over the slot's
    // tiles (t0 .. t0+cnt-1), for the locate's first level.
    if (SLOTS && threadIdx.x < R && m0 + (int)threadIdx.x < B) {
        const int row = threadIdx.x;
        float2 ra = make_float2(-INFINITY, 0.0f);
        if constexpr (MANY && SLOTS) ra = run_agg[row];
        fold_partials(&ra.x, &ra.y, left, [&](int i) { return unpack_f2(stage[i][row]); });
        sagg[(size_t)(m0 + row) * kSlotAggMax + slot] = ra;
    }
    wait_all_mem();
}

// ---------------------------------------------------------------------------
// Locate and sample.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_draft_locate(const typename DT::T* __restrict__ L,
                                                           const typename DT::T* __restrict__ A,
                                                           const typename DT::T* __restrict__ Bm,
                                                           const int32_t* __restrict__ x0, int32_t* tok,
                                                           float* __restrict__ p_out, double* __restrict__ lse_out,
                                                           const float2* __restrict__ part,
                                                           const typename DT::T* __restrict__ H, int B, int gamma,
                                                           int V, int r, int k, int nT, SeedArg seed_arg, ConfOut co)
{
    const uint64_t seed = seed_of(seed_arg);
    typedef TileTraits<DT> TT;
    __shared__ __attribute__((aligned(1024))) char lds[TT::kLdsBytes];
    __shared__ BlockScratch bs;
    __shared__ double sh_cprev;

    const int b = blockIdx.x;
    const float2* pr = part + (size_t)b * nT;
    const int per = (nT + kThreads - 1) / kThreads;
    const int t0 = min((int)threadIdx.x * per, nT), t1 = min(t0 + per, nT);
    float mloc = -INFINITY;
    for (int i = t0; i < t1; ++i) mloc = fmaxf(mloc, pr[i].x);
    const float M = block_max(mloc, bs);
    const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
    const Located loc = locate(
        nT, [&](int i) { const float2 q = pr[i]; return tile_mass(q.x, (double)q.y, M); }, u, bs, &sh_cprev);

    const int n0 = loc.idx * TT::kCols;
    const int prev = cond_token(x0, tok, b, gamma, k, V);
    if (co.z && (threadIdx.x >> 6) == 0) markov_confidence<DT>(A, co, prev, r, b * gamma + (k - 1));
    const auto* lrow = L + ((size_t)b * gamma + (k - 1)) * V;
    const float mt = pr[loc.idx].x;
    const double scale = tile_mass(mt, 1.0, M);
    const float ml = row_mlog2(mt);
    double wsel;
    int j;
    if constexpr (std::is_same<DT, Bf16>::value) {
        floatx4 f[4];
        row_tile_vm(lrow, H ? H + ((size_t)b * gamma + (k - 1)) * r : A, Bm, H ? 0 : prev, V, r, n0, lds, f);
        if ((threadIdx.x >> 6) != 0) return;
        j = scan_vm_tile(
            n0, b, scale, loc.cprev, loc.tau,
            [&](int vb, int i, int col) {
                return col < V && mt != -INFINITY ? (double)softmax_w(f[vb][i], ml) : 0.0;
            },
            &wsel);
    } else {
        float f[TT::kNB];
        row_tile_f(lrow, H ? H + ((size_t)b * gamma + (k - 1)) * r : A, Bm, H ? 0 : prev, V, r, n0, lds, f);
        if ((threadIdx.x >> 6) != 0) return;
        const int l16 = threadIdx.x & 15;
        double w[TT::kNB];
#pragma unroll
        for (int nb = 0; nb < TT::kNB; ++nb) {
            const bool ok = n0 + 16 * nb + l16 < V && mt != -INFINITY;
            w[nb] = ok ? (double)softmax_w(f[nb], ml) : 0.0;
        }
        j = scan_tile_weights<TT::kNB>(w, scale, loc.cprev, loc.tau, &wsel);
    }
    if (threadIdx.x == 0) {
        tok[b * gamma + (k - 1)] = min(n0 + j, V - 1);
        p_out[b * gamma + (k - 1)] = (float)(scale * wsel / loc.S);
        lse_out[b * gamma + (k - 1)] = (double)M + log(loc.S);
    }
}

// bf16: one wave per request, for rows of at most 64*PER tiles.  The A
// operand of the request's conditioning token is loaded first; lane l loads
// its contiguous slice of the row's tile partials into registers with all
// loads in flight at once; the partials are combined with wave scans (no
// barriers, no LDS) by the same rule as locate(); the chosen tile is
// recomputed by the wave alone from its own LDS copy of the Bm tile.
// First tile of the next step's tile kernel, read ahead into L2.  Workgroup
// b of this launch and workgroup b of the tile launch that follows it are
// both placed on XCD b mod 8 (workgroups are dispatched to the XCDs
// round-robin by index), so when the AG locate's second wave reads the 256
// L rows and the 256 Bm rows of that workgroup's first tile (64 KB, by LDS
// DMA into a kilobyte nothing reads), the tile kernel finds them in its XCD's
// L2 instead of starting with a full HBM round trip.  Addresses are clamped
// into the arrays as the tile kernel clamps them (rows past the batch read the
// last row; columns stop at V - 8).
__device__ __forceinline__ void prefetch_first_tile(const uint16_t* __restrict__ L, const uint16_t* __restrict__ Bm,
                                                    int b, int B, int gamma, int V, int k_next, int nT, int nM,
                                                    int S, char* sink)
{
    const int G = S * nM;
    if (b >= G) return;
    const int lid = xcd_logical_id(b, G);
    const int mblk = lid % nM, slot = lid / nM;
    int t0, ts, cnt;
    slot_tiles(slot, S, nT, &t0, &ts, &cnt);
    if (cnt <= 0) return;
    const int lane = threadIdx.x & 63;
    const int col = min(t0 * kTcols + 8 * (lane & 7), V - 8);
#pragma unroll 4
    for (int i = 0; i < kTileRows / 8; ++i) {
        const int rb = min(mblk * kTileRows + 8 * i, B - 1);  // wave-uniform
        const int row = min(mblk * kTileRows + 8 * i + (lane >> 3), B - 1);
        dma16(L + ((size_t)rb * gamma + (k_next - 1)) * V,
              (uint32_t)(((size_t)(row - rb) * gamma * V + col) * 2), sink);
    }
#pragma unroll 4
    for (int i = 0; i < kAgRank / 8; ++i) dma16(Bm + (size_t)(8 * i) * V, (uint32_t)(((lane >> 3) * V + col) * 2), sink);
    wait_all_mem();
}

// The budget schedule carried by the last step's locate launch (SCHED): one
// extra workgroup (index 0) of kSchedWgThreads threads, keys and scratch in
// the locate's LDS tile buffer.  (Measured on MI355X: 512 threads were
// slower than 256, and index 0 was 0.3-0.7 us per step faster than index B.)
constexpr int kSchedWgThreads = 256;
static_assert(sizeof(SelectScratch<kSchedWgThreads>) <= kSchedKeysOffset, "select scratch");

template <int KS, int PER, bool AG, bool SCHED = false, bool SLOTS = false>
__global__ __launch_bounds__(SCHED ? kSchedWgThreads : 128) void k_draft_locate_bf16(const uint16_t* __restrict__ L,
                                                          const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ Bm,
                                                          const int32_t* __restrict__ x0, int32_t* tok,
                                                          float* __restrict__ p_out, double* __restrict__ lse_out,
                                                          const float2* __restrict__ part, uint16_t* __restrict__ ag,
                                                          const uint16_t* __restrict__ H, int B, int gamma, int V,
                                                          int r, int k, int nT, int nM_next, int S_next,
                                                          SeedArg seed_arg, ConfOut co, SchedArg sa)
{
    __shared__ __attribute__((aligned(1024))) char lds[kBmTileBytes];
    if constexpr (SCHED) {
        // Workgroup 0 is the budget schedule (dispatched first: it takes longer
        // than a request's locate); it shares nothing with the others, which
        // take requests b = blockIdx.x - 1.
        if (blockIdx.x == 0) {
            budget_select<kSchedWgThreads>(sa.z, sa.temps, B, gamma, sa.admit, sa.surv, sa.len,
                                           reinterpret_cast<uint32_t*>(lds + kSchedKeysOffset),
                                           *reinterpret_cast<SelectScratch<kSchedWgThreads>*>(lds));
            return;
        }
    }
    const uint64_t seed = seed_of(seed_arg);
    // AG (not the last step): a second wave reads the next tile launch's
    // first tile ahead; it shares nothing with the first wave.
    if (threadIdx.x >= 64) {
        if constexpr (AG) {
            __shared__ __attribute__((aligned(1024))) char sink[1024];
            prefetch_first_tile(L, Bm, blockIdx.x, B, gamma, V, k + 1, nT, nM_next, S_next, sink);
        }
        return;
    }
    // With AG (rank 256) the sampled token's A row is copied into `ag` in MFMA
    // order for the next step's tile kernel.  (Measured on MI355X: reading
    // that one row after the sample is faster than reading the chosen tile's
    // 64 candidate rows, 32 KB, alongside its Bm tile: 7.78 against 8.02 us
    // per launch, 8.4 MB less traffic.)
    const int b = blockIdx.x - (SCHED ? 1 : 0);
    const int lane = threadIdx.x & 63;
    // The partial loads go first: the A-operand loads wait for the token.
    // SLOTS: the tile launch wrote slot aggregates (its S_next = Sp slots,
    // at most kSlotAggMax; such launches never carry the schedule, so every
    // tile launch of the call has the same slots).  Only those are read now,
    // 2 KB per row instead of the row's 8 bytes per tile (at 2020 tiles a
    // wave's full slices take 3-4 us to arrive, a 2 KB read 1.3 us), and the
    // chosen slot's tiles after them.  (A compile-time choice: loads pending
    // on one side of a run-time branch would make the compiler wait for every
    // load where the paths join.  The aggregates' address comes from ag: an
    // extra kernel argument measured 0.2 us slower per launch.)
    const int Sp = S_next;
    const float2* sagg = reinterpret_cast<const float2*>(reinterpret_cast<const char*>(ag) + slot_agg_offset(B));
    const float2* pr = part + (size_t)b * nT;
    float2 q[SLOTS ? 1 : PER];
    int i0 = 0;
    float2 qs[4];
    int i0s = 0;
    if constexpr (SLOTS) load_slices<4>(sagg + (size_t)b * kSlotAggMax, Sp, make_float2(-INFINITY, 0.0f), qs, &i0s);
    else load_slices<PER>(pr, nT, make_float2(-INFINITY, 0.0f), q, &i0);
    const int prev = cond_token(x0, tok, b, gamma, k, V);
    uint4 a[1][8];
    {
        const uint16_t* arow[1] = { H ? H + ((size_t)b * gamma + (k - 1)) * r : A + (size_t)prev * r };
        load_a_frags<1>(arow, r, a);
    }
    // Confidence weights in the A operand's order (lane group G holds
    // k = 32ks + 8G .. +7), for the Markov-conditioned confidence logit.
    uint4 wcf[8];
    if (co.z) {
        const uint16_t* wc = static_cast<const uint16_t*>(co.wc);
        const int kq8 = 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) wcf[ks] = ld16(wc + min(32 * ks + kq8, r - 8));
    }
    float M, mt = 0.0f;
    Located loc;
    if constexpr (SLOTS) {
        // First level: the slots in index order (each a contiguous tile range),
        // masses from their aggregates; the row max is the max of the slot maxima.
        M = wave_max(fmaxf(fmaxf(qs[0].x, qs[1].x), fmaxf(qs[2].x, qs[3].x)));
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
        const Located ls = wave_locate_slices<4>(
            i0s, [&](int j) { return tile_mass(qs[j].x, (double)qs[j].y, M); }, u, reinterpret_cast<double*>(lds));
        // Second level: the chosen slot's tiles (at most kManyTiles), one per
        // lane, scanned from the mass before the slot.  Where rounding leaves
        // every running sum in the slot at or below tau, its last tile of
        // positive mass is taken (as wave_locate_slices does within a slice).
        int t0, ts, cnt;
        slot_tiles(ls.idx, Sp, nT, &t0, &ts, &cnt);
        const float2 qt = pr[t0 + min(lane, cnt - 1) * ts];
        const double mm = lane < cnt ? tile_mass(qt.x, (double)qt.y, M) : 0.0;
        const double inc = wave_incl_scan(mm);
        const uint64_t hit = __ballot(mm > 0.0 && ls.cprev + inc > ls.tau);
        const uint64_t pos = __ballot(mm > 0.0);
        const int sel = hit ? __builtin_ctzll(hit) : pos ? 63 - __builtin_clzll(pos) : 0;
        loc.S = ls.S;
        loc.tau = ls.tau;
        loc.idx = t0 + sel * ts;
        loc.cprev = ls.cprev + __shfl(inc - mm, sel, 64);
        mt = __shfl(qt.x, sel, 64);
    } else {
        float mloc = -INFINITY;
#pragma unroll
        for (int j = 0; j < PER; ++j) mloc = fmaxf(mloc, q[j].x);
        M = wave_max(mloc);
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
        // Tile masses relative to the row max, kept when the registers allow.
        constexpr bool kCache = PER <= 32;
        double ms[kCache ? PER : 1];
        if constexpr (kCache) {
#pragma unroll
            for (int j = 0; j < PER; ++j) ms[j] = tile_mass(q[j].x, (double)q[j].y, M);
        }
        loc = wave_locate_slices<PER>(
            i0,
            [&](int j) {
                if constexpr (kCache) return ms[j];
                else return tile_mass(q[j].x, (double)q[j].y, M);
            },
            u, reinterpret_cast<double*>(lds));
    }
    const int idx = loc.idx;
    const double cprev = loc.cprev, tau = loc.tau, S = loc.S;

    const int n0 = idx * kTcols;
    // Max of the chosen tile (one level: reloaded, the partials are cached;
    // its latency hides behind the tile's own loads).
    if constexpr (!SLOTS) mt = pr[idx].x;
    floatx4 f[4];
    row_tile_vm_wave<KS>(L + ((size_t)b * gamma + (k - 1)) * V, a, Bm, V, r, n0, lds, f);
    if (co.z) {
        // z = z0 + <A[prev], wc> from the A operand already in registers
        // (pieces past r are zero): 64 products per lane in (k step, element)
        // order, then the four lane groups by the xor-16 / xor-32 butterflies.
        float sdot = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) sdot = __builtin_fmaf(Bf16::get(a[0][ks], e), Bf16::get(wcf[ks], e), sdot);
        sdot = sum_xor16_32(sdot);
        if (lane == 0) co.z[b * gamma + (k - 1)] = co.z0[b * gamma + (k - 1)] + sdot;
    }
    const double scale = tile_mass(mt, 1.0, M);
    const float ml = row_mlog2(mt);
    double wsel;
    const int j = scan_row_tile_lanes(
        n0, scale, cprev, tau,
        [&](int col, auto pick) { return col < V && mt != -INFINITY ? (double)softmax_w(pick(f), ml) : 0.0; },
        &wsel);
    const int xk = min(n0 + j, V - 1);
    if constexpr (AG) {
        if (lane < 32) {  // piece (ks, G) = (lane >> 2, lane & 3) of A[xk]: elements 8 * lane .. +7
            const uint4 v = *reinterpret_cast<const uint4*>(A + (size_t)xk * kAgRank + lane * 8);
            *reinterpret_cast<uint4*>(ag + ag_offset(b, lane >> 2, lane & 3)) = v;
        }
    }
    if (lane == 0) {
        tok[b * gamma + (k - 1)] = xk;
        p_out[b * gamma + (k - 1)] = (float)(scale * wsel / S);
        lse_out[b * gamma + (k - 1)] = (double)M + log(S);
    }
}

// ---------------------------------------------------------------------------
// RNN sequential head (menfem.com note, Key Contributions: the head variant
// that keeps the whole in-block prefix in a recurrent state instead of the
// first-order Markov dependency).  Before draft step k:
//     h_k = tanh(W h_{k-1} + A[x_{k-1}]),  h_0 = 0,
// stored as row (b, k-1) of H in the element type; it replaces A[x_{k-1}] as
// the operand of the rank-r bias.  Wt is W transposed (Wt[j][i] multiplies
// h_{k-1}[j] into output i), so for a fixed j the lanes read consecutive
// outputs with 16-byte loads.  One workgroup of r threads per request: the
// products are summed in fp32 over kPer slices of j (thread (g, slice)
// covers kPer consecutive outputs), the slices added in order to A[x][i],
// then fp32 tanh and a round to the element type.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t store_elem(Bf16, float f) { return f32_to_bf16_rne(f); }
__device__ __forceinline__ float store_elem(F32, float f) { return f; }

template <class DT>
__global__ __launch_bounds__(kMaxRank) void k_rnn_state(const typename DT::T* __restrict__ A,
                                                        const typename DT::T* __restrict__ Wt,
                                                        const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
                                                        typename DT::T* H, int B, int gamma, int V, int r, int k)
{
    typedef typename DT::T T;
    constexpr int kPer = 16 / sizeof(T);  // outputs per 16-byte load of a row of Wt
    __shared__ float hp[kMaxRank];
    __shared__ float part[kPer][kMaxRank];
    const int b = blockIdx.x, t = threadIdx.x;
    const int x = cond_token(x0, tok, b, gamma, k, V);
    const T* arow = A + (size_t)x * r;
    T* hout = H + ((size_t)b * gamma + (k - 1)) * r;
    if (k >= 2 && t < r) hp[t] = DT::to_f32(H[((size_t)b * gamma + (k - 2)) * r + t]);
    __syncthreads();
    if (k >= 2) {
        // Thread t: outputs kPer*g .. +kPer-1 (g = t mod r/kPer) over the
        // slice jj = t / (r/kPer) of j, one 16-byte load of Wt per j.
        const int ng = r / kPer, g = t % ng, jj = t / ng, per = r / kPer;
        float s[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) s[e] = 0.0f;
        if (t < r) {
#pragma unroll 8
            for (int j = jj * per; j < (jj + 1) * per; ++j) {
                const uint4 w = ld16(Wt + (size_t)j * r + kPer * g);
                const float h = hp[j];
#pragma unroll
                for (int e = 0; e < kPer; ++e) s[e] = __builtin_fmaf(DT::get(w, e), h, s[e]);
            }
#pragma unroll
            for (int e = 0; e < kPer; ++e) part[jj][kPer * g + e] = s[e];
        }
        __syncthreads();
    }
    if (t < r) {
        float pre = DT::to_f32(arow[t]);
        if (k >= 2) {
#pragma unroll
            for (int q = 0; q < kPer; ++q) pre += part[q][t];
        }
        hout[t] = store_elem(DT{}, tanhf(pre));
    }
}

hipError_t launch_draft_step(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, int k, SeedArg seed, int32_t* tok, float* p, double* lse,
                             const float* z0, const void* wc, float* z_out, const void* Wt, void* H, void* ws,
                             const WsLayout& lay, hipStream_t s, const SchedArg* sched)
{
    const ConfOut co{ z0, wc, z_out };
    if (H) {  // RNN head: this step's operand rows
        if (dtype == 1)
            hipLaunchKernelGGL(k_rnn_state<Bf16>, dim3(B), dim3(kMaxRank), 0, s, static_cast<const uint16_t*>(A),
                               static_cast<const uint16_t*>(Wt), x0, tok, static_cast<uint16_t*>(H), B, gamma, V, r, k);
        else
            hipLaunchKernelGGL(k_rnn_state<F32>, dim3(B), dim3(kMaxRank), 0, s, static_cast<const float*>(A),
                               static_cast<const float*>(Wt), x0, tok, static_cast<float*>(H), B, gamma, V, r, k);
    }
    float2* part = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.draft_part);
    uint16_t* ag = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.ag);
    const int nT = n_tiles(dtype, V);
    // The one-wave locate (bf16, up to 4096 tiles) hands the next step its A
    // rows in MFMA order when the rank is 256.
    const bool wave_locate = dtype == 1 && nT <= 64 * 64;
    const bool ag_path = wave_locate && r == kAgRank && !H;  // (RNN head: the next operand is the state, not A[x])
    // bf16 tile grid: nM row blocks x S persistent slots.
    const int nM = (B + kTileRows - 1) / kTileRows;
    const int S = draft_tile_slots(B, nT);
    const bool many = B % kTileRows == 0 && (nT + S - 1) / S > kPartTiles;
    // The schedule rides in the first tile launch when one slot fewer leaves
    // every slot's tile count as it is (the launch takes as long, and the
    // freed CU runs the schedule), else in the last locate launch.
    const bool first_tiles_sched = schedule_in_first_tiles(dtype, B, gamma, V);
    const bool sch_tiles = sched != nullptr && k == 1 && first_tiles_sched;
    const bool sch_locate = sched != nullptr && k == gamma && !first_tiles_sched;
    const SchedArg none{ nullptr, nullptr, 0, nullptr, nullptr };
    const int St = sch_tiles ? S - 1 : S;  // slots of this step's tile launch
    // Slot aggregates for the one-wave locate, where its workgroups share CUs
    // (B > 256): each then reads 2 KB of aggregates and one slot's tiles
    // instead of its row's 8 bytes per tile.  (Measured on MI355X at
    // V = 129280: B = 1024, the locate 14.3 -> 10.8 us per launch and the step
    // 0.4-1.3% shorter; B = 256, one workgroup per CU, its waves end earlier
    // but the launch, held by its slowest workgroups, does not.)
    // Such shapes never carry the schedule in a tile launch, so every tile
    // launch of a call has the same slots and the aggregates the same ranges.
    float2* sagg = wave_locate && B > kTileRows && St <= kSlotAggMax
                       ? reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.slot_agg)
                       : nullptr;
    // The locate finds the aggregates at ag + slot_agg_offset(B): every layout keeps them there.
    if (sagg && lay.slot_agg != lay.ag + slot_agg_offset(B)) return hipErrorInvalidValue;
    if (dtype == 1) {
        const bool k8 = (r + 31) / 32 == 8, full = B % kTileRows == 0;
        auto kern = sagg ? (k8 ? (many ? k_draft_tiles_bf16<8, true, true, true>
                                       : full ? k_draft_tiles_bf16<8, true, false, true>
                                              : k_draft_tiles_bf16<8, false, false, true>)
                               : (many ? k_draft_tiles_bf16<0, true, true, true>
                                       : k_draft_tiles_bf16<0, false, false, true>))
                         : (k8 ? (many ? k_draft_tiles_bf16<8, true, true>
                                       : full ? k_draft_tiles_bf16<8, true> : k_draft_tiles_bf16<8, false>)
                               : (many ? k_draft_tiles_bf16<0, true, true> : k_draft_tiles_bf16<0, false>));
        launch_timed(K_DRAFT_TILES, kern, dim3(St * nM + (sch_tiles ? 1 : 0)), dim3(64 * kTileWaves), s,
                     static_cast<const uint16_t*>(L), static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(Bm), x0, tok,
                     static_cast<const uint16_t*>(ag_path && k >= 2 ? ag : nullptr), static_cast<const uint16_t*>(H),
                     B, gamma, V, r, k, nT, nM, St, part, sagg, sch_tiles ? *sched : none);
    } else {
        const int nM32 = (B + 255) / 256;
        launch_timed(K_DRAFT_TILES, k_draft_tiles_f32, dim3(nT * nM32), dim3(kThreads), s, static_cast<const float*>(L),
                           static_cast<const float*>(A), static_cast<const float*>(Bm), x0, tok,
                           static_cast<const float*>(H), B, gamma, V, r, k, nT, nM32, part);
    }
    if (wave_locate) {
        const bool k8 = (r + 31) / 32 == 8, small = nT <= 64 * 32, wag = ag_path && k < gamma;
        const bool sch = sch_locate;  // (wag is false at k = gamma)
        auto kern = sagg ? (sch ? (k8 ? k_draft_locate_bf16<8, 4, false, true, true>
                                      : k_draft_locate_bf16<0, 4, false, true, true>)
                                : k8 ? (wag ? k_draft_locate_bf16<8, 4, true, false, true>
                                            : k_draft_locate_bf16<8, 4, false, false, true>)
                                     : k_draft_locate_bf16<0, 4, false, false, true>)
                  : sch ? (small ? (k8 ? k_draft_locate_bf16<8, 32, false, true> : k_draft_locate_bf16<0, 32, false, true>)
                                 : (k8 ? k_draft_locate_bf16<8, 64, false, true> : k_draft_locate_bf16<0, 64, false, true>))
                  : small ? (k8 ? (wag ? k_draft_locate_bf16<8, 32, true> : k_draft_locate_bf16<8, 32, false>)
                                : k_draft_locate_bf16<0, 32, false>)
                          : (k8 ? (wag ? k_draft_locate_bf16<8, 64, true> : k_draft_locate_bf16<8, 64, false>)
                                : k_draft_locate_bf16<0, 64, false>);
        const SchedArg sa = sch ? *sched : none;
        launch_timed(K_DRAFT_LOCATE, kern, dim3(B + (sch ? 1 : 0)), dim3(sch ? kSchedWgThreads : wag ? 128 : 64), s,
                     static_cast<const uint16_t*>(L), static_cast<const uint16_t*>(A),
                     static_cast<const uint16_t*>(Bm), x0, tok, p, lse, part, ag, static_cast<const uint16_t*>(H), B,
                     gamma, V, r, k, nT, nM, S, seed, co, sa);
    } else if (dtype == 1) {
        launch_timed(K_DRAFT_LOCATE, k_draft_locate<Bf16>, dim3(B), dim3(kThreads), s, static_cast<const uint16_t*>(L),
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm), x0, tok, p, lse, part,
                           static_cast<const uint16_t*>(H), B, gamma, V, r, k, nT, seed, co);
    } else
        launch_timed(K_DRAFT_LOCATE, k_draft_locate<F32>, dim3(B), dim3(kThreads), s, static_cast<const float*>(L),
                           static_cast<const float*>(A), static_cast<const float*>(Bm), x0, tok, p, lse, part,
                           static_cast<const float*>(H), B, gamma, V, r, k, nT, seed, co);
    return hipGetLastError();
}

int draft_tile_slots(int B, int nT)
{
    const int nM = (B + kTileRows - 1) / kTileRows;
    return tile_slots(nT, nM, cu_count(), B % kTileRows == 0 ? kManyTiles : kPartTiles);
}

bool schedule_in_first_tiles(int dtype, int B, int gamma, int V)
{
    if (dtype != 1 || (long long)B * gamma > kSchedMaxKeys || B > kTileRows) return false;
    const int nT = n_tiles(dtype, V), S = draft_tile_slots(B, nT);
    return S > 1 && (nT + S - 2) / (S - 1) == (nT + S - 1) / S;
}

bool draft_step_can_schedule(int dtype, int B, int gamma, int V)
{
    return dtype == 1 && (long long)B * gamma <= kSchedMaxKeys &&
           (n_tiles(dtype, V) <= 64 * 64 || schedule_in_first_tiles(dtype, B, gamma, V));
}

}  // namespace dspark
