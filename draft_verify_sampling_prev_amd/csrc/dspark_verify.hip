// dspark_verify.hip -- exact rejection-sampling verification on gfx950.
//
// Rule (menfem.com note on arXiv 2607.05147, Methodology; paperlayer.ai
// summary, section 2): drafted token x_k is kept with probability
// min(1, p_t(x_k) / p_d(x_k)), positions are checked left to right and the
// first rejection discards every later token.  After the a accepted tokens
// one more token is emitted: at a rejection, a sample of
// normalise(max(0, p_t - p_d)) at the rejected position; when all ell
// verified tokens pass (ell = 0 included: paperlayer.ai summary, Appendix A),
// a sample of p_t at position ell + 1.
//
// Launch sequence (all fixed-shape; per-request lengths are read on the
// device, so the sequence can be captured in a HIP graph):
//   k_row_partials (target)  grid = chunks x (B*gamma): row (b,k) with
//                            k <= ell_b -> chunk max and sum of exp (fp64).
//   k_accept_bonus           one wave per request: lse_t and p_t(x_k) of its
//                            verified rows, accept draws, first rejection;
//                            appends the requests with a rejection to the
//                            residual list.  In the same launch, while
//                            B*V*s <= 80 MB, chunks x B workgroups: target
//                            row ell_b + 1 of every request (the bonus row)
//                            -> chunk max and sum of exp.
//   k_resid_tiles            Markov MFMA tiles of the rejected draft rows
//                            fused with the target row: per tile sums of
//                            max(0, p_t - p_d) and of p_t, stored in the
//                            request's row of the residual partials.
//   k_row_partials (bonus)   otherwise: grid = chunks x B, the bonus rows of
//                            the requests without a rejection.
//   k_final                  one workgroup per request: locate and sample
//                            the last token, write the emitted tokens.
#include <limits.h>

#include <algorithm>
#include <type_traits>

#include "dspark_internal.hpp"
#include "dspark_locate.hpp"
#include "dspark_markov.hpp"
#include "dspark_tile.hpp"

namespace dspark {

__device__ __forceinline__ int clamp_len(int l, int gamma) { return min(max(l, 0), gamma); }
__device__ __forceinline__ int clamp_tok(int x, int V) { return min(max(x, 0), V - 1); }

__device__ __forceinline__ int cond_token_v(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                            int gamma, int k, int V)
{
    return clamp_tok((k == 1) ? x0[b] : tok[b * gamma + (k - 2)], V);
}

// A log-normaliser split into two floats, hi + lo = lse to ~2^-48 relative.
// A row's log-normaliser as the base-2 offset used by resid_weight:
// c = lse * log2(e), rounded to float.
__device__ __forceinline__ float lse_log2(double lse) { return (float)(lse * kLog2eD); }

// Residual weight of one vocabulary entry: w = max(0, p_t - p_d) with
// p = exp(x - lse) = 2^(x log2 e - c), one FMA and the hardware base-2
// exponential (the exponent carries an absolute error of a few 1e-6, from
// rounding log2 e and c to float); *pt receives p_t.  The same expression is
// used by the residual tile pass and by the final rescan, so the weights the
// final sample scans are exactly those summed into the tile partials.
__device__ __forceinline__ float resid_weight(float f, float t, float cd, float ct, float* pt)
{
    const float ptv = __builtin_amdgcn_exp2f(__builtin_fmaf(t, kLog2e, -ct));
    const float pdv = __builtin_amdgcn_exp2f(__builtin_fmaf(f, kLog2e, -cd));
    *pt = ptv;
    const float w = ptv - pdv;
    return w > 0.0f ? w : 0.0f;
}

// ---------------------------------------------------------------------------
// Chunk max / sum of exp over a target row: 8192 elements per workgroup,
// every element loaded once with 16-byte loads and kept in registers between
// the max and the sum.
// ---------------------------------------------------------------------------
// Rows: kRowTarget, row = b*gamma + k-1 for k <= ell_b; kRowBonusAll, row = b,
// target row ell_b of every request (the bonus row, computed before it is
// known whether all ell_b drafts are accepted, the only case that uses it);
// kRowBonusAccepted, the same row of the requests whose drafts were all
// accepted (after the accept scan).
constexpr int kRowTarget = 0, kRowBonusAll = 1, kRowBonusAccepted = 2;

template <class DT>
__device__ __forceinline__ void row_partials(const typename DT::T* __restrict__ Tg, const int32_t* __restrict__ len,
                                             const int32_t* __restrict__ accepted, int gamma, int V, int nC, int mode,
                                             int c, int row, float* __restrict__ om, double* __restrict__ os,
                                             BlockScratch& bs)
{
    int b, trow;
    if (mode == kRowTarget) {
        b = row / gamma;
        trow = row - b * gamma;
        if (trow >= clamp_len(len[b], gamma)) return;  // uniform over the workgroup
    } else {
        b = row;
        trow = clamp_len(len[b], gamma);
        if (mode == kRowBonusAccepted && accepted[b] < trow) return;
    }
    const typename DT::T* x = Tg + ((size_t)b * (gamma + 1) + trow) * V;
    constexpr int PV = DT::kPerVec;
    constexpr int NV = kChunkElems / (kThreads * PV);
    const int e0 = c * kChunkElems;
    uint4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = e0 + (i * kThreads + (int)threadIdx.x) * PV;
        v[i] = e < V ? ld16(x + e) : make_uint4(0u, 0u, 0u, 0u);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = e0 + (i * kThreads + (int)threadIdx.x) * PV;
        if (e < V) {
#pragma unroll
            for (int j = 0; j < PV; ++j) mloc = fmaxf(mloc, DT::get(v[i], j));
        }
    }
    const float M = block_max(mloc, bs);
    // exp(x - M) is 0 for x = -inf; each 16-byte vector is summed in fp32, vectors in fp64.
    const float ml = row_mlog2(M);
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = e0 + (i * kThreads + (int)threadIdx.x) * PV;
        if (e < V) {
            float sv = 0.0f;
#pragma unroll
            for (int j = 0; j < PV; ++j) sv += softmax_w(DT::get(v[i], j), ml);
            s += (double)sv;
        }
    }
    s = block_sum(M == -INFINITY ? 0.0 : s, bs);
    if (threadIdx.x == 0) {
        om[(size_t)row * nC + c] = M;
        os[(size_t)row * nC + c] = s;
    }
}

// Grid chunks x rows (target: rows B*gamma; bonus: rows B).
template <class DT>
__global__ __launch_bounds__(kThreads) void k_row_partials(const typename DT::T* __restrict__ Tg,
                                                           const int32_t* __restrict__ len,
                                                           const int32_t* __restrict__ accepted, int gamma, int V,
                                                           int nC, int mode, float* __restrict__ om,
                                                           double* __restrict__ os, int32_t* __restrict__ clear_count)
{
    __shared__ BlockScratch bs;
    // The residual-list counter of the accept kernel, which runs next on the stream.
    if (clear_count && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *clear_count = 0;
    row_partials<DT>(Tg, len, accepted, gamma, V, nC, mode, blockIdx.x, blockIdx.y, om, os, bs);
}

// ---------------------------------------------------------------------------
// Target log-normalisers, p_t(x_k) and the accept scan: one wave per request.
//
// Lane c holds chunk c's (max, sum of exp) partials of every verified row
// (all loads issued before the first reduction); per row the wave reduces
// them to the log-normaliser, lane kk keeps row kk's, loads T[b][kk][x_kk]
// and draws its accept uniform, and a ballot gives the first rejection.  A
// request with a rejection takes the next slot of the residual list with an
// atomic add on the counter that the target row pass cleared: the list is
// compact but in no fixed order, and nothing downstream depends on the order
// (every row's residual tile results depend only on the row).
// ---------------------------------------------------------------------------
constexpr int kAcceptWaves = 4;
constexpr double kBonusInAcceptBytes = 80.0 * 1024 * 1024;  // B * V * element size
static_assert(64 * kAcceptWaves == kThreads, "the accept and row-pass workgroups share one launch");

template <class DT>
__device__ __forceinline__ void lse_accept(
    const typename DT::T* __restrict__ Tg, const float* __restrict__ pd, const int32_t* __restrict__ len,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, const float* __restrict__ tgm,
    const double* __restrict__ tgs, int B, int gamma, int V, int nC, int rnn, SeedArg seed_arg,
    int32_t* __restrict__ accepted, int32_t* __restrict__ n_out, float* __restrict__ target_p,
    double* __restrict__ lse_t, int4* __restrict__ resid_list,
    int32_t* __restrict__ resid_count, int wg)
{
    const uint64_t seed = seed_of(seed_arg);
    const int b = wg * kAcceptWaves + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (b >= B) return;
    const size_t row0 = (size_t)b * gamma;
    // Every load of rows k < gamma is issued before the length arrives (all
    // in bounds; rows past ell_b are loaded and ignored), so the chain is
    // {length, partials, p_d, tokens} -> T[x_k] -> residual slot.
    float pdk = 1.0f;
    int xk = 0;
    if (lane < gamma) {
        pdk = pd[row0 + lane];
        xk = clamp_tok(tok[row0 + lane], V);
    }
    const int l = clamp_len(len[b], gamma);
    // Row kk's log-normaliser: M = max of the chunk maxima, S = sum over
    // chunks of s_c exp(m_c - M), lse = M + ln S.  Lane kk keeps (M, S) of row kk.
    float Mk = 0.0f;
    double Sk = 1.0;
    if (nC <= 64) {
        float mv[kMaxGamma];
        double sv[kMaxGamma];
#pragma unroll
        for (int kk = 0; kk < kMaxGamma; ++kk) {
            mv[kk] = -INFINITY;
            sv[kk] = 0.0;
            if (kk < gamma && lane < nC) {
                mv[kk] = tgm[(row0 + kk) * nC + lane];
                sv[kk] = tgs[(row0 + kk) * nC + lane];
            }
        }
#pragma unroll
        for (int kk = 0; kk < kMaxGamma; ++kk) {
            if (kk < l) {
                const float M = wave_max(mv[kk]);
                const double S = wave_sum(tile_mass(mv[kk], sv[kk], M));
                if (lane == kk) {
                    Mk = M;
                    Sk = S;
                }
            }
        }
    } else {
        for (int kk = 0; kk < l; ++kk) {
            const float* m = tgm + (row0 + kk) * nC;
            const double* s = tgs + (row0 + kk) * nC;
            float M = -INFINITY;
            for (int c = lane; c < nC; c += 64) M = fmaxf(M, m[c]);
            M = wave_max(M);
            double S = 0.0;
            for (int c = lane; c < nC; c += 64) S += tile_mass(m[c], s[c], M);
            S = wave_sum(S);
            if (lane == kk) {
                Mk = M;
                Sk = S;
            }
        }
    }
    bool reject = false;
    if (lane < l) {
        const double lse = (double)Mk + log(Sk);
        lse_t[row0 + lane] = lse;
        const double tx = (double)DT::to_f32(Tg[((size_t)b * (gamma + 1) + lane) * V + xk]);
        const double ptk = exp(tx - lse);
        const double ratio = ptk / (double)pdk;
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(lane + 1), 1u);
        reject = !(u < (float)ratio);
        if (target_p) target_p[row0 + lane] = (float)ptk;
    } else if (target_p && lane < gamma) {
        target_p[row0 + lane] = 0.0f;
    }
    const uint64_t rej = __ballot(reject);
    const int a = rej ? __builtin_ctzll(rej) : l;
    if (lane == 0) {
        accepted[b] = a;
        n_out[b] = a + 1;
        if (a < l) {
            const int ks = a + 1;
            // operand row of the rejected position's draft logits: A[x_{ks-1}],
            // or with the RNN head the state row (b, ks-1)
            const int xprev = rnn ? b * gamma + ks - 1 : ks == 1 ? x0[b] : tok[row0 + ks - 2];
            const int idx = atomicAdd(resid_count, 1);
            resid_list[idx] = make_int4(b, ks, xprev, 0);
        }
    }
}

// The accept scan (workgroups 0 .. nAcc-1, one wave per request) and, when
// the grid has more workgroups, in the same launch the bonus row's chunk
// partials of every request (workgroup nAcc + b*nC + c: chunk c of target row
// ell_b of request b).  The bonus row is needed only where all ell_b drafts
// are accepted, but its index does not depend on the accept scan, so it can
// be read while the scan's dependent loads are in flight instead of by a
// launch of its own after the scan (the launcher does so while that read is
// small; otherwise the rows that are needed are read after the scan).
template <class DT>
__global__ __launch_bounds__(kThreads) void k_accept_bonus(
    const typename DT::T* __restrict__ Tg, const float* __restrict__ pd, const int32_t* __restrict__ len,
    const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, const float* __restrict__ tgm,
    const double* __restrict__ tgs, int B, int gamma, int V, int nC, int rnn, SeedArg seed_arg,
    int32_t* __restrict__ accepted, int32_t* __restrict__ n_out, float* __restrict__ target_p,
    double* __restrict__ lse_t, int4* __restrict__ resid_list,
    int32_t* __restrict__ resid_count, int nAcc, float* __restrict__ bm, double* __restrict__ bsum)
{
    __shared__ BlockScratch bs;
    const int wg = blockIdx.x;
    if (wg < nAcc) {
        lse_accept<DT>(Tg, pd, len, x0, tok, tgm, tgs, B, gamma, V, nC, rnn, seed_arg, accepted, n_out, target_p,
                       lse_t, resid_list, resid_count, wg);
        return;
    }
    const int q = wg - nAcc, b = q / nC;
    row_partials<DT>(Tg, len, accepted, gamma, V, nC, kRowBonusAll, q - b * nC, b, bm, bsum, bs);
}

// Row m of the compacted residual list: request b at its first rejected
// position ks, conditioned on token x (x_{ks-1}), as written by the accept scan.
// Every field is clamped into range, so a row read past the count (stale
// workspace) still addresses valid memory; such rows are never reported.
struct ResidRow {
    int b, ks, x;
};
__device__ __forceinline__ ResidRow resid_decode(int4 q, int B, int gamma, int V)
{
    ResidRow r;
    r.b = min(max(q.x, 0), B - 1);
    r.ks = min(max(q.y, 1), gamma);
    r.x = min(max(q.z, 0), V - 1);
    return r;
}
__device__ __forceinline__ ResidRow resid_row(const int4* __restrict__ resid_list, int m, int B, int gamma, int V)
{
    const int4 q = resid_list[m];
    ResidRow r;
    r.b = min(max(q.x, 0), B - 1);
    r.ks = min(max(q.y, 1), gamma);
    r.x = min(max(q.z, 0), V - 1);
    return r;
}

// ---------------------------------------------------------------------------
// Residual tiles, fp32: one 4-wave workgroup per (tile, 256-row block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_resid_tiles_f32(
    const float* __restrict__ Tg, const float* __restrict__ L, const float* __restrict__ A,
    const float* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ accepted,
    const int4* __restrict__ resid_list, const int32_t* __restrict__ resid_count, int B, int gamma, int V, int r, int nT,
    int nM, int nA, float2* __restrict__ rpart)
{
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<F32>()];
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int tile = lid / nM, mblk = lid % nM;
    const int cnt = *resid_count;
    if (mblk * 256 >= cnt) return;  // whole workgroup idle (uniform)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = tile * kTileN;
    const int mw0 = mblk * 256 + wave * 64;
    const bool compute = mw0 < cnt;

    const float* arow[4];
    floatx4 acc[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const ResidRow ra = resid_row(resid_list, min(mw0 + 16 * mb + (lane & 15), cnt - 1), B, gamma, nA);
        arow[mb] = A + (size_t)ra.x * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const ResidRow rr = resid_row(resid_list, min(row, cnt - 1), B, gamma, nA);
            const float* lrow = L + ((size_t)rr.b * gamma + (rr.ks - 1)) * V;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                acc[mb][nb][i] = (compute && row < cnt && col < V) ? lrow[col] : 0.0f;
            }
        }
    }
    markov_tile<F32, 4>(Bm, V, r, n0, arow, compute, lds, acc);
    if (!compute) return;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const ResidRow rr = resid_row(resid_list, min(row, cnt - 1), B, gamma, nA);
            const float* trow = Tg + ((size_t)rr.b * (gamma + 1) + (rr.ks - 1)) * V;
            const float ld = lse_log2(lse_d[(size_t)rr.b * gamma + rr.ks - 1]);
            const float lt = lse_log2(lse_t[(size_t)rr.b * gamma + rr.ks - 1]);
            double sw = 0.0, sp = 0.0;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                if (col < V) {
                    float ptv;
                    sw += (double)resid_weight(acc[mb][nb][i], trow[col], ld, lt, &ptv);
                    sp += (double)ptv;
                }
            }
            sw = sum16(sw);
            sp = sum16(sp);
            if ((lane & 15) == 0 && row < cnt) rpart[(size_t)rr.b * nT + tile] = make_float2((float)sw, (float)sp);
        }
    }
}

// ---------------------------------------------------------------------------
// Residual tiles, bf16: persistent 8-wave workgroups over 64-column tiles in
// vocabulary-major MFMA form (dspark_tile.hpp), the same pipeline as the
// draft tile kernel: Bm tiles through four LDS buffers, the rejected rows'
// draft logits (L) and target logits (T) loaded into registers one tile
// ahead, and the per-tile sums staged in LDS.  (With the L and T registers,
// holding a second tile's logits for a deferred epilogue would not fit the
// register file.)  Loads per iteration and wave: the L and T rows of two
// batch blocks (four load_row16) and the Bm DMA (wait_stage).
// ---------------------------------------------------------------------------
constexpr int kResPartTiles = 12;

// Rank of workgroup b among the G workgroups of a launch in the order the
// hardware starts them when every CU takes one at a time: workgroups go to
// the 8 XCDs round-robin (b mod 8), and within an XCD the q-th one (q = b/8)
// lands on CU q mod cpx, behind the ones before it on that CU (measured on
// MI355X: with one workgroup per CU, a workgroup that exits at once does not
// let a later one past an earlier one still running on its CU).  Rank
// p*8*cpx + x*n_p + (q mod cpx) for position p = q / cpx (n_p workgroups of
// the XCD at that position): position 0 of every CU first, consecutive
// ranks on one XCD.  A bijection of [0, G) when G is a multiple of 8; the
// XCD-grouped order of xcd_logical_id otherwise.
__device__ __forceinline__ int resid_item(int b, int G, int cpx)
{
    if ((G & 7) || cpx <= 0) return xcd_logical_id(b, G);
    const int x = b & 7, q = b >> 3, Qx = G >> 3;
    const int p = q / cpx, n = min(cpx, Qx - p * cpx);
    return p * 8 * cpx + x * n + (q - p * cpx);
}

// Byte offset of the draft's slot-aggregate rows from the residual tile sums
// in the verify workspace (residual tile sums, bonus chunk maxima and sums,
// the A-row hand-over, each rounded up to 256 bytes): B > 256 kernels reach
// the per-slot residual sums there without a kernel argument (the launcher
// checks the layout agrees).
__host__ __device__ inline size_t rslot_offset(int B, int V)
{
    const size_t nT = (size_t)(V + kTcols - 1) / kTcols, nC = (size_t)(V + kChunkElems - 1) / kChunkElems;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return up((size_t)B * nT * 8) + up((size_t)B * nC * 4) + up((size_t)B * nC * 8) + up(ag_bytes(B));
}

template <int KS, bool SLOTS = false>
__global__ __launch_bounds__(64 * kTileWaves) void k_resid_tiles_bf16(
    const uint16_t* __restrict__ Tg, const uint16_t* __restrict__ L, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ accepted,
    const int4* __restrict__ resid_list, const int32_t* __restrict__ resid_count, int B, int gamma, int V, int r, int nT,
    int nM, int S, int nA, int cpx, float2* __restrict__ rpart)
{
    constexpr int NW = kTileWaves, R = kTileRows;
    __shared__ __attribute__((aligned(1024))) char s0[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s1[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s2[kBmTileBytes];
    __shared__ __attribute__((aligned(1024))) char s3[kBmTileBytes];
    __shared__ unsigned long long stage[kResPartTiles][R];  // float2 pairs, stored as one 64-bit word each

    // Work items (slot, row block) of the row blocks that hold rejected rows,
    // slot-major, so the row blocks of a slot are consecutive items; items
    // past them exit at once.  Items go to workgroups in dispatch order
    // (resid_item), so whatever the rejected count, the active items take
    // the first workgroup of every CU and a slot's row blocks share an XCD.
    const int cntr = *resid_count;
    const int nMa = min(nM, (cntr + R - 1) / R);
    const int item = resid_item(blockIdx.x, gridDim.x, cpx);
    if (item >= S * nMa) return;  // uniform
    const int mblk = item % nMa, slot = item / nMa;
    const int m0 = mblk * R;
    int t0, ts, cnt;
    slot_tiles(slot, S, nT, &t0, &ts, &cnt);
    if (cnt <= 0) return;  // uniform
    const int w = wave_id(), lane = threadIdx.x & 63, G = lane >> 4, c = lane & 15;
    // Batch block bb of wave w holds the workgroup's rows 128bb + 16w .. +15,
    // so the first rejected rows spread over all waves (and SIMDs) and a
    // block past the last rejected row is skipped.
    auto row_of = [&](int bb) { return 128 * bb + 16 * w; };
    const bool act0 = m0 + row_of(0) < cntr, act1 = m0 + row_of(1) < cntr;

    uint4 a[2][8];  // B operand: the rows' A vectors (loaded in the prologue)
    const uint16_t* lrow[2];
    const uint16_t* trow[2];
    int lrow_idx[2];
    int rowb[2] = { 0, 0 };  // request of this lane's row in each active block (its partials' row)
    float ld[2], lt[2];
    int4 rec[2];  // the rows' records (decoded after the first Bm tile is issued)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) rec[bb] = resid_list[min(m0 + row_of(bb) + c, cntr - 1)];
    const int nks = KS > 0 ? KS : (r + 31) / 32;

    auto load_lt = [&](auto nbb, int i, uint4 (&lv)[2][2], uint4 (&tv)[2][2]) {
        const bool dummy = i >= cnt;
#pragma unroll
        for (int bb = 0; bb < decltype(nbb)::value; ++bb) {
            load_row16(lrow[bb], (t0 + i * ts) * kTcols, V, dummy, lv[bb]);
            load_row16(trow[bb], (t0 + i * ts) * kTcols, V, dummy, tv[bb]);
        }
    };
    const BmDmaLanes<NW> dml = bm_dma_lanes<NW>(V, r);
    auto dma = [&](int i, char* buf) { dma_bm_tile_pre<NW>(Bm, V, r, (t0 + i * ts) * kTcols, i >= cnt, buf, dml); };
    auto dma_block = [&](int i, char* buf, int t) {
        dma_bm_block_pre<NW>(Bm, V, (t0 + i * ts) * kTcols, i >= cnt, buf, dml, t);
    };

    // Row sums of tile i from its logits f (accumulators) and target values,
    // for the first NBB batch blocks.  Every lane of a row ends with the same
    // bits, so the staging store needs no lane predicate.
    auto epilogue = [&](auto nbb, int i, const floatx4 (&f)[4][decltype(nbb)::value], const uint4 (&tv)[2][2]) {
        constexpr int NBB = decltype(nbb)::value;
#pragma unroll
        for (int bb = 0; bb < NBB; ++bb) {
            // Per 4-column block in column order, the block sums pairwise, then
            // the xor-16 / xor-32 butterflies (short chains, no LDS).
            float sw[4], sp[4];
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                const floatx4 t = bf16x4_to_f32(row16_block(tv[bb], vb));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float ptv;
                    const float w = resid_weight(f[vb][bb][e], t[e], ld[bb], lt[bb], &ptv);
                    sw[vb] = e == 0 ? w : sw[vb] + w;
                    sp[vb] = e == 0 ? ptv : sp[vb] + ptv;
                }
            }
            stage[i][row_of(bb) + c] = pack_f2(sum_xor16_32((sw[0] + sw[1]) + (sw[2] + sw[3])),
                                               sum_xor16_32((sp[0] + sp[1]) + (sp[2] + sp[3])));
        }
    };
    // The vocabulary's tail tile: target values of columns at or past V
    // become -inf, so their residual weight and target probability are 0
    // (V is a multiple of 8: a 16-byte group is entirely in or out).
    auto mask_tail = [&](auto nbb, int i, uint4 (&tv)[2][2]) {
        const int n0 = (t0 + i * ts) * kTcols;
        if (n0 + kTcols > V) {  // uniform
            const uint4 ninf = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
#pragma unroll
            for (int bb = 0; bb < decltype(nbb)::value; ++bb)
#pragma unroll
                for (int h = 0; h < kRow16Loads; ++h)
                    if (n0 + 16 * G + 8 * h >= V) tv[bb][h] = ninf;
        }
    };
    // L and T values of two tiles in flight: the four unrolled bodies
    // alternate between two register sets, so no copy waits on a load just issued.
    uint4 l0[2][2], t0r[2][2], l1[2][2], t1r[2][2];
    // The whole pipeline for a wave whose first NB batch blocks hold rejected
    // rows (NB = 2, 1 or 0, uniform per wave): only those blocks' L and T rows
    // are loaded, and every wait counts exactly this path's loads.  All waves
    // take part in every tile's DMA and barrier.
    auto run = [&](auto nbb) {
        constexpr int NB = decltype(nbb)::value;
        constexpr int NL = 2 * kRow16Loads * NB;  // L and T row loads per tile
        constexpr int NA = 10 * NB;               // after the first tile: A operand (8 per block), normalisers (2)
        auto body = [&](int i, const char* cur, char* nxt, uint4 (&lc)[2][2], uint4 (&tc)[2][2], uint4 (&ln)[2][2],
                        uint4 (&tn)[2][2]) {
            if (KS > 0) wait_stage<NL, 32 / NW, NA>(i);
            else if (i == 0) wait_all_mem();  // run-time rank
            else wait_stage<NL, 32 / NW, NA>(i);
            barrier_lds();  // Bm tile i has landed in cur; every wave is done with nxt
            issue_fence();
            load_lt(nbb, i + 1, ln, tn);
            issue_fence();
            if (i == 0) {  // ramp-up: tiles 1 and 2 (buffers s1, s2) behind tile 3
                dma(1, s1);
                issue_fence();
                dma(2, s2);
                issue_fence();
            }
            // Bm tile i+3: with a compile-time rank its DMA instructions go
            // between the MFMAs (see the draft tile kernel).
            if constexpr (KS == 0) {
                dma(i + 3, nxt);
                issue_fence();
            }
            auto hook = [&](int ks) {
                if ((ks & 1) == 0) dma_block(i + 3, nxt, ks >> 1);
            };
            if constexpr (NB > 0) {
                mask_tail(nbb, i, tc);
                floatx4 acc[4][NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                    for (int vb = 0; vb < 4; ++vb) acc[vb][bb] = bf16x4_to_f32(row16_block(lc[bb], vb));
                const uint4(&an)[NB][8] = *reinterpret_cast<const uint4(*)[NB][8]>(&a[0]);
                if constexpr (KS > 0) tile_mma_vm<NB, KS>(an, cur, nks, acc, hook);
                else tile_mma_vm<NB, KS>(an, cur, nks, acc);
                epilogue(nbb, i, acc, tc);
            } else if constexpr (KS > 0) {
                for (int t = 0; t < 32 / NW; ++t) dma_block(i + 3, nxt, t);
                issue_fence();
            }
        };

        // Prologue: the rows' records were loaded first; the first Bm tile
        // does not depend on them and is issued before they are used; then
        // the first L and T tiles, the A-operand gather and the rows'
        // normalisers (NA loads after the first tile).
        issue_fence();
        dma(0, s0);
        issue_fence();
        if constexpr (NB > 0) {
            const uint16_t* arn[NB];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const ResidRow rr = resid_decode(rec[bb], B, gamma, nA);
                arn[bb] = A + (size_t)rr.x * r;
                lrow[bb] = L + ((size_t)rr.b * gamma + (rr.ks - 1)) * V;
                trow[bb] = Tg + ((size_t)rr.b * (gamma + 1) + (rr.ks - 1)) * V;
                lrow_idx[bb] = rr.b * gamma + rr.ks - 1;
                rowb[bb] = rr.b;
            }
            load_lt(nbb, 0, l0, t0r);
            issue_fence();
            load_a_frags<NB>(arn, r, *reinterpret_cast<uint4(*)[NB][8]>(&a[0]));
            double lsd[NB], lst[NB];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                lsd[bb] = lse_d[lrow_idx[bb]];
                lst[bb] = lse_t[lrow_idx[bb]];
            }
            issue_fence();
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                ld[bb] = lse_log2(lsd[bb]);
                lt[bb] = lse_log2(lst[bb]);
            }
        }
        // Tile 0 is peeled off the loop (see the draft tile kernel).
        body(0, s0, s3, l0, t0r, l1, t1r);
        // Whole rounds of four tiles, then at most three more (see the draft
        // tile kernel: no exit between the bodies of the loop).
        int i = 1;
        for (; i + 4 <= cnt; i += 4) {
            body(i, s1, s0, l1, t1r, l0, t0r);
            body(i + 1, s2, s1, l0, t0r, l1, t1r);
            body(i + 2, s3, s2, l1, t1r, l0, t0r);
            body(i + 3, s0, s3, l0, t0r, l1, t1r);
        }
        const int rest = cnt - i;
        if (rest == 1) {
            body(i, s1, s0, l1, t1r, l0, t0r);
        } else if (rest == 2) {
            body(i, s1, s0, l1, t1r, l0, t0r);
            body(i + 1, s2, s1, l0, t0r, l1, t1r);
        } else if (rest == 3) {
            body(i, s1, s0, l1, t1r, l0, t0r);
            body(i + 1, s2, s1, l0, t0r, l1, t1r);
            body(i + 2, s3, s2, l1, t1r, l0, t0r);
        }
    };
    if (act1) run(std::integral_constant<int, 2>{});
    else if (act0) run(std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 0>{});
    // As in the draft tile kernel: LDS wait and barrier for the staging, the
    // dummy loads drain while the sums are written.  The partials go to the
    // row of the request (rpart is indexed by request, so the final kernel
    // can read them before it knows whether the request was rejected); each
    // wave writes its own rows, lane group G taking tiles G, G+4, ...
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int row = row_of(bb) + c;
        if (m0 + row < cntr)
            for (int i = G; i < cnt; i += 4) rpart[(size_t)rowb[bb] * nT + t0 + i * ts] = unpack_f2(stage[i][row]);
    }
    // SLOTS (B > 256): the request's sums over this slot's tiles, in tile
    // order, for the final kernel's first level.
    if (SLOTS && G == 0) {
        float2* rslot = reinterpret_cast<float2*>(reinterpret_cast<char*>(rpart) + rslot_offset(B, V));
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int row = row_of(bb) + c;
            if (m0 + row < cntr) {
                float2 sum = make_float2(0.0f, 0.0f);
                for (int i = 0; i < cnt; ++i) {
                    const float2 v = unpack_f2(stage[i][row]);
                    sum.x += v.x;
                    sum.y += v.y;
                }
                rslot[(size_t)rowb[bb] * kSlotAggMax + slot] = sum;
            }
        }
    }
    wait_all_mem();
}

// ---------------------------------------------------------------------------
// Final token of each request.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_final(
    const typename DT::T* __restrict__ Tg, const typename DT::T* __restrict__ L, const typename DT::T* __restrict__ A,
    const typename DT::T* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ len,
    const int32_t* __restrict__ accepted, const float2* __restrict__ rpart, const float* __restrict__ bm,
    const double* __restrict__ bsum, int gamma, int V, int r, int nT, int nC, int rnn, SeedArg seed_arg,
    int32_t* __restrict__ out_tok)
{
    const uint64_t seed = seed_of(seed_arg);
    typedef typename DT::T T;
    typedef TileTraits<DT> TT;
    __shared__ __attribute__((aligned(1024))) char lds[TT::kLdsBytes];
    __shared__ BlockScratch bs;
    __shared__ double sh_cprev;
    __shared__ int sh_tok;

    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63;
    const int l = clamp_len(len[b], gamma);
    const int a = accepted[b];

    if (a < l) {
        // ---- residual at the first rejected position ks -------------------
        const int ks = a + 1;
        const float2* rq = rpart + (size_t)b * nT;
        // Total residual mass decides between the residual and its p_t fallback.
        double sloc = 0.0;
        {
            const int per = (nT + kThreads - 1) / kThreads;
            const int i0 = min(t * per, nT), i1 = min(i0 + per, nT);
            for (int i = i0; i < i1; ++i) sloc += (double)rq[i].x;
        }
        const bool degen = !(block_sum(sloc, bs) > 0.0);
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)ks, 2u);
        const Located loc = locate(
            nT, [&](int i) { const float2 q = rq[i]; return (double)(degen ? q.y : q.x); }, u, bs, &sh_cprev);

        const int n0 = loc.idx * TT::kCols;
        const T* trow = Tg + ((size_t)b * (gamma + 1) + (ks - 1)) * V;
        const T* lrow = L + ((size_t)b * gamma + (ks - 1)) * V;
        const int prev = rnn ? b * gamma + ks - 1 : cond_token_v(x0, tok, b, gamma, ks, V);
        const float ld = lse_log2(lse_d[(size_t)b * gamma + ks - 1]);
        const float lt = lse_log2(lse_t[(size_t)b * gamma + ks - 1]);
        auto weight = [&](float fv, float tv) {
            float ptv;
            const float wr = resid_weight(fv, tv, ld, lt, &ptv);
            return (double)(degen ? ptv : wr);
        };
        if constexpr (std::is_same<DT, Bf16>::value) {
            floatx4 f[4];
            row_tile_vm(lrow, A, Bm, prev, V, r, n0, lds, f);
            if ((t >> 6) == 0) {
                uint4 tv[2];
                load_row16(trow, n0, V, false, tv);
                floatx4 tf[4];
#pragma unroll
                for (int vb = 0; vb < 4; ++vb) tf[vb] = bf16x4_to_f32(row16_block(tv, vb));
                double wsel;
                const int j = scan_vm_tile(
                    n0, 0, 1.0, loc.cprev, loc.tau,
                    [&](int vb, int i, int col) { return col < V ? weight(f[vb][i], tf[vb][i]) : 0.0; }, &wsel);
                if (lane == 0) sh_tok = clamp_tok(n0 + j, V);
            }
        } else {
            float f[TT::kNB];
            row_tile_f(lrow, A, Bm, prev, V, r, n0, lds, f);
            if ((t >> 6) == 0) {
                double wv[TT::kNB];
#pragma unroll
                for (int nb = 0; nb < TT::kNB; ++nb) {
                    const int col = n0 + 16 * nb + (lane & 15);
                    wv[nb] = col < V ? weight(f[nb], DT::to_f32(trow[col])) : 0.0;
                }
                double wsel;
                const int j = scan_tile_weights<TT::kNB>(wv, 1.0, loc.cprev, loc.tau, &wsel);
                if (lane == 0) sh_tok = clamp_tok(n0 + j, V);
            }
        }
    } else {
        // ---- bonus token from target row l (position l + 1) ----------------
        const float* pm = bm + (size_t)b * nC;
        const double* ps = bsum + (size_t)b * nC;
        const int per = (nC + kThreads - 1) / kThreads;
        const int c0 = min(t * per, nC), c1 = min(c0 + per, nC);
        float mloc = -INFINITY;
        for (int c = c0; c < c1; ++c) mloc = fmaxf(mloc, pm[c]);
        const float M = block_max(mloc, bs);
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(l + 1), 3u);
        const Located loc = locate(nC, [&](int c) { return tile_mass(pm[c], ps[c], M); }, u, bs, &sh_cprev);

        // rescan the chunk in index order: 32 contiguous elements per thread
        const float mc = pm[loc.idx];
        const float mcl = row_mlog2(mc);
        const double scale = tile_mass(mc, 1.0, M);
        const T* x = Tg + ((size_t)b * (gamma + 1) + l) * V;
        constexpr int EPT = kChunkElems / kThreads;  // 32
        const int e0 = loc.idx * kChunkElems + t * EPT;
        double wv[EPT];
        double tsum = 0.0;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int e = e0 + j;
            double wj = 0.0;
            if (e < V && mc != -INFINITY) {
                const float xv = DT::to_f32(x[e]);
                wj = (double)softmax_w(xv, mcl);
            }
            wv[j] = wj;
            tsum += wj;
        }
        double tot;
        const double tpre = block_excl_scan(tsum, bs, &tot);
        int hit = INT_MAX, lastpos = -1;
        double run = tpre;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            run += wv[j];
            if (hit == INT_MAX && loc.cprev + scale * run > loc.tau) hit = e0 + j;
            if (wv[j] > 0.0) lastpos = e0 + j;
        }
        const int th = block_min_int(hit, bs);
        const int tl = block_max_int(lastpos, bs);
        if (t == 0) sh_tok = clamp_tok(th != INT_MAX ? th : max(tl, 0), V);
    }
    __syncthreads();
    const int token = sh_tok;
    for (int kk = t; kk <= gamma; kk += kThreads)
        out_tok[(size_t)b * (gamma + 1) + kk] = kk < a ? tok[(size_t)b * gamma + kk] : (kk == a ? token : -1);
}

// ---------------------------------------------------------------------------
// Final token, bf16: one wave per request.  Residual: the residual tile sums
// are located with wave scans and the chosen tile is recomputed by the wave
// from its own LDS copy of the Bm tile (row_tile_vm_wave), in the MFMA batch
// column the row had in the residual pass.  Bonus: the target chunk is
// located from the chunk partials; each lane sums the weights of 128
// contiguous elements of the chunk, the lane slice holding the crossing is
// found by a wave scan, and that slice (handed over through LDS by the lane
// that loaded it) is rescanned two elements per lane.
//
// The small loads that do not depend on the accept count go out with the
// length and the accept count: the request's bonus chunk partials (unused,
// and possibly stale, when the request has a rejection) and per position k = lane + 1
// its conditioning token, draft token and both log-normalisers.  The
// residual tile sums (the request's row of the residual partials) are read
// in the residual branch only: issued in every workgroup they cost more than
// the round trip they save (measured on MI355X, B = 256, V = 129280: 9.7
// against 8.4 us per launch).  SLOTS (B > 256, at most 256 residual slots):
// the request's per-slot sums are read instead (2 KB), then the chosen
// slot's tile sums (measured on MI355X, B = 1024, V = 129280: 10.2-11.2
// against 11.7-15.0 us per launch).
// ---------------------------------------------------------------------------

// Holds v in a register at this point, so the load that produced it is not
// moved into the one branch that uses it (behind the accept count).
template <class X>
__device__ __forceinline__ void pin_reg(X& v)
{
    asm volatile("" : "+v"(v));
}

template <int KS, int PER, bool SLOTS = false>
__global__ __launch_bounds__(64) void k_final_bf16(
    const uint16_t* __restrict__ Tg, const uint16_t* __restrict__ L, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ len,
    const int32_t* __restrict__ accepted, const float2* __restrict__ rpart, const float* __restrict__ bm,
    const double* __restrict__ bsum, int gamma, int V, int r, int nT, int nC, int rmode, SeedArg seed_arg,
    int32_t* __restrict__ out_tok)
{
    // rmode: the RNN head flag; with SLOTS also the residual slot count
    // (bits 1-9) and the batch size (bits 10 and up), which locate the
    // per-slot residual sums without more kernel arguments.
    const int rnn = SLOTS ? (rmode & 1) : rmode;
    const uint64_t seed = seed_of(seed_arg);
    __shared__ __attribute__((aligned(1024))) char lds[kBmTileBytes];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const size_t row0 = (size_t)b * gamma;

    const int l = clamp_len(len[b], gamma);
    const int a = accepted[b];
    int xc = 0, tk = 0;       // position lane+1: conditioning token x_lane, draft token x_{lane+1}
    double lsd = 0.0, lst = 0.0;  // and the draft / target log-normalisers of its row
    if (lane < gamma) {
        if (!rnn) xc = lane == 0 ? x0[b] : tok[row0 + lane - 1];  // the RNN head has no x0 (null)
        tk = tok[row0 + lane];
        lsd = lse_d[row0 + lane];
        lst = lse_t[row0 + lane];
    }
    // nC <= 64 * 4 chunks (lengths up to 2^21), slices of at most 4 per lane.
    const float* pm = bm + (size_t)b * nC;
    const double* ps = bsum + (size_t)b * nC;
    const int cper = (nC + 63) / 64, c0l = lane * cper;
    float cm[4];
    double cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ci = min(c0l + j, nC - 1);
        const bool ok = j < cper && c0l + j < nC;
        cm[j] = ok ? pm[ci] : -INFINITY;
        cs[j] = ok ? ps[ci] : 0.0;
    }
    pin_reg(xc);
    pin_reg(lsd);
    pin_reg(lst);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pin_reg(cm[j]);
        pin_reg(cs[j]);
    }
    int token;

    if (a < l) {
        // ---- residual at the first rejected position ks = a + 1 -----------
        const int ks = a + 1;
        // SLOTS (B > 256): the request's per-slot sums first (2 KB, Sr <= 256
        // slots of contiguous tiles), then the chosen slot's tile sums, as the
        // draft locate reads its slot aggregates; else the row's tile sums.
        float2 q[SLOTS ? 1 : PER];
        float2 qs[4];
        int i0 = 0, i0s = 0;
        const int Sr = (rmode >> 1) & 511;
        if constexpr (SLOTS) {
            const float2* rslot =
                reinterpret_cast<const float2*>(reinterpret_cast<const char*>(rpart) + rslot_offset(rmode >> 10, V));
            load_slices<4>(rslot + (size_t)b * kSlotAggMax, Sr, make_float2(0.0f, 0.0f), qs, &i0s);
        } else {
            load_slices<PER>(rpart + (size_t)b * nT, nT, make_float2(0.0f, 0.0f), q, &i0);
        }
        uint4 af[1][8];
        {
            const int xr = rnn ? (int)row0 + a : clamp_tok(__shfl(xc, a, 64), V);
            const uint16_t* arow[1] = { A + (size_t)xr * r };
            load_a_frags<1>(arow, r, af);
        }
        float sw = 0.0f;
        if constexpr (SLOTS) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sw += qs[j].x;
        } else {
#pragma unroll
            for (int j = 0; j < PER; ++j) sw += q[j].x;
        }
        const bool degen = !(wave_last(wave_incl_scan((double)sw)) > 0.0);  // no residual mass: sample p_t
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)ks, 2u);
        Located loc;
        if constexpr (SLOTS) {
            const Located ls = wave_locate_slices<4>(
                i0s, [&](int j) { return (double)(degen ? qs[j].y : qs[j].x); }, u, reinterpret_cast<double*>(lds));
            // the chosen slot's tiles (at most 12), one per lane, from the mass
            // before the slot; without a crossing, its last tile of positive mass
            int t0, ts, cnt;
            slot_tiles(ls.idx, Sr, nT, &t0, &ts, &cnt);
            const float2 qt = rpart[(size_t)b * nT + t0 + min(lane, cnt - 1) * ts];
            const double mm = lane < cnt ? (double)(degen ? qt.y : qt.x) : 0.0;
            const double inc = wave_incl_scan(mm);
            const uint64_t hit = __ballot(mm > 0.0 && ls.cprev + inc > ls.tau);
            const uint64_t pos = __ballot(mm > 0.0);
            const int sel = hit ? __builtin_ctzll(hit) : pos ? 63 - __builtin_clzll(pos) : 0;
            loc.S = ls.S;
            loc.tau = ls.tau;
            loc.idx = t0 + sel * ts;
            loc.cprev = ls.cprev + __shfl(inc - mm, sel, 64);
        } else {
            loc = wave_locate_slices<PER>(
                i0, [&](int j) { return (double)(degen ? q[j].y : q[j].x); }, u, reinterpret_cast<double*>(lds));
        }

        const int n0 = loc.idx * kTcols;
        const uint16_t* trow = Tg + ((size_t)b * (gamma + 1) + (ks - 1)) * V;
        uint4 tv[2];
        load_row16(trow, n0, V, false, tv);
        floatx4 f[4];
        row_tile_vm_wave<KS>(L + (row0 + (ks - 1)) * V, af, Bm, V, r, n0, lds, f);
        const float ld = lse_log2(__shfl(lsd, a, 64));
        const float lt = lse_log2(__shfl(lst, a, 64));
        floatx4 tf[4];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) tf[vb] = bf16x4_to_f32(row16_block(tv, vb));
        double wsel;
        const int j = scan_row_tile_lanes(
            n0, 1.0, loc.cprev, loc.tau,
            [&](int col, auto pick) {
                if (col >= V) return 0.0;
                float ptv;
                const float wr = resid_weight(pick(f), pick(tf), ld, lt, &ptv);
                return (double)(degen ? ptv : wr);
            },
            &wsel);
        token = clamp_tok(n0 + j, V);
    } else {
        // ---- bonus token from target row l (position l + 1) ----------------
        const float M = wave_max(fmaxf(fmaxf(cm[0], cm[1]), fmaxf(cm[2], cm[3])));
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(l + 1), 3u);
        const Located loc = wave_locate_slices<4>(c0l, [&](int j) { return tile_mass(cm[j], cs[j], M); }, u,
                                                  reinterpret_cast<double*>(lds));

        // The chosen chunk's maximum, from the lane whose slice holds it.
        const int own = loc.idx / cper, jo = loc.idx - lane * cper;
        float mine = cm[0];
#pragma unroll
        for (int j = 1; j < 4; ++j)
            if (j == jo) mine = cm[j];
        const float mc = __shfl(mine, own, 64);
        const float mcl = row_mlog2(mc);
        const double scale = tile_mass(mc, 1.0, M);
        const uint16_t* x = Tg + ((size_t)b * (gamma + 1) + l) * V;
        constexpr int EPL = kChunkElems / 64;  // 128 elements per lane
        const int c0 = loc.idx * kChunkElems;
        auto w_of = [&](int e, float xv) { return e < V && mc != -INFINITY ? (double)softmax_w(xv, mcl) : 0.0; };
        // Pass 1: lane totals over contiguous 128-element slices (16-byte
        // loads, all in flight at once; V is a multiple of 8, so a group
        // that starts below V is loaded unclamped).
        const int e0 = c0 + lane * EPL;
        uint4 xv[EPL / 8];
#pragma unroll
        for (int qv = 0; qv < EPL / 8; ++qv) xv[qv] = ld16(x + min(e0 + 8 * qv, V - 8));
        double tl = 0.0;
#pragma unroll
        for (int qv = 0; qv < EPL / 8; ++qv) {
            float tv = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) tv += (float)w_of(e0 + 8 * qv + jj, Bf16::get(xv[qv], jj));
            tl += (double)tv;
        }
        const double inc = wave_incl_scan(tl);
        const double off = wave_excl_from_incl(inc);
        const uint64_t mh = __ballot(tl > 0.0 && loc.cprev + scale * inc > loc.tau);
        const uint64_t mp = __ballot(tl > 0.0);
        int src;
        if (mh) src = __builtin_ctzll(mh);
        else if (mp) src = 63 - __builtin_clzll(mp);
        else src = 0;
        // Pass 2: the chosen slice, two elements per lane, scanned in index
        // order.  Lane src hands its 128 values over through LDS (past the
        // locate scratch): lane L takes the 32-bit word L, elements 2L, 2L+1.
        uint4* xs = reinterpret_cast<uint4*>(lds + 1024);
        if (lane == src) {
#pragma unroll
            for (int qv = 0; qv < EPL / 8; ++qv) xs[qv] = xv[qv];
        }
        __builtin_amdgcn_wave_barrier();  // one wave: its LDS accesses complete in order
        const uint32_t pair = reinterpret_cast<const uint32_t*>(xs)[lane];
        __builtin_amdgcn_wave_barrier();
        const double base = __shfl(off, src, 64);
        const int s0 = c0 + src * EPL + 2 * lane;
        const double w0 = s0 < V ? w_of(s0, __uint_as_float(pair << 16)) : 0.0;
        const double w1 = s0 + 1 < V ? w_of(s0 + 1, __uint_as_float(pair & 0xFFFF0000u)) : 0.0;
        const double pin = wave_incl_scan(w0 + w1);
        const double pex = pin - (w0 + w1);
        const double r0 = base + pex + w0, r1 = base + pex + w0 + w1;
        const bool h0 = loc.cprev + scale * r0 > loc.tau, h1 = loc.cprev + scale * r1 > loc.tau;
        const uint64_t ch = __ballot(h0 || h1);
        const uint64_t cp = __ballot(w0 > 0.0 || w1 > 0.0);
        int e;
        if (ch) {
            const int sl = __builtin_ctzll(ch);
            const int which = __shfl((int)(h0 ? 0 : 1), sl, 64);
            e = c0 + src * EPL + 2 * sl + which;
        } else if (cp) {
            const int sl = 63 - __builtin_clzll(cp);
            const int which = __shfl((int)(w1 > 0.0 ? 1 : 0), sl, 64);
            e = c0 + src * EPL + 2 * sl + which;
        } else {
            e = 0;
        }
        token = clamp_tok(e, V);
    }
    // gamma <= 16: one lane per output slot.
    if (lane <= gamma) out_tok[(size_t)b * (gamma + 1) + lane] = lane < a ? tk : (lane == a ? token : -1);
}

template <class DT>
static hipError_t verify_t(const void* Tg_, const void* L_, const void* A_, const void* Bm_, const int32_t* x0,
                           const int32_t* tok, const float* pd, const double* lse_d, const int32_t* len, int B,
                           int gamma, int V, int r, SeedArg seed, int32_t* accepted, int32_t* out_tok,
                           int32_t* n_out, float* target_p, const void* H, void* ws, const WsLayout& lay, hipStream_t s)
{
    // RNN head: the operand rows are the draft's states H[b][k-1] (row b*gamma + k-1) instead of A[x].
    const int rnn = H ? 1 : 0, nA = H ? B * gamma : V;
    if (H) A_ = H;
    typedef typename DT::T T;
    const T* Tg = static_cast<const T*>(Tg_);
    const T* L = static_cast<const T*>(L_);
    const T* A = static_cast<const T*>(A_);
    const T* Bm = static_cast<const T*>(Bm_);
    char* w = static_cast<char*>(ws);
    float* tgm = reinterpret_cast<float*>(w + lay.tgt_m);
    double* tgs = reinterpret_cast<double*>(w + lay.tgt_s);
    double* lse_t = reinterpret_cast<double*>(w + lay.lse_t);
    int4* rlist = reinterpret_cast<int4*>(w + lay.resid_list);
    int32_t* rcnt = reinterpret_cast<int32_t*>(w + lay.resid_count);
    float2* rpart = reinterpret_cast<float2*>(w + lay.res_part);
    float* bm = reinterpret_cast<float*>(w + lay.bon_m);
    double* bsum = reinterpret_cast<double*>(w + lay.bon_s);
    const int nT = n_tiles(std::is_same<DT, Bf16>::value ? 1 : 0, V), nC = n_chunks(V);
    // bf16: the residual pass's tile slots, and whether it also writes
    // per-(request, slot) residual sums for the final kernel's two-level
    // locate (B > 256, at most kSlotAggMax slots).  They go to the draft's
    // slot-aggregate rows, which the draft call has finished reading, and
    // both kernels find them at rslot_offset past the residual tile sums.
    const int Sr = tile_slots(nT, (B + kTileRows - 1) / kTileRows, cu_count(), kResPartTiles);
    const bool rslot = std::is_same<DT, Bf16>::value && B > kTileRows && B < (1 << 21) && Sr <= kSlotAggMax;
    if (rslot && lay.slot_agg != lay.res_part + rslot_offset(B, V)) return hipErrorInvalidValue;

    launch_timed(K_TARGET_PARTIALS, k_row_partials<DT>, dim3(nC, B * gamma), dim3(kThreads), s, Tg, len, accepted,
                 gamma, V, nC, kRowTarget, tgm, tgs, rcnt);
    // Bonus rows inside the accept launch while reading them for every
    // request stays small next to the launch it saves (measured on MI355X:
    // B = 256, V = 129280 bf16, 66 MB: 2 us per step faster; B = 1024, 265 MB:
    // 33-60 us slower).
    const bool bonus_in_accept = (double)B * V * sizeof(T) <= kBonusInAcceptBytes;
    const int nAcc = (B + kAcceptWaves - 1) / kAcceptWaves;
    launch_timed(K_ACCEPT, k_accept_bonus<DT>, dim3(nAcc + (bonus_in_accept ? nC * B : 0)), dim3(kThreads), s, Tg, pd,
                 len, x0, tok, tgm, tgs, B, gamma, V, nC, rnn, seed, accepted, n_out, target_p, lse_t, rlist, rcnt,
                 nAcc, bm, bsum);
    // The bf16 residual-pass and final-token kernels.  The variants without
    // per-slot sums are named first: the code object holds kernels in the
    // order they are first named, and with the slot variants ahead of them
    // the same machine code ran slower (measured on MI355X, B = 256, V =
    // 129280: residual pass 30.9 against 30.4 us, final 8.3 against 8.2 us).
    const bool k8 = (r + 31) / 32 == 8;
    auto resid_kern = k8 ? k_resid_tiles_bf16<8> : k_resid_tiles_bf16<0>;
    auto final_kern = nT <= 64 * 32 ? (k8 ? k_final_bf16<8, 32> : k_final_bf16<0, 32>)
                                    : (k8 ? k_final_bf16<8, 64> : k_final_bf16<0, 64>);
    if (rslot) {
        resid_kern = k8 ? k_resid_tiles_bf16<8, true> : k_resid_tiles_bf16<0, true>;
        final_kern = k8 ? k_final_bf16<8, 32, true> : k_final_bf16<0, 32, true>;
    }
    if (std::is_same<DT, Bf16>::value) {
        const int nM = (B + kTileRows - 1) / kTileRows;
        const int S = Sr;
        launch_timed(K_RESID_TILES, resid_kern, dim3(S * nM), dim3(64 * kTileWaves), s,
                           reinterpret_cast<const uint16_t*>(Tg), reinterpret_cast<const uint16_t*>(L),
                           reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(Bm), x0, tok,
                           lse_d, lse_t, accepted, rlist, rcnt, B, gamma, V, r, nT, nM, S, nA, cu_count() / 8,
                           rpart);
    } else {
        const int nM = (B + 255) / 256;
        launch_timed(K_RESID_TILES, k_resid_tiles_f32, dim3(nT * nM), dim3(kThreads), s,
                           reinterpret_cast<const float*>(Tg), reinterpret_cast<const float*>(L),
                           reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(Bm), x0, tok, lse_d,
                           lse_t, accepted, rlist, rcnt, B, gamma, V, r, nT, nM, nA, rpart);
    }
    if (!bonus_in_accept)
        launch_timed(K_BONUS_PARTIALS, k_row_partials<DT>, dim3(nC, B), dim3(kThreads), s, Tg, len, accepted, gamma, V,
                     nC, kRowBonusAccepted, bm, bsum, (int32_t*)nullptr);
    if (std::is_same<DT, Bf16>::value && nT <= 64 * 64 && nC <= 64 * 4) {
        launch_timed(K_FINAL, final_kern, dim3(B), dim3(64), s, reinterpret_cast<const uint16_t*>(Tg),
                           reinterpret_cast<const uint16_t*>(L), reinterpret_cast<const uint16_t*>(A),
                           reinterpret_cast<const uint16_t*>(Bm), x0, tok, lse_d, lse_t, len, accepted, rpart, bm,
                           bsum, gamma, V, r, nT, nC, rslot ? rnn | Sr << 1 | B << 10 : rnn, seed, out_tok);
    } else {
        launch_timed(K_FINAL, k_final<DT>, dim3(B), dim3(kThreads), s, Tg, L, A, Bm, x0, tok, lse_d, lse_t, len,
                           accepted, rpart, bm, bsum, gamma, V, r, nT, nC, rnn, seed, out_tok);
    }
    return hipGetLastError();
}

hipError_t launch_verify(int dtype, const void* Tg, const void* L, const void* A, const void* Bm, const int32_t* x0,
                         const int32_t* tok, const float* pd, const double* lse_d, const int32_t* len, int B,
                         int gamma, int V, int r, SeedArg seed, int32_t* accepted, int32_t* out_tok,
                         int32_t* n_out, float* target_p, const void* H, void* ws, const WsLayout& lay,
                         hipStream_t s)
{
    if (dtype == 1)
        return verify_t<Bf16>(Tg, L, A, Bm, x0, tok, pd, lse_d, len, B, gamma, V, r, seed, accepted, out_tok, n_out,
                              target_p, H, ws, lay, s);
    return verify_t<F32>(Tg, L, A, Bm, x0, tok, pd, lse_d, len, B, gamma, V, r, seed, accepted, out_tok, n_out,
                         target_p, H, ws, lay, s);
}

}  // namespace dspark
