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
//   k_target_lse             one wave per row: lse_t and p_t(x_k).
//   k_accept                 one workgroup: accept draws per request; compacts
//                            the requests with a rejection.
//   k_resid_tiles            Markov MFMA tiles of the rejected draft rows
//                            fused with the target row: per tile sums of
//                            max(0, p_t - p_d) and of p_t.
//   k_row_partials (bonus)   grid = chunks x B: target row ell_b + 1 of
//                            requests without a rejection.
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
struct SplitLse {
    float hi, lo;
};
__device__ __forceinline__ SplitLse split_lse(double v)
{
    SplitLse s;
    s.hi = (float)v;
    s.lo = (float)(v - (double)s.hi);
    return s;
}

// Residual weight of one vocabulary entry: w = max(0, p_t - p_d) with
// p = exp((x - hi) - lo) in fp32; *pt receives p_t.  The same expression is
// used by the residual tile pass and by the final rescan, so the weights the
// final sample scans are exactly those summed into the tile partials.
__device__ __forceinline__ float resid_weight(float f, float t, SplitLse d, SplitLse tg, float* pt)
{
    const float ptv = exp_fast((t - tg.hi) - tg.lo);
    const float pdv = exp_fast((f - d.hi) - d.lo);
    *pt = ptv;
    const float w = ptv - pdv;
    return w > 0.0f ? w : 0.0f;
}

// ---------------------------------------------------------------------------
// Chunk max / sum of exp over a target row: 8192 elements per workgroup,
// every element loaded once with 16-byte loads and kept in registers between
// the max and the sum.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_row_partials(const typename DT::T* __restrict__ Tg,
                                                           const int32_t* __restrict__ len,
                                                           const int32_t* __restrict__ accepted, int B, int gamma,
                                                           int V, int nC, int bonus, float* __restrict__ om,
                                                           double* __restrict__ os)
{
    __shared__ BlockScratch bs;
    const int c = blockIdx.x;
    const int row = blockIdx.y;
    int b, trow;
    if (!bonus) {
        b = row / gamma;
        trow = row - b * gamma;
        if (trow >= clamp_len(len[b], gamma)) return;
    } else {
        b = row;
        const int l = clamp_len(len[b], gamma);
        if (accepted[b] < l) return;
        trow = l;
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
    const float ml = M * kLog2e;
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

// ---------------------------------------------------------------------------
// Target log-normaliser and p_t(x_k) of every verified row: one wave per row.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_target_lse(const typename DT::T* __restrict__ Tg,
                                                         const int32_t* __restrict__ tok,
                                                         const int32_t* __restrict__ len,
                                                         const float* __restrict__ tgm,
                                                         const double* __restrict__ tgs, int B, int gamma, int V,
                                                         int nC, double* __restrict__ lse_t, double* __restrict__ pt)
{
    const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= B * gamma) return;
    const int b = row / gamma, kk = row - b * gamma;
    if (kk >= clamp_len(len[b], gamma)) return;
    const float* m = tgm + (size_t)row * nC;
    const double* s = tgs + (size_t)row * nC;
    float M = -INFINITY;
    for (int c = lane; c < nC; c += 64) M = fmaxf(M, m[c]);
    M = wave_max(M);
    double S = 0.0;
    for (int c = lane; c < nC; c += 64) S += tile_mass(m[c], s[c], M);
    S = wave_sum(S);
    if (lane == 0) {
        const double lse = (double)M + log(S);
        lse_t[row] = lse;
        const int x = clamp_tok(tok[row], V);
        const double tx = (double)DT::to_f32(Tg[((size_t)b * (gamma + 1) + kk) * V + x]);
        pt[row] = exp(tx - lse);
    }
}

// ---------------------------------------------------------------------------
// Accept scan: one workgroup of 1024 threads, one request per thread.
// ---------------------------------------------------------------------------
constexpr int kAcceptThreads = 1024;

__global__ __launch_bounds__(kAcceptThreads) void k_accept(const float* __restrict__ pd, const int32_t* __restrict__ len,
                                                           const double* __restrict__ pt, int B, int gamma,
                                                           uint64_t seed, int32_t* __restrict__ accepted,
                                                           int32_t* __restrict__ n_out, float* __restrict__ target_p,
                                                           int32_t* __restrict__ resid_idx,
                                                           int32_t* __restrict__ resid_list,
                                                           int32_t* __restrict__ resid_count)
{
    __shared__ int wsum[kAcceptThreads / 64];
    __shared__ int base;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (t == 0) base = 0;
    __syncthreads();
    for (int b0 = 0; b0 < B; b0 += kAcceptThreads) {
        const int b = b0 + t;
        int rej = 0;
        if (b < B) {
            const int l = clamp_len(len[b], gamma);
            int a = l;
            for (int kk = 0; kk < gamma; ++kk) {
                const size_t row = (size_t)b * gamma + kk;
                if (kk < l) {
                    const double ptk = pt[row];
                    const double ratio = ptk / (double)pd[row];
                    const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(kk + 1), 1u);
                    if (a == l && !(u < (float)ratio)) a = kk;
                    if (target_p) target_p[row] = (float)ptk;
                } else if (target_p) {
                    target_p[row] = 0.0f;
                }
            }
            accepted[b] = a;
            n_out[b] = a + 1;
            rej = a < l;
        }
        int inc = rej;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int n = __shfl_up(inc, o, 64);
            if (lane >= o) inc += n;
        }
        __syncthreads();
        if (lane == 63) wsum[w] = inc;
        __syncthreads();
        int off = base, tot = 0;
        for (int i = 0; i < kAcceptThreads / 64; ++i) {
            if (i < w) off += wsum[i];
            tot += wsum[i];
        }
        const int idx = off + inc - rej;
        if (b < B) {
            resid_idx[b] = rej ? idx : -1;
            if (rej) resid_list[idx] = b;
        }
        __syncthreads();
        if (t == 0) base += tot;
        __syncthreads();
    }
    if (t == 0) *resid_count = base;
}

// Row m of the compacted residual list: request b at its first rejected position ks.
struct ResidRow {
    int b, ks;
};
__device__ __forceinline__ ResidRow resid_row(const int32_t* __restrict__ resid_list,
                                              const int32_t* __restrict__ accepted, int m)
{
    ResidRow r;
    r.b = resid_list[m];
    r.ks = accepted[r.b] + 1;
    return r;
}

// ---------------------------------------------------------------------------
// Residual tiles, fp32: one 4-wave workgroup per (tile, 256-row block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_resid_tiles_f32(
    const float* __restrict__ Tg, const float* __restrict__ L, const float* __restrict__ A,
    const float* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ resid_list, const int32_t* __restrict__ resid_count, int gamma, int V, int r, int nT,
    int nM, double* __restrict__ rw, double* __restrict__ rp)
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
        const ResidRow ra = resid_row(resid_list, accepted, min(mw0 + 16 * mb + (lane & 15), cnt - 1));
        arow[mb] = A + (size_t)cond_token_v(x0, tok, ra.b, gamma, ra.ks, V) * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const ResidRow rr = resid_row(resid_list, accepted, min(row, cnt - 1));
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
            const ResidRow rr = resid_row(resid_list, accepted, min(row, cnt - 1));
            const float* trow = Tg + ((size_t)rr.b * (gamma + 1) + (rr.ks - 1)) * V;
            const SplitLse ld = split_lse(lse_d[(size_t)rr.b * gamma + rr.ks - 1]);
            const SplitLse lt = split_lse(lse_t[(size_t)rr.b * gamma + rr.ks - 1]);
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
            if ((lane & 15) == 0 && row < cnt) {
                rw[(size_t)row * nT + tile] = sw;
                rp[(size_t)row * nT + tile] = sp;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Residual tiles, bf16: persistent workgroups of NW waves (dspark_tile.hpp)
// over 64-column tiles; each LDS buffer holds the Bm tile, the rejected
// rows' draft-logit tile and their target tile, all staged by DMA.
// ---------------------------------------------------------------------------
template <int NW, int KS>
__global__ __launch_bounds__(64 * NW) void k_resid_tiles_bf16(
    const uint16_t* __restrict__ Tg, const uint16_t* __restrict__ L, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ resid_list, const int32_t* __restrict__ resid_count, int gamma, int V, int r, int nT,
    int nM, int S, double* __restrict__ rw, double* __restrict__ rp)
{
    constexpr int R = 32 * NW;
    constexpr int kRowBytes = R * kTrowBytes;
    constexpr int kBuf = kBmTileBytes + 2 * kRowBytes;
    __shared__ __attribute__((aligned(1024))) char buf0[kBuf];
    __shared__ __attribute__((aligned(1024))) char buf1[kBuf];
    __shared__ SplitLse sh_lse[R][2];

    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int mblk = lid % nM, slot = lid / nM;
    const int cnt = *resid_count;
    const int m0 = mblk * R;
    if (m0 >= cnt || slot >= nT) return;  // uniform
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int mw = m0 + 32 * w;
    const bool active = mw < cnt;

    uint4 a[2][8];
    {
        const uint16_t* arow[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const ResidRow ra = resid_row(resid_list, accepted, min(mw + 16 * mb + (lane & 15), cnt - 1));
            arow[mb] = A + (size_t)cond_token_v(x0, tok, ra.b, gamma, ra.ks, V) * r;
        }
        load_a_frags<2>(arow, r, a);
    }
    int lidx[4], tidx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const ResidRow rr = resid_row(resid_list, accepted, min(m0 + dma_row_of<NW>(t), cnt - 1));
        lidx[t] = rr.b * gamma + rr.ks - 1;
        tidx[t] = rr.b * (gamma + 1) + rr.ks - 1;
    }
    for (int i = threadIdx.x; i < R; i += 64 * NW) {
        const int m = m0 + i;
        SplitLse d{ 0.f, 0.f }, t{ 0.f, 0.f };
        if (m < cnt) {
            const ResidRow rr = resid_row(resid_list, accepted, m);
            d = split_lse(lse_d[(size_t)rr.b * gamma + rr.ks - 1]);
            t = split_lse(lse_t[(size_t)rr.b * gamma + rr.ks - 1]);
        }
        sh_lse[i][0] = d;
        sh_lse[i][1] = t;
    }
    const int nks = KS > 0 ? KS : (r + 31) / 32;

    persistent_tiles(
        slot, nT, S, buf0, buf1,
        [&](int tile, char* buf) {
            dma_bm_tile<NW>(Bm, V, r, tile * kTcols, 32 * nks, buf);
            dma_row_tile<NW>(L, lidx, V, tile * kTcols, buf + kBmTileBytes);
            dma_row_tile<NW>(Tg, tidx, V, tile * kTcols, buf + kBmTileBytes + kRowBytes);
        },
        [&](int tile, const char* buf) {
            if (!active) return;
            floatx4 acc[2][4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4{ 0.f, 0.f, 0.f, 0.f };
            tile_mma64<2, KS>(a, buf, nks, acc);
            const int n0 = tile * kTcols;
            const int nl = lane & 15;
            const bool tail = n0 + kTcols > V;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                floatx4 tv[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    acc[mb][nb] += row_vals(buf + kBmTileBytes, 32 * w + 16 * mb, nb);
                    tv[nb] = row_vals(buf + kBmTileBytes + kRowBytes, 32 * w + 16 * mb, nb);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = 32 * w + 16 * mb + 4 * (lane >> 4) + i;
                    const SplitLse ld = sh_lse[lr][0], ltg = sh_lse[lr][1];
                    double sw = 0.0, sp = 0.0;
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) {
                        float ptv;
                        float wr = resid_weight(acc[mb][nb][i], tv[nb][i], ld, ltg, &ptv);
                        if (tail && n0 + 16 * nb + nl >= V) wr = ptv = 0.0f;
                        sw += (double)wr;
                        sp += (double)ptv;
                    }
                    sw = sum16(sw);
                    sp = sum16(sp);
                    const int row = m0 + lr;
                    if (nl == 0 && row < cnt) {
                        rw[(size_t)row * nT + tile] = sw;
                        rp[(size_t)row * nT + tile] = sp;
                    }
                }
            }
        },
        [&]() {});
}

// ---------------------------------------------------------------------------
// Final token of each request.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_final(
    const typename DT::T* __restrict__ Tg, const typename DT::T* __restrict__ L, const typename DT::T* __restrict__ A,
    const typename DT::T* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ len,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ resid_idx, const double* __restrict__ rw,
    const double* __restrict__ rp, const float* __restrict__ bm, const double* __restrict__ bsum, int gamma, int V,
    int r, int nT, int nC, uint64_t seed, int32_t* __restrict__ out_tok)
{
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
        const int m = resid_idx[b];
        const double* w = rw + (size_t)m * nT;
        const double* p = rp + (size_t)m * nT;
        // Total residual mass decides between the residual and its p_t fallback.
        double sloc = 0.0;
        {
            const int per = (nT + kThreads - 1) / kThreads;
            const int i0 = min(t * per, nT), i1 = min(i0 + per, nT);
            for (int i = i0; i < i1; ++i) sloc += w[i];
        }
        const bool degen = !(block_sum(sloc, bs) > 0.0);
        const double* src = degen ? p : w;
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)ks, 2u);
        const Located loc = locate(nT, [&](int i) { return src[i]; }, u, bs, &sh_cprev);

        const int n0 = loc.idx * TT::kCols;
        const T* trow = Tg + ((size_t)b * (gamma + 1) + (ks - 1)) * V;
        float f[TT::kNB];
        row_tile_f(L + ((size_t)b * gamma + (ks - 1)) * V, A, Bm, cond_token_v(x0, tok, b, gamma, ks, V), V, r, n0,
                   lds, f);
        if ((t >> 6) == 0) {
            const SplitLse ld = split_lse(lse_d[(size_t)b * gamma + ks - 1]);
            const SplitLse lt = split_lse(lse_t[(size_t)b * gamma + ks - 1]);
            double wv[TT::kNB];
#pragma unroll
            for (int nb = 0; nb < TT::kNB; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                wv[nb] = 0.0;
                if (col < V) {
                    float ptv;
                    const float wr = resid_weight(f[nb], DT::to_f32(trow[col]), ld, lt, &ptv);
                    wv[nb] = (double)(degen ? ptv : wr);
                }
            }
            double wsel;
            const int j = scan_tile_weights<TT::kNB>(wv, 1.0, loc.cprev, loc.tau, &wsel);
            if (lane == 0) sh_tok = clamp_tok(n0 + j, V);
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
        const float mcl = mc * kLog2e;
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

template <class DT>
static hipError_t verify_t(const void* Tg_, const void* L_, const void* A_, const void* Bm_, const int32_t* x0,
                           const int32_t* tok, const float* pd, const double* lse_d, const int32_t* len, int B,
                           int gamma, int V, int r, uint64_t seed, int32_t* accepted, int32_t* out_tok,
                           int32_t* n_out, float* target_p, void* ws, const WsLayout& lay, hipStream_t s)
{
    typedef typename DT::T T;
    const T* Tg = static_cast<const T*>(Tg_);
    const T* L = static_cast<const T*>(L_);
    const T* A = static_cast<const T*>(A_);
    const T* Bm = static_cast<const T*>(Bm_);
    char* w = static_cast<char*>(ws);
    float* tgm = reinterpret_cast<float*>(w + lay.tgt_m);
    double* tgs = reinterpret_cast<double*>(w + lay.tgt_s);
    double* lse_t = reinterpret_cast<double*>(w + lay.lse_t);
    double* ptw = reinterpret_cast<double*>(w + lay.pt);
    int32_t* ridx = reinterpret_cast<int32_t*>(w + lay.resid_idx);
    int32_t* rlist = reinterpret_cast<int32_t*>(w + lay.resid_list);
    int32_t* rcnt = reinterpret_cast<int32_t*>(w + lay.resid_count);
    double* rw = reinterpret_cast<double*>(w + lay.res_w);
    double* rp = reinterpret_cast<double*>(w + lay.res_p);
    float* bm = reinterpret_cast<float*>(w + lay.bon_m);
    double* bsum = reinterpret_cast<double*>(w + lay.bon_s);
    const int nT = n_tiles(std::is_same<DT, Bf16>::value ? 1 : 0, V), nC = n_chunks(V);

    prof_begin(K_TARGET_PARTIALS, s);
    hipLaunchKernelGGL(k_row_partials<DT>, dim3(nC, B * gamma), dim3(kThreads), 0, s, Tg, len, accepted, B, gamma, V,
                       nC, 0, tgm, tgs);
    hipLaunchKernelGGL(k_target_lse<DT>, dim3((B * gamma + 3) / 4), dim3(kThreads), 0, s, Tg, tok, len, tgm, tgs, B,
                       gamma, V, nC, lse_t, ptw);
    prof_end(K_TARGET_PARTIALS, s);
    prof_begin(K_ACCEPT, s);
    hipLaunchKernelGGL(k_accept, dim3(1), dim3(kAcceptThreads), 0, s, pd, len, ptw, B, gamma, seed, accepted, n_out,
                       target_p, ridx, rlist, rcnt);
    prof_end(K_ACCEPT, s);
    prof_begin(K_RESID_TILES, s);
    if (std::is_same<DT, Bf16>::value) {
        constexpr int NW = 4;
        const int nM = (B + 32 * NW - 1) / (32 * NW);
        const int S = std::min(nT, (cu_count() + nM - 1) / nM);
        auto kern = (r + 31) / 32 == 8 ? k_resid_tiles_bf16<NW, 8> : k_resid_tiles_bf16<NW, 0>;
        hipLaunchKernelGGL(kern, dim3(S * nM), dim3(64 * NW), 0, s,
                           reinterpret_cast<const uint16_t*>(Tg), reinterpret_cast<const uint16_t*>(L),
                           reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(Bm), x0, tok,
                           lse_d, lse_t, accepted, rlist, rcnt, gamma, V, r, nT, nM, S, rw, rp);
    } else {
        const int nM = (B + 255) / 256;
        hipLaunchKernelGGL(k_resid_tiles_f32, dim3(nT * nM), dim3(kThreads), 0, s,
                           reinterpret_cast<const float*>(Tg), reinterpret_cast<const float*>(L),
                           reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(Bm), x0, tok, lse_d,
                           lse_t, accepted, rlist, rcnt, gamma, V, r, nT, nM, rw, rp);
    }
    prof_end(K_RESID_TILES, s);
    prof_begin(K_BONUS_PARTIALS, s);
    hipLaunchKernelGGL(k_row_partials<DT>, dim3(nC, B), dim3(kThreads), 0, s, Tg, len, accepted, B, gamma, V, nC, 1,
                       bm, bsum);
    prof_end(K_BONUS_PARTIALS, s);
    prof_begin(K_FINAL, s);
    hipLaunchKernelGGL(k_final<DT>, dim3(B), dim3(kThreads), 0, s, Tg, L, A, Bm, x0, tok, lse_d, lse_t, len, accepted,
                       ridx, rw, rp, bm, bsum, gamma, V, r, nT, nC, seed, out_tok);
    prof_end(K_FINAL, s);
    return hipGetLastError();
}

hipError_t launch_verify(int dtype, const void* Tg, const void* L, const void* A, const void* Bm, const int32_t* x0,
                         const int32_t* tok, const float* pd, const double* lse_d, const int32_t* len, int B,
                         int gamma, int V, int r, uint64_t seed, int32_t* accepted, int32_t* out_tok,
                         int32_t* n_out, float* target_p, void* ws, const WsLayout& lay, hipStream_t s)
{
    if (dtype == 1)
        return verify_t<Bf16>(Tg, L, A, Bm, x0, tok, pd, lse_d, len, B, gamma, V, r, seed, accepted, out_tok, n_out,
                              target_p, ws, lay, s);
    return verify_t<F32>(Tg, L, A, Bm, x0, tok, pd, lse_d, len, B, gamma, V, r, seed, accepted, out_tok, n_out,
                         target_p, ws, lay, s);
}

}  // namespace dspark
