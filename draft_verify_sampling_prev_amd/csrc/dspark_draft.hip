// dspark_draft.hip -- one semi-autoregressive draft step on gfx950.
//
// The sequential stage samples the block left to right; position k is drawn
// from softmax(L[b,k,:] + A[x_{k-1}] Bm) where x_{k-1} is the token just
// sampled (x_0 the last committed token) -- paperlayer.ai summary of arXiv
// 2607.05147, section 3.1; llm-wiki.hwlabs.dev explainer, Markov-head
// diagram.  Each step is two launches:
//
//   k_draft_tiles   Markov MFMA tile fused with the vocabulary pass: per
//                   (row, 128-column tile) it writes the tile max m_t (fp32)
//                   and s_t = sum exp(f - m_t) (fp64).  The biased logits f
//                   are never written to memory.  bf16: persistent kernel of
//                   8-wave workgroups over 256-row x 128-column tiles
//                   (dspark_tile.hpp), about one workgroup per CU; fp32:
//                   one 4-wave workgroup per tile (dspark_markov.hpp).
//   k_draft_locate  one workgroup per request.  Combines the tile partials in
//                   tile order (fp64), draws u = U(seed, b, k, 0), finds the
//                   tile where the running mass passes u*S, recomputes that
//                   one tile with the same MFMA sequence (bit-identical f) and
//                   scans it in index order.  Inverse-CDF sampling at
//                   temperature 1: token = min{ j : C_j > u*S }.
#include <limits.h>

#include <algorithm>

#include "dspark_internal.hpp"
#include "dspark_locate.hpp"
#include "dspark_markov.hpp"
#include "dspark_tile.hpp"

namespace dspark {

// Conditioning token of request b at draft step k (1-based), clamped into the
// vocabulary so that an out-of-range caller token can never address outside A.
__device__ __forceinline__ int cond_token(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                          int gamma, int k, int V)
{
    int x = (k == 1) ? x0[b] : tok[b * gamma + (k - 2)];
    return min(max(x, 0), V - 1);
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
            const float ml = mx * kLog2e;
            float sv = 0.0f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sv += softmax_w(fv[nb], ml);
            sv = sum16f(sv);
            if (mx == -INFINITY) sv = 0.0f;
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
                                                              int B, int gamma, int V, int r, int k, int nT, int nM,
                                                              float* __restrict__ pm, double* __restrict__ ps)
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
        arow[mb] = A + (size_t)cond_token(x0, tok, ra, gamma, k, V) * r;
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
        if ((lane & 15) < 4 && row < B) {
            pm[(size_t)row * nT + tile] = m[mb];
            ps[(size_t)row * nT + tile] = (double)sv[mb];
        }
    }
}

// ---------------------------------------------------------------------------
// bf16: persistent.  Workgroup `lid` owns row block mblk = lid % nM (32*NW
// rows) and the 64-column tiles slot, slot + S, ... (slot = lid / nM).  LDS
// holds two (Bm tile, L tile) buffers; the DMA of tile i+1 is issued before
// the MFMAs of tile i.
// ---------------------------------------------------------------------------
template <int NW, int KS>
__global__ __launch_bounds__(64 * NW) void k_draft_tiles_bf16(
    const uint16_t* __restrict__ L, const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
    const int32_t* __restrict__ x0, const int32_t* tok, int B, int gamma, int V, int r, int k, int nT, int nM, int S,
    float* __restrict__ pm, double* __restrict__ ps)
{
    constexpr int R = 32 * NW;
    constexpr int kBuf = kBmTileBytes + R * kTrowBytes;
    __shared__ __attribute__((aligned(1024))) char buf0[kBuf];
    __shared__ __attribute__((aligned(1024))) char buf1[kBuf];

    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int mblk = lid % nM, slot = lid / nM;
    if (slot >= nT) return;
    const int w = wave_id(), lane = threadIdx.x & 63;
    const int m0 = mblk * R;
    const int mw = m0 + 32 * w;  // first row of this wave
    const bool active = mw < B;

    uint4 a[2][8];
    {
        const uint16_t* arow[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int ra = min(mw + 16 * mb + (lane & 15), B - 1);
            arow[mb] = A + (size_t)cond_token(x0, tok, ra, gamma, k, V) * r;
        }
        load_a_frags<2>(arow, r, a);
    }
    int ridx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ridx[t] = min(m0 + dma_row_of<NW>(t), B - 1) * gamma + (k - 1);
    const int nks = KS > 0 ? KS : (r + 31) / 32;

    // Software pipeline: the row partials of tile i (VALU) are computed while
    // the MFMAs of tile i+1 run (fprev holds tile i's logits f = acc + L),
    // and stored after the next loop-top barrier.
    floatx4 fprev[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) fprev[mb][nb] = floatx4{ 0.f, 0.f, 0.f, 0.f };
    int prev = -1, done = -1;  // tile held in fprev; tile whose partials wait in pm_r / ps_r
    float pm_r[2] = { 0.f, 0.f }, ps_r[2] = { 0.f, 0.f };
    auto store = [&]() {
        if (done < 0) return;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int row = mw + 16 * mb + 4 * (lane >> 4) + (lane & 15);
            if ((lane & 15) < 4 && row < B) {
                pm[(size_t)row * nT + done] = pm_r[mb];
                ps[(size_t)row * nT + done] = (double)ps_r[mb];
            }
        }
        done = -1;
    };
    auto finish = [&]() {  // partials of tile `prev` from fprev into pm_r / ps_r
        tile_row_partials<2, 4>(fprev, (prev + 1) * kTcols > V, V - prev * kTcols, pm_r, ps_r);
        done = prev;
    };
    persistent_tiles(
        slot, nT, S, buf0, buf1,
        [&](int tile, char* buf) {
            dma_bm_tile<NW>(Bm, V, r, tile * kTcols, 32 * nks, buf);
            dma_row_tile<NW>(L, ridx, V, tile * kTcols, buf + kBmTileBytes);
        },
        [&](int tile, const char* buf) {
            if (!active) return;
            floatx4 acc[2][4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4{ 0.f, 0.f, 0.f, 0.f };
            tile_mma64<2, KS>(a, buf, nks, acc);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) acc[mb][nb] += row_vals(buf + kBmTileBytes, 32 * w + 16 * mb, nb);
            finish();  // math of the previous tile; interleaves with the MFMAs above
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) fprev[mb][nb] = acc[mb][nb];
            prev = tile;
        },
        [&]() { store(); });
    if (active) {
        store();
        finish();
        store();
    }
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
                                                           const float* __restrict__ pm, const double* __restrict__ ps,
                                                           int B, int gamma, int V, int r, int k, int nT,
                                                           uint64_t seed)
{
    typedef TileTraits<DT> TT;
    __shared__ __attribute__((aligned(1024))) char lds[TT::kLdsBytes];
    __shared__ BlockScratch bs;
    __shared__ double sh_cprev;

    const int b = blockIdx.x;
    const float* pmr = pm + (size_t)b * nT;
    const double* psr = ps + (size_t)b * nT;
    const int per = (nT + kThreads - 1) / kThreads;
    const int t0 = min((int)threadIdx.x * per, nT), t1 = min(t0 + per, nT);
    float mloc = -INFINITY;
    for (int i = t0; i < t1; ++i) mloc = fmaxf(mloc, pmr[i]);
    const float M = block_max(mloc, bs);
    const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
    const Located loc = locate(nT, [&](int i) { return tile_mass(pmr[i], psr[i], M); }, u, bs, &sh_cprev);

    const int n0 = loc.idx * TT::kCols;
    const int prev = cond_token(x0, tok, b, gamma, k, V);
    float f[TT::kNB];
    row_tile_f(L + ((size_t)b * gamma + (k - 1)) * V, A, Bm, prev, V, r, n0, lds, f);
    if ((threadIdx.x >> 6) != 0) return;
    const float mt = pmr[loc.idx];
    const double scale = tile_mass(mt, 1.0, M);
    const int l16 = threadIdx.x & 15;
    const float ml = mt * kLog2e;
    double w[TT::kNB];
#pragma unroll
    for (int nb = 0; nb < TT::kNB; ++nb) {
        const bool ok = n0 + 16 * nb + l16 < V && mt != -INFINITY;
        w[nb] = ok ? (double)softmax_w(f[nb], ml) : 0.0;
    }
    double wsel;
    const int j = scan_tile_weights<TT::kNB>(w, scale, loc.cprev, loc.tau, &wsel);
    if (threadIdx.x == 0) {
        tok[b * gamma + (k - 1)] = min(n0 + j, V - 1);
        p_out[b * gamma + (k - 1)] = (float)(scale * wsel / loc.S);
        lse_out[b * gamma + (k - 1)] = (double)M + log(loc.S);
    }
}

hipError_t launch_draft_step(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, int k, uint64_t seed, int32_t* tok, float* p, double* lse,
                             void* ws, const WsLayout& lay, hipStream_t s)
{
    char* w = static_cast<char*>(ws);
    float* pm = reinterpret_cast<float*>(w + lay.draft_m);
    double* ps = reinterpret_cast<double*>(w + lay.draft_s);
    const int nT = n_tiles(dtype, V);
    prof_begin(K_DRAFT_TILES, s);
    if (dtype == 1) {
        constexpr int NW = 8;
        const int nM = (B + 32 * NW - 1) / (32 * NW);
        const int S = std::min(nT, (cu_count() + nM - 1) / nM);
        auto kern = (r + 31) / 32 == 8 ? k_draft_tiles_bf16<NW, 8> : k_draft_tiles_bf16<NW, 0>;
        hipLaunchKernelGGL(kern, dim3(S * nM), dim3(64 * NW), 0, s, static_cast<const uint16_t*>(L),
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm), x0, tok, B, gamma, V,
                           r, k, nT, nM, S, pm, ps);
    } else {
        const int nM = (B + 255) / 256;
        hipLaunchKernelGGL(k_draft_tiles_f32, dim3(nT * nM), dim3(kThreads), 0, s, static_cast<const float*>(L),
                           static_cast<const float*>(A), static_cast<const float*>(Bm), x0, tok, B, gamma, V, r, k,
                           nT, nM, pm, ps);
    }
    prof_end(K_DRAFT_TILES, s);
    prof_begin(K_DRAFT_LOCATE, s);
    if (dtype == 1)
        hipLaunchKernelGGL(k_draft_locate<Bf16>, dim3(B), dim3(kThreads), 0, s, static_cast<const uint16_t*>(L),
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm), x0, tok, p, lse, pm, ps,
                           B, gamma, V, r, k, nT, seed);
    else
        hipLaunchKernelGGL(k_draft_locate<F32>, dim3(B), dim3(kThreads), 0, s, static_cast<const float*>(L),
                           static_cast<const float*>(A), static_cast<const float*>(Bm), x0, tok, p, lse, pm, ps, B,
                           gamma, V, r, k, nT, seed);
    prof_end(K_DRAFT_LOCATE, s);
    return hipGetLastError();
}

}  // namespace dspark
