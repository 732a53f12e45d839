// dspark_draft.hip -- one semi-autoregressive draft step on gfx950.
//
// The sequential stage samples the block left to right; position k is drawn
// from softmax(L[b,k,:] + A[x_{k-1}] Bm) where x_{k-1} is the token just
// sampled (x_0 the last committed token) -- paperlayer.ai summary of arXiv
// 2607.05147, section 3.1; llm-wiki.hwlabs.dev explainer, Markov-head
// diagram.  Each step is two launches:
//
//   k_draft_tiles   grid = (V/128 tiles) x (B/256 row blocks), 4 waves.
//                   Markov MFMA tile (dspark_markov.hpp) fused with the
//                   vocabulary pass: per (row, tile) it writes the tile max
//                   m_t (fp32) and s_t = sum exp(f - m_t) (fp64).  The biased
//                   logits f are never written to memory.
//   k_draft_locate  one workgroup per request.  Combines the tile partials in
//                   tile order (fp64), draws u = U(seed, b, k, 0), finds the
//                   tile where the running mass passes u*S, recomputes that
//                   one tile with the same MFMA routine (bit-identical f) and
//                   scans it in index order.  Inverse-CDF sampling at
//                   temperature 1: token = min{ j : C_j > u*S }.
#include <limits.h>

#include "dspark_internal.hpp"
#include "dspark_markov.hpp"

namespace dspark {

// Conditioning token of request b at draft step k (1-based), clamped into the
// vocabulary so that an out-of-range caller token can never address outside A.
__device__ __forceinline__ int cond_token(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                          int gamma, int k, int V)
{
    int x = (k == 1) ? x0[b] : tok[b * gamma + (k - 2)];
    return min(max(x, 0), V - 1);
}

template <class DT>
__global__ __launch_bounds__(kThreads) void k_draft_tiles(const typename DT::T* __restrict__ L,
                                                          const typename DT::T* __restrict__ A,
                                                          const typename DT::T* __restrict__ Bm,
                                                          const int32_t* __restrict__ x0, const int32_t* tok, int B,
                                                          int gamma, int V, int r, int k, int nT, int nM,
                                                          float* __restrict__ pm, double* __restrict__ ps)
{
    typedef typename DT::T T;
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<DT>()];

    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int tile = lid / nM, mblk = lid % nM;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = tile * kTileN;
    const int mw0 = mblk * 256 + wave * 64;
    const bool compute = mw0 < B;

    const T* arow[4];
    floatx4 acc[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int ra = min(mw0 + 16 * mb + (lane & 15), B - 1);
        arow[mb] = A + (size_t)cond_token(x0, tok, ra, gamma, k, V) * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const T* lrow = L + ((size_t)min(row, B - 1) * gamma + (k - 1)) * V;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                acc[mb][nb][i] = (compute && row < B && col < V) ? DT::to_f32(lrow[col]) : 0.0f;
            }
        }
    }

    markov_tile<DT, 4>(Bm, V, r, n0, arow, compute, lds, acc);
    if (!compute) return;

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            float f[8];
            float mx = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                f[nb] = col < V ? acc[mb][nb][i] : -INFINITY;
                mx = fmaxf(mx, f[nb]);
            }
            mx = max16(mx);
            double s = 0.0;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
                if (f[nb] != -INFINITY) s += (double)exp_fast(f[nb] - mx);
            s = sum16(s);
            if ((lane & 15) == 0 && row < B) {
                pm[(size_t)row * nT + tile] = mx;
                ps[(size_t)row * nT + tile] = s;
            }
        }
    }
}

// Tile mass relative to the row maximum M; tiles with no finite logit weigh 0.
__device__ __forceinline__ double tile_mass(float m, double s, float M)
{
    return m == -INFINITY ? 0.0 : s * exp((double)m - (double)M);
}

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
    typedef typename DT::T T;
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<DT>()];
    __shared__ BlockScratch bs;
    __shared__ double sh_cprev;

    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const float* pmr = pm + (size_t)b * nT;
    const double* psr = ps + (size_t)b * nT;

    // ---- combine tile partials: row max, then masses in tile order --------
    const int per = (nT + kThreads - 1) / kThreads;
    const int t0 = min(t * per, nT), t1 = min(t0 + per, nT);
    float mloc = -INFINITY;
    for (int i = t0; i < t1; ++i) mloc = fmaxf(mloc, pmr[i]);
    const float M = block_max(mloc, bs);
    double sloc = 0.0;
    for (int i = t0; i < t1; ++i) sloc += tile_mass(pmr[i], psr[i], M);
    double S = 0.0;
    const double off = block_excl_scan(sloc, bs, &S);

    const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)k, 0u);
    const double tau = (double)u * S;

    // first tile whose running mass exceeds tau (fallback: last tile with mass)
    int hit = INT_MAX, lastpos = -1;
    double c = off, cprev_hit = 0.0, cprev_last = 0.0;
    for (int i = t0; i < t1; ++i) {
        const double mi = tile_mass(pmr[i], psr[i], M);
        const double cb = c;
        c += mi;
        if (hit == INT_MAX && c > tau) {
            hit = i;
            cprev_hit = cb;
        }
        if (mi > 0.0) {
            lastpos = i;
            cprev_last = cb;
        }
    }
    if (t == 0) sh_cprev = 0.0;
    const int tstar_hit = block_min_int(hit, bs);
    const int tstar_last = block_max_int(lastpos, bs);
    const bool use_hit = tstar_hit != INT_MAX;
    const int tstar = use_hit ? tstar_hit : max(tstar_last, 0);
    if (use_hit ? (hit == tstar) : (lastpos == tstar)) sh_cprev = use_hit ? cprev_hit : cprev_last;
    __syncthreads();
    const double cprev = sh_cprev;

    // ---- recompute the chosen tile for this row (wave 0 computes) ---------
    const int wave = t >> 6, lane = t & 63;
    const int n0 = tstar * kTileN;
    const int prev = cond_token(x0, tok, b, gamma, k, V);
    const T* arow[1] = { A + (size_t)prev * r };
    const T* lrow = L + ((size_t)b * gamma + (k - 1)) * V;
    floatx4 acc[1][8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int col = n0 + 16 * nb + (lane & 15);
        const float v = col < V ? DT::to_f32(lrow[col]) : 0.0f;
        acc[0][nb] = floatx4{ v, v, v, v };
    }
    markov_tile<DT, 1>(Bm, V, r, n0, arow, wave == 0, lds, acc);

    if (wave != 0) return;
    const float mt = pmr[tstar];
    const double scale = tile_mass(mt, 1.0, M);
    const int l16 = lane & 15;
    double carry = 0.0;
    int jhit = -1, jlast = -1;
    double whit = 0.0, wlast = 0.0;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const int col = n0 + 16 * nb + l16;
        const float f = acc[0][nb][0];
        const double w = (col < V && f != -INFINITY && mt != -INFINITY) ? (double)exp_fast(f - mt) : 0.0;
        double v = w;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const double n = __shfl_up(v, o, 16);
            if (l16 >= o) v += n;
        }
        const double cum = carry + v;
        carry = __shfl(cum, 15, 16);
        const bool cond = cprev + scale * cum > tau;
        const uint64_t mc = __ballot(cond) & 0xFFFFull;
        const uint64_t mp = __ballot(w > 0.0) & 0xFFFFull;
        if (jhit < 0 && mc) {
            const int lsel = __builtin_ctzll(mc);
            jhit = 16 * nb + lsel;
            whit = __shfl(w, lsel, 64);
        }
        if (mp) {
            const int lsel = 63 - __builtin_clzll(mp);
            jlast = 16 * nb + lsel;
            wlast = __shfl(w, lsel, 64);
        }
    }
    if (lane == 0) {
        const int j = jhit >= 0 ? jhit : max(jlast, 0);
        const double wj = jhit >= 0 ? whit : wlast;
        const int x = min(n0 + j, V - 1);
        tok[b * gamma + (k - 1)] = x;
        p_out[b * gamma + (k - 1)] = (float)(scale * wj / S);
        lse_out[b * gamma + (k - 1)] = (double)M + log(S);
    }
}

template <class DT>
static hipError_t draft_step_t(const void* L, const void* A, const void* Bm, const int32_t* x0, int B, int gamma,
                               int V, int r, int k, uint64_t seed, int32_t* tok, float* p, double* lse, void* ws,
                               const WsLayout& lay, hipStream_t s)
{
    typedef typename DT::T T;
    char* w = static_cast<char*>(ws);
    float* pm = reinterpret_cast<float*>(w + lay.draft_m);
    double* ps = reinterpret_cast<double*>(w + lay.draft_s);
    const int nT = n_tiles(V);
    const int nM = (B + 255) / 256;
    prof_begin(K_DRAFT_TILES, s);
    hipLaunchKernelGGL(k_draft_tiles<DT>, dim3(nT * nM), dim3(kThreads), 0, s, static_cast<const T*>(L),
                       static_cast<const T*>(A), static_cast<const T*>(Bm), x0, tok, B, gamma, V, r, k, nT, nM, pm,
                       ps);
    prof_end(K_DRAFT_TILES, s);
    prof_begin(K_DRAFT_LOCATE, s);
    hipLaunchKernelGGL(k_draft_locate<DT>, dim3(B), dim3(kThreads), 0, s, static_cast<const T*>(L),
                       static_cast<const T*>(A), static_cast<const T*>(Bm), x0, tok, p, lse, pm, ps, B, gamma, V, r,
                       k, nT, seed);
    prof_end(K_DRAFT_LOCATE, s);
    return hipGetLastError();
}

hipError_t launch_draft_step(int dtype, const void* L, const void* A, const void* Bm, const int32_t* x0, int B,
                             int gamma, int V, int r, int k, uint64_t seed, int32_t* tok, float* p, double* lse,
                             void* ws, const WsLayout& lay, hipStream_t s)
{
    if (dtype == 1) return draft_step_t<Bf16>(L, A, Bm, x0, B, gamma, V, r, k, seed, tok, p, lse, ws, lay, s);
    return draft_step_t<F32>(L, A, Bm, x0, B, gamma, V, r, k, seed, tok, p, lse, ws, lay, s);
}

}  // namespace dspark
