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
//   k_accept                 one workgroup: per request combine chunk
//                            partials -> lse_t, p_t(x_k), ratio, accept
//                            draws; compacts the requests with a rejection.
//   k_resid_tiles            Markov MFMA tiles of the rejected draft rows
//                            fused with the target row: per tile sums of
//                            max(0, p_t - p_d) and of p_t.
//   k_row_partials (bonus)   grid = chunks x B: target row ell_b + 1 of
//                            requests without a rejection.
//   k_final                  one workgroup per request: locate and sample
//                            the last token, write the emitted tokens.
#include <limits.h>

#include "dspark_internal.hpp"
#include "dspark_markov.hpp"

namespace dspark {

__device__ __forceinline__ int clamp_len(int l, int gamma) { return min(max(l, 0), gamma); }
__device__ __forceinline__ int clamp_tok(int x, int V) { return min(max(x, 0), V - 1); }

__device__ __forceinline__ int cond_token_v(const int32_t* __restrict__ x0, const int32_t* __restrict__ tok, int b,
                                            int gamma, int k, int V)
{
    return clamp_tok((k == 1) ? x0[b] : tok[b * gamma + (k - 2)], V);
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
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = e0 + (i * kThreads + (int)threadIdx.x) * PV;
        if (e < V) {
#pragma unroll
            for (int j = 0; j < PV; ++j) {
                const float xv = DT::get(v[i], j);
                if (xv != -INFINITY) s += (double)exp_fast(xv - M);
            }
        }
    }
    s = block_sum(s, bs);
    if (threadIdx.x == 0) {
        om[(size_t)row * nC + c] = M;
        os[(size_t)row * nC + c] = s;
    }
}

__device__ __forceinline__ double part_mass(float m, double s, float M)
{
    return m == -INFINITY ? 0.0 : s * exp((double)m - (double)M);
}

// ---------------------------------------------------------------------------
// Accept scan: one workgroup of 1024 threads, one request per thread.
// ---------------------------------------------------------------------------
constexpr int kAcceptThreads = 1024;

template <class DT>
__global__ __launch_bounds__(kAcceptThreads) void k_accept(
    const typename DT::T* __restrict__ Tg, const int32_t* __restrict__ tok, const float* __restrict__ pd,
    const int32_t* __restrict__ len, const float* __restrict__ tgm, const double* __restrict__ tgs, int B, int gamma,
    int V, int nC, uint64_t seed, double* __restrict__ lse_t, int32_t* __restrict__ accepted,
    int32_t* __restrict__ n_out, float* __restrict__ target_p, int32_t* __restrict__ resid_idx,
    int32_t* __restrict__ resid_list, int32_t* __restrict__ resid_count)
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
                if (kk < l) {
                    const size_t row = (size_t)b * gamma + kk;
                    const float* m = tgm + row * nC;
                    const double* s = tgs + row * nC;
                    float M = -INFINITY;
                    for (int c = 0; c < nC; ++c) M = fmaxf(M, m[c]);
                    double S = 0.0;
                    for (int c = 0; c < nC; ++c) S += part_mass(m[c], s[c], M);
                    const double lse = (double)M + log(S);
                    lse_t[row] = lse;
                    const int x = clamp_tok(tok[row], V);
                    const double tx = (double)DT::to_f32(Tg[((size_t)b * (gamma + 1) + kk) * V + x]);
                    const double pt = exp(tx - lse);
                    const double ratio = pt / (double)pd[row];
                    const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(kk + 1), 1u);
                    if (a == l && !(u < (float)ratio)) a = kk;
                    if (target_p) target_p[row] = (float)pt;
                } else if (target_p) {
                    target_p[(size_t)b * gamma + kk] = 0.0f;
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

// ---------------------------------------------------------------------------
// Residual tiles: rows are the compacted requests with a rejection; row m is
// request b = resid_list[m] at its first rejected position ks = a_b + 1.
// ---------------------------------------------------------------------------
template <class DT>
__global__ __launch_bounds__(kThreads) void k_resid_tiles(
    const typename DT::T* __restrict__ Tg, const typename DT::T* __restrict__ L, const typename DT::T* __restrict__ A,
    const typename DT::T* __restrict__ Bm, const int32_t* __restrict__ x0, const int32_t* __restrict__ tok,
    const double* __restrict__ lse_d, const double* __restrict__ lse_t, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ resid_list, const int32_t* __restrict__ resid_count, int gamma, int V, int r, int nT,
    int nM, double* __restrict__ rw, double* __restrict__ rp)
{
    typedef typename DT::T T;
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<DT>()];
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int tile = lid / nM, mblk = lid % nM;
    const int cnt = *resid_count;
    if (mblk * 256 >= cnt) return;  // whole workgroup idle (uniform)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = tile * kTileN;
    const int mw0 = mblk * 256 + wave * 64;
    const bool compute = mw0 < cnt;

    const T* arow[4];
    floatx4 acc[4][8];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int ra = min(mw0 + 16 * mb + (lane & 15), cnt - 1);
        const int ba = resid_list[ra];
        arow[mb] = A + (size_t)cond_token_v(x0, tok, ba, gamma, accepted[ba] + 1, V) * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mw0 + 16 * mb + 4 * (lane >> 4) + i;
            const int bb = resid_list[min(row, cnt - 1)];
            const int ks = accepted[bb] + 1;
            const T* lrow = L + ((size_t)bb * gamma + (ks - 1)) * V;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                acc[mb][nb][i] = (compute && row < cnt && col < V) ? DT::to_f32(lrow[col]) : 0.0f;
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
            const int bb = resid_list[min(row, cnt - 1)];
            const int ks = accepted[bb] + 1;
            const T* trow = Tg + ((size_t)bb * (gamma + 1) + (ks - 1)) * V;
            const double ld = lse_d[(size_t)bb * gamma + ks - 1];
            const double lt = lse_t[(size_t)bb * gamma + ks - 1];
            double sw = 0.0, sp = 0.0;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + (lane & 15);
                if (col < V) {
                    const double pdj = exp_to_double((double)acc[mb][nb][i] - ld);
                    const double ptj = exp_to_double((double)DT::to_f32(trow[col]) - lt);
                    const double dj = ptj - pdj;
                    sw += dj > 0.0 ? dj : 0.0;
                    sp += ptj;
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
// Locate within a list of n non-negative masses (given by mass(i)) the first
// index whose running sum exceeds tau (fallback: last index with positive
// mass).  Returns the index and the running sum before it.  All threads.
// ---------------------------------------------------------------------------
template <class MassFn>
__device__ __forceinline__ int block_locate(int n, MassFn mass, double tau, double off, BlockScratch& bs,
                                            double* sh_cprev, double* cprev_out)
{
    const int t = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int i0 = min(t * per, n), i1 = min(i0 + per, n);
    int hit = INT_MAX, lastpos = -1;
    double c = off, cph = 0.0, cpl = 0.0;
    for (int i = i0; i < i1; ++i) {
        const double mi = mass(i);
        const double cb = c;
        c += mi;
        if (hit == INT_MAX && c > tau) {
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
    const int idx = use_hit ? th : max(tl, 0);
    if (use_hit ? (hit == idx) : (lastpos == idx && tl >= 0)) *sh_cprev = use_hit ? cph : cpl;
    __syncthreads();
    *cprev_out = *sh_cprev;
    return idx;
}

template <class MassFn>
__device__ __forceinline__ double block_prefix_setup(int n, MassFn mass, BlockScratch& bs, double* total)
{
    const int t = threadIdx.x;
    const int per = (n + kThreads - 1) / kThreads;
    const int i0 = min(t * per, n), i1 = min(i0 + per, n);
    double sloc = 0.0;
    for (int i = i0; i < i1; ++i) sloc += mass(i);
    return block_excl_scan(sloc, bs, total);
}

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
    __shared__ __attribute__((aligned(16))) char lds[markov_lds_bytes<DT>()];
    __shared__ BlockScratch bs;
    __shared__ double sh_cprev;
    __shared__ int sh_tok;

    const int b = blockIdx.x;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int l = clamp_len(len[b], gamma);
    const int a = accepted[b];

    if (a < l) {
        // ---- residual at the first rejected position ks -------------------
        const int ks = a + 1;
        const int m = resid_idx[b];
        const double* w = rw + (size_t)m * nT;
        const double* p = rp + (size_t)m * nT;
        double Sw = 0.0;
        double off = block_prefix_setup(nT, [&](int i) { return w[i]; }, bs, &Sw);
        const bool degen = !(Sw > 0.0);
        const double* src = degen ? p : w;
        double S = Sw;
        if (degen) off = block_prefix_setup(nT, [&](int i) { return p[i]; }, bs, &S);
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)ks, 2u);
        const double tau = (double)u * S;
        double cprev;
        const int tstar = block_locate(nT, [&](int i) { return src[i]; }, tau, off, bs, &sh_cprev, &cprev);

        const int n0 = tstar * kTileN;
        const T* arow[1] = { A + (size_t)cond_token_v(x0, tok, b, gamma, ks, V) * r };
        const T* lrow = L + ((size_t)b * gamma + (ks - 1)) * V;
        const T* trow = Tg + ((size_t)b * (gamma + 1) + (ks - 1)) * V;
        floatx4 acc[1][8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int col = n0 + 16 * nb + (lane & 15);
            const float v = col < V ? DT::to_f32(lrow[col]) : 0.0f;
            acc[0][nb] = floatx4{ v, v, v, v };
        }
        markov_tile<DT, 1>(Bm, V, r, n0, arow, wave == 0, lds, acc);
        if (wave == 0) {
            const double ld = lse_d[(size_t)b * gamma + ks - 1];
            const double lt = lse_t[(size_t)b * gamma + ks - 1];
            const int l16 = lane & 15;
            double carry = 0.0;
            int jhit = -1, jlast = -1;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = n0 + 16 * nb + l16;
                double wj = 0.0;
                if (col < V) {
                    const double ptj = exp_to_double((double)DT::to_f32(trow[col]) - lt);
                    if (degen) {
                        wj = ptj;
                    } else {
                        const double pdj = exp_to_double((double)acc[0][nb][0] - ld);
                        const double dj = ptj - pdj;
                        wj = dj > 0.0 ? dj : 0.0;
                    }
                }
                double v = wj;
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const double n = __shfl_up(v, o, 16);
                    if (l16 >= o) v += n;
                }
                const double cum = carry + v;
                carry = __shfl(cum, 15, 16);
                const uint64_t mc = __ballot(cprev + cum > tau) & 0xFFFFull;
                const uint64_t mp = __ballot(wj > 0.0) & 0xFFFFull;
                if (jhit < 0 && mc) jhit = 16 * nb + __builtin_ctzll(mc);
                if (mp) jlast = 16 * nb + (63 - __builtin_clzll(mp));
            }
            if (lane == 0) sh_tok = clamp_tok(n0 + (jhit >= 0 ? jhit : max(jlast, 0)), V);
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
        double S = 0.0;
        const double off = block_prefix_setup(nC, [&](int c) { return part_mass(pm[c], ps[c], M); }, bs, &S);
        const float u = philox_uniform(seed, (uint32_t)b, (uint32_t)(l + 1), 3u);
        const double tau = (double)u * S;
        double cprev;
        const int cstar =
            block_locate(nC, [&](int c) { return part_mass(pm[c], ps[c], M); }, tau, off, bs, &sh_cprev, &cprev);

        // rescan the chunk in index order: 32 contiguous elements per thread
        const float mc = pm[cstar];
        const double scale = part_mass(mc, 1.0, M);
        const T* x = Tg + ((size_t)b * (gamma + 1) + l) * V;
        constexpr int EPT = kChunkElems / kThreads;  // 32
        const int e0 = cstar * kChunkElems + t * EPT;
        double wv[EPT];
        double tsum = 0.0;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int e = e0 + j;
            double wj = 0.0;
            if (e < V && mc != -INFINITY) {
                const float xv = DT::to_f32(x[e]);
                if (xv != -INFINITY) wj = (double)exp_fast(xv - mc);
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
            if (hit == INT_MAX && cprev + scale * run > tau) hit = e0 + j;
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
    int32_t* ridx = reinterpret_cast<int32_t*>(w + lay.resid_idx);
    int32_t* rlist = reinterpret_cast<int32_t*>(w + lay.resid_list);
    int32_t* rcnt = reinterpret_cast<int32_t*>(w + lay.resid_count);
    double* rw = reinterpret_cast<double*>(w + lay.res_w);
    double* rp = reinterpret_cast<double*>(w + lay.res_p);
    float* bm = reinterpret_cast<float*>(w + lay.bon_m);
    double* bsum = reinterpret_cast<double*>(w + lay.bon_s);
    const int nT = n_tiles(V), nC = n_chunks(V);
    const int nM = (B + 255) / 256;

    prof_begin(K_TARGET_PARTIALS, s);
    hipLaunchKernelGGL(k_row_partials<DT>, dim3(nC, B * gamma), dim3(kThreads), 0, s, Tg, len, accepted, B, gamma, V,
                       nC, 0, tgm, tgs);
    prof_end(K_TARGET_PARTIALS, s);
    prof_begin(K_ACCEPT, s);
    hipLaunchKernelGGL(k_accept<DT>, dim3(1), dim3(kAcceptThreads), 0, s, Tg, tok, pd, len, tgm, tgs, B, gamma, V, nC,
                       seed, lse_t, accepted, n_out, target_p, ridx, rlist, rcnt);
    prof_end(K_ACCEPT, s);
    prof_begin(K_RESID_TILES, s);
    hipLaunchKernelGGL(k_resid_tiles<DT>, dim3(nT * nM), dim3(kThreads), 0, s, Tg, L, A, Bm, x0, tok, lse_d, lse_t,
                       accepted, rlist, rcnt, gamma, V, r, nT, nM, rw, rp);
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
