// dspark_markov.hpp -- the Markov-head bias contraction on MFMA, fp32 path
// (v_mfma_f32_16x16x4_f32; the bf16 path lives in dspark_tile.hpp).
//
// For a set of rows m (each row names a request whose conditioning token is
// x_m and a backbone logit row L_m), one 128-column vocabulary tile
// [n0, n0 + 128) of
//     f[m][n] = L_m[n] + sum_i A[x_m][i] * Bm[i][n]
// is computed by one wavefront per 16 * MB rows with 16x16 MFMA blocks, fp32
// accumulation initialised with the backbone logit.  The bias term is the
// low-rank Markov transition of the sequential head (paperlayer.ai summary of
// arXiv 2607.05147, section 3.1; menfem.com note, Methodology: rank-256
// factorisation; llm-wiki.hwlabs.dev explainer, Markov-head diagram).
//
// Data flow: A rows are gathered straight from global memory into MFMA
// A-operand registers (each lane reads 8 consecutive k of its row).  Bm is
// [r][V] row-major, so its k index is the strided one; it is staged through
// LDS in 32-row chunks, transposed on the way in (4 rows x 4 columns per
// thread, re-packed in registers) so that the B operand is two 16-byte LDS
// reads per lane.  Two LDS buffers alternate so the global loads of chunk c+1
// overlap the MFMAs of chunk c.
//
// Output layout (both dtypes): acc[mb][nb][i] holds row
//   16*mb + 4*(lane>>4) + i  and column  n0 + 16*nb + (lane&15).
// Each output element depends only on its own A row, its own Bm column, its
// initial value and the fixed k-step order, so recomputing one row later with
// the same routine reproduces it bit for bit.
#pragma once

#include "dspark_device.hpp"

namespace dspark {

constexpr int kTileN = 128;  // vocabulary columns per wave tile

// Bm rows per LDS chunk (kChunk), LDS pitch per column in elements, bytes per buffer.
template <class DT> struct MarkovLds;

template <> struct MarkovLds<F32> {
    static constexpr int kChunk = 32;
    static constexpr int kPitch = kChunk + 4;
    static constexpr int kBufBytes = kTileN * kPitch * 4;            // 18432
};

template <class DT> constexpr int markov_lds_bytes() { return 2 * MarkovLds<DT>::kBufBytes; }

// ---------------------------------------------------------------------------
// Staging of one Bm chunk (rows [k0, k0+kChunk) x columns [n0, n0+128)) into LDS
// laid out as column-major [n][k] with pitch kPitch.  Rows >= r and columns
// >= V are zero-filled.  Split into a global-load half and an LDS-store half
// so the caller can keep the loads in flight.
// ---------------------------------------------------------------------------
template <class DT> struct BmStage;

template <> struct BmStage<F32> {
    // one item per thread: 4 consecutive k rows x 4 consecutive columns
    uint4 v[4];
    __device__ __forceinline__ void load(const float* __restrict__ Bm, int V, int r, int n0, int k0)
    {
        const int kq = threadIdx.x >> 5, cg = threadIdx.x & 31;
        const int col = n0 + 4 * cg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 4 * kq + i;
            if (k < r && col < V) v[i] = ld16(Bm + (size_t)k * V + col);
            else v[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void store(char* buf) const
    {
        float* s = reinterpret_cast<float*>(buf);
        const int kq = threadIdx.x >> 5, cg = threadIdx.x & 31;
        uint4 c0 = make_uint4(v[0].x, v[1].x, v[2].x, v[3].x);
        uint4 c1 = make_uint4(v[0].y, v[1].y, v[2].y, v[3].y);
        uint4 c2 = make_uint4(v[0].z, v[1].z, v[2].z, v[3].z);
        uint4 c3 = make_uint4(v[0].w, v[1].w, v[2].w, v[3].w);
        const int n = 4 * cg;
        constexpr int P = MarkovLds<F32>::kPitch;
        *reinterpret_cast<uint4*>(s + (n + 0) * P + 4 * kq) = c0;
        *reinterpret_cast<uint4*>(s + (n + 1) * P + 4 * kq) = c1;
        *reinterpret_cast<uint4*>(s + (n + 2) * P + 4 * kq) = c2;
        *reinterpret_cast<uint4*>(s + (n + 3) * P + 4 * kq) = c3;
    }
};

// ---------------------------------------------------------------------------
// MFMA fragments for one 32-wide k step.  Lane l holds, for its row / column
// (l & 15), the 8 consecutive k values 8*(l>>4) .. 8*(l>>4)+7 of the step; A
// and B use the same k assignment, so the contraction is over all 32 k.
// ---------------------------------------------------------------------------
template <class DT> struct Frag;

template <> struct Frag<F32> {
    uint4 v0, v1;
    __device__ __forceinline__ void load_a(const float* __restrict__ arow, int k, int r)
    {
        if (k < r) {
            v0 = ld16(arow + k);
            v1 = ld16(arow + k + 4);
        } else {
            v0 = v1 = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void load_b(const char* buf, int n, int kk)
    {
        const float* s = reinterpret_cast<const float*>(buf) + n * MarkovLds<F32>::kPitch + kk;
        v0 = *reinterpret_cast<const uint4*>(s);
        v1 = *reinterpret_cast<const uint4*>(s + 4);
    }
    __device__ __forceinline__ static floatx4 mma(const Frag& a, const Frag& b, floatx4 c)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v0.x), __uint_as_float(b.v0.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v0.y), __uint_as_float(b.v0.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v0.z), __uint_as_float(b.v0.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v0.w), __uint_as_float(b.v0.w), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v1.x), __uint_as_float(b.v1.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v1.y), __uint_as_float(b.v1.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v1.z), __uint_as_float(b.v1.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v1.w), __uint_as_float(b.v1.w), c, 0, 0, 0);
        return c;
    }
};

// ---------------------------------------------------------------------------
// markov_tile: all 256 threads of the workgroup must call it (it contains
// workgroup barriers).  Waves with compute == false only help with staging.
//   arow[mb]  : pointer to A[x] for the lane's row (16*mb + (lane&15)) of
//               this wave, valid for every lane (callers clamp tokens).
//   acc       : on entry the initial values (backbone logits), on exit f.
// ---------------------------------------------------------------------------
template <class DT, int MB>
__device__ __forceinline__ void markov_tile(const typename DT::T* __restrict__ Bm, int V, int r, int n0,
                                            const typename DT::T* const (&arow)[MB], bool compute, char* lds,
                                            floatx4 (&acc)[MB][8])
{
    const int lane = threadIdx.x & 63;
    const int kq8 = 8 * (lane >> 4);
    const int nlane = lane & 15;
    constexpr int KC = MarkovLds<DT>::kChunk;
    const int nchunks = (r + KC - 1) / KC;
    char* buf[2] = { lds, lds + MarkovLds<DT>::kBufBytes };

    BmStage<DT> st;
    st.load(Bm, V, r, n0, 0);
    for (int c = 0; c < nchunks; ++c) {
        st.store(buf[c & 1]);
        __syncthreads();
        if (c + 1 < nchunks) st.load(Bm, V, r, n0, (c + 1) * KC);
        if (compute) {
#pragma unroll
            for (int s = 0; s < KC / 32; ++s) {
                const int kg = c * KC + s * 32 + kq8;  // global k of this lane's 8 values
                if (c * KC + s * 32 >= r) break;
                Frag<DT> a[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) a[mb].load_a(arow[mb], kg, r);
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    Frag<DT> b;
                    b.load_b(buf[c & 1], 16 * nb + nlane, s * 32 + kq8);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = Frag<DT>::mma(a[mb], b, acc[mb][nb]);
                }
            }
        }
    }
    __syncthreads();  // LDS may be reused by the caller after this point
}

}  // namespace dspark
