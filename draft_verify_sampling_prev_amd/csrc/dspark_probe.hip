// dspark_probe.hip -- a load-only kernel that bounds the draft tile kernel
// from above (measurement tooling, built as its own library; not part of the
// dspark C ABI).
//
// k_probe_tile_reads reads exactly the bytes one launch of the bf16 draft
// tile kernel reads from HBM, split over the same workgroups: slot s of S
// takes the same contiguous range of 64-column tiles, and for each tile the
// 128-byte pieces of the B rows of L at draft step k and of the r rows of Bm,
// as 16-byte loads, two batches of eight per thread in flight.  It does no
// arithmetic beyond folding the loaded words into one word per thread (so the
// loads are kept).  Its duration is the time any kernel with the tile
// kernel's traffic and access order needs on the part; the tile kernel's own
// duration over it is the fraction of that ceiling the kernel reaches.
// (The tile kernel also reads its rows' A vectors, 128 KB per workgroup from
// L2; they are not read here.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace {

constexpr int kThreadsP = 512;
constexpr int kBatch = 8;  // 16-byte loads per thread per batch

// The tile kernel's split of nT tiles over S slots: contiguous ranges.
__device__ inline void slot_range(int s, int S, int nT, int* t0, int* cnt)
{
    const int q = nT / S, rem = nT - q * S;
    *t0 = s * q + min(s, rem);
    *cnt = q + (s < rem ? 1 : 0);
}

__global__ __launch_bounds__(kThreadsP) void k_probe_tile_reads(const uint16_t* __restrict__ L,
                                                                const uint16_t* __restrict__ Bm, int B, int gamma,
                                                                int V, int r, int k, int nT, int S,
                                                                unsigned* __restrict__ sink)
{
    int t0, cnt;
    slot_range(blockIdx.x, S, nT, &t0, &cnt);
    const int rows = B + r;
    const int per_tile = rows * 8;                 // 16-byte pieces per tile
    const int total = cnt * per_tile;
    const int lim = V - 8;
    // Piece p: tile p / per_tile, row (p % per_tile) / 8, chunk p % 8.
    auto piece = [&](int p) -> uint4 {
        p = min(p, total - 1);  // the last batch may run past the range: re-read the last piece
        const int t = p / per_tile, rem = p - t * per_tile;
        const int row = rem >> 3, c = rem & 7;
        const int col = min((t0 + t) * 64 + 8 * c, lim);
        const uint16_t* src = row < B ? L + ((size_t)row * gamma + (k - 1)) * V + col
                                      : Bm + (size_t)(row - B) * V + col;
        return *reinterpret_cast<const uint4*>(src);
    };
    const int nb = (total + kThreadsP * kBatch - 1) / (kThreadsP * kBatch);
    unsigned acc = 0;
    uint4 b0[kBatch], b1[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) b0[j] = piece(j * kThreadsP + threadIdx.x);
    for (int b = 0; b < nb; b += 2) {
        if (b + 1 < nb) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) b1[j] = piece(((b + 1) * kBatch + j) * kThreadsP + threadIdx.x);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) acc ^= b0[j].x ^ b0[j].y ^ b0[j].z ^ b0[j].w;
        if (b + 1 >= nb) break;
        if (b + 2 < nb) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) b0[j] = piece(((b + 2) * kBatch + j) * kThreadsP + threadIdx.x);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) acc ^= b1[j].x ^ b1[j].y ^ b1[j].z ^ b1[j].w;
    }
    sink[blockIdx.x * kThreadsP + threadIdx.x] = acc;
}

}  // namespace

// Times the load-only kernel: one untimed round over draft steps k = 1..gamma,
// then `reps` rounds, each launch with a pair of events bound to its dispatch
// (hipExtLaunchKernelGGL), so each interval is the kernel's own execution.
// Reads L [B][gamma][V] and Bm [r][V] (device, bf16 bit patterns) split over
// `slots` workgroups of 512 threads as the draft tile kernel splits its tiles;
// sink: device, at least slots * 512 words, overwritten.  Synchronises the
// stream.  *avg_us receives the mean duration per launch.  Returns a
// hipError_t code (0 on success).  Requires B, r, gamma, reps >= 1, V >= 8 a
// multiple of 8, 1 <= slots <= ceil(V / 64).
extern "C" int dspark_probe_time_tile_reads(const void* L, const void* Bm, int B, int gamma, int V, int r, int slots,
                                            int reps, unsigned* sink, hipStream_t stream, double* avg_us)
{
    const int nT = (V + 63) / 64;
    if (!L || !Bm || !sink || !avg_us || B < 1 || r < 1 || gamma < 1 || reps < 1 || V < 8 || (V & 7) || slots < 1 ||
        slots > nT)
        return (int)hipErrorInvalidValue;
    const uint16_t* l = static_cast<const uint16_t*>(L);
    const uint16_t* bm = static_cast<const uint16_t*>(Bm);
    for (int k = 1; k <= gamma; ++k)
        hipLaunchKernelGGL(k_probe_tile_reads, dim3(slots), dim3(kThreadsP), 0, stream, l, bm, B, gamma, V, r, k, nT,
                           slots, sink);
    const int n = reps * gamma;
    std::vector<hipEvent_t> ev(2 * n, nullptr);
    hipError_t err = hipSuccess;
    for (int i = 0; i < 2 * n && err == hipSuccess; ++i) err = hipEventCreate(&ev[i]);
    for (int i = 0; i < n && err == hipSuccess; ++i) {
        hipExtLaunchKernelGGL(k_probe_tile_reads, dim3(slots), dim3(kThreadsP), 0, stream, ev[2 * i], ev[2 * i + 1],
                              0, l, bm, B, gamma, V, r, 1 + i % gamma, nT, slots, sink);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipStreamSynchronize(stream);
    double total = 0.0;
    for (int i = 0; i < n && err == hipSuccess; ++i) {
        float ms = 0.0f;
        err = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
        total += ms;
    }
    for (hipEvent_t e : ev)
        if (e) (void)hipEventDestroy(e);
    if (err == hipSuccess) *avg_us = 1000.0 * total / n;
    return (int)err;
}
