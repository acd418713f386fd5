// Compaction of the kept set.
//
// TokenGate (spke.com article, pruned-forward phase): the layers above the gate
// process only the kept tokens and never create KV entries for pruned ones, so
// the kept residuals are copied into a dense [M, d_model] block, with each kept
// token's gate score and its original in-sequence position.
//
// One wavefront per kept row; 16-byte lanes, a whole row in flight per wave
// (a 4 KiB bf16 row is 4 loads per lane issued back to back).
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void gather_rows_kernel(
    const char* __restrict__ x, int64_t x_stride_bytes, int row_bytes,
    const float* __restrict__ scores, const int* __restrict__ kept_idx, int64_t m_tot,
    int n_seqs, const int* __restrict__ cu_seqlens, const int* __restrict__ cu_kept,
    char* __restrict__ x_kept, float* __restrict__ s_kept, int* __restrict__ pos_kept) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (m >= m_tot) return;
    const int src = kept_idx[m];
    const u32x4* __restrict__ srow = (const u32x4*)(x + (int64_t)src * x_stride_bytes);
    u32x4* __restrict__ drow = (u32x4*)(x_kept + m * (int64_t)row_bytes);
    const int nvec = row_bytes >> 4;
    int c = lane;
    for (; c + 64 * (kUnroll - 1) < nvec; c += 64 * kUnroll) {
        u32x4 t[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) t[u] = __builtin_nontemporal_load(srow + c + 64 * u);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) drow[c + 64 * u] = t[u];
    }
    for (; c < nvec; c += 64) drow[c] = __builtin_nontemporal_load(srow + c);
    if (lane == 0) {
        if (s_kept) s_kept[m] = scores[src];
        if (pos_kept) {
            const int s = find_seq(cu_kept, n_seqs, m);
            pos_kept[m] = src - cu_seqlens[s];
        }
    }
}

}  // namespace

int launch_gather(const void* x, int esize, int d_model, int64_t x_stride, const float* scores,
                  const int* kept_idx, int64_t m_tot, int n_seqs, const int* cu_seqlens,
                  const int* cu_kept, void* x_kept, float* s_kept, int* pos_kept, hipStream_t st) {
    if (m_tot == 0) return TG_OK;
    const int64_t blocks = (m_tot + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0, st,
                       (const char*)x, x_stride * esize, d_model * esize, scores, kept_idx, m_tot,
                       n_seqs, cu_seqlens, cu_kept, (char*)x_kept, s_kept, pos_kept);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
