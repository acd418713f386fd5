// Top-K selection with the question always kept.
//
// TokenGate (spke.com article, section on how learned token pruning works):
// a top-K selector keeps the highest-scoring tokens at the gate layer; only the
// document part of the prompt is prunable, the question never is.
//
// One workgroup per sequence.  MSB-first radix select (11 + 11 + 10 bits) over
// order-preserving 32-bit keys finds the threshold key T of the K_eff-th
// document token and the number r of tokens equal to T that are kept; a
// stable in-order compaction then writes the kept indices ascending.  Ties at T
// are resolved to the lowest indices by an exclusive prefix count, never by
// atomics, so the result is deterministic.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kItems = 4;   // consecutive tokens per thread in the compaction sweep

// Monotone map float -> uint32: larger score <=> larger key.  -0.0 and +0.0
// map to one key; every NaN maps to 0, below -inf (whose key is 0x007fffff).
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive block-wide prefix sum over kThreads threads; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wtot[w] = x;
    __syncthreads();
    if (w == 0) {
        uint32_t t = lane < kWaves ? wtot[lane] : 0u;
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            uint32_t y = __shfl_up(t, o, 64);
            if (lane >= o) t += y;
        }
        if (lane < kWaves) wtot[lane] = t;
    }
    __syncthreads();
    const uint32_t wex = w ? wtot[w - 1] : 0u;
    *total = wtot[kWaves - 1];
    __syncthreads();
    return wex + x - v;
}

__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu_seqlens,
    const int* __restrict__ doc_begin, const int* __restrict__ doc_end,
    const int* __restrict__ k_doc, const int* __restrict__ cu_kept, int* __restrict__ kept_idx) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t wtot[kWaves];
    __shared__ uint32_t sh_bucket, sh_above;

    const int s = blockIdx.x;
    const int tid = threadIdx.x;
    const int start = cu_seqlens[s];
    const int n = cu_seqlens[s + 1] - start;
    const int db = doc_begin[s], de = doc_end[s];
    const int nd = de - db;
    const int k = max(0, min(k_doc[s], nd));
    const float* __restrict__ sc = scores + start;
    int* __restrict__ out = kept_idx + cu_kept[s];
    const uint32_t m_s = (uint32_t)(cu_kept[s + 1] - cu_kept[s]);   // bound on output slots

    // Keep document keys > T, plus the first r (in index order) equal to T.
    uint32_t T;
    int r;
    if (k == nd) {            // whole document kept (NaN keys are 0 == T)
        T = 0u;
        r = 0x7fffffff;
    } else if (k == 0) {      // no document token kept (key 0xffffffff never occurs)
        T = 0xffffffffu;
        r = 0;
    } else {
        uint32_t prefix = 0u, pmask = 0u;
        int remaining = k;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const uint32_t bmask = pass == 2 ? 1023u : 2047u;
            for (int i = tid; i < kBins; i += kThreads) hist[i] = 0u;
            __syncthreads();
            for (int i = tid; i < nd; i += kThreads) {
                const uint32_t key = score_key(sc[db + i]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & bmask], 1u);
            }
            __syncthreads();
            // Thread t owns bins 2047-2t (hi) and 2046-2t (lo): a prefix over
            // threads is a suffix over bins, i.e. the count of larger keys.
            const uint32_t c_hi = hist[kBins - 1 - 2 * tid];
            const uint32_t c_lo = hist[kBins - 2 - 2 * tid];
            uint32_t tot;
            const uint32_t above = block_excl_scan(c_hi + c_lo, wtot, &tot);
            const uint32_t rem = (uint32_t)remaining;
            if (above < rem && rem <= above + c_hi) {
                sh_bucket = kBins - 1 - 2 * tid;
                sh_above = above;
            } else if (above + c_hi < rem && rem <= above + c_hi + c_lo) {
                sh_bucket = kBins - 2 - 2 * tid;
                sh_above = above + c_hi;
            }
            __syncthreads();
            remaining -= (int)sh_above;
            prefix |= sh_bucket << shift;
            pmask |= bmask << shift;
            __syncthreads();
        }
        T = prefix;
        r = remaining;
    }

    // In-order compaction.  a: always-kept (outside the document or key > T);
    // b: document key == T.  Output slot = #a before + min(#b before, r).
    uint32_t run_a = 0u, run_b = 0u;
    for (int base = 0; base < n; base += kThreads * kItems) {
        const int i0 = base + tid * kItems;
        uint32_t fa = 0u, fb = 0u;
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const int i = i0 + e;
            if (i < n) {
                const bool isdoc = (i >= db) && (i < de);
                if (!isdoc) {
                    fa |= 1u << e;
                } else {
                    const uint32_t key = score_key(sc[i]);
                    if (key > T) fa |= 1u << e;
                    else if (key == T) fb |= 1u << e;
                }
            }
        }
        const uint32_t packed = (uint32_t)__popc(fa) | ((uint32_t)__popc(fb) << 16);
        uint32_t tot;
        const uint32_t ex = block_excl_scan(packed, wtot, &tot);
        uint32_t ca = run_a + (ex & 0xffffu);
        uint32_t cb = run_b + (ex >> 16);
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
            const bool a = (fa >> e) & 1u, b = (fb >> e) & 1u;
            const uint32_t slot = ca + min(cb, (uint32_t)r);
            if ((a || (b && cb < (uint32_t)r)) && slot < m_s) out[slot] = start + i0 + e;
            ca += a;
            cb += b;
        }
        run_a += tot & 0xffffu;
        run_b += tot >> 16;
    }
}

}  // namespace

int launch_topk(const float* scores, int n_seqs, const int* cu_seqlens, const int* doc_begin,
                const int* doc_end, const int* k_doc, const int* cu_kept, int* kept_idx,
                hipStream_t st) {
    if (n_seqs == 0) return TG_OK;
    hipLaunchKernelGGL(topk_select_kernel, dim3(n_seqs), dim3(kThreads), 0, st, scores,
                       cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, kept_idx);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
