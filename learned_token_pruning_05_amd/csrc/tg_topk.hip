// Top-K selection with the question always kept.
//
// TokenGate (spke.com article, section on how learned token pruning works):
// a top-K selector keeps the highest-scoring tokens at the gate layer; only the
// document part of the prompt is prunable, the question never is.
//
// Scores map to order-preserving 32-bit keys (larger score <=> larger key; -0
// and +0 share a key; NaN is key 0, below -inf).  Per sequence the selector
// needs the key T of the K_eff-th document token and r, the number of tokens
// with key == T that are kept (the r lowest-indexed ones).  Four launches over
// 2048-token chunks, no spin-waits:
//   Z  zero the per-sequence state and histogram;
//   A  every chunk adds a histogram of the top 11 key bits; the last chunk of
//      the sequence to finish (atomic ticket) finds the bucket b1 holding T;
//   B  every chunk counts its always-kept tokens (outside the document, or top
//      bits above b1) and appends the keys in bucket b1 to a candidate list;
//      the last chunk selects T among the candidates (two more radix passes in
//      LDS), finishes the per-chunk kept / tie counts and scans them into
//      per-chunk output offsets;
//   D  every chunk writes its kept indices in order: slot = offset + (kept
//      before it in the chunk, from wave ballots) with ties capped at r.
// Ties are decided by index order through prefix counts, never by the order of
// atomics, so the output is deterministic.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kItems = 8;
constexpr int kChunk = kThreads * kItems;   // 2048 tokens per workgroup
constexpr int kBins = 2048;
constexpr int kMaxChunks = 2048;            // max_seqlen <= 4 Mi tokens

struct SeqState {
    uint32_t ticket_a, ticket_b;
    uint32_t b1, above1;       // bucket of T in the top 11 bits; doc keys in higher buckets
    uint32_t n_cand;
    uint32_t T;
    int32_t r;
    uint32_t pad;
};

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t load_acq(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-sequence view shared by every kernel.
struct SeqInfo {
    int start, n, db, de, k;
    __device__ SeqInfo(int s, const int* cu, const int* b, const int* e, const int* kd) {
        start = cu[s];
        n = cu[s + 1] - start;
        db = b[s];
        de = e[s];
        k = max(0, min(kd[s], de - db));
    }
    __device__ bool needs_select() const { return k > 0 && k < de - db; }
    __device__ int n_chunks() const { return (n + kChunk - 1) / kChunk; }
};

// Exclusive prefix over kThreads threads of one value; *total = sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[w] = x;
    __syncthreads();
    uint32_t wex = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t t = sh[i];
        wex += i < w ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return wex + x - v;
}

// Find the bucket (of `nb` <= 2048 histogram bins in LDS) that holds the
// rem-th largest key: returns bucket and the count in higher buckets.
__device__ void find_bucket(const uint32_t* hist, uint32_t rem, uint32_t* sh_scan, uint32_t* out_b,
                            uint32_t* out_above) {
    // thread t owns the 8 bins 2047-8t .. 2040-8t (descending)
    uint32_t c[8], sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c[i] = hist[kBins - 1 - 8 * threadIdx.x - i];
        sum += c[i];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan(sum, sh_scan, &tot);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (above < rem && rem <= above + c[i]) {
            *out_b = kBins - 1 - 8 * threadIdx.x - i;
            *out_above = above;
        }
        above += c[i];
    }
    __syncthreads();
}

// ------------------------------------------------------------------ Z ----
__global__ __launch_bounds__(kThreads) void topk_zero_kernel(SeqState* st, uint32_t* hist1) {
    const int s = blockIdx.x;
    if (threadIdx.x < sizeof(SeqState) / 4) ((uint32_t*)&st[s])[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist1[(int64_t)s * kBins + i] = 0u;
}

// ------------------------------------------------------------------ A ----
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, SeqState* st, uint32_t* hist1) {
    // n_s <= max_seqlen (host contract) keeps every chunk inside the grid
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t sh_scan[kWaves];
    __shared__ uint32_t sh_last;
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select() || c >= q.n_chunks()) return;
    for (int i = tid; i < kBins; i += kThreads) h[i] = 0u;
    __syncthreads();
    const float* sc = scores + q.start;
    const int c0 = c * kChunk;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int i = c0 + j * kThreads + tid;
        if (i >= q.db && i < q.de) atomicAdd(&h[score_key(sc[i]) >> 21], 1u);
    }
    __syncthreads();
    uint32_t* gh = hist1 + (int64_t)s * kBins;
    for (int i = tid; i < kBins; i += kThreads)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    __threadfence();
    __syncthreads();
    if (tid == 0) sh_last = atomicAdd(&st[s].ticket_a, 1u) == (uint32_t)(q.n_chunks() - 1);
    __syncthreads();
    if (!sh_last) return;
    __threadfence();
    for (int i = tid; i < kBins; i += kThreads) h[i] = load_acq(&gh[i]);
    __syncthreads();
    __shared__ uint32_t sh_b, sh_above;
    find_bucket(h, (uint32_t)q.k, sh_scan, &sh_b, &sh_above);
    if (tid == 0) {
        st[s].b1 = sh_b;
        st[s].above1 = sh_above;
    }
}

// ------------------------------------------------------------------ B ----
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, int nch_max, SeqState* st,
    uint32_t* __restrict__ chunk_a0, uint32_t* __restrict__ base_a, uint32_t* __restrict__ base_b,
    uint2* __restrict__ cand) {
    __shared__ uint32_t sh_scan[kWaves];
    __shared__ uint32_t sh_misc[4];
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t ca[kMaxChunks], cb[kMaxChunks];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select() || c >= q.n_chunks()) return;
    const uint32_t b1 = st[s].b1;
    const float* sc = scores + q.start;
    const int c0 = c * kChunk;
    uint32_t a0 = 0, ncand = 0;
    uint32_t keys[kItems];
    uint32_t cmask = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int i = c0 + j * kThreads + tid;
        keys[j] = 0u;
        if (i < q.n) {
            if (i < q.db || i >= q.de) {
                ++a0;
            } else {
                const uint32_t key = score_key(sc[i]);
                keys[j] = key;
                const uint32_t top = key >> 21;
                if (top > b1) ++a0;
                else if (top == b1) {
                    cmask |= 1u << j;
                    ++ncand;
                }
            }
        }
    }
    // workgroup totals: always-kept count and candidate count
    uint32_t tot_a0, tot_c;
    block_excl_scan(a0, sh_scan, &tot_a0);
    const uint32_t my_c = block_excl_scan(ncand, sh_scan, &tot_c);
    if (tid == 0) {
        chunk_a0[(int64_t)s * nch_max + c] = tot_a0;
        sh_misc[0] = tot_c ? atomicAdd(&st[s].n_cand, tot_c) : 0u;
    }
    __syncthreads();
    uint32_t slot = sh_misc[0] + my_c;
    uint2* cs = cand + q.start;
#pragma unroll
    for (int j = 0; j < kItems; ++j)
        if ((cmask >> j) & 1u) cs[slot++] = make_uint2(keys[j], (uint32_t)(c0 + j * kThreads + tid));
    __threadfence();
    __syncthreads();
    if (tid == 0) sh_misc[1] = atomicAdd(&st[s].ticket_b, 1u) == (uint32_t)(q.n_chunks() - 1);
    __syncthreads();
    if (!sh_misc[1]) return;

    // ---- last chunk of the sequence: exact threshold among the candidates
    __threadfence();
    const uint32_t n_cand = load_acq(&st[s].n_cand);
    uint32_t rem = (uint32_t)q.k - st[s].above1;     // 1 <= rem <= n_cand
    uint32_t prefix = b1 << 21, pmask = 0xffe00000u;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t bmask = pass == 0 ? 2047u : 1023u;
        for (int i = tid; i < kBins; i += kThreads) h[i] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < n_cand; i += kThreads) {
            const uint32_t key = ((const uint32_t*)cs)[2 * i];
            if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & bmask], 1u);
        }
        __syncthreads();
        find_bucket(h, rem, sh_scan, &sh_misc[2], &sh_misc[3]);
        rem -= sh_misc[3];
        prefix |= sh_misc[2] << shift;
        pmask |= bmask << shift;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int32_t r = (int32_t)rem;
    // per-chunk counts of candidates above / equal to T
    const int nch = q.n_chunks();
    for (int i = tid; i < nch; i += kThreads) {
        ca[i] = 0u;
        cb[i] = 0u;
    }
    __syncthreads();
    for (uint32_t i = tid; i < n_cand; i += kThreads) {
        const uint2 e = cs[i];
        if (e.x > T) atomicAdd(&ca[e.y / kChunk], 1u);
        else if (e.x == T) atomicAdd(&cb[e.y / kChunk], 1u);
    }
    __syncthreads();
    // exclusive scan over chunks (in order) of kept (a) and tie (b) counts
    uint32_t run_a = 0, run_b = 0;
    for (int base = 0; base < nch; base += kThreads) {
        const int i = base + tid;
        uint32_t va = 0, vb = 0;
        if (i < nch) {
            va = ca[i] + load_acq(&chunk_a0[(int64_t)s * nch_max + i]);
            vb = cb[i];
        }
        uint32_t ta, tb;
        const uint32_t ea = block_excl_scan(va, sh_scan, &ta);
        const uint32_t eb = block_excl_scan(vb, sh_scan, &tb);
        if (i < nch) {
            base_a[(int64_t)s * nch_max + i] = run_a + ea;
            base_b[(int64_t)s * nch_max + i] = run_b + eb;
        }
        run_a += ta;
        run_b += tb;
    }
    if (tid == 0) {
        st[s].T = T;
        st[s].r = r;
    }
    (void)lane;
    (void)w;
}

// ------------------------------------------------------------------ D ----
__global__ __launch_bounds__(kThreads) void topk_write_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, const int* __restrict__ cu_kept,
    int nch_max, const SeqState* __restrict__ st, const uint32_t* __restrict__ base_a,
    const uint32_t* __restrict__ base_b, int* __restrict__ kept_idx) {
    __shared__ uint32_t cnt[2][kItems * kWaves];
    __shared__ uint32_t pre[2][kItems * kWaves];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const SeqInfo q(s, cu, db, de, kd);
    if (c >= q.n_chunks()) return;
    int* __restrict__ out = kept_idx + cu_kept[s];
    const uint32_t m_s = (uint32_t)(cu_kept[s + 1] - cu_kept[s]);
    const int c0 = c * kChunk;
    const int nd = q.de - q.db;
    if (!q.needs_select()) {
        // whole document kept (k == n_doc) or none of it (k == 0)
        const bool all = q.k == nd;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const int i = c0 + j * kThreads + tid;
            if (i >= q.n) continue;
            const bool doc = i >= q.db && i < q.de;
            uint32_t slot;
            if (all) slot = (uint32_t)i;
            else if (doc) continue;
            else slot = (uint32_t)(i < q.db ? i : i - nd);
            if (slot < m_s) out[slot] = q.start + i;
        }
        return;
    }
    const uint32_t T = st[s].T;
    const uint32_t r = (uint32_t)st[s].r;
    const float* sc = scores + q.start;
    uint64_t ma[kItems], mb[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int i = c0 + j * kThreads + tid;
        bool fa = false, fb = false;
        if (i < q.n) {
            if (i < q.db || i >= q.de) {
                fa = true;
            } else {
                const uint32_t key = score_key(sc[i]);
                fa = key > T;
                fb = key == T;
            }
        }
        ma[j] = __ballot(fa);
        mb[j] = __ballot(fb);
        if (lane == 0) {
            cnt[0][j * kWaves + w] = (uint32_t)__popcll(ma[j]);
            cnt[1][j * kWaves + w] = (uint32_t)__popcll(mb[j]);
        }
    }
    __syncthreads();
    if (tid < 2) {
        uint32_t run = 0;
        for (int x = 0; x < kItems * kWaves; ++x) {
            pre[tid][x] = run;
            run += cnt[tid][x];
        }
    }
    __syncthreads();
    const uint32_t ba = base_a[(int64_t)s * nch_max + c];
    const uint32_t bb = base_b[(int64_t)s * nch_max + c];
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const bool fa = (ma[j] >> lane) & 1ull, fb = (mb[j] >> lane) & 1ull;
        if (!fa && !fb) continue;
        const uint32_t pa = ba + pre[0][j * kWaves + w] + (uint32_t)__popcll(ma[j] & below);
        const uint32_t pb = bb + pre[1][j * kWaves + w] + (uint32_t)__popcll(mb[j] & below);
        if (fb && pb >= r) continue;
        const uint32_t slot = pa + min(pb, r);
        if (slot < m_s) out[slot] = q.start + c0 + j * kThreads + tid;
    }
}

struct TopkLayout {
    size_t st, hist, a0, ba, bb, cand, total;
};

inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

TopkLayout topk_layout(int n_seqs, int64_t n_tokens, int max_seqlen) {
    const int64_t nch = (max_seqlen + kChunk - 1) / kChunk;
    TopkLayout L;
    size_t o = 0;
    L.st = o;   o += al256((size_t)n_seqs * sizeof(SeqState));
    L.hist = o; o += al256((size_t)n_seqs * kBins * 4);
    L.a0 = o;   o += al256((size_t)n_seqs * nch * 4);
    L.ba = o;   o += al256((size_t)n_seqs * nch * 4);
    L.bb = o;   o += al256((size_t)n_seqs * nch * 4);
    L.cand = o; o += al256((size_t)n_tokens * 8);
    L.total = o;
    return L;
}

}  // namespace

size_t topk_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen) {
    return topk_layout(n_seqs, n_tokens, max_seqlen).total;
}

int topk_max_seqlen() { return kMaxChunks * kChunk; }

int launch_topk(const float* scores, int n_seqs, int64_t n_tokens, int max_seqlen,
                const int* cu_seqlens, const int* doc_begin, const int* doc_end, const int* k_doc,
                const int* cu_kept, int* kept_idx, void* ws, hipStream_t stm) {
    if (n_seqs == 0 || max_seqlen == 0) return TG_OK;
    const TopkLayout L = topk_layout(n_seqs, n_tokens, max_seqlen);
    char* w = (char*)ws;
    SeqState* st = (SeqState*)(w + L.st);
    uint32_t* hist = (uint32_t*)(w + L.hist);
    uint32_t* a0 = (uint32_t*)(w + L.a0);
    uint32_t* ba = (uint32_t*)(w + L.ba);
    uint32_t* bb = (uint32_t*)(w + L.bb);
    uint2* cand = (uint2*)(w + L.cand);
    const int nch = (max_seqlen + kChunk - 1) / kChunk;
    const dim3 grid(nch, n_seqs);
    hipLaunchKernelGGL(topk_zero_kernel, dim3(n_seqs), dim3(kThreads), 0, stm, st, hist);
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, stm, scores, cu_seqlens, doc_begin,
                       doc_end, k_doc, st, hist);
    hipLaunchKernelGGL(topk_filter_kernel, grid, dim3(kThreads), 0, stm, scores, cu_seqlens, doc_begin,
                       doc_end, k_doc, nch, st, a0, ba, bb, cand);
    hipLaunchKernelGGL(topk_write_kernel, grid, dim3(kThreads), 0, stm, scores, cu_seqlens, doc_begin,
                       doc_end, k_doc, cu_kept, nch, (const SeqState*)st, (const uint32_t*)ba,
                       (const uint32_t*)bb, kept_idx);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
