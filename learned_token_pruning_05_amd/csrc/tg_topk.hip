// Top-K selection with the question always kept.
//
// TokenGate (spke.com article, section on how learned token pruning works):
// a top-K selector keeps the highest-scoring tokens at the gate layer; only the
// document part of the prompt is prunable, the question never is.
//
// Scores map to order-preserving 32-bit keys (larger score <=> larger key; -0
// and +0 share a key; NaN is key 0, below -inf).  Per sequence the selector
// needs the key T of the K_eff-th document token and r, the number of tokens
// with key == T that are kept (the r lowest-indexed ones).  Five launches, no
// cross-workgroup waiting, no zero-filled state, and every pass over all
// tokens spread over many workgroups:
//   H  every 4096-token chunk writes the 2048-bin histogram of its document
//      keys' top 11 bits (plain stores, one row per chunk);
//   B  one workgroup per sequence sums the chunk histograms and finds the
//      bucket b1 holding T;
//   F  every 2048-token chunk counts its always-kept tokens (outside the
//      document, or top bits above b1) and compacts its bucket-b1 keys, with
//      their indices, into its own slice of a candidate buffer;
//   S  one workgroup per sequence gathers the candidates (a few per cent of the
//      tokens) into LDS, finds T and r with two more radix passes, and turns
//      the per-chunk kept / tie counts into output offsets;
//   W  every 2048-token chunk writes its kept indices in order: slot = chunk
//      offset + kept tokens before it (wave ballots), ties capped at r.
// Ties are decided by index order through prefix counts, never by the order of
// atomics, so the output is deterministic.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBins = 2048;
constexpr int kHistChunk = 4096;            // tokens per histogram workgroup
constexpr int kHistThreads = 1024;
constexpr int kWriteChunk = 2048;           // tokens per write workgroup
constexpr int kWriteThreads = 256;
constexpr int kWriteItems = kWriteChunk / kWriteThreads;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxWriteChunks = 2048;       // max_seqlen <= 4 Mi tokens
constexpr int kCandCap = 8192;              // candidates kept in LDS (else in the workspace)

struct SeqState {
    uint32_t T;
    int32_t r;
};

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
};

// LDS histogram add; a wave whose active lanes all hit one bin adds once.
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t bin, bool active) {
    const uint64_t act = __ballot(active);
    if (!act) return;
    const int lead = __builtin_ctzll(act);
    const uint32_t b0 = __shfl(bin, lead, 64);
    const uint64_t same = __ballot(active && bin == b0);
    if (same == act) {
        if ((int)(threadIdx.x & 63) == lead) atomicAdd(&h[b0], (uint32_t)__popcll(act));
    } else if (active) {
        atomicAdd(&h[bin], 1u);
    }
}

// Exclusive prefix over the workgroup of one value; *total = sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
    constexpr int NW = NT / 64;
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
    for (int i = 0; i < NW; ++i) {
        const uint32_t t = sh[i];
        wex += i < w ? t : 0u;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return wex + x - v;
}

// Bucket (of 2048 LDS bins, bin 2047 = largest) holding the rem-th largest key,
// and the count in higher bins.  Every thread gets the answer.
__device__ void find_bucket(const uint32_t* hist, uint32_t rem, uint32_t* sh_scan, uint32_t* sh_out,
                            uint32_t* out_b, uint32_t* out_above) {
    constexpr int PER = kBins / kSelThreads;   // 2 bins per thread, descending
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = hist[kBins - 1 - PER * threadIdx.x - i];
        sum += c[i];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan<kSelThreads>(sum, sh_scan, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (above < rem && rem <= above + c[i]) {
            sh_out[0] = kBins - 1 - PER * threadIdx.x - i;
            sh_out[1] = above;
        }
        above += c[i];
    }
    __syncthreads();
    *out_b = sh_out[0];
    *out_above = sh_out[1];
    __syncthreads();
}

// ------------------------------------------------------------------ H ----
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, int nch_hist, uint32_t* __restrict__ part) {
    __shared__ uint32_t h[kBins];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kHistChunk;
    if (!q.needs_select() || c0 >= q.n) return;
    for (int i = tid; i < kBins; i += kHistThreads) h[i] = 0u;
    __syncthreads();
    const float* sc = scores + q.start;
    constexpr int PER = kHistChunk / kHistThreads;   // all of a thread's scores loaded first
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = c0 + j * kHistThreads + tid;
        v[j] = (i >= q.db && i < q.de) ? sc[i] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = c0 + j * kHistThreads + tid;
        hist_add(h, score_key(v[j]) >> 21, i >= q.db && i < q.de);
    }
    __syncthreads();
    uint32_t* dst = part + ((int64_t)s * nch_hist + c) * kBins;
    for (int i = tid; i < kBins; i += kHistThreads) dst[i] = h[i];
}

// ------------------------------------------------------------------ B ----
struct SelState {
    uint32_t b1, above1;
};

__global__ __launch_bounds__(kSelThreads) void topk_bucket_kernel(
    const int* __restrict__ cu, const int* __restrict__ db, const int* __restrict__ de,
    const int* __restrict__ kd, int nch_hist, const uint32_t* __restrict__ part,
    SelState* __restrict__ sel) {
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t sh_scan[kSelWaves];
    __shared__ uint32_t sh_out[2];
    const int s = blockIdx.x, tid = threadIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select()) return;
    const int nh = (q.n + kHistChunk - 1) / kHistChunk;
    const uint32_t* ps = part + (int64_t)s * nch_hist * kBins;
    for (int b = tid; b < kBins; b += kSelThreads) {
        uint32_t t = 0;
        int c = 0;
        for (; c + 8 <= nh; c += 8) {   // eight rows in flight
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ps[(int64_t)(c + u) * kBins + b];
#pragma unroll
            for (int u = 0; u < 8; ++u) t += v[u];
        }
        for (; c < nh; ++c) t += ps[(int64_t)c * kBins + b];
        h[b] = t;
    }
    __syncthreads();
    uint32_t b1, above1;
    find_bucket(h, (uint32_t)q.k, sh_scan, sh_out, &b1, &above1);
    if (tid == 0) sel[s] = SelState{b1, above1};
}

// ------------------------------------------------------------------ F ----
__global__ __launch_bounds__(kWriteThreads) void topk_filter_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, int nch_write,
    const SelState* __restrict__ sel, uint32_t* __restrict__ chunk_a0, uint32_t* __restrict__ chunk_nc,
    uint2* __restrict__ cand_g) {
    constexpr int NW = kWriteThreads / 64;
    __shared__ uint32_t cnt[2][kWriteItems * NW];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kWriteChunk;
    if (!q.needs_select() || c0 >= q.n) return;
    const uint32_t b1 = sel[s].b1;
    const float* sc = scores + q.start;
    float v[kWriteItems];
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const int i = c0 + j * kWriteThreads + tid;
        v[j] = i < q.n ? sc[i] : 0.0f;
    }
    uint64_t mc[kWriteItems];
    uint32_t keys[kWriteItems];
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const int i = c0 + j * kWriteThreads + tid;
        const bool in = i < q.n;
        const bool doc = in && i >= q.db && i < q.de;
        keys[j] = score_key(v[j]);
        const uint32_t top = keys[j] >> 21;
        const uint64_t ma = __ballot(in && (!doc || top > b1));
        mc[j] = __ballot(doc && top == b1);
        if (lane == 0) {
            cnt[0][j * NW + w] = (uint32_t)__popcll(ma);
            cnt[1][j * NW + w] = (uint32_t)__popcll(mc[j]);
        }
    }
    __syncthreads();
    // in-order rank of this wave-slice's candidates within the chunk
    uint32_t pre_c = 0, tot_a = 0, tot_c = 0, my_pre[kWriteItems];
#pragma unroll
    for (int x = 0; x < kWriteItems * NW; ++x) {
        const int j = x / NW, ww = x % NW;
        if (ww == w) my_pre[j] = pre_c;
        pre_c += cnt[1][x];
        tot_a += cnt[0][x];
    }
    tot_c = pre_c;
    uint2* cs = cand_g + q.start + c0;   // this chunk's slice
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j)
        if ((mc[j] >> lane) & 1ull)
            cs[my_pre[j] + (uint32_t)__popcll(mc[j] & below)] =
                make_uint2(keys[j], (uint32_t)(c0 + j * kWriteThreads + tid));
    if (tid == 0) {
        chunk_a0[(int64_t)s * nch_write + c] = tot_a;
        chunk_nc[(int64_t)s * nch_write + c] = tot_c;
    }
}

// ------------------------------------------------------------------ S ----
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const int* __restrict__ cu, const int* __restrict__ db, const int* __restrict__ de,
    const int* __restrict__ kd, int nch_write, const SelState* __restrict__ sel,
    const uint32_t* __restrict__ chunk_a0, const uint32_t* __restrict__ chunk_nc,
    const uint2* __restrict__ cand_g, SeqState* __restrict__ st, uint32_t* __restrict__ base_a,
    uint32_t* __restrict__ base_b) {
    __shared__ uint32_t h[kBins];
    __shared__ uint32_t ca[kMaxWriteChunks], cb[kMaxWriteChunks], coff[kMaxWriteChunks + 1];
    __shared__ uint2 cand[kCandCap];
    __shared__ uint32_t sh_scan[kSelWaves];
    __shared__ uint32_t sh_out[2];
    const int s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select()) return;   // the write kernel handles "all" and "none" directly
    const int nch = (q.n + kWriteChunk - 1) / kWriteChunk;
    const uint32_t b1 = sel[s].b1, above1 = sel[s].above1;

    // candidate offsets per chunk (exclusive scan of the chunk counts)
    {
        uint32_t run = 0;
        for (int b0 = 0; b0 < nch; b0 += kSelThreads) {
            const int i = b0 + tid;
            const uint32_t v = i < nch ? chunk_nc[(int64_t)s * nch_write + i] : 0u;
            uint32_t tot;
            const uint32_t e = block_excl_scan<kSelThreads>(v, sh_scan, &tot);
            if (i < nch) {
                coff[i] = run + e;
                ca[i] = chunk_a0[(int64_t)s * nch_write + i];
                cb[i] = 0u;
            }
            run += tot;
        }
        if (tid == 0) coff[nch] = run;
        __syncthreads();
    }
    const uint32_t nc = coff[nch];
    const uint2* cg = cand_g + q.start;
    // candidate g of the sequence lives in chunk c at slice position g - coff[c]
    auto cand_at = [&](uint32_t g) {
        int lo = 0, hi = nch;   // coff[lo] <= g < coff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (coff[mid] <= g) lo = mid; else hi = mid;
        }
        return cg[(int64_t)lo * kWriteChunk + (g - coff[lo])];
    };
    const bool in_lds = nc <= kCandCap;
    if (in_lds) {
        // a wave per chunk copies the chunk's slice (coalesced) to its offset
        for (int c = w; c < nch; c += kSelWaves) {
            const uint32_t o = coff[c], n_c = coff[c + 1] - o;
            const uint2* src = cg + (int64_t)c * kWriteChunk;
            for (uint32_t i = lane; i < n_c; i += 64) cand[o + i] = src[i];
        }
        __syncthreads();
    }
    auto get = [&](uint32_t g) { return in_lds ? cand[g] : cand_at(g); };

    // two radix passes among the candidates: T and r
    uint32_t rem = (uint32_t)q.k - above1;          // 1 <= rem <= nc
    uint32_t prefix = b1 << 21, pmask = 0xffe00000u;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        const uint32_t bmask = pass == 0 ? 2047u : 1023u;
        for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0u;
        __syncthreads();
        // eight candidates per thread per round, their loads issued together
        // (from the workspace they are global reads)
        constexpr int U = 8;
        for (uint32_t i0 = 0; i0 < nc; i0 += kSelThreads * U) {
            uint32_t key[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + u * kSelThreads + tid;
                key[u] = i < nc ? get(i).x : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + u * kSelThreads + tid;
                hist_add(h, (key[u] >> shift) & bmask, i < nc && (key[u] & pmask) == prefix);
            }
        }
        __syncthreads();
        uint32_t bk, ab;
        find_bucket(h, rem, sh_scan, sh_out, &bk, &ab);
        rem -= ab;
        prefix |= bk << shift;
        pmask |= bmask << shift;
    }
    const uint32_t T = prefix;
    const uint32_t r = rem;

    // candidates above / equal to T, per write chunk (a wave per chunk, counted
    // by ballots over its slice); offsets by exclusive scan
    for (int c = w; c < nch; c += kSelWaves) {
        const uint32_t o = coff[c], n_c = coff[c + 1] - o;
        const uint2* src = cg + (int64_t)c * kWriteChunk;
        uint32_t na = 0, nb = 0;
        constexpr int V = 4;   // four slices of 64 per round, loads together
        for (uint32_t i0 = 0; i0 < n_c; i0 += 64 * V) {
            uint32_t key[V];
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const uint32_t i = i0 + u * 64 + lane;
                key[u] = i < n_c ? (in_lds ? cand[o + i].x : src[i].x) : 0u;
            }
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const uint32_t i = i0 + u * 64 + lane;
                na += (uint32_t)__popcll(__ballot(i < n_c && key[u] > T));
                nb += (uint32_t)__popcll(__ballot(i < n_c && key[u] == T));
            }
        }
        if (lane == 0) {
            ca[c] += na;
            cb[c] = nb;
        }
    }
    __syncthreads();
    uint32_t run_a = 0, run_b = 0;
    for (int b0 = 0; b0 < nch; b0 += kSelThreads) {
        const int i = b0 + tid;
        const uint32_t va = i < nch ? ca[i] : 0u, vb = i < nch ? cb[i] : 0u;
        uint32_t ta, tb;
        const uint32_t ea = block_excl_scan<kSelThreads>(va, sh_scan, &ta);
        const uint32_t eb = block_excl_scan<kSelThreads>(vb, sh_scan, &tb);
        if (i < nch) {
            base_a[(int64_t)s * nch_write + i] = run_a + ea;
            base_b[(int64_t)s * nch_write + i] = run_b + eb;
        }
        run_a += ta;
        run_b += tb;
    }
    if (tid == 0) {
        st[s].T = T;
        st[s].r = (int32_t)r;
    }
}

// ------------------------------------------------------------------ W ----
__global__ __launch_bounds__(kWriteThreads) void topk_write_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, const int* __restrict__ cu_kept,
    int nch_write, const SeqState* __restrict__ st, const uint32_t* __restrict__ base_a,
    const uint32_t* __restrict__ base_b, int* __restrict__ kept_idx) {
    constexpr int NW = kWriteThreads / 64;
    __shared__ uint32_t cnt[2][kWriteItems * NW];
    __shared__ uint32_t pre[2][kWriteItems * NW];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kWriteChunk;
    if (c0 >= q.n) return;
    int* __restrict__ out = kept_idx + cu_kept[s];
    const uint32_t m_s = (uint32_t)(cu_kept[s + 1] - cu_kept[s]);
    const int nd = q.de - q.db;
    if (!q.needs_select()) {
        // whole document kept (k == n_doc) or none of it (k == 0)
        const bool all = q.k == nd;
#pragma unroll
        for (int j = 0; j < kWriteItems; ++j) {
            const int i = c0 + j * kWriteThreads + tid;
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
    float v[kWriteItems];
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const int i = c0 + j * kWriteThreads + tid;
        v[j] = i < q.n ? sc[i] : 0.0f;
    }
    uint64_t ma[kWriteItems], mb[kWriteItems];
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const int i = c0 + j * kWriteThreads + tid;
        bool fa = false, fb = false;
        if (i < q.n) {
            if (i < q.db || i >= q.de) {
                fa = true;
            } else {
                const uint32_t key = score_key(v[j]);
                fa = key > T;
                fb = key == T;
            }
        }
        ma[j] = __ballot(fa);
        mb[j] = __ballot(fb);
        if (lane == 0) {
            cnt[0][j * NW + w] = (uint32_t)__popcll(ma[j]);
            cnt[1][j * NW + w] = (uint32_t)__popcll(mb[j]);
        }
    }
    __syncthreads();
    if (tid < 2) {
        uint32_t run = 0;
        for (int x = 0; x < kWriteItems * NW; ++x) {
            pre[tid][x] = run;
            run += cnt[tid][x];
        }
    }
    __syncthreads();
    const uint32_t ba = base_a[(int64_t)s * nch_write + c];
    const uint32_t bb = base_b[(int64_t)s * nch_write + c];
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const bool fa = (ma[j] >> lane) & 1ull, fb = (mb[j] >> lane) & 1ull;
        if (!fa && !fb) continue;
        const uint32_t pa = ba + pre[0][j * NW + w] + (uint32_t)__popcll(ma[j] & below);
        const uint32_t pb = bb + pre[1][j * NW + w] + (uint32_t)__popcll(mb[j] & below);
        if (fb && pb >= r) continue;
        const uint32_t slot = pa + min(pb, r);
        if (slot < m_s) out[slot] = q.start + c0 + j * kWriteThreads + tid;
    }
}

struct TopkLayout {
    size_t st, sel, part, a0, nc, ba, bb, cand, total;
};

inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

TopkLayout topk_layout(int n_seqs, int64_t n_tokens, int max_seqlen) {
    const int64_t nch_h = (max_seqlen + kHistChunk - 1) / kHistChunk;
    const int64_t nch_w = (max_seqlen + kWriteChunk - 1) / kWriteChunk;
    TopkLayout L;
    size_t o = 0;
    L.st = o;   o += al256((size_t)n_seqs * sizeof(SeqState));
    L.sel = o;  o += al256((size_t)n_seqs * sizeof(SelState));
    L.part = o; o += al256((size_t)n_seqs * nch_h * kBins * 4);
    L.a0 = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.nc = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.ba = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.bb = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.cand = o; o += al256((size_t)n_tokens * 8);
    L.total = o;
    return L;
}

// Random-K selector mode: uniform scores in [0, 1) from SplitMix64 (Steele,
// Lea and Flood 2014): output t of the generator seeded with `seed` is the
// finalizer of seed + (t+1) * 0x9E3779B97F4A7C15, so each token's draw is
// independent of the others.  The score is the top 30 bits d of the draw as the
// positive normal fp32 with bit pattern 2^23 + d: it orders exactly like d, and
// d's top bits spread the scores over the selector's radix buckets.
__global__ __launch_bounds__(256) void random_scores_kernel(uint64_t seed, int64_t n, float* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    uint64_t z = seed + (uint64_t)(t + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    out[t] = __uint_as_float((uint32_t)(z >> 34) + 0x00800000u);
}

}  // namespace

size_t random_k_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen) {
    return al256((size_t)n_tokens * 4) + topk_workspace_bytes(n_seqs, n_tokens, max_seqlen);
}

int launch_random_k(uint64_t seed, int n_seqs, int64_t n_tokens, int max_seqlen, const int* cu_seqlens,
                    const int* doc_begin, const int* doc_end, const int* k_doc, const int* cu_kept,
                    int* kept_idx, void* ws, hipStream_t stm) {
    if (n_seqs == 0 || n_tokens == 0) return TG_OK;
    float* sc = (float*)ws;
    hipLaunchKernelGGL(random_scores_kernel, dim3((unsigned)((n_tokens + 255) / 256)), dim3(256), 0, stm, seed,
                       n_tokens, sc);
    if (hipGetLastError() != hipSuccess) return TG_ERR_HIP;
    return launch_topk(sc, n_seqs, n_tokens, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, kept_idx,
                       (char*)ws + al256((size_t)n_tokens * 4), stm);
}

size_t topk_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen) {
    return topk_layout(n_seqs, n_tokens, max_seqlen).total;
}

int topk_max_seqlen() { return kMaxWriteChunks * kWriteChunk; }

int launch_topk(const float* scores, int n_seqs, int64_t n_tokens, int max_seqlen,
                const int* cu_seqlens, const int* doc_begin, const int* doc_end, const int* k_doc,
                const int* cu_kept, int* kept_idx, void* ws, hipStream_t stm) {
    if (n_seqs == 0 || max_seqlen == 0) return TG_OK;
    const TopkLayout L = topk_layout(n_seqs, n_tokens, max_seqlen);
    char* w = (char*)ws;
    SeqState* st = (SeqState*)(w + L.st);
    SelState* sel = (SelState*)(w + L.sel);
    uint32_t* part = (uint32_t*)(w + L.part);
    uint32_t* a0 = (uint32_t*)(w + L.a0);
    uint32_t* nc = (uint32_t*)(w + L.nc);
    uint32_t* ba = (uint32_t*)(w + L.ba);
    uint32_t* bb = (uint32_t*)(w + L.bb);
    uint2* cand = (uint2*)(w + L.cand);
    const int nch_h = (max_seqlen + kHistChunk - 1) / kHistChunk;
    const int nch_w = (max_seqlen + kWriteChunk - 1) / kWriteChunk;
    hipLaunchKernelGGL(topk_hist_kernel, dim3(nch_h, n_seqs), dim3(kHistThreads), 0, stm, scores,
                       cu_seqlens, doc_begin, doc_end, k_doc, nch_h, part);
    hipLaunchKernelGGL(topk_bucket_kernel, dim3(n_seqs), dim3(kSelThreads), 0, stm, cu_seqlens, doc_begin,
                       doc_end, k_doc, nch_h, (const uint32_t*)part, sel);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(nch_w, n_seqs), dim3(kWriteThreads), 0, stm, scores,
                       cu_seqlens, doc_begin, doc_end, k_doc, nch_w, (const SelState*)sel, a0, nc, cand);
    hipLaunchKernelGGL(topk_select_kernel, dim3(n_seqs), dim3(kSelThreads), 0, stm, cu_seqlens, doc_begin,
                       doc_end, k_doc, nch_w, (const SelState*)sel, (const uint32_t*)a0, (const uint32_t*)nc,
                       (const uint2*)cand, st, ba, bb);
    hipLaunchKernelGGL(topk_write_kernel, dim3(nch_w, n_seqs), dim3(kWriteThreads), 0, stm, scores,
                       cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, nch_w, (const SeqState*)st,
                       (const uint32_t*)ba, (const uint32_t*)bb, kept_idx);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
