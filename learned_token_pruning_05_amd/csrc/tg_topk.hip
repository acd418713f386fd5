// Top-K selection with the question always kept, and the compaction that
// follows it.
//
// TokenGate (spke.com article, section on how learned token pruning works):
// a top-K selector keeps the highest-scoring tokens at the gate layer; only the
// document part of the prompt is prunable, the question never is; the layers
// above the gate see only the kept tokens.
//
// Scores map to order-preserving 32-bit keys (larger score <=> larger key; -0
// and +0 share a key; NaN is key 0, below -inf).  Per sequence the selector
// needs the key T of the K_eff-th document token and r, the number of tokens
// with key == T that are kept (the r lowest-indexed ones).  A batch whose
// sequences all fit in 16 Ki tokens takes one launch, in 64 Ki tokens two (S,
// below: one workgroup per sequence finds T and r, then W).  Longer sequences
// take four launches, with no cross-workgroup waiting:
//   C  zero the per-sequence counters (histogram, ticket, list length): a
//      kernel, not a memset, so that the call can be captured into a graph
//      and replayed;
//   H  every 4096-token chunk builds the LDS histogram of its document keys'
//      top 12 bits and adds its non-zero bins to the sequence's histogram with
//      atomics;
//   F  every 2048-token chunk finds the bucket b1 holding T from the summed
//      histogram, counts its always-kept tokens (outside the
//      document, or top bits above b1) and appends its bucket-b1 keys, with
//      their indices, to the sequence's candidate list (space reserved with
//      one atomic per chunk); the last chunk of the sequence to finish finds
//      T and r with two more radix passes over the candidates (a few per cent
//      of the tokens) and turns the per-chunk kept / tie counts into output
//      offsets;
//   W  every 2048-token chunk writes its kept indices in order: slot = chunk
//      offset + kept tokens before it (wave ballots), ties capped at r.
// Ties are decided by index order through prefix counts, never by the order of
// atomics (atomics only count and reserve space in an unordered list), so the
// output is deterministic.  A workgroup that is not last leaves after its
// ticket: nothing ever waits for another workgroup.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBits1 = 12;
constexpr int kBins1 = 1 << kBits1;          // first-level buckets: the key's top 12 bits
constexpr int kShift1 = 32 - kBits1;
constexpr int kBins2 = 1024;                 // two more passes of 10 bits among the candidates
constexpr int kHistChunk = 4096;             // tokens per histogram workgroup
constexpr int kHistThreads = 1024;
constexpr int kChunk = 2048;                 // tokens per filter / write workgroup
constexpr int kFiltThreads = 512;
constexpr int kFiltWaves = kFiltThreads / 64;
constexpr int kFiltItems = kChunk / kFiltThreads;
constexpr int kWriteThreads = 256;
constexpr int kWriteItems = kChunk / kWriteThreads;
constexpr int kWCnt = kWriteItems * (kWriteThreads / 64);   // wave-slices of a write chunk
constexpr int kMaxChunks = 2048;             // max_seqlen <= 4 Mi tokens
constexpr int kCandCap = 4096;               // candidates the select step keeps in LDS (else read from HBM)

// Per-sequence counters, zeroed by the C kernel at the start of every call.
struct SeqCtl {
    uint32_t hist[kBins1];   // document keys' top-12-bit counts, summed by atomics
    uint32_t ticket_f;       // filter workgroups done
    uint32_t n_cand;         // length of the sequence's candidate list
    uint32_t pad[62];
};
static_assert(sizeof(SeqCtl) % 256 == 0, "counters stay 256-B aligned");

struct SelState {
    uint32_t b1, above1;   // first-level bucket of T, document tokens in higher buckets
};

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
    __device__ bool needs_select() const { return seq_selects(db, de, k); }
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

// Bucket (of NB LDS bins, bin NB-1 = largest) holding the rem-th largest key,
// and the count in higher bins.  Every thread gets the answer.
template <int NB, int NT>
__device__ void find_bucket(const uint32_t* hist, uint32_t rem, uint32_t* sh_scan, uint32_t* sh_out,
                            uint32_t* out_b, uint32_t* out_above) {
    constexpr int PER = NB / NT;   // bins per thread, descending
    static_assert(PER * NT == NB, "bins must spread evenly");
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = hist[NB - 1 - PER * threadIdx.x - i];
        sum += c[i];
    }
    uint32_t tot;
    uint32_t above = block_excl_scan<NT>(sum, sh_scan, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (above < rem && rem <= above + c[i]) {
            sh_out[0] = NB - 1 - PER * threadIdx.x - i;
            sh_out[1] = above;
        }
        above += c[i];
    }
    __syncthreads();
    *out_b = sh_out[0];
    *out_above = sh_out[1];
    __syncthreads();
}

// The last of `n_parts` workgroups to reach this point gets true.  Every thread
// calls it after its global writes.  The barrier orders the workgroup's writes
// before thread 0's device-scope release fence (one L2 write-back per
// workgroup) and ticket; in the last workgroup thread 0's acquire fence (one
// cache invalidation) and the second barrier order every thread's later reads
// after all the other workgroups' writes.  Nobody waits: the others simply
// leave.
__device__ __forceinline__ bool last_to_arrive(uint32_t* ticket, uint32_t n_parts, int* sh_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const bool last = atomicAdd(ticket, 1u) == n_parts - 1u;
        if (last) __threadfence();
        *sh_flag = last;
    }
    __syncthreads();
    return *sh_flag != 0;
}

// ------------------------------------------------------------------ C ----
__global__ __launch_bounds__(256) void topk_clear_kernel(const int* __restrict__ cu, const int* __restrict__ db,
                                                         const int* __restrict__ de, const int* __restrict__ kd,
                                                         SeqCtl* __restrict__ ctl) {
    const int s = blockIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select()) return;
    u32x4* p = (u32x4*)(ctl + s);
    for (int i = threadIdx.x; i < (int)(sizeof(SeqCtl) / 16); i += 256) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ H ----
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, SeqCtl* __restrict__ ctl) {
    __shared__ uint32_t h[kBins1];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kHistChunk;
    if (!q.needs_select() || c0 >= q.n) return;
    for (int i = tid; i < kBins1; i += kHistThreads) h[i] = 0u;
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
        hist_add(h, score_key(v[j]) >> kShift1, i >= q.db && i < q.de);
    }
    __syncthreads();
    SeqCtl* g = ctl + s;
    for (int i = tid; i < kBins1; i += kHistThreads) {
        const uint32_t x = h[i];
        if (x) atomicAdd(&g->hist[i], x);
    }
}

// ------------------------------------------------------------------ F ----
// Select step, run by the last filter workgroup of a sequence: T and r from the
// candidate list, then the per-chunk output offsets.
struct SelectLds {
    uint32_t h[kBins2];
    uint32_t ca[kMaxChunks], cb[kMaxChunks];
    uint2 cand[kCandCap];
    uint32_t sh_scan[kFiltWaves];
    uint32_t sh_out[2];
};

__device__ void select_step(const SeqInfo& q, int s, int nch_write, const SelState& se,
                            const uint32_t* __restrict__ n_cand, const uint32_t* __restrict__ chunk_a0,
                            const uint2* __restrict__ cg, SeqState* __restrict__ st,
                            uint32_t* __restrict__ base_a, uint32_t* __restrict__ base_b, SelectLds& L) {
    constexpr int NT = kFiltThreads;
    const int tid = threadIdx.x;
    const int nch = (q.n + kChunk - 1) / kChunk;
    // One memory round trip for every input: the list length, the per-chunk
    // counts and the list itself, read ahead up to the LDS capacity (inside
    // the sequence's list region, which holds a slot per document token;
    // entries past the length are not used).
    const uint32_t n_doc = (uint32_t)(q.de - q.db);
    constexpr int CPT = kMaxChunks / NT;   // per-chunk counts per thread, at most
    uint32_t a0[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int i = u * NT + tid;
        a0[u] = i < nch ? chunk_a0[(int64_t)s * nch_write + i] : 0u;
    }
    constexpr int U = kCandCap / NT;
    uint2 v[U];
    const uint32_t n_read = min(n_doc, (uint32_t)kCandCap);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = u * NT + tid;
        v[u] = i < n_read ? cg[i] : make_uint2(0u, 0u);
    }
    // the length last, so that waiting for it leaves nothing else waiting
    const uint32_t nc = min(__hip_atomic_load(n_cand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), n_doc);
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int i = u * NT + tid;
        if (i < nch) {
            L.ca[i] = a0[u];
            L.cb[i] = 0u;
        }
    }
    // the list, coalesced, into LDS
    const bool in_lds = nc <= kCandCap;
    if (in_lds) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = u * NT + tid;
            if (i < nc) L.cand[i] = v[u];
        }
    }
    __syncthreads();
    auto get = [&](uint32_t g) { return in_lds ? L.cand[g] : cg[g]; };

    // two radix passes of 10 bits among the candidates: T and r
    uint32_t rem = (uint32_t)q.k - se.above1;   // 1 <= rem <= nc
    uint32_t prefix = se.b1 << kShift1, pmask = ~0u << kShift1;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 10 : 0;
        for (int i = tid; i < kBins2; i += NT) L.h[i] = 0u;
        __syncthreads();
        constexpr int U = 8;   // eight candidates per thread per round, loads together
        for (uint32_t i0 = 0; i0 < nc; i0 += NT * U) {
            uint32_t key[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + u * NT + tid;
                key[u] = i < nc ? get(i).x : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + u * NT + tid;
                hist_add(L.h, (key[u] >> shift) & (kBins2 - 1u), i < nc && (key[u] & pmask) == prefix);
            }
        }
        __syncthreads();
        uint32_t bk, ab;
        find_bucket<kBins2, NT>(L.h, rem, L.sh_scan, L.sh_out, &bk, &ab);
        rem -= ab;
        prefix |= bk << shift;
        pmask |= (kBins2 - 1u) << shift;
    }
    const uint32_t T = prefix;
    const uint32_t r = rem;

    // candidates above / equal to T, counted per chunk (LDS atomics add counts
    // only); offsets by exclusive scans over the chunks
    for (uint32_t i = tid; i < nc; i += NT) {
        const uint2 e = get(i);
        const uint32_t c = e.y / kChunk;
        if (c >= (uint32_t)nch) continue;   // only with inconsistent metadata
        if (e.x > T) atomicAdd(&L.ca[c], 1u);
        else if (e.x == T) atomicAdd(&L.cb[c], 1u);
    }
    __syncthreads();
    uint32_t run_a = 0, run_b = 0;
    for (int b0 = 0; b0 < nch; b0 += NT) {
        const int i = b0 + tid;
        const uint32_t va = i < nch ? L.ca[i] : 0u, vb = i < nch ? L.cb[i] : 0u;
        uint32_t ta, tb;
        const uint32_t ea = block_excl_scan<NT>(va, L.sh_scan, &ta);
        const uint32_t eb = block_excl_scan<NT>(vb, L.sh_scan, &tb);
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

__global__ __launch_bounds__(kFiltThreads) void topk_filter_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, int nch_write, SeqCtl* __restrict__ ctl,
    uint32_t* __restrict__ chunk_a0, uint2* __restrict__ cand_g,
    SeqState* __restrict__ st, uint32_t* __restrict__ base_a, uint32_t* __restrict__ base_b) {
    __shared__ uint32_t cnt[2][kFiltItems * kFiltWaves];
    __shared__ int sh_last;
    __shared__ uint32_t sh_off;
    __shared__ SelectLds L;
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kChunk;
    if (!q.needs_select() || c0 >= q.n) return;
    SeqCtl* g = ctl + s;
    const float* sc = scores + q.start;
    float v[kFiltItems];
#pragma unroll
    for (int j = 0; j < kFiltItems; ++j) {
        const int i = c0 + j * kFiltThreads + tid;
        v[j] = i < q.n ? sc[i] : 0.0f;
    }
    // the bucket b1 holding T, from the sequence's summed histogram (every
    // workgroup of the sequence finds the same one)
    SelState se;
    find_bucket<kBins1, kFiltThreads>(g->hist, (uint32_t)q.k, L.sh_scan, L.sh_out, &se.b1, &se.above1);
    uint64_t mc[kFiltItems];
    uint32_t keys[kFiltItems];
#pragma unroll
    for (int j = 0; j < kFiltItems; ++j) {
        const int i = c0 + j * kFiltThreads + tid;
        const bool in = i < q.n;
        const bool doc = in && i >= q.db && i < q.de;
        keys[j] = score_key(v[j]);
        const uint32_t top = keys[j] >> kShift1;
        const uint64_t ma = __ballot(in && (!doc || top > se.b1));
        mc[j] = __ballot(doc && top == se.b1);
        if (lane == 0) {
            cnt[0][j * kFiltWaves + w] = (uint32_t)__popcll(ma);
            cnt[1][j * kFiltWaves + w] = (uint32_t)__popcll(mc[j]);
        }
    }
    __syncthreads();
    // rank of this wave-slice's candidates within the chunk, and the chunk's
    // place in the sequence's list (one reservation per chunk)
    uint32_t pre_c = 0, tot_a = 0, my_pre[kFiltItems];
#pragma unroll
    for (int x = 0; x < kFiltItems * kFiltWaves; ++x) {
        const int j = x / kFiltWaves, ww = x % kFiltWaves;
        if (ww == w) my_pre[j] = pre_c;
        pre_c += cnt[1][x];
        tot_a += cnt[0][x];
    }
    if (tid == 0) {
        sh_off = pre_c ? atomicAdd(&g->n_cand, pre_c) : 0u;
        chunk_a0[(int64_t)s * nch_write + c] = tot_a;
    }
    __syncthreads();
    uint2* cs = cand_g + q.start + sh_off;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kFiltItems; ++j)
        if ((mc[j] >> lane) & 1ull)
            cs[my_pre[j] + (uint32_t)__popcll(mc[j] & below)] =
                make_uint2(keys[j], (uint32_t)(c0 + j * kFiltThreads + tid));
    const int nch = (q.n + kChunk - 1) / kChunk;
    if (!last_to_arrive(&g->ticket_f, (uint32_t)nch, &sh_last)) return;
    // every chunk's candidates are in
    select_step(q, s, nch_write, se, &g->n_cand, chunk_a0, cand_g + q.start, st, base_a, base_b, L);
}

// ------------------------------------------------------------------ W ----
// Kept tokens of one 2048-token chunk: per token whether it is kept and its
// output slot (ascending original index within the sequence).  Returns the
// chunk's first slot and its kept count.
struct ChunkKept {
    uint32_t base, count;
};

__device__ ChunkKept chunk_kept(const SeqInfo& q, int c0, const float* __restrict__ sc,
                                const SeqState* __restrict__ st, int s, uint32_t ba, uint32_t bb,
                                uint32_t (*cnt)[kWCnt], uint32_t (*pre)[kWCnt + 1], uint32_t* slot_out,
                                bool* kept_out) {
    constexpr int NW = kWriteThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nd = q.de - q.db;
    const bool sel = q.needs_select();
    const bool all = !sel && q.k == nd;
    // every score load issued before T and r are needed (one memory round
    // trip); items past the sequence end read its last score, unused
    float v[kWriteItems];
    if (sel) {
#pragma unroll
        for (int j = 0; j < kWriteItems; ++j) v[j] = sc[min(c0 + j * kWriteThreads + tid, q.n - 1)];
    }
    uint32_t T = 0, r = 0;
    if (sel) {
        T = st[s].T;
        r = (uint32_t)st[s].r;
    }
    uint64_t ma[kWriteItems], mb[kWriteItems];
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const int i = c0 + j * kWriteThreads + tid;
        bool fa = false, fb = false;
        if (i < q.n) {
            if (i < q.db || i >= q.de) {
                fa = true;
            } else if (sel) {
                const uint32_t key = score_key(v[j]);
                fa = key > T;
                fb = key == T;
            } else {
                fa = all;
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
        pre[tid][kWriteItems * NW] = run;   // chunk totals
    }
    __syncthreads();
    // without selection the slots follow from the spans: everything kept, or
    // the document dropped
    if (!sel) {
        ba = all ? (uint32_t)c0 : (uint32_t)(c0 <= q.db ? c0 : (c0 >= q.de ? c0 - nd : q.db));
        bb = 0;
    }
    const uint32_t base = ba + min(bb, r);
    const uint32_t n_b = pre[1][kWriteItems * NW];
    const uint32_t count = pre[0][kWriteItems * NW] + (r > bb ? min(r - bb, n_b) : 0u);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j) {
        const bool fa = (ma[j] >> lane) & 1ull, fb = (mb[j] >> lane) & 1ull;
        const uint32_t pa = ba + pre[0][j * NW + w] + (uint32_t)__popcll(ma[j] & below);
        const uint32_t pb = bb + pre[1][j * NW + w] + (uint32_t)__popcll(mb[j] & below);
        const bool kept = fa || (fb && pb < r);
        const uint32_t slot = pa + min(pb, r);
        kept_out[j] = kept;
        slot_out[j] = slot;
    }
    return ChunkKept{base, count};
}

__global__ __launch_bounds__(kWriteThreads) void topk_write_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, const int* __restrict__ cu_kept,
    int nch_write, const SeqState* __restrict__ st, const uint32_t* __restrict__ base_a,
    const uint32_t* __restrict__ base_b, int* __restrict__ kept_idx) {
    __shared__ uint32_t cnt[2][kWCnt];
    __shared__ uint32_t pre[2][kWCnt + 1];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const SeqInfo q(s, cu, db, de, kd);
    const int c0 = c * kChunk;
    if (c0 >= q.n) return;
    int* __restrict__ out = kept_idx + cu_kept[s];
    const uint32_t m_s = (uint32_t)(cu_kept[s + 1] - cu_kept[s]);
    const bool sel = q.needs_select();
    const uint32_t ba = sel ? base_a[(int64_t)s * nch_write + c] : 0u;
    const uint32_t bb = sel ? base_b[(int64_t)s * nch_write + c] : 0u;
    uint32_t slot[kWriteItems];
    bool kept[kWriteItems];
    chunk_kept(q, c0, scores + q.start, st, s, ba, bb, cnt, pre, slot, kept);
#pragma unroll
    for (int j = 0; j < kWriteItems; ++j)
        if (kept[j] && slot[j] < m_s) out[slot[j]] = q.start + c0 + j * kWriteThreads + tid;
}

// ------------------------------------------------------------------ S ----
// Sequences of at most 64 Ki tokens: one 1024-thread workgroup per sequence
// holds the sequence's keys in registers and finds T and r itself.  Wave w
// holds tokens [64 E w, 64 E (w+1)), item e of lane l being token
// 64 (E w + e) + l, so the thread order is the token order.  An item holds
// the score key of a document token, else 0xffffffff, above every score key
// (a token outside the document is always kept; an item past the end of the
// sequence comes after every real token, so it never takes a real slot).
// Three radix passes (11, 11 and 10 bits) over LDS histograms of the document
// keys give T and r.
//   - Up to 16 Ki tokens the same workgroup then places the kept tokens:
//     "key > T" and "key == T" ballots, per-wave counts and a scan over the 16
//     waves give every kept token its slot, as in the write pass.  One launch.
//   - Up to 64 Ki tokens it writes T, r and the per-chunk output offsets (a
//     wave's items are one or two 2048-token chunks) and the write pass W
//     places the tokens: two launches.  Placing 32-64 tokens per lane on one
//     CU would cost more than the second launch.
// Longer sequences take the chunked passes above, which spread the histogram
// over many CUs.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallMax = kSmallThreads * 16;   // 16 Ki tokens: one launch
constexpr int kMidMax = kSmallThreads * 64;     // 64 Ki tokens: two launches
constexpr uint32_t kOutKey = 0xffffffffu;       // no score key is this large (+inf is 0xff800000)

struct SmallLds {
    uint32_t h[2048 + 64];   // bins, then one sink slot per lane
    uint32_t sh_scan[kSmallWaves];
    uint32_t sh_out[2];
    uint32_t cnt[2][2 * kSmallWaves];
};

// Keys of the workgroup's sequence (layout above) and (T, r) such that
// "key > T, or key == T among the first r" keeps exactly the sequence's
// tokens: the radix passes when the document is pruned; T = 0, r = all when
// the whole document is kept (NaN scores have key 0); T = 0xfffffffe, r = 0
// when none of it is (no score key equals that).  T and r come back uniform.
template <int E>
__device__ __forceinline__ void small_select(const SeqInfo& q, const float* __restrict__ sc, int first,
                                             uint32_t (&key)[E], SmallLds& L, uint32_t* T_out, uint32_t* r_out) {
    const int tid = threadIdx.x;
    // every load unconditional, all in flight at once: a buffer resource over
    // the sequence's scores reads zeros past its end, and one offset register
    // serves every item (item e adds 256 e bytes as the scalar offset)
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sc, (uint32_t)q.n * 4u);
#pragma unroll
    for (int e = 0; e < E; ++e)
        key[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, first * 4, 256 * e, 0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = first + 64 * e;
        const uint32_t dm = 0u - (uint32_t)(i >= q.db && i < q.de);   // all ones for a document token
        key[e] = (score_key(__uint_as_float(key[e])) & dm) | ~dm;     // else kOutKey
    }
    uint32_t T, r;
    if (q.needs_select()) {
        uint32_t rem = (uint32_t)q.k, prefix = 0, pmask = 0;
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
            const uint32_t nbm = pass < 2 ? 2047u : 1023u;
            for (int i = tid; i < 2048; i += kSmallThreads) L.h[i] = 0u;
            __syncthreads();
            // a lane whose item is not counted adds to a slot of its own past
            // the bins: no branch, and no pile-up on one address.  After the
            // first pass the prefix test alone excludes 0xffffffff: its top
            // 11 bits (2047) are above those of every score key (+inf: 2044).
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool act = pass == 0 ? key[e] != kOutKey : (key[e] & pmask) == prefix;
                atomicAdd(&L.h[act ? (key[e] >> shift) & nbm : 2048u + (tid & 63)], 1u);
            }
            __syncthreads();
            uint32_t bk, ab;
            if (pass < 2) find_bucket<2048, kSmallThreads>(L.h, rem, L.sh_scan, L.sh_out, &bk, &ab);
            else find_bucket<1024, kSmallThreads>(L.h, rem, L.sh_scan, L.sh_out, &bk, &ab);
            rem -= ab;
            prefix |= bk << shift;
            pmask |= nbm << shift;
        }
        T = prefix;
        r = rem;
    } else if (q.k > 0) {
        T = 0u;
        r = 0xffffffffu;
    } else {
        T = 0xfffffffeu;
        r = 0u;
    }
    *T_out = __builtin_amdgcn_readfirstlane(T);
    *r_out = __builtin_amdgcn_readfirstlane(r);
}

template <int E>
__global__ __launch_bounds__(kSmallThreads) void topk_small_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, const int* __restrict__ cu_kept,
    int* __restrict__ kept_idx) {
    __shared__ SmallLds L;
    const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SeqInfo q(s, cu, db, de, kd);
    if (q.n <= 0) return;
    const int first = w * E * 64 + lane;   // token of item 0; item e adds 64 e
    uint32_t key[E];
    uint32_t T, r;
    small_select<E>(q, scores + q.start, first, key, L, &T, &r);

    // T is re-made opaque for every item, so each item's two compares stay
    // next to their use instead of 2E lane masks being computed up front
    // (they would spill)
    uint32_t na = 0, nb = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        __asm__ volatile("" : "+s"(T));
        na += (uint32_t)__popcll(__ballot(key[e] > T));
        nb += (uint32_t)__popcll(__ballot(key[e] == T));
    }
    if (lane == 0) {
        L.cnt[0][w] = na;
        L.cnt[1][w] = nb;
    }
    __syncthreads();
    uint32_t ba = 0, bb = 0;
    for (int x = 0; x < w; ++x) {
        ba += L.cnt[0][x];
        bb += L.cnt[1][x];
    }
    int* __restrict__ out = kept_idx + cu_kept[s];
    const uint32_t m_s = (uint32_t)(cu_kept[s + 1] - cu_kept[s]);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        __asm__ volatile("" : "+s"(T));
        const bool fa = key[e] > T, fb = key[e] == T;
        const uint64_t ma = __ballot(fa), mb = __ballot(fb);
        const uint32_t pa = ba + (uint32_t)__popcll(ma & below);
        const uint32_t pb = bb + (uint32_t)__popcll(mb & below);
        const uint32_t slot = pa + min(pb, r);
        if ((fa || (fb && pb < r)) && slot < m_s) out[slot] = q.start + first + 64 * e;
        ba += (uint32_t)__popcll(ma);
        bb += (uint32_t)__popcll(mb);
    }
}

// T, r and the per-chunk output offsets of a pruned sequence of up to 64 Ki
// tokens, for the write pass.  A wave's 64 E tokens are E / 32 whole chunks.
template <int E>
__global__ __launch_bounds__(kSmallThreads) void topk_mid_kernel(
    const float* __restrict__ scores, const int* __restrict__ cu, const int* __restrict__ db,
    const int* __restrict__ de, const int* __restrict__ kd, int nch_write, SeqState* __restrict__ st,
    uint32_t* __restrict__ base_a, uint32_t* __restrict__ base_b) {
    constexpr int CPW = E * 64 / kChunk;   // chunks per wave
    static_assert(CPW * kChunk == E * 64 && CPW * kSmallWaves <= 2 * kSmallWaves, "whole chunks per wave");
    __shared__ SmallLds L;
    const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SeqInfo q(s, cu, db, de, kd);
    if (!q.needs_select()) return;   // the write pass places these from the spans alone
    const int first = w * E * 64 + lane;
    uint32_t key[E];
    uint32_t T, r;
    small_select<E>(q, scores + q.start, first, key, L, &T, &r);
    // per chunk: always-kept tokens (key > T) and ties (key == T); items past
    // the end only ever count in the sequence's last chunk
    // (per-lane counts, then one sum over the wave: no lane masks kept alive)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        uint32_t na = 0, nb = 0;
#pragma unroll
        for (int e = c * (E / CPW); e < (c + 1) * (E / CPW); ++e) {
            na += (uint32_t)(key[e] > T);
            nb += (uint32_t)(key[e] == T);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            na += __shfl_xor(na, o, 64);
            nb += __shfl_xor(nb, o, 64);
        }
        if (lane == 0) {
            L.cnt[0][w * CPW + c] = na;
            L.cnt[1][w * CPW + c] = nb;
        }
    }
    __syncthreads();
    const int nch = (q.n + kChunk - 1) / kChunk;
    if (tid < nch) {
        uint32_t ba = 0, bb = 0;
        for (int x = 0; x < tid; ++x) {
            ba += L.cnt[0][x];
            bb += L.cnt[1][x];
        }
        base_a[(int64_t)s * nch_write + tid] = ba;
        base_b[(int64_t)s * nch_write + tid] = bb;
    }
    if (tid == 0) {
        st[s].T = T;
        st[s].r = (int32_t)r;
    }
}

template <int E>
void launch_small(const float* scores, int n_seqs, const int* cu, const int* db, const int* de, const int* kd,
                  const int* cu_kept, int* kept_idx, hipStream_t stm) {
    hipLaunchKernelGGL(topk_small_kernel<E>, dim3(n_seqs), dim3(kSmallThreads), 0, stm, scores, cu, db, de, kd,
                       cu_kept, kept_idx);
}

struct TopkLayout {
    size_t ctl, st, a0, ba, bb, cand, total;
};

inline size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

TopkLayout topk_layout(int n_seqs, int64_t n_tokens, int max_seqlen) {
    const int64_t nch_w = (max_seqlen + kChunk - 1) / kChunk;
    TopkLayout L;
    size_t o = 0;
    L.ctl = o;  o += al256((size_t)n_seqs * sizeof(SeqCtl));
    L.st = o;   o += al256((size_t)n_seqs * sizeof(SeqState));
    L.a0 = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.ba = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.bb = o;   o += al256((size_t)n_seqs * nch_w * 4);
    L.cand = o; o += al256((size_t)n_tokens * 8);
    L.total = o;
    return L;
}

// Random-K selector mode: scores from SplitMix64 (Steele, Lea and Flood 2014):
// output t of the generator seeded with `seed` is the finalizer of
// seed + (t+1) * 0x9E3779B97F4A7C15, so each token's draw is independent of
// the others.  The score is the top 30 bits d of the draw as the positive
// normal fp32 with bit pattern 2^23 + d: it orders exactly like d, and d's top
// bits spread the scores over the selector's radix buckets.
__global__ __launch_bounds__(256) void random_scores_kernel(uint64_t seed, int64_t n, float* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    uint64_t z = seed + (uint64_t)(t + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    out[t] = __uint_as_float((uint32_t)(z >> 34) + 0x00800000u);
}

struct TopkPtrs {
    SeqCtl* ctl;
    SeqState* st;
    uint32_t *a0, *ba, *bb;
    uint2* cand;
};

TopkPtrs topk_ptrs(void* ws, int n_seqs, int64_t n_tokens, int max_seqlen) {
    const TopkLayout L = topk_layout(n_seqs, n_tokens, max_seqlen);
    char* w = (char*)ws;
    return TopkPtrs{(SeqCtl*)(w + L.ctl),  (SeqState*)(w + L.st),  (uint32_t*)(w + L.a0),
                    (uint32_t*)(w + L.ba), (uint32_t*)(w + L.bb), (uint2*)(w + L.cand)};
}

// C (unless the counters are already zero), H, F: after these the
// per-sequence T, r and chunk offsets are in place.
void launch_select_passes(const float* scores, int n_seqs, int max_seqlen, const int* cu_seqlens,
                          const int* doc_begin, const int* doc_end, const int* k_doc, const TopkPtrs& P,
                          bool counters_zeroed, hipStream_t stm) {
    const int nch_h = (max_seqlen + kHistChunk - 1) / kHistChunk;
    const int nch_w = (max_seqlen + kChunk - 1) / kChunk;
    if (!counters_zeroed)
        hipLaunchKernelGGL(topk_clear_kernel, dim3(n_seqs), dim3(256), 0, stm, cu_seqlens, doc_begin, doc_end,
                           k_doc, P.ctl);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(nch_h, n_seqs), dim3(kHistThreads), 0, stm, scores, cu_seqlens,
                       doc_begin, doc_end, k_doc, P.ctl);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(nch_w, n_seqs), dim3(kFiltThreads), 0, stm, scores, cu_seqlens,
                       doc_begin, doc_end, k_doc, nch_w, P.ctl, P.a0, P.cand, P.st, P.ba, P.bb);
}

}  // namespace

size_t random_k_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen) {
    return al256((size_t)n_tokens * 4) + topk_workspace_bytes(n_seqs, n_tokens, max_seqlen);
}

int launch_random_k(uint64_t seed, int n_seqs, int64_t n_tokens, int max_seqlen, const int* cu_seqlens,
                    const int* doc_begin, const int* doc_end, const int* k_doc, const int* cu_kept,
                    int* kept_idx, void* ws, hipStream_t stm) {
    if (n_seqs == 0 || n_tokens == 0) return TG_OK;
    float* sc = (float*)((char*)ws + topk_workspace_bytes(n_seqs, n_tokens, max_seqlen));
    hipLaunchKernelGGL(random_scores_kernel, dim3((unsigned)((n_tokens + 255) / 256)), dim3(256), 0, stm, seed,
                       n_tokens, sc);
    if (hipGetLastError() != hipSuccess) return TG_ERR_HIP;
    return launch_topk(sc, n_seqs, n_tokens, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, kept_idx,
                       ws, stm);
}

size_t topk_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen) {
    return topk_layout(n_seqs, n_tokens, max_seqlen).total;
}

int topk_max_seqlen() { return kMaxChunks * kChunk; }

bool topk_sel_zero(int n_seqs, int64_t n_tokens, int max_seqlen, const int* doc_begin, const int* doc_end,
                   const int* k_doc, void* ws, SelZero* out) {
    if (n_seqs == 0 || max_seqlen <= kMidMax) return false;
    const TopkPtrs P = topk_ptrs(ws, n_seqs, n_tokens, max_seqlen);
    static_assert(sizeof(SeqCtl) % 16 == 0, "whole 16-B stores");
    *out = SelZero{(uint32_t*)P.ctl, (int64_t)(sizeof(SeqCtl) / 4), (int)(sizeof(SeqCtl) / 4), doc_begin, doc_end,
                   k_doc, n_seqs};
    return true;
}

int launch_topk(const float* scores, int n_seqs, int64_t n_tokens, int max_seqlen,
                const int* cu_seqlens, const int* doc_begin, const int* doc_end, const int* k_doc,
                const int* cu_kept, int* kept_idx, void* ws, hipStream_t stm, bool counters_zeroed) {
    if (n_seqs == 0 || max_seqlen == 0) return TG_OK;
    if (max_seqlen <= kSmallMax) {
        if (max_seqlen <= 4096)
            launch_small<4>(scores, n_seqs, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, kept_idx, stm);
        else
            launch_small<16>(scores, n_seqs, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, kept_idx, stm);
        return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
    }
    const TopkPtrs P = topk_ptrs(ws, n_seqs, n_tokens, max_seqlen);
    const int nch_w = (max_seqlen + kChunk - 1) / kChunk;
    if (max_seqlen <= kMidMax) {
        if (max_seqlen <= kMidMax / 2)
            hipLaunchKernelGGL(topk_mid_kernel<32>, dim3(n_seqs), dim3(kSmallThreads), 0, stm, scores, cu_seqlens,
                               doc_begin, doc_end, k_doc, nch_w, P.st, P.ba, P.bb);
        else
            hipLaunchKernelGGL(topk_mid_kernel<64>, dim3(n_seqs), dim3(kSmallThreads), 0, stm, scores, cu_seqlens,
                               doc_begin, doc_end, k_doc, nch_w, P.st, P.ba, P.bb);
    } else {
        launch_select_passes(scores, n_seqs, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc, P, counters_zeroed,
                             stm);
    }
    hipLaunchKernelGGL(topk_write_kernel, dim3(nch_w, n_seqs), dim3(kWriteThreads), 0, stm, scores, cu_seqlens,
                       doc_begin, doc_end, k_doc, cu_kept, nch_w, (const SeqState*)P.st, (const uint32_t*)P.ba,
                       (const uint32_t*)P.bb, kept_idx);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
