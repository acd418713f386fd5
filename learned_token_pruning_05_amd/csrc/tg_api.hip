// C ABI of libtokengate: argument validation (before any HIP call) and launch.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "tg_common.hpp"

using namespace tg;

// Scratch of tg_topk_select_noalloc: one array per GPU, allocated with the
// code object when the library loads on that device and held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host that name is only a stand-in for the device variable); it resolves the
// array's device address once per device with hipGetSymbolAddress and passes
// that.
constexpr size_t kScratchBytes = 6u << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::atomic<void*> g_scratch_ptr[kScratchDevices];

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks of the front-half calls: TG_OK (launch), -1 (valid, nothing to do) or
// the error status.  No HIP call.
int gate_check(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d_model, int64_t x_row_stride,
               const void* w1, const float* w2, float b2, int32_t d_hid, const float* scores) {
    if (n_tokens < 0 || d_model <= 0 || d_hid <= 0 || !isfinite(b2)) return TG_ERR_INVALID_ARG;
    if (x_dtype != TG_F32 && x_dtype != TG_BF16) return TG_ERR_INVALID_ARG;
    if (d_model % 8 != 0 || x_row_stride < d_model || x_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    if (n_tokens == 0) return -1;
    if (!x || !w1 || !w2 || !scores || !aligned16(x) || !aligned16(w1)) return TG_ERR_INVALID_ARG;
    if (x_dtype == TG_BF16) {
        if (d_model % 64 != 0) return TG_ERR_UNSUPPORTED;
        if (d_hid != 64 && d_hid != 128 && d_hid != 192 && d_hid != 256) return TG_ERR_UNSUPPORTED;
        if (x_row_stride >= (1 << 23)) return TG_ERR_UNSUPPORTED;   // per-workgroup offsets are 32-bit
    } else if (d_hid > 1024 || d_model > 2048) {
        return TG_ERR_UNSUPPORTED;
    }
    return TG_OK;
}

int gate_launch(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d_model, int64_t x_row_stride,
                const void* w1, const float* b1, const float* w2, float b2, int32_t d_hid, float* scores,
                void* stream, const SelZero* zero = nullptr) {
    hipStream_t st = (hipStream_t)stream;
    if (x_dtype == TG_BF16)
        return launch_gate_bf16((const bf16*)x, n_tokens, d_model, x_row_stride, (const bf16*)w1, b1, w2, b2,
                                d_hid, scores, st, zero);
    return launch_gate_f32((const float*)x, n_tokens, d_model, x_row_stride, (const float*)w1, b1, w2, b2, d_hid,
                           scores, st);
}

int topk_check(const float* scores, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
               const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end, const int32_t* k_doc,
               const int32_t* cu_kept, const int32_t* kept_idx, const void* workspace, size_t workspace_bytes) {
    if (n_seqs < 0 || n_tokens_total < 0 || n_tokens_total > INT32_MAX || max_seqlen < 0 ||
        max_seqlen > n_tokens_total)
        return TG_ERR_INVALID_ARG;
    if (max_seqlen > topk_max_seqlen()) return TG_ERR_UNSUPPORTED;
    if (n_seqs == 0 || n_tokens_total == 0) return -1;
    if (!cu_seqlens || !doc_begin || !doc_end || !k_doc || !cu_kept || !kept_idx || !scores)
        return TG_ERR_INVALID_ARG;
    const size_t need = topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return TG_ERR_WORKSPACE;
    return TG_OK;
}

int gather_check(const void* x, int32_t x_dtype, int32_t d_model, int64_t x_row_stride, const float* scores,
                 const int32_t* kept_idx, int64_t n_kept_total, int32_t n_seqs, const int32_t* cu_seqlens,
                 const int32_t* cu_kept, const void* x_kept, const float* scores_kept, const int32_t* pos_kept) {

    if (n_kept_total < 0 || n_seqs < 0 || d_model <= 0) return TG_ERR_INVALID_ARG;
    if (x_dtype != TG_F32 && x_dtype != TG_BF16) return TG_ERR_INVALID_ARG;
    if (d_model % 8 != 0 || x_row_stride < d_model || x_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    if (n_kept_total == 0) return -1;
    if (!x || !kept_idx || !x_kept || !aligned16(x) || !aligned16(x_kept)) return TG_ERR_INVALID_ARG;
    if (scores_kept && !scores) return TG_ERR_INVALID_ARG;
    if (pos_kept && (n_seqs < 1 || !cu_seqlens || !cu_kept)) return TG_ERR_INVALID_ARG;
    return TG_OK;
}

// Device address of the current device's `scratch` array (resolved on the
// device's first call, then cached; threads that race here store the same
// address).
int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return TG_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TG_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return TG_OK;
}

// ------------------------------------------------------------ TG_DEBUG ----
// With TG_DEBUG=1 in the environment (read at every call), the entry points
// that take device metadata copy it to the host (synchronising `stream`) and
// check what the kernels otherwise trust; a violation returns
// TG_ERR_INVALID_ARG before anything is launched.
bool debug_on() {
    const char* e = getenv("TG_DEBUG");
    return e && e[0] == '1' && e[1] == 0;
}

bool fetch_i32(const int32_t* dev, int64_t n, std::vector<int32_t>& h, void* stream) {
    h.assign((size_t)std::max<int64_t>(n, 0), 0);
    if (n <= 0) return true;
    if (!dev) return false;
    if (hipMemcpyAsync(h.data(), dev, (size_t)n * 4, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
        return false;
    return hipStreamSynchronize((hipStream_t)stream) == hipSuccess;
}

// offsets[0] == 0, non-decreasing, offsets[S] == total, every span <= max_len
bool offsets_ok(const std::vector<int32_t>& cu, int32_t n_seqs, int64_t total, int64_t max_len) {
    if ((int64_t)cu.size() != (int64_t)n_seqs + 1 || cu[0] != 0 || cu[n_seqs] != total) return false;
    for (int32_t s = 0; s < n_seqs; ++s)
        if (cu[s + 1] < cu[s] || (int64_t)cu[s + 1] - cu[s] > max_len) return false;
    return true;
}

// The selector's metadata: spans inside their sequences, budgets >= 0, and
// cu_kept equal to tg_kept_counts of the rest.
int debug_check_select(int32_t n_seqs, int64_t n_tokens, int32_t max_seqlen, const int32_t* cu_seqlens,
                       const int32_t* doc_begin, const int32_t* doc_end, const int32_t* k_doc,
                       const int32_t* cu_kept, int64_t n_kept_total, void* stream) {
    std::vector<int32_t> cu, b, e, k, ck, ref(n_seqs + 1);
    if (!fetch_i32(cu_seqlens, n_seqs + 1, cu, stream) || !fetch_i32(doc_begin, n_seqs, b, stream) ||
        !fetch_i32(doc_end, n_seqs, e, stream) || !fetch_i32(k_doc, n_seqs, k, stream) ||
        !fetch_i32(cu_kept, n_seqs + 1, ck, stream))
        return TG_ERR_HIP;
    if (!offsets_ok(cu, n_seqs, n_tokens, max_seqlen)) return TG_ERR_INVALID_ARG;
    if (tg_kept_counts(n_seqs, cu.data(), b.data(), e.data(), k.data(), ref.data()) != TG_OK)
        return TG_ERR_INVALID_ARG;
    if (ref != ck || (n_kept_total >= 0 && ck[n_seqs] != n_kept_total)) return TG_ERR_INVALID_ARG;
    return TG_OK;
}

// kept_idx inside its sequence (so the gather never reads outside x) and
// ascending there.
int debug_check_kept(int32_t n_seqs, const int32_t* cu_seqlens, const int32_t* cu_kept, const int32_t* kept_idx,
                     int64_t n_kept_total, void* stream) {
    std::vector<int32_t> cu, ck, ki;
    if (!fetch_i32(cu_seqlens, n_seqs + 1, cu, stream) || !fetch_i32(cu_kept, n_seqs + 1, ck, stream) ||
        !fetch_i32(kept_idx, n_kept_total, ki, stream))
        return TG_ERR_HIP;
    if (cu.empty() || !offsets_ok(cu, n_seqs, cu.back(), INT32_MAX) || !offsets_ok(ck, n_seqs, n_kept_total, INT32_MAX))
        return TG_ERR_INVALID_ARG;
    for (int32_t s = 0; s < n_seqs; ++s)
        for (int32_t m = ck[s]; m < ck[s + 1]; ++m)
            if (ki[m] < cu[s] || ki[m] >= cu[s + 1] || (m > ck[s] && ki[m] <= ki[m - 1])) return TG_ERR_INVALID_ARG;
    return TG_OK;
}

// The attention's metadata: cu_kept offsets of n_kept_total rows with no
// sequence above max_kept_seqlen (when given), positions >= 0 and strictly
// increasing within each sequence (the kernels take causality from the kept
// order).
int debug_check_attn(int32_t n_seqs, int64_t n_kept_total, int32_t max_kept_seqlen, const int32_t* cu_kept,
                     const int32_t* pos, void* stream) {
    std::vector<int32_t> ck, ps;
    if (!fetch_i32(cu_kept, n_seqs + 1, ck, stream)) return TG_ERR_HIP;
    if (!offsets_ok(ck, n_seqs, n_kept_total, max_kept_seqlen >= 0 ? max_kept_seqlen : INT32_MAX))
        return TG_ERR_INVALID_ARG;
    if (pos) {
        if (!fetch_i32(pos, n_kept_total, ps, stream)) return TG_ERR_HIP;
        for (int32_t s = 0; s < n_seqs; ++s)
            for (int32_t m = ck[s]; m < ck[s + 1]; ++m)
                if (ps[m] < 0 || (m > ck[s] && ps[m] <= ps[m - 1])) return TG_ERR_INVALID_ARG;
    }
    return TG_OK;
}

}  // namespace

extern "C" {

const char* tg_status_string(int status) {
    switch (status) {
        case TG_OK: return "TG_OK";
        case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG";
        case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
        case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE";
        case TG_ERR_HIP: return "TG_ERR_HIP";
        default: return "TG_ERR_UNKNOWN";
    }
}

int tg_kept_counts(int32_t n_seqs, const int32_t* cu_seqlens_h, const int32_t* doc_begin_h,
                   const int32_t* doc_end_h, const int32_t* k_doc_h, int32_t* cu_kept_h) {
    if (n_seqs < 0 || !cu_seqlens_h || !cu_kept_h) return TG_ERR_INVALID_ARG;
    if (n_seqs > 0 && (!doc_begin_h || !doc_end_h || !k_doc_h)) return TG_ERR_INVALID_ARG;
    if (cu_seqlens_h[0] != 0) return TG_ERR_INVALID_ARG;
    int64_t acc = 0;
    cu_kept_h[0] = 0;
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int64_t n = (int64_t)cu_seqlens_h[s + 1] - cu_seqlens_h[s];
        const int32_t b = doc_begin_h[s], e = doc_end_h[s], k = k_doc_h[s];
        if (n < 0 || b < 0 || b > e || e > n || k < 0) return TG_ERR_INVALID_ARG;
        const int64_t nd = e - b;
        acc += (k < nd ? k : nd) + (n - nd);
        if (acc > INT32_MAX) return TG_ERR_INVALID_ARG;
        cu_kept_h[s + 1] = (int32_t)acc;
    }
    return TG_OK;
}

int tg_random_budgets(uint64_t seed, int32_t n_seqs, const int32_t* doc_begin_h, const int32_t* doc_end_h,
                      int32_t* k_doc_h) {
    if (n_seqs < 0) return TG_ERR_INVALID_ARG;
    if (n_seqs > 0 && (!doc_begin_h || !doc_end_h || !k_doc_h)) return TG_ERR_INVALID_ARG;
    for (int32_t s = 0; s < n_seqs; ++s)
        if (doc_begin_h[s] < 0 || doc_end_h[s] < doc_begin_h[s]) return TG_ERR_INVALID_ARG;
    for (int32_t s = 0; s < n_seqs; ++s) {
        // SplitMix64 output s: the finalizer of seed + (s + 1) * golden-ratio increment
        uint64_t z = seed + (uint64_t)(s + 1) * 0x9E3779B97F4A7C15ull;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        const uint64_t n = (uint64_t)(doc_end_h[s] - doc_begin_h[s]) + 1;
        k_doc_h[s] = (int32_t)(((unsigned __int128)(z >> 11) * n) >> 53);
    }
    return TG_OK;
}

int tg_gate_score(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d_model,
                  int64_t x_row_stride, const void* w1, const float* b1, const float* w2,
                  float b2, int32_t d_hid, float* scores, void* stream) {
    const int st = gate_check(x, x_dtype, n_tokens, d_model, x_row_stride, w1, w2, b2, d_hid, scores);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    return gate_launch(x, x_dtype, n_tokens, d_model, x_row_stride, w1, b1, w2, b2, d_hid, scores, stream);
}

size_t tg_topk_workspace_bytes(int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen) {
    if (n_seqs < 0 || n_tokens_total < 0 || max_seqlen < 0) return 0;
    return topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen);
}

int tg_topk_select(const float* scores, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                   const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                   const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx,
                   void* workspace, size_t workspace_bytes, void* stream) {
    const int st = topk_check(scores, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc,
                              cu_kept, kept_idx, workspace, workspace_bytes);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    if (debug_on())
        if (const int e = debug_check_select(n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                                             k_doc, cu_kept, -1, stream))
            return e;
    return launch_topk(scores, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                       k_doc, cu_kept, kept_idx, workspace, (hipStream_t)stream);
}

size_t tg_topk_noalloc_max_bytes(void) { return kScratchBytes; }

int tg_topk_select_noalloc(const float* scores, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                           const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                           const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx, void* stream) {
    if (n_seqs < 0 || n_tokens_total < 0 || n_tokens_total > INT32_MAX || max_seqlen < 0 ||
        max_seqlen > n_tokens_total)
        return TG_ERR_INVALID_ARG;
    if (max_seqlen > topk_max_seqlen()) return TG_ERR_UNSUPPORTED;
    if (topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen) > kScratchBytes) return TG_ERR_UNSUPPORTED;
    if (n_seqs == 0 || n_tokens_total == 0) return TG_OK;
    if (!cu_seqlens || !doc_begin || !doc_end || !k_doc || !cu_kept || !kept_idx || !scores)
        return TG_ERR_INVALID_ARG;
    if (debug_on())
        if (const int e = debug_check_select(n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                                             k_doc, cu_kept, -1, stream))
            return e;
    void* ws = nullptr;
    if (const int e = scratch_ptr(&ws)) return e;
    return launch_topk(scores, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept,
                       kept_idx, ws, (hipStream_t)stream);
}

size_t tg_random_k_workspace_bytes(int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen) {
    if (n_seqs < 0 || n_tokens_total < 0 || max_seqlen < 0) return 0;
    return random_k_workspace_bytes(n_seqs, n_tokens_total, max_seqlen);
}

int tg_random_k_select(uint64_t seed, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                       const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                       const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (n_seqs < 0 || n_tokens_total < 0 || n_tokens_total > INT32_MAX || max_seqlen < 0 ||
        max_seqlen > n_tokens_total)
        return TG_ERR_INVALID_ARG;
    if (max_seqlen > topk_max_seqlen()) return TG_ERR_UNSUPPORTED;
    if (n_seqs == 0 || n_tokens_total == 0) return TG_OK;
    if (!cu_seqlens || !doc_begin || !doc_end || !k_doc || !cu_kept || !kept_idx) return TG_ERR_INVALID_ARG;
    const size_t need = random_k_workspace_bytes(n_seqs, n_tokens_total, max_seqlen);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return TG_ERR_WORKSPACE;
    if (debug_on())
        if (const int e = debug_check_select(n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                                             k_doc, cu_kept, -1, stream))
            return e;
    return launch_random_k(seed, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc,
                           cu_kept, kept_idx, workspace, (hipStream_t)stream);
}

int tg_gather_kept(const void* x, int32_t x_dtype, int32_t d_model, int64_t x_row_stride,
                   const float* scores, const int32_t* kept_idx, int64_t n_kept_total,
                   int32_t n_seqs, const int32_t* cu_seqlens, const int32_t* cu_kept,
                   void* x_kept, float* scores_kept, int32_t* pos_kept, void* stream) {
    const int st = gather_check(x, x_dtype, d_model, x_row_stride, scores, kept_idx, n_kept_total, n_seqs,
                                cu_seqlens, cu_kept, x_kept, scores_kept, pos_kept);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    if (debug_on() && cu_seqlens && cu_kept)
        if (const int e = debug_check_kept(n_seqs, cu_seqlens, cu_kept, kept_idx, n_kept_total, stream)) return e;
    const int esize = x_dtype == TG_BF16 ? 2 : 4;
    return launch_gather(x, esize, d_model, x_row_stride, scores, kept_idx, n_kept_total, n_seqs,
                         cu_seqlens, cu_kept, x_kept, scores_kept, pos_kept, (hipStream_t)stream);
}

int tg_gated_select(const void* x, int32_t x_dtype, int64_t n_tokens_total, int32_t d_model,
                    int64_t x_row_stride, const void* w1, const float* b1, const float* w2, float b2,
                    int32_t d_hid, int32_t n_seqs, int32_t max_seqlen, const int32_t* cu_seqlens,
                    const int32_t* doc_begin, const int32_t* doc_end, const int32_t* k_doc,
                    const int32_t* cu_kept, int64_t n_kept_total, float* scores, int32_t* kept_idx,
                    void* x_kept, float* scores_kept, int32_t* pos_kept, void* workspace,
                    size_t workspace_bytes, void* stream) {
    // every stage is validated before the first launch
    const int sg = gate_check(x, x_dtype, n_tokens_total, d_model, x_row_stride, w1, w2, b2, d_hid, scores);
    if (sg != TG_OK && sg != -1) return sg;
    const int stk = topk_check(scores, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                               k_doc, cu_kept, kept_idx, workspace, workspace_bytes);
    if (stk != TG_OK && stk != -1) return stk;
    const int sga = gather_check(x, x_dtype, d_model, x_row_stride, scores, kept_idx, n_kept_total, n_seqs,
                                 cu_seqlens, cu_kept, x_kept, scores_kept, pos_kept);
    if (sga != TG_OK && sga != -1) return sga;
    if (debug_on() && stk == TG_OK)
        if (const int e = debug_check_select(n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                                             k_doc, cu_kept, n_kept_total, stream))
            return e;
    // where the selector needs counters zeroed first, the bf16 gate does it,
    // so the selector launches no clear kernel
    SelZero sz{};
    const bool gate_zeroes = sg == TG_OK && stk == TG_OK && x_dtype == TG_BF16 &&
                             topk_sel_zero(n_seqs, n_tokens_total, max_seqlen, doc_begin, doc_end, k_doc, workspace,
                                           &sz);
    if (sg == TG_OK) {
        const int st = gate_launch(x, x_dtype, n_tokens_total, d_model, x_row_stride, w1, b1, w2, b2, d_hid,
                                   scores, stream, gate_zeroes ? &sz : nullptr);
        if (st != TG_OK) return st;
    }
    if (stk == TG_OK) {
        const int st = launch_topk(scores, n_seqs, n_tokens_total, max_seqlen, cu_seqlens, doc_begin, doc_end,
                                   k_doc, cu_kept, kept_idx, workspace, (hipStream_t)stream, gate_zeroes);
        if (st != TG_OK) return st;
    }
    if (sga == TG_OK) {
        const int esize = x_dtype == TG_BF16 ? 2 : 4;
        return launch_gather(x, esize, d_model, x_row_stride, scores, kept_idx, n_kept_total, n_seqs, cu_seqlens,
                             cu_kept, x_kept, scores_kept, pos_kept, (hipStream_t)stream);
    }
    return TG_OK;
}

size_t tg_attn_workspace_bytes(int32_t n_seqs, int64_t n_kept_total, int32_t n_kv_heads,
                               int32_t head_dim) {
    if (n_seqs < 0 || n_kept_total < 0 || n_kv_heads <= 0 || head_dim <= 0) return 0;
    return attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, nullptr, nullptr,
                                 nullptr);
}

}  // extern "C"

namespace {

// Checks shared by the attention entry points; q-side checks only when q_side.
int attn_check(bool q_side, const void* q, int64_t q_row_stride, int32_t max_kept_seqlen,
               int32_t n_q_heads, float tau, const void* out, int64_t kv_row_stride,
               int32_t n_seqs, int64_t n_kept_total, int32_t n_kv_heads, int32_t head_dim,
               double rope_base, const void* workspace, size_t workspace_bytes) {
    if (!isfinite(rope_base)) return TG_ERR_INVALID_ARG;
    if (n_seqs < 0 || n_kept_total < 0 || n_kept_total > INT32_MAX) return TG_ERR_INVALID_ARG;
    if (n_kv_heads <= 0) return TG_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
    if (q_side) {
        if (!(tau > 0.0f) || !isfinite(tau) || max_kept_seqlen < 0) return TG_ERR_INVALID_ARG;
        if (n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
        const int grp = n_q_heads / n_kv_heads;
        if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return TG_ERR_UNSUPPORTED;
        if (q_row_stride < (int64_t)n_q_heads * head_dim || q_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    } else {
        if (kv_row_stride < (int64_t)n_kv_heads * head_dim || kv_row_stride % 8 != 0)
            return TG_ERR_INVALID_ARG;
    }
    if (n_kept_total == 0) return -1;   // valid, nothing to do
    if (n_seqs < 1) return TG_ERR_INVALID_ARG;
    if (q_side) {
        if (max_kept_seqlen < 1 || max_kept_seqlen > n_kept_total) return TG_ERR_INVALID_ARG;
        if (!q || !out || !aligned16(q) || !aligned16(out)) return TG_ERR_INVALID_ARG;
    }
    const size_t need = attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, nullptr,
                                              nullptr, nullptr);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
        return TG_ERR_WORKSPACE;
    return TG_OK;
}

// Under TG_DEBUG, a call that reads a prepared cache first compares the
// header the pre-pass left in it with its own arguments: the sizes, the rotary
// base and a hash of cu_kept must be those the cache was prepared with.
int debug_check_cache(const void* cache, int32_t n_seqs, int64_t n_kept_total, int32_t n_kv_heads,
                      int32_t head_dim, double rope_base, const int32_t* cu_kept, void* stream) {
    size_t off_hdr = 0;
    attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, nullptr, nullptr, nullptr, nullptr,
                          &off_hdr);
    CacheHeader h{};
    if (hipMemcpyAsync(&h, (const char*)cache + off_hdr, sizeof h, hipMemcpyDeviceToHost, (hipStream_t)stream) !=
        hipSuccess)
        return TG_ERR_HIP;
    std::vector<int32_t> ck;
    if (!fetch_i32(cu_kept, (int64_t)n_seqs + 1, ck, stream)) return TG_ERR_HIP;   // synchronises the stream
    uint64_t hash = 0;
    for (int64_t i = 0; i <= n_seqs; ++i) hash += cu_hash_term(ck[(size_t)i], i);
    const bool rope = rope_base > 0.0;
    if (h.magic != kCacheMagic || h.n_seqs != n_seqs || h.m_tot != n_kept_total || h.hkv != n_kv_heads ||
        h.d != head_dim || (h.rope_base > 0.0) != rope || (rope && h.rope_base != rope_base) || h.cu_hash != hash)
        return TG_ERR_INVALID_ARG;
    return TG_OK;
}

void attn_fill(AttnArgs& a, int32_t n_seqs, int64_t n_kept_total, int32_t n_kv_heads,
               int32_t head_dim, double rope_base, const void* workspace) {
    size_t off_k, off_vt, off_cs, off_split, off_hdr;
    attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, &off_k, &off_vt, &off_cs, &off_split,
                          &off_hdr);
    a.ws_hdr = (CacheHeader*)((char*)workspace + off_hdr);
    a.rope_base = rope_base;
    a.n_seqs = n_seqs;
    a.m_tot = n_kept_total;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.rope = rope_base > 0.0;
    a.rope_log2_base = a.rope ? log2(rope_base) : 0.0;
    char* ws = (char*)workspace;
    a.ws_k = (bf16*)(ws + off_k);
    a.ws_vt = (bf16*)(ws + off_vt);
    a.ws_cs = (float2*)(ws + off_cs);
    a.mp = attn_padded_rows(n_seqs, n_kept_total);
    a.ws_tk = off_split ? (uint32_t*)(ws + off_split) : nullptr;
    a.ws_part = off_split ? (float*)(ws + off_split + (((size_t)kSplitCap * 4 + 255) & ~(size_t)255)) : nullptr;
}

}  // namespace

extern "C" {

int tg_attn_prepare(const void* k, const void* v, int64_t kv_row_stride, const float* key_score,
                    const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs, int64_t n_kept_total,
                    int32_t n_kv_heads, int32_t head_dim, double rope_base, void* workspace,
                    size_t workspace_bytes, void* stream) {
    const int st = attn_check(false, nullptr, 0, 0, 0, 1.0f, nullptr, kv_row_stride, n_seqs,
                              n_kept_total, n_kv_heads, head_dim, rope_base, workspace, workspace_bytes);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    if (!k || !v || !key_score || !pos || !cu_kept || !aligned16(k) || !aligned16(v)) return TG_ERR_INVALID_ARG;
    if (debug_on())
        if (const int e = debug_check_attn(n_seqs, n_kept_total, -1, cu_kept, pos, stream)) return e;
    AttnArgs a{};
    attn_fill(a, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, workspace);
    a.k = (const bf16*)k;
    a.v = (const bf16*)v;
    a.kv_stride = kv_row_stride;
    a.key_score = key_score;
    a.pos = pos;
    a.cu_kept = cu_kept;
    return launch_attn_prep(a, (hipStream_t)stream);
}

int tg_attn_forward(const void* q, int64_t q_row_stride, const float* head_gain, float tau,
                    const int32_t* cu_kept, int32_t n_seqs, int64_t n_kept_total,
                    int32_t max_kept_seqlen, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    double rope_base, void* out, float* lse, const void* workspace,
                    size_t workspace_bytes, void* stream) {
    const int st = attn_check(true, q, q_row_stride, max_kept_seqlen, n_q_heads, tau, out, 0, n_seqs,
                              n_kept_total, n_kv_heads, head_dim, rope_base, workspace, workspace_bytes);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    if (!head_gain || !cu_kept) return TG_ERR_INVALID_ARG;
    if (debug_on()) {
        if (const int e = debug_check_attn(n_seqs, n_kept_total, max_kept_seqlen, cu_kept, nullptr, stream)) return e;
        if (const int e = debug_check_cache(workspace, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, cu_kept,
                                            stream))
            return e;
    }
    AttnArgs a{};
    attn_fill(a, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, workspace);
    a.q = (const bf16*)q;
    a.q_stride = q_row_stride;
    a.gain = head_gain;
    a.qk_scale_log2 = (float)(1.4426950408889634 / (sqrt((double)head_dim) * (double)tau));
    a.cu_kept = cu_kept;
    a.max_kept_seqlen = max_kept_seqlen;
    a.hq = n_q_heads;
    a.out = (bf16*)out;
    a.lse = lse;
    return launch_attn_fwd(a, (hipStream_t)stream);
}

int tg_keybias_attn_prefill(const void* q, const void* k, const void* v, int64_t q_row_stride,
                            int64_t kv_row_stride, const float* key_score, const float* head_gain,
                            float tau, const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs,
                            int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, double rope_base, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    // validate both halves before launching either
    int st = attn_check(false, nullptr, 0, 0, 0, 1.0f, nullptr, kv_row_stride, n_seqs, n_kept_total,
                        n_kv_heads, head_dim, rope_base, workspace, workspace_bytes);
    if (st == TG_OK || st == -1)
        st = attn_check(true, q, q_row_stride, max_kept_seqlen, n_q_heads, tau, out, 0, n_seqs,
                        n_kept_total, n_kv_heads, head_dim, rope_base, workspace, workspace_bytes);
    if (st == -1) return TG_OK;
    if (st != TG_OK) return st;
    if (!k || !v || !key_score || !pos || !cu_kept || !head_gain || !aligned16(k) || !aligned16(v))
        return TG_ERR_INVALID_ARG;
    st = tg_attn_prepare(k, v, kv_row_stride, key_score, pos, cu_kept, n_seqs, n_kept_total, n_kv_heads,
                         head_dim, rope_base, workspace, workspace_bytes, stream);
    if (st != TG_OK) return st;
    return tg_attn_forward(q, q_row_stride, head_gain, tau, cu_kept, n_seqs, n_kept_total,
                           max_kept_seqlen, n_q_heads, n_kv_heads, head_dim, rope_base, out, lse,
                           workspace, workspace_bytes, stream);
}

size_t tg_attn_decode_workspace_bytes(int32_t n_seqs, int32_t max_kept_seqlen, int32_t n_q_heads,
                                      int32_t head_dim) {
    if (n_seqs < 0 || max_kept_seqlen < 0 || n_q_heads <= 0 || (head_dim != 64 && head_dim != 128)) return 0;
    return decode_workspace_bytes(n_seqs, max_kept_seqlen, n_q_heads, head_dim);
}

int tg_attn_decode(const void* q, int64_t q_row_stride, const int32_t* q_pos, const float* head_gain,
                   float tau, const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs,
                   int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_base, const void* cache, size_t cache_bytes, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (!isfinite(rope_base)) return TG_ERR_INVALID_ARG;
    if (n_seqs < 0 || n_kept_total < 0 || n_kept_total > INT32_MAX) return TG_ERR_INVALID_ARG;
    if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
    const int grp = n_q_heads / n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return TG_ERR_UNSUPPORTED;
    if (!(tau > 0.0f) || !isfinite(tau)) return TG_ERR_INVALID_ARG;
    if (q_row_stride < (int64_t)n_q_heads * head_dim) return TG_ERR_INVALID_ARG;
    if (max_kept_seqlen < 0 || max_kept_seqlen > n_kept_total || (n_kept_total > 0 && max_kept_seqlen < 1))
        return TG_ERR_INVALID_ARG;
    if (n_seqs == 0 && n_kept_total > 0) return TG_ERR_INVALID_ARG;   // kept keys but no sequence
    if (n_seqs == 0) return TG_OK;
    if (!q || !q_pos || !head_gain || !cu_kept || !out || (n_kept_total > 0 && !pos)) return TG_ERR_INVALID_ARG;
    if (debug_on())
        if (const int e = debug_check_attn(n_seqs, n_kept_total, max_kept_seqlen, cu_kept, pos, stream)) return e;
    const size_t cache_need = attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, nullptr,
                                                    nullptr, nullptr);
    if (!cache || cache_bytes < cache_need || ((uintptr_t)cache & 255u) != 0) return TG_ERR_WORKSPACE;
    const size_t need = decode_workspace_bytes(n_seqs, max_kept_seqlen, n_q_heads, head_dim);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return TG_ERR_WORKSPACE;
    if (debug_on())
        if (const int e = debug_check_cache(cache, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, cu_kept,
                                            stream))
            return e;
    const int64_t mp = attn_padded_rows(n_seqs, n_kept_total);
    // buffer offsets into one head's K' rows ((D+16)*2 B each) stay 32-bit
    if ((int64_t)(head_dim + 16) * 2 * mp >= ((int64_t)1 << 32)) return TG_ERR_UNSUPPORTED;
    size_t off_k, off_vt, off_cs;
    attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, &off_k, &off_vt, &off_cs);
    DecodeArgs a{};
    a.q = (const bf16*)q;
    a.q_stride = q_row_stride;
    a.q_pos = q_pos;
    a.gain = head_gain;
    a.qk_scale_log2 = (float)(1.4426950408889634 / (sqrt((double)head_dim) * (double)tau));
    a.pos = pos;
    a.cu_kept = cu_kept;
    a.n_seqs = n_seqs;
    a.m_tot = n_kept_total;
    a.max_kept_seqlen = max_kept_seqlen;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.rope = rope_base > 0.0;
    a.rope_log2_base = a.rope ? log2(rope_base) : 0.0;
    a.ws_k = (const bf16*)((const char*)cache + off_k);
    a.ws_vt = (const bf16*)((const char*)cache + off_vt);
    a.mp = mp;
    a.out = (bf16*)out;
    a.lse = lse;
    a.ws = workspace;
    return launch_attn_decode(a, (hipStream_t)stream);
}

}  // extern "C"

extern "C" {

size_t tg_attn_gate_grads_workspace_bytes(int32_t n_seqs, int64_t n_kept_total, int32_t max_kept_seqlen,
                                          int32_t n_q_heads, int32_t head_dim) {
    if (n_seqs < 0 || n_kept_total < 0 || max_kept_seqlen < 0 || n_q_heads <= 0 ||
        (head_dim != 64 && head_dim != 128))
        return 0;
    return bwd_workspace_bytes(n_seqs, n_kept_total, max_kept_seqlen, n_q_heads, head_dim);
}

int tg_attn_gate_grads(const void* q, int64_t q_row_stride, const void* v, int64_t kv_row_stride,
                       const float* key_score, const float* head_gain, float tau, const int32_t* cu_kept,
                       int32_t n_seqs, int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, double rope_base, const void* out,
                       const float* lse, const void* d_out, int64_t d_out_row_stride, const void* cache,
                       size_t cache_bytes, float* d_score, float* d_gain, float* d_tau, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!isfinite(rope_base)) return TG_ERR_INVALID_ARG;
    if (n_seqs < 0 || n_kept_total < 0 || n_kept_total > INT32_MAX) return TG_ERR_INVALID_ARG;
    if (n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return TG_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return TG_ERR_UNSUPPORTED;
    const int grp = n_q_heads / n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return TG_ERR_UNSUPPORTED;
    if (!(tau > 0.0f) || !isfinite(tau)) return TG_ERR_INVALID_ARG;
    if (q_row_stride < (int64_t)n_q_heads * head_dim || q_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    if (kv_row_stride < (int64_t)n_kv_heads * head_dim || kv_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    if (d_out_row_stride < (int64_t)n_q_heads * head_dim || d_out_row_stride % 8 != 0) return TG_ERR_INVALID_ARG;
    if (max_kept_seqlen < 0 || max_kept_seqlen > n_kept_total || (n_kept_total > 0 && max_kept_seqlen < 1))
        return TG_ERR_INVALID_ARG;
    if (!d_gain || !d_tau) return TG_ERR_INVALID_ARG;
    if (n_seqs == 0 && n_kept_total > 0) return TG_ERR_INVALID_ARG;   // kept tokens but no sequence
    if (n_seqs == 0 || n_kept_total == 0) {
        // no causal pair: every gradient is zero
        return launch_gate_grads_zero(n_q_heads, d_gain, d_tau, (hipStream_t)stream);
    }
    if (!q || !v || !key_score || !head_gain || !cu_kept || !out || !lse || !d_out || !d_score)
        return TG_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(v) || !aligned16(out) || !aligned16(d_out)) return TG_ERR_INVALID_ARG;
    if (debug_on())
        if (const int e = debug_check_attn(n_seqs, n_kept_total, max_kept_seqlen, cu_kept, nullptr, stream)) return e;
    const size_t cache_need = attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, nullptr,
                                                    nullptr, nullptr);
    if (!cache || cache_bytes < cache_need || ((uintptr_t)cache & 255u) != 0) return TG_ERR_WORKSPACE;
    const size_t need = bwd_workspace_bytes(n_seqs, n_kept_total, max_kept_seqlen, n_q_heads, head_dim);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) return TG_ERR_WORKSPACE;
    if (debug_on())
        if (const int e = debug_check_cache(cache, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, cu_kept,
                                            stream))
            return e;
    const int64_t mp = attn_padded_rows(n_seqs, n_kept_total);
    // buffer offsets into one head's prepared rows stay 32-bit
    if ((int64_t)(head_dim + 16) * 2 * mp >= ((int64_t)1 << 32)) return TG_ERR_UNSUPPORTED;
    size_t off_k, off_vt, off_cs;
    attn_workspace_layout(n_seqs, n_kept_total, n_kv_heads, head_dim, &off_k, &off_vt, &off_cs);
    BwdArgs a{};
    a.q = (const bf16*)q;
    a.q_stride = q_row_stride;
    a.v = (const bf16*)v;
    a.kv_stride = kv_row_stride;
    a.o = (const bf16*)out;
    a.lse = lse;
    a.dout = (const bf16*)d_out;
    a.do_stride = d_out_row_stride;
    a.key_score = key_score;
    a.gain = head_gain;
    a.tau = tau;
    a.qk_scale_log2 = (float)(1.4426950408889634 / (sqrt((double)head_dim) * (double)tau));
    a.cu_kept = cu_kept;
    a.n_seqs = n_seqs;
    a.m_tot = n_kept_total;
    a.max_kept_seqlen = max_kept_seqlen;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.rope = rope_base > 0.0;
    a.ws_k = (const bf16*)((const char*)cache + off_k);
    a.ws_cs = (const float2*)((const char*)cache + off_cs);
    a.mp = mp;
    a.d_score = d_score;
    a.d_gain = d_gain;
    a.d_tau = d_tau;
    a.ws = workspace;
    return launch_attn_gate_grads(a, (hipStream_t)stream);
}

}  // extern "C"
