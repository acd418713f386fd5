// Shared types and helpers of the libtokengate kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tokengate.h"

namespace tg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-sequence counters that the top-K's four-launch form needs zeroed before
// its histogram pass: `words` uint32 at base + s * stride for every sequence s
// that selects (0 < min(k_doc, n_doc) < n_doc).  In tg_gated_select the gate's
// workgroups zero them at their start, so the selector launches no clear
// kernel.  base == nullptr: nothing to zero.
struct SelZero {
    uint32_t* base;
    int64_t stride;
    int words;
    const int* db;
    const int* de;
    const int* kd;
    int n_seqs;
};

__device__ __host__ __forceinline__ bool seq_selects(int db, int de, int kd) {
    const int nd = de - db;
    const int k = kd < nd ? kd : nd;
    return k > 0 && k < nd;
}

// Launchers, one per kernel family.  Each returns TG_OK or TG_ERR_HIP.
int launch_gate_bf16(const bf16* x, int64_t n, int d_model, int64_t x_stride, const bf16* w1,
                     const float* b1, const float* w2, float b2, int d_hid, float* scores,
                     hipStream_t st, const SelZero* zero = nullptr);
int launch_gate_f32(const float* x, int64_t n, int d_model, int64_t x_stride, const float* w1,
                    const float* b1, const float* w2, float b2, int d_hid, float* scores,
                    hipStream_t st);
size_t topk_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen);
int topk_max_seqlen();
// counters_zeroed: the counters of topk_sel_zero are already zero (the gate
// cleared them), so the four-launch form skips its clear kernel.
int launch_topk(const float* scores, int n_seqs, int64_t n_tokens, int max_seqlen,
                const int* cu_seqlens, const int* doc_begin, const int* doc_end, const int* k_doc,
                const int* cu_kept, int* kept_idx, void* ws, hipStream_t st, bool counters_zeroed = false);
// Whether the selector for this batch needs counters zeroed beforehand, and
// where they are in ws (false: it needs none).
bool topk_sel_zero(int n_seqs, int64_t n_tokens, int max_seqlen, const int* doc_begin, const int* doc_end,
                   const int* k_doc, void* ws, SelZero* out);
size_t random_k_workspace_bytes(int n_seqs, int64_t n_tokens, int max_seqlen);
int launch_random_k(uint64_t seed, int n_seqs, int64_t n_tokens, int max_seqlen, const int* cu_seqlens,
                    const int* doc_begin, const int* doc_end, const int* k_doc, const int* cu_kept,
                    int* kept_idx, void* ws, hipStream_t st);
int launch_gather(const void* x, int esize, int d_model, int64_t x_stride, const float* scores,
                  const int* kept_idx, int64_t m_tot, int n_seqs, const int* cu_seqlens,
                  const int* cu_kept, void* x_kept, float* s_kept, int* pos_kept, hipStream_t st);

// What the pre-pass prepared, in the last 256 B of the workspace: the calls
// that read the cache compare it with their own arguments under TG_DEBUG.
struct CacheHeader {
    uint32_t magic;
    int32_t n_seqs, hkv, d;
    int64_t m_tot;
    double rope_base;
    uint64_t cu_hash;   // sum over i of cu_hash_term(cu_kept[i], i), mod 2^64
};
constexpr uint32_t kCacheMagic = 0x4b564754u;
__host__ __device__ __forceinline__ uint64_t cu_hash_term(int32_t x, int64_t i) {
    return ((uint64_t)(uint32_t)x + 1u) * (2u * (uint64_t)i + 1u) * 0x9E3779B97F4A7C15ull;
}

struct AttnArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    int64_t q_stride, kv_stride;
    const float* key_score;
    const float* gain;
    float qk_scale_log2;   // log2(e) / (sqrt(D) * tau)
    const int* pos;
    const int* cu_kept;
    int n_seqs;
    int64_t m_tot;
    int max_kept_seqlen;
    int hq, hkv, d;
    double rope_log2_base;  // log2(rope base); <= -1e300 when rotary embedding is off
    bool rope;
    bf16* out;
    float* lse;
    // workspace carve-up
    bf16* ws_k;       // [Hkv][Mp][D]  rotated keys, per-sequence padded rows
    bf16* ws_vt;      // [Hkv][D][Mp]  values, transposed
    float2* ws_cs;    // [M][D/2]      (cos, sin) per kept token and frequency
    int64_t mp;       // padded row count
    // key-split scratch (null when the workspace holds none): one ticket per
    // split query tile, zeroed by the pre-pass and left at zero by every
    // forward; one partial (O, offset, sum) slot per forward workgroup
    uint32_t* ws_tk;
    float* ws_part;
    CacheHeader* ws_hdr;
    double rope_base;
};
constexpr int kSplitCap = 512;   // workgroups of a key-split forward grid, at most

int64_t attn_padded_rows(int n_seqs, int64_t m_tot);
// off_split (optional): offset of the key-split scratch, 0 when none is reserved;
// off_hdr (optional): offset of the CacheHeader
size_t attn_workspace_layout(int n_seqs, int64_t m_tot, int hkv, int d, size_t* off_k,
                             size_t* off_vt, size_t* off_cs, size_t* off_split = nullptr,
                             size_t* off_hdr = nullptr);
int launch_attn_prep(const AttnArgs& a, hipStream_t st);
int launch_attn_fwd(const AttnArgs& a, hipStream_t st);

struct DecodeArgs {
    const bf16* q;          // [n_seqs] rows of [Hq][D], q_stride elements apart
    int64_t q_stride;
    const int* q_pos;       // [n_seqs] original position of each new query
    const float* gain;
    float qk_scale_log2;    // log2(e) / (sqrt(D) * tau)
    const int* pos;         // [M] kept positions
    const int* cu_kept;
    int n_seqs;
    int64_t m_tot;
    int max_kept_seqlen;
    int hq, hkv, d;
    double rope_log2_base;
    bool rope;
    const bf16* ws_k;       // the prepared cache (see AttnArgs)
    const bf16* ws_vt;
    int64_t mp;
    bf16* out;              // [n_seqs][Hq][D]
    float* lse;             // [Hq][n_seqs] or null
    void* ws;               // decode partials
};
struct BwdArgs {
    const bf16* q;          // [M] rows of [Hq][D], q_stride elements apart
    int64_t q_stride;
    const bf16* v;          // [M] rows of [Hkv][D], kv_stride elements apart
    int64_t kv_stride;
    const bf16* o;          // forward output [M][Hq][D]
    const float* lse;       // forward LSE [Hq][M] (natural log)
    const bf16* dout;       // [M] rows of [Hq][D], do_stride elements apart
    int64_t do_stride;
    const float* key_score; // [M]
    const float* gain;      // [Hq]
    float tau;
    float qk_scale_log2;    // log2(e) / (sqrt(D) * tau)
    const int* cu_kept;
    int n_seqs;
    int64_t m_tot;
    int max_kept_seqlen;
    int hq, hkv, d;
    bool rope;
    const bf16* ws_k;       // the prepared cache (see AttnArgs)
    const float2* ws_cs;
    int64_t mp;
    float* d_score;         // [M]
    float* d_gain;          // [Hq]
    float* d_tau;           // [1]
    void* ws;
};
size_t bwd_workspace_bytes(int n_seqs, int64_t m_tot, int max_kept, int hq, int d);
int launch_attn_gate_grads(const BwdArgs& a, hipStream_t st);
int launch_gate_grads_zero(int hq, float* d_gain, float* d_tau, hipStream_t st);

int decode_chunks(int max_kept_seqlen);
size_t decode_part_o_bytes(int n_seqs, int max_kept_seqlen, int hq, int d);
size_t decode_workspace_bytes(int n_seqs, int max_kept_seqlen, int hq, int d);
int launch_attn_decode(const DecodeArgs& a, hipStream_t st);

// Raises `fn`'s dynamic LDS limit to `bytes` on the current device, once per
// device: `done` records the devices already set (devices past 63 are set on
// every call).  Concurrent first calls may both set the same value, which is
// harmless; the mask itself is atomic.
inline int set_dyn_lds_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_HIP;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return TG_OK;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return TG_ERR_HIP;
    if (bit) done.fetch_or(bit, std::memory_order_release);
    return TG_OK;
}

// Compute units of the current device, queried once per device (devices past
// 63 are queried on every call).
inline int device_cu_count(int* n_cu) {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TG_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *n_cu = c;
            return TG_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return TG_ERR_HIP;
    if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
    *n_cu = c;
    return TG_OK;
}

// Buffer resource over `bytes` bytes from `base` (raw, untyped 32-bit
// elements): reads at per-lane offsets beyond it return zero instead of
// faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct global -> LDS copy (buffer_load_dwordx4 ... lds): 16 B per lane from
// rsrc at byte offset voff + soff (soff wave-uniform) into LDS bytes
// [ldst + 16 lane, ldst + 16 lane + 16) (ldst wave-uniform).
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* ldst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)ldst, 16, (int)voff,
                                              (int)soff, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LDS / export counters left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (7 << 4) | (0xf << 8); }

// Wait until at most n (wave-uniform, 0..12) vector-memory operations remain.
__device__ __forceinline__ void wait_vm_le(int n) {
    switch (n) {
        case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
        case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
        case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
        case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
        case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
        case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
        case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
        case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
        case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
        case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
        case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
        default: __builtin_amdgcn_s_waitcnt(0); break;
    }
}

// Upper-bound search: the sequence s with cu[s] <= m < cu[s+1] (cu non-decreasing,
// cu[0] <= m < cu[n]).
__device__ __forceinline__ int find_seq(const int* __restrict__ cu, int n, int64_t m) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] <= m) lo = mid; else hi = mid;
    }
    return lo;
}

// First padded workspace row of kept sequence s: a multiple of 8 (16-byte
// aligned bf16 rows for vector loads), and sequences never overlap.
__device__ __host__ __forceinline__ int64_t padded_seq_start(int64_t cu_kept_s, int s) {
    return (cu_kept_s + 16 * (int64_t)s + 15) & ~(int64_t)15;
}

// Column of key row r in the V^T workspace: within every aligned group of 16
// keys the middle two quads are swapped (keys 4-7 <-> 8-11), which is the key
// order of the P^T operand taken straight from the S^T accumulators, so one
// 16-B LDS read gives a lane its whole A-operand slice.  An involution.
__device__ __host__ __forceinline__ int64_t vt_col(int64_t r) {
    return (r & ~(int64_t)12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

}  // namespace tg
