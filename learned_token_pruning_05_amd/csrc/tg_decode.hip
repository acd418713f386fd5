// One decode step of token-gated attention over the kept-only cache.
//
// TokenGate ([ES] "¿Qué es la atención con control de acceso por tokens…?"):
// above the gate layer only kept tokens have keys and values, and every kept
// key carries its gate-score bias.  A token generated after the prefill
// attends to that cache with the prefill's logit
//     l_j = <R(q, q_pos), R(k_j, pos_j)> / (sqrt(D) tau) + g_h s_j
// over the kept keys of its sequence with pos_j <= q_pos.
//
// The cache is the one tg_attn_prepare writes: rotated K' rows with the
// bias columns (s_hi, s_lo, s_hi, 1, 1) and V^T with its permuted columns.  One
// query per sequence makes this a matrix-vector product, so it is bound by
// reading the cache (K' (D+16) x 2 B + V^T D x 2 B per key and kv head), not by
// arithmetic: split over keys.  The split kernel gives each workgroup 64 keys
// of one kv head and all its q heads (GQA heads share the key and value
// reads): the tiles arrive by LDS-direct loads, logits and the P.V sums run
// in fp32 on the VALU, and each workgroup leaves an unnormalised partial
// (max, sum, O).  The combine kernel merges the partials of a sequence.
#include <math.h>

#include <algorithm>

#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kDecKeys = 64;       // keys per split workgroup
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxGrp = 8;      // q heads per kv head
constexpr int kDecMaxSub = 4;      // 64-key tiles per split workgroup

struct DecFreqs {
    double rev[64];   // base^(-2f/D) / (2 pi): turns of frequency f per position
};

template <int D>
struct DecLds {
    // rows padded by one 16-B chunk (odd pitch: the 16-B reads of 16
    // consecutive rows hit 16 distinct 4-bank groups); pad slots hold a
    // duplicate that is never read
    static constexpr int KD = D + 16;
    static constexpr int KCHUNK = KD / 8;
    static constexpr int KROW = KCHUNK + 1;
    static constexpr int VCHUNK = kDecKeys / 8;
    static constexpr int VROW = VCHUNK + 1;
    static constexpr int K_INSTR = kDecKeys * KROW / 64;   // 64-lane load instructions per tile
    static constexpr int V_INSTR = D * VROW / 64;
    static constexpr int KT = kDecKeys * KROW * 8;          // tile sizes in elements
    static constexpr int VT = D * VROW * 8;
    // ring slots: one when a workgroup streams a single tile, else two
    __host__ __device__ static int slots(int nsub) { return nsub > 1 ? 2 : 1; }
    static size_t smem(int grp, int nsub) {
        return (size_t)(slots(nsub) * KT + slots(nsub) * VT) * 2 + (size_t)grp * D * 4 + (size_t)grp * kDecKeys * 4 +
               (size_t)nsub * kDecKeys * 4 + (size_t)4 * grp * 4;
    }
    static_assert(kDecKeys * KROW % 64 == 0 && D * VROW % 64 == 0, "tiles must be whole load instructions");
};

template <int D>
__global__ __launch_bounds__(kDecThreads, 2) void attn_decode_split_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const int* __restrict__ q_pos,
    const float* __restrict__ gain, float qk_scale_log2, const int* __restrict__ pos,
    const int* __restrict__ cu_kept, int hq, int grp, int64_t mp, const bf16* __restrict__ ws_k,
    const bf16* __restrict__ ws_vt, DecFreqs fr, int rope, int nsub, int n_chunks, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
    using L = DecLds<D>;
    constexpr int HALF = D / 2;
    constexpr int KT = L::KT, VT = L::VT;                               // tile sizes (elements)
    constexpr int OPT = kDecMaxGrp * D / kDecThreads;                  // output items per thread (max)
    // dynamic LDS, sized for this launch's grp and nsub (two workgroups fit a CU)
    extern __shared__ __attribute__((aligned(16))) char dsm[];
    bf16* const ks = (bf16*)dsm;                       // [2][KT] K' ring
    bf16* const vs = ks + L::slots(nsub) * KT;         // [slots][VT] V^T ring
    float* const qs = (float*)(vs + L::slots(nsub) * VT);   // [grp][D] rotated, scaled queries
    float* const ts = qs + grp * D;                    // [grp][64] logits, then probabilities
    int* const pk = (int*)(ts + grp * kDecKeys);       // [nsub][64] key positions
    float* const gs = (float*)(pk + nsub * kDecKeys);  // [grp] g log2 e
    float* const mh = gs + grp;                        // [grp] running max
    float* const lh = mh + grp;                        // [grp] running sum
    float* const sc = lh + grp;                        // [grp] rescale factor of this tile
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int key_begin = chunk * nsub * kDecKeys;
    if (key_begin >= ms) return;   // the combine kernel reads only chunks that hold keys
    const int n_tiles = min(nsub, (ms - key_begin + kDecKeys - 1) / kDecKeys);
    const int h0 = hk * grp;
    const int qp = q_pos[s];

    // K' and V^T tiles straight into LDS through a two-slot ring.  Buffer
    // resources over this sequence's rows: reads past the cache return zeros.
    const int64_t prow0 = padded_seq_start(cs0, s);
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(ws_k + ((int64_t)hk * mp + prow0) * L::KD, (uint32_t)((mp - prow0) * L::KD * 2));
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(ws_vt + (int64_t)hk * D * mp + prow0, (uint32_t)(((int64_t)D * mp - prow0) * 2));
    auto load_tile = [&](int t, int slot) {
        const uint32_t key0 = (uint32_t)(key_begin + t * kDecKeys);
        for (int i = wave; i < L::K_INSTR; i += kDecWaves) {
            const int sl = i * 64 + lane;
            const int r = sl / L::KROW, c = sl % L::KROW;
            const uint32_t off = (uint32_t)((r * L::KD + (c < L::KCHUNK ? c : 0) * 8) * 2);
            lds_load16_buf(krs, off, key0 * (L::KD * 2), ks + slot * KT + i * 512);
        }
        for (int i = wave; i < L::V_INSTR; i += kDecWaves) {
            const int sl = i * 64 + lane;
            const int r = sl / L::VROW, c = sl % L::VROW;
            const uint32_t off = (uint32_t)(((uint32_t)r * (uint32_t)mp + (c < L::VCHUNK ? c : 0) * 8) * 2);
            lds_load16_buf(vrs, off, key0 * 2, vs + slot * VT + i * 512);
        }
    };
    // this wave's load instructions per tile (what may stay in flight)
    const int per_tile = (L::K_INSTR - wave + kDecWaves - 1) / kDecWaves + (L::V_INSTR - wave + kDecWaves - 1) / kDecWaves;
    // The chunk's key positions and the query elements are loaded before the
    // tile loads are issued, so they do not queue behind the tiles
    // (vector-memory counts retire in order: a load issued after the tiles
    // completes only after them).  A thread holds at most one position
    // (n_tiles * 64 <= kDecThreads) and two query items (grp * D / 2 <=
    // 2 kDecThreads).
    static_assert(kDecMaxSub * kDecKeys <= kDecThreads && kDecMaxGrp * D / 2 <= 2 * kDecThreads, "items per thread");
    const int pkey = key_begin + tid;
    const int pv = tid < n_tiles * kDecKeys && pkey < ms ? pos[cs0 + pkey] : INT32_MAX;
    float qa[2], qb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = tid + u * kDecThreads;
        qa[u] = qb[u] = 0.0f;
        if (it < grp * HALF) {
            const bf16* qr = q + (int64_t)s * q_stride + (int64_t)(h0 + it / HALF) * D;
            qa[u] = (float)qr[it % HALF];
            qb[u] = (float)qr[it % HALF + HALF];
        }
    }
    load_tile(0, 0);
    if (n_tiles > 1) load_tile(1, 1);

    // key positions of the chunk, and the rotated, scaled queries (fp32, not
    // rounded): item (head g, rotate-half pair f); the angle is reduced in fp64
    // to [-1/2, 1/2] turns and fed to the hardware sine and cosine
    if (tid < n_tiles * kDecKeys) pk[tid] = pv;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = tid + u * kDecThreads;
        if (it >= grp * HALF) break;
        const int g = it / HALF, f = it % HALF;
        const float a = qa[u], b = qb[u];
        float y1 = a, y2 = b;
        if (rope) {
            const double t = (double)qp * fr.rev[f];
            const float tr = (float)(t - rint(t));
            const float sn = __builtin_amdgcn_sinf(tr), cn = __builtin_amdgcn_cosf(tr);
            y1 = a * cn - b * sn;
            y2 = b * cn + a * sn;
        }
        qs[g * D + f] = y1 * qk_scale_log2;
        qs[g * D + f + HALF] = y2 * qk_scale_log2;
    }
    if (tid < grp) {
        gs[tid] = gain[h0 + tid] * kLog2e;
        mh[tid] = -INFINITY;
        lh[tid] = 0.0f;
    }
    float oacc[OPT];
#pragma unroll
    for (int j = 0; j < OPT; ++j) oacc[j] = 0.0f;

    for (int t = 0; t < n_tiles; ++t) {
        const int slot = t & 1;
        if (t + 1 < n_tiles) wait_vm_le(per_tile);   // tile t landed; tile t+1 may be in flight
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bf16* kt = ks + slot * KT;
        const bf16* vt = vs + slot * VT;
        // log2-domain logits: item (head g, key r); a wave covers 64 keys of one head
        for (int it = tid; it < grp * kDecKeys; it += kDecThreads) {
            const int g = it / kDecKeys, r = it % kDecKeys;
            float x = -INFINITY;
            if (pk[t * kDecKeys + r] <= qp) {
                const bf16* kr = kt + r * L::KROW * 8;
                const float* qg = qs + g * D;
                float acc = 0.0f;
#pragma unroll 4
                for (int c = 0; c < D / 8; ++c) {
                    const bf16x8 kv = *(const bf16x8*)(kr + c * 8);
                    const f32x4 qa = *(const f32x4*)(qg + c * 8);
                    const f32x4 qb = *(const f32x4*)(qg + c * 8 + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(qa[e], (float)kv[e], acc);
                        acc = fmaf(qb[e], (float)kv[e + 4], acc);
                    }
                }
                x = acc + gs[g] * ((float)kr[D] + (float)kr[D + 1]);   // s = s_hi + s_lo
            }
            ts[g * kDecKeys + r] = x;
        }
        __syncthreads();
        // online softmax per head (a wave per head): new max, rescale factor,
        // probabilities, running sum
        for (int g = wave; g < grp; g += kDecWaves) {
            const float x = ts[g * kDecKeys + lane];
            float mx = x;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float m_old = mh[g];
            const float m_new = fmaxf(m_old, mx);
            const float p = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - m_new);
            ts[g * kDecKeys + (int)vt_col(lane)] = p;   // in V^T column order (every read above is done)
            float l = p;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
            if (lane == 0) {
                const float f = m_old == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_old - m_new);
                sc[g] = f;
                mh[g] = m_new;
                lh[g] = lh[g] * f + l;
            }
        }
        __syncthreads();
        // unnormalised P.V: item (head g, channel d); the probabilities sit in
        // V^T column order, so both operands are read 16 B at a time
#pragma unroll
        for (int j = 0; j < OPT; ++j) {
            const int it = tid + j * kDecThreads;
            if (it >= grp * D) break;
            const int g = it / D, d = it % D;
            const bf16* vr = vt + d * L::VROW * 8;
            const float* pg = ts + g * kDecKeys;
            float acc = oacc[j] * sc[g];
#pragma unroll 2
            for (int c8 = 0; c8 < kDecKeys / 8; ++c8) {
                const bf16x8 vv = *(const bf16x8*)(vr + c8 * 8);
                const f32x4 pa = *(const f32x4*)(pg + c8 * 8);
                const f32x4 pb = *(const f32x4*)(pg + c8 * 8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = fmaf(pa[e], (float)vv[e], acc);
                    acc = fmaf(pb[e], (float)vv[e + 4], acc);
                }
            }
            oacc[j] = acc;
        }
        __syncthreads();   // slot t & 1 is free again
        if (t + 2 < n_tiles) load_tile(t + 2, slot);
    }
    const int64_t pbase = ((int64_t)s * n_chunks + chunk) * hq + h0;
    if (tid < grp) part_ml[pbase + tid] = make_float2(mh[tid], lh[tid]);
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
        const int it = tid + j * kDecThreads;
        if (it < grp * D) part_o[(pbase + it / D) * D + it % D] = oacc[j];
    }
}

// One workgroup of NT threads per (sequence, q head) merges the partials of
// the sequence's chunks; SUB = NT / D lanes per channel, lane `sub` of channel
// d taking the chunks c = sub (mod SUB).  With J > 0 (at most SUB * J <= NT
// chunks) the merge costs one memory round trip: thread c loads chunk c's
// (max, sum), every lane then issues its J O loads, and while those are in
// flight the maxima reduce to one m and thread c leaves the chunk weight
// 2^(m_c - m) in LDS.  With J = 0 (longer sequences) batches of NT chunk
// weights go through LDS in turn, eight O loads per lane in flight.  Either
// way every lane sums its chunks in chunk order.  No visible key: O = 0,
// LSE = -inf.
template <int D, int NT, int J>
__global__ __launch_bounds__(NT) void attn_decode_combine_kernel(
    const int* __restrict__ cu_kept, int hq, int chunk_keys, int n_chunks, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, bf16* __restrict__ out, float* __restrict__ lse) {
    constexpr int SUB = NT / D;   // lanes per channel
    static_assert(SUB * J <= NT, "one (max, sum) load per thread");
    __shared__ float wsh[NT];
    __shared__ float red[NT];
    const int s = blockIdx.x / hq, h = blockIdx.x % hq, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ms = cu_kept[s + 1] - cu_kept[s];
    const int nc = min((ms + chunk_keys - 1) / chunk_keys, n_chunks);   // ms <= max_kept_seqlen by contract
    const float2* ml = part_ml + (int64_t)s * n_chunks * hq + h;     // chunk c at ml[c * hq]
    const float* po = part_o + ((int64_t)s * n_chunks * hq + h) * D;  // chunk c at po[c * hq * D]

    auto block_reduce = [&](float v, bool is_max) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float u = __shfl_xor(v, o, 64);
            v = is_max ? fmaxf(v, u) : v + u;
        }
        if (lane == 0) red[wave] = v;
        __syncthreads();
        float r = red[0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
        __syncthreads();
        return r;
    };

    const int d = tid % D, sub = tid / D;
    float m, l = 0.0f, o = 0.0f;
    if constexpr (J > 0) {
        // the (max, sum) load first: vector-memory counts retire in order, so
        // waiting for it leaves the O loads issued after it in flight
        const float2 v = tid < nc ? ml[(int64_t)tid * hq] : make_float2(-INFINITY, 0.0f);
        // straight-line loads (a chunk past the end reads chunk 0's slot, which
        // every sequence has, and is replaced by 0), so the wait for v can
        // leave them outstanding
        float ov[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int c = sub + SUB * j;
            const float x = po[((int64_t)(c < nc ? c : 0) * hq) * D + d];
            ov[j] = c < nc ? x : 0.0f;
        }
        m = block_reduce(v.x, true);
        const float wc = v.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(v.x - m);
        wsh[tid] = wc;   // 0 past the last chunk
        l = block_reduce(wc * v.y, false);   // its barriers also publish wsh
#pragma unroll
        for (int j = 0; j < J; ++j) o += wsh[sub + SUB * j] * ov[j];
    } else {
        float mx = -INFINITY;
        for (int c = tid; c < nc; c += NT) mx = fmaxf(mx, ml[(int64_t)c * hq].x);
        m = block_reduce(mx, true);
        for (int c0 = 0; c0 < nc; c0 += NT) {
            const int c = c0 + tid;
            float wc = 0.0f;
            if (c < nc && m != -INFINITY) {
                const float2 v = ml[(int64_t)c * hq];
                if (v.x != -INFINITY) {
                    wc = __builtin_amdgcn_exp2f(v.x - m);
                    l += wc * v.y;
                }
            }
            wsh[tid] = wc;
            __syncthreads();
            const int nb = min(NT, nc - c0);
#pragma unroll 8
            for (int j = sub; j < nb; j += SUB) o += wsh[j] * po[((int64_t)(c0 + j) * hq) * D + d];
            __syncthreads();
        }
        l = block_reduce(l, false);
    }
    red[tid] = o;
    __syncthreads();
    if (tid < D) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < SUB; ++j) t += red[j * D + tid];
        out[((int64_t)s * hq + h) * D + tid] = (bf16)(l > 0.0f ? t / l : 0.0f);
    }
    const int n_seqs = (int)gridDim.x / hq;
    if (lse && tid == 0) lse[(int64_t)h * n_seqs + s] = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// The combine launch for n_chunks chunks per sequence: 1024 threads from 128
// chunks on, else 256; the one-round form with the smallest J that covers
// them, up to 64 per lane.
template <int D, int NT>
void launch_combine_nt(const DecodeArgs& a, int chunk_keys, int n_chunks, const float* part_o,
                       const float2* part_ml, hipStream_t st) {
    constexpr int SUB = NT / D;
    const int jn = (n_chunks + SUB - 1) / SUB;
    const dim3 grid((unsigned)(a.n_seqs * a.hq)), block(NT);
#define TG_COMBINE(JJ)                                                                                       \
    hipLaunchKernelGGL((attn_decode_combine_kernel<D, NT, JJ>), grid, block, 0, st, a.cu_kept, a.hq,      \
                       chunk_keys, n_chunks, part_o, part_ml, a.out, a.lse)
    if (jn <= 4) TG_COMBINE(4);
    else if (jn <= 8) TG_COMBINE(8);
    else if (jn <= 16) TG_COMBINE(16);
    else if (jn <= 24 && SUB * 24 <= NT) TG_COMBINE(24);
    else if (jn <= 32 && SUB * 32 <= NT) TG_COMBINE(32);
    else if (jn <= 48 && SUB * 48 <= NT) TG_COMBINE(48);
    else if (jn <= 64 && SUB * 64 <= NT) TG_COMBINE(64);
    else TG_COMBINE(0);
#undef TG_COMBINE
}

template <int D>
int launch_decode_d(const DecodeArgs& a, hipStream_t st) {
    using L = DecLds<D>;
    const int grp = a.hq / a.hkv;
    // 64-key tiles per split workgroup.  Up to 1536 (tile, kv head, sequence)
    // jobs each workgroup takes one tile through a one-slot ring (~38 KB of LDS,
    // four workgroups per CU, every tile's loads in flight at once); more jobs
    // give 2-4 tiles per workgroup through a two-slot ring, two per CU.
    const int64_t jobs = (int64_t)decode_chunks(a.max_kept_seqlen) * a.hkv * a.n_seqs;
    const int nsub = jobs <= 1536 ? 1 : (int)std::min<int64_t>(kDecMaxSub, (jobs + 511) / 512);
    const int chunk_keys = nsub * kDecKeys;
    const int n_chunks = a.max_kept_seqlen > 0 ? (a.max_kept_seqlen + chunk_keys - 1) / chunk_keys : 1;
    float* part_o = (float*)a.ws;
    float2* part_ml = (float2*)((char*)a.ws + decode_part_o_bytes(a.n_seqs, a.max_kept_seqlen, a.hq, D));
    DecFreqs fr;
    for (int f = 0; f < 64; ++f)
        fr.rev[f] = a.rope && f < D / 2 ? exp2(-(2.0 * f / D) * a.rope_log2_base) / 6.283185307179586 : 0.0;
    if (a.m_tot > 0) {
        const size_t shm = L::smem(kDecMaxGrp, kDecMaxSub);   // the attribute covers every launch
        static std::atomic<uint64_t> lds_set{0};
        if (const int e = set_dyn_lds_once((const void*)attn_decode_split_kernel<D>, (int)shm, lds_set)) return e;
        hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3((unsigned)n_chunks, a.hkv, a.n_seqs),
                           dim3(kDecThreads), L::smem(grp, nsub), st, a.q, a.q_stride, a.q_pos, a.gain,
                           a.qk_scale_log2, a.pos, a.cu_kept, a.hq, grp, a.mp, a.ws_k, a.ws_vt, fr, (int)a.rope,
                           nsub, n_chunks, part_o, part_ml);
    }
    if (n_chunks >= 128)
        launch_combine_nt<D, 1024>(a, chunk_keys, n_chunks, part_o, part_ml, st);
    else
        launch_combine_nt<D, kDecThreads>(a, chunk_keys, n_chunks, part_o, part_ml, st);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace

int decode_chunks(int max_kept_seqlen) { return max_kept_seqlen > 0 ? (max_kept_seqlen + kDecKeys - 1) / kDecKeys : 1; }

size_t decode_part_o_bytes(int n_seqs, int max_kept_seqlen, int hq, int d) {
    return ((size_t)n_seqs * decode_chunks(max_kept_seqlen) * hq * d * 4 + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int n_seqs, int max_kept_seqlen, int hq, int d) {
    const size_t ml = ((size_t)n_seqs * decode_chunks(max_kept_seqlen) * hq * 8 + 255) & ~(size_t)255;
    return decode_part_o_bytes(n_seqs, max_kept_seqlen, hq, d) + ml;
}

int launch_attn_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.n_seqs == 0) return TG_OK;
    switch (a.d) {
        case 64: return launch_decode_d<64>(a, st);
        case 128: return launch_decode_d<128>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace tg
