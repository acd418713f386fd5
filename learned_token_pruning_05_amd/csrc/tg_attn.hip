// Token-gated (key-bias) causal GQA attention over the kept tokens.
//
// TokenGate (spke.com article, section on token-gated attention): each kept
// token's gate score becomes an additive bias on the attention logits above
// the gate, scaled by a learnable per-head gain, with a learnable temperature.
// Logit used (the pages print no formula):
//     l_ij = <R(q_i,pos_i), R(k_j,pos_j)> / (sqrt(D) tau) + g_h s_j,
// causal on original positions, R = rotary embedding on original positions.
//
// Work split.
//  1. attn_prep_k_kernel: per kept token, rotary angles in fp64 (reduced mod 2pi)
//     -> fp32 (cos, sin) table; keys rotated in fp32, rounded to bf16 and stored
//     head-major [Hkv][row][D] so a 64-key tile is one contiguous 16 KiB block.
//  2. attn_prep_v_kernel: values transposed to [Hkv][D][row] so the P.V MFMA
//     operand (8 keys per lane at fixed d) is two 8-byte LDS reads.
//     Rows are padded per sequence (16-byte aligned starts).
//  3. attn_fwd_kernel: FlashAttention-style online softmax in the log2 domain.
//     S^T = K.Q^T on 32x32x16 bf16 MFMA puts one query per lane (lane & 31), so
//     row statistics are per-lane scalars combined across the two 32-lane
//     halves with one permlane32 swap; P^T feeds O^T = V^T.P^T directly from
//     the S^T accumulator registers (8 consecutive accumulators are exactly
//     one 16-key MFMA step, with the V^T operand read in the matching key
//     order).  Scale and bias fold into one FMA per logit:
//         t = qk * log2(e)/(sqrt(D) tau) + g_h log2(e) s_j,  p = exp2(t - m).
//     All q heads of a KV group that fit in the workgroup share each K/V tile.
//     Causality uses the kept order (positions increase within a sequence, so
//     pos_j <= pos_i  <=>  j <= i).
#include <math.h>

#include "tg_common.hpp"

namespace tg {

int64_t attn_padded_rows(int n_seqs, int64_t m_tot) {
    return ((m_tot + 8 * (int64_t)n_seqs + 8) + 63) & ~(int64_t)63;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t attn_workspace_layout(int n_seqs, int64_t m_tot, int hkv, int d, size_t* off_k,
                             size_t* off_vt, size_t* off_cs) {
    const int64_t mp = attn_padded_rows(n_seqs, m_tot);
    const size_t kb = align256((size_t)hkv * mp * d * 2);
    const size_t vb = align256((size_t)hkv * mp * d * 2);
    const size_t cb = align256((size_t)(m_tot > 0 ? m_tot : 1) * (d / 2) * sizeof(float2));
    if (off_k) *off_k = 0;
    if (off_vt) *off_vt = kb;
    if (off_cs) *off_cs = kb + vb;
    return kb + vb + cb;
}

namespace {

constexpr int kBN = 64;   // keys per tile

// ---------------------------------------------------------------- pre-pass --
// One thread per (kept token, chunk of 8 frequency pairs).
template <int D>
__global__ __launch_bounds__(256) void attn_prep_k_kernel(
    const bf16* __restrict__ k, int64_t kv_stride, const int* __restrict__ pos,
    const int* __restrict__ cu_kept, int n_seqs, int64_t m_tot, int hkv, int64_t mp,
    double log2_base, int rope, bf16* __restrict__ ws_k, float2* __restrict__ ws_cs) {
    constexpr int HALF = D / 2, NCH = HALF / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m = gid / NCH;
    const int c = (int)(gid % NCH);
    if (m >= m_tot) return;
    const int s = find_seq(cu_kept, n_seqs, m);
    const int64_t prow = padded_seq_start(cu_kept[s], s) + (m - cu_kept[s]);
    float cs_c[8], cs_s[8];
    if (rope) {
        const double p = (double)pos[m];
        const double two_pi = 6.283185307179586;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int f = c * 8 + e;
            const double inv_freq = exp2(-(2.0 * f / D) * log2_base);
            const double ang = p * inv_freq;
            const double red = ang - two_pi * rint(ang / two_pi);
            float sn, cn;
            sincosf((float)red, &sn, &cn);
            cs_c[e] = cn;
            cs_s[e] = sn;
        }
        float4* dst = (float4*)(ws_cs + m * HALF + c * 8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) dst[e / 2] = make_float4(cs_c[e], cs_s[e], cs_c[e + 1], cs_s[e + 1]);
    }
    for (int h = 0; h < hkv; ++h) {
        const bf16* src = k + m * kv_stride + (int64_t)h * D;
        bf16x8 x1 = *(const bf16x8*)(src + c * 8);
        bf16x8 x2 = *(const bf16x8*)(src + HALF + c * 8);
        if (rope) {
            bf16x8 y1, y2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = (float)x1[e], b = (float)x2[e];
                y1[e] = (bf16)(a * cs_c[e] - b * cs_s[e]);
                y2[e] = (bf16)(b * cs_c[e] + a * cs_s[e]);
            }
            x1 = y1;
            x2 = y2;
        }
        bf16* dst = ws_k + ((int64_t)h * mp + prow) * D;
        *(bf16x8*)(dst + c * 8) = x1;
        *(bf16x8*)(dst + HALF + c * 8) = x2;
    }
}

// One thread per (kept token, kv head, chunk of 8 channels); tokens fastest so
// the transposed 2-byte stores of a wave are contiguous.
template <int D>
__global__ __launch_bounds__(256) void attn_prep_v_kernel(
    const bf16* __restrict__ v, int64_t kv_stride, const int* __restrict__ cu_kept, int n_seqs,
    int64_t m_tot, int hkv, int64_t mp, bf16* __restrict__ ws_vt) {
    constexpr int NCH = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t m = gid % m_tot;
    const int64_t rest = gid / m_tot;
    const int c = (int)(rest % NCH);
    const int h = (int)(rest / NCH);
    if (h >= hkv) return;
    const int s = find_seq(cu_kept, n_seqs, m);
    const int64_t prow = padded_seq_start(cu_kept[s], s) + (m - cu_kept[s]);
    const bf16x8 x = *(const bf16x8*)(v + m * kv_stride + (int64_t)h * D + c * 8);
    bf16* dst = ws_vt + ((int64_t)h * D + c * 8) * mp + prow;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[(int64_t)e * mp] = x[e];
}

// ------------------------------------------------------------- main kernel --
template <int D>
struct AttnLds {
    static constexpr int KLD = D + 8;      // K tile row (elements): 16-B reads conflict-free
    static constexpr int VLD = kBN + 4;    // V^T tile row: 8-B reads conflict-free
    static constexpr int K_ELEMS = kBN * KLD;
    static constexpr int V_ELEMS = D * VLD;
    static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 2 + 4 * kBN * 4;
};

// HW q heads per workgroup (1, 2 or 4); each of the 4 waves owns 32 query tokens
// of one head; WB = 4 / HW waves per head; BMT = 32 * WB tokens per workgroup.
template <int D, int HW>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const bf16* __restrict__ ws_k,
    const bf16* __restrict__ ws_vt, const float2* __restrict__ ws_cs, int rope,
    const float* __restrict__ key_score, const float* __restrict__ gain, float qk_scale_log2,
    const int* __restrict__ cu_kept, int n_seqs, int64_t m_tot, int64_t mp, int hq, int grp,
    int n_qtiles, bf16* __restrict__ out, float* __restrict__ lse) {
    using L = AttnLds<D>;
    constexpr int WB = 4 / HW;
    constexpr int BMT = 32 * WB;
    constexpr int KS = D / 16;      // MFMA k-steps over head_dim
    constexpr int DB = D / 32;      // 32-row blocks of O^T
    constexpr int KCH = kBN * D / 8 / 256;   // 16-B chunks of the K tile per thread
    constexpr int VCH = D * kBN / 8 / 256;   // ... of the V^T tile
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int il = lane & 31, half = lane >> 5;

    // largest query tiles first (causal work grows with the tile index)
    const int tile_rev = blockIdx.x / n_seqs;
    const int s = blockIdx.x % n_seqs;
    const int qt = n_qtiles - 1 - tile_rev;
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int q0 = qt * BMT;
    if (q0 >= ms) return;

    const int nsub = grp / HW;
    const int hk = blockIdx.y / nsub;
    const int hbase = hk * grp + (blockIdx.y % nsub) * HW;
    const int h = hbase + wave / WB;
    const int qb = q0 + (wave % WB) * 32;    // first query (sequence-local) of this wave
    const int qi = qb + il;                  // this lane's query
    const bool qvalid = qi < ms;
    const int64_t prow0 = padded_seq_start(cs0, s);
    const int kend = min(ms, q0 + BMT);
    const int n_kt = (kend + kBN - 1) / kBN;

    // ---- Q fragment (B operand of S^T = K Q^T), rotary applied in fp32
    bf16x8 qf[KS];
    {
        const bf16* qrow = q + (int64_t)(cs0 + (qvalid ? qi : 0)) * q_stride + (int64_t)h * D;
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            qf[t] = qvalid ? *(const bf16x8*)(qrow + t * 16 + half * 8) : bf16x8{};
        }
        if (rope && qvalid) {
            const float2* csr = ws_cs + (int64_t)(cs0 + qi) * (D / 2);
#pragma unroll
            for (int t = 0; t < KS / 2; ++t) {
                const float4* c4 = (const float4*)(csr + t * 16 + half * 8);
                bf16x8 y1, y2;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float4 cc = c4[e2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = e2 * 2 + u;
                        const float cn = u ? cc.z : cc.x, sn = u ? cc.w : cc.y;
                        const float a = (float)qf[t][e], b = (float)qf[t + KS / 2][e];
                        y1[e] = (bf16)(a * cn - b * sn);
                        y2[e] = (bf16)(b * cn + a * sn);
                    }
                }
                qf[t] = y1;
                qf[t + KS / 2] = y2;
            }
        }
    }
    const float gl = gain[h] * kLog2e;

    // ---- tile staging
    u32x4 kreg[KCH], vreg[VCH];
    float breg = 0.0f;
    const bf16* kbase = ws_k + ((int64_t)hk * mp + prow0) * D;
    const bf16* vbase = ws_vt + (int64_t)hk * D * mp + prow0;
    auto load_tile = [&](int kt) {
        const int j0 = kt * kBN;
        const bool tail = j0 + kBN > kend;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int ch = tid + 256 * c;
            const int r = ch / (D / 8), cc = ch % (D / 8);
            kreg[c] = (!tail || j0 + r < kend) ? *(const u32x4*)(kbase + (int64_t)(j0 + r) * D + cc * 8)
                                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int ch = tid + 256 * c;
            const int dr = ch / (kBN / 8), cc = ch % (kBN / 8);
            const int j = j0 + cc * 8;
            if (!tail || j + 8 <= kend) {
                vreg[c] = *(const u32x4*)(vbase + (int64_t)dr * mp + j);
            } else {
                const bf16* p = vbase + (int64_t)dr * mp + j;
                bf16x8 t8;
#pragma unroll
                for (int e = 0; e < 8; ++e) t8[e] = (j + e < kend) ? p[e] : (bf16)0.0f;
                vreg[c] = *(u32x4*)&t8;
            }
        }
        if (tid < HW * kBN) {
            const int jj = tid % kBN, hh = tid / kBN;
            breg = (j0 + jj < kend) ? gain[hbase + hh] * kLog2e * key_score[cs0 + j0 + jj] : 0.0f;
        }
    };
    auto store_tile = [&](int buf) {
        char* base = smem + buf * L::BUF_BYTES;
        bf16* ks = (bf16*)base;
        bf16* vs = ks + L::K_ELEMS;
        float* bs = (float*)(vs + L::V_ELEMS);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int ch = tid + 256 * c;
            *(u32x4*)(ks + (ch / (D / 8)) * L::KLD + (ch % (D / 8)) * 8) = kreg[c];
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int ch = tid + 256 * c;
            bf16* dst = vs + (ch / (kBN / 8)) * L::VLD + (ch % (kBN / 8)) * 8;
            // VLD rows are 8-byte aligned: two 8-byte stores
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            ((u32x2*)dst)[0] = u32x2{vreg[c][0], vreg[c][1]};
            ((u32x2*)dst)[1] = u32x2{vreg[c][2], vreg[c][3]};
        }
        if (tid < HW * kBN) bs[tid] = breg;
    };

    f32x16 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    (void)gl;

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < n_kt) load_tile(kt + 1);
        const int j0 = kt * kBN;
        if (j0 <= qb + 31) {   // some key of this tile is visible to this wave
            const char* base = smem + buf * L::BUF_BYTES;
            const bf16* ks = (const bf16*)base;
            const bf16* vs = ks + L::K_ELEMS;
            const float* bs = (const float*)(vs + L::V_ELEMS) + (wave / WB) * kBN;

            f32x16 st[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                st[blk] = f32x16{};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    const bf16x8 a = *(const bf16x8*)(ks + (blk * 32 + il) * L::KLD + t * 16 + half * 8);
                    st[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], st[blk], 0, 0, 0);
                }
            }
            // st[blk][r] <-> key j0 + blk*32 + (r/4)*8 + half*4 + r%4, query qi
            const bool need_mask = j0 + kBN - 1 > qb;
            float mx = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int jl = blk * 32 + g * 8 + half * 4;
                    const float4 b4 = *(const float4*)(bs + jl);
                    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float t = fmaf(st[blk][g * 4 + e], qk_scale_log2, bb[e]);
                        if (need_mask && j0 + jl + e > qi) t = -INFINITY;
                        st[blk][g * 4 + e] = t;
                        mx = fmaxf(mx, t);
                    }
                }
            }
            {
                auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            float lsum = 0.0f;
            bf16x8 pb[4];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(st[blk][r] - m_new);
                    lsum += p;
                    pb[blk * 2 + (r >> 3)][r & 7] = (bf16)p;
                }
            }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
            // O^T += V^T P^T, 16 keys per step
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const bf16* vr = vs + (b * 32 + il) * L::VLD + u * 16 + half * 4;
                    const bf16x4 lo = *(const bf16x4*)vr;
                    const bf16x4 hi = *(const bf16x4*)(vr + 8);
                    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[b], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < n_kt) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: combine the two halves' partial sums, normalise, store
    float l_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!qvalid) return;
    const float inv = 1.0f / l_tot;
    bf16* orow = out + ((int64_t)(cs0 + qi) * hq + h) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[b][g * 4 + e] * inv);
            *(bf16x4*)(orow + b * 32 + g * 8 + half * 4) = v4;
        }
    }
    if (lse && half == 0) lse[(int64_t)h * m_tot + cs0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, int HW>
int launch_fwd(const AttnArgs& a, hipStream_t st) {
    constexpr int BMT = 32 * (4 / HW);
    const int grp = a.hq / a.hkv;
    const int n_qtiles = (a.max_kept_seqlen + BMT - 1) / BMT;
    const dim3 grid((unsigned)(n_qtiles * a.n_seqs), (unsigned)(a.hkv * (grp / HW)));
    const size_t shm = 2 * (size_t)AttnLds<D>::BUF_BYTES;
    static bool attr_set = false;   // idempotent; racing first calls set the same value
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)attn_fwd_kernel<D, HW>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
            return TG_ERR_HIP;
        attr_set = true;
    }
    hipLaunchKernelGGL((attn_fwd_kernel<D, HW>), grid, dim3(256), shm, st, a.q, a.q_stride, a.ws_k,
                       a.ws_vt, a.ws_cs, (int)a.rope, a.key_score, a.gain, a.qk_scale_log2,
                       a.cu_kept, a.n_seqs, a.m_tot, a.mp, a.hq, grp, n_qtiles, a.out, a.lse);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

template <int D>
int launch_all(const AttnArgs& a, hipStream_t st) {
    {
        const int64_t threads = a.m_tot * (D / 16);
        hipLaunchKernelGGL(attn_prep_k_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, a.k, a.kv_stride, a.pos, a.cu_kept, a.n_seqs, a.m_tot, a.hkv, a.mp,
                           a.rope_log2_base, (int)a.rope, a.ws_k, a.ws_cs);
        if (hipGetLastError() != hipSuccess) return TG_ERR_HIP;
    }
    {
        const int64_t threads = a.m_tot * a.hkv * (D / 8);
        hipLaunchKernelGGL(attn_prep_v_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           st, a.v, a.kv_stride, a.cu_kept, a.n_seqs, a.m_tot, a.hkv, a.mp, a.ws_vt);
        if (hipGetLastError() != hipSuccess) return TG_ERR_HIP;
    }
    const int grp = a.hq / a.hkv;
    switch (grp) {
        case 1: return launch_fwd<D, 1>(a, st);
        case 2: return launch_fwd<D, 2>(a, st);
        case 4:
        case 8: return launch_fwd<D, 4>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace

int launch_attn(const AttnArgs& a, hipStream_t st) {
    if (a.m_tot == 0) return TG_OK;
    switch (a.d) {
        case 64: return launch_all<64>(a, st);
        case 128: return launch_all<128>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace tg
