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
//  1. attn_prep_kernel (one workgroup per 64 kept tokens and kv head):
//     - rotary angles pos * base^(-2f/D) in fp64, reduced mod 2pi, then fp32
//       (cos, sin), kept as a per-token table for the queries;
//     - keys rotated in fp32 and rounded to bf16 into K' rows [Hkv][row][D+16]
//       whose 16 extra columns carry the key score split in two bf16 halves
//       (s_hi, s_lo, s_hi, 0...), so the bias rides inside the QK MFMA;
//     - values transposed through LDS to V^T [Hkv][D][row] (coalesced stores),
//       the layout the P.V MFMA operand wants, with the middle two quads of
//       every 16-key group swapped (vt_col) to match the P^T operand's order.
//     Rows are padded per sequence so every sequence starts on a 16-row
//     boundary.
//  2. attn_fwd_kernel: FlashAttention-style online softmax in the log2 domain.
//     Queries are rotated, scaled by log2(e)/(sqrt(D) tau) and rounded to bf16
//     once per workgroup; their 16 extra columns hold (g_hi, g_hi, g_lo, 0...)
//     with g = g_h log2(e), so one extra MFMA k-step adds
//     g_hi s_hi + g_hi s_lo + g_lo s_hi = g s (to ~2^-16 relative) and the MFMA
//     output is already the log2-domain logit.  S^T = K'.Q'^T on 32x32x16 bf16
//     MFMA puts one query per lane (lane & 31): row statistics are per-lane
//     scalars combined across the two 32-lane halves with one permlane32 swap;
//     P^T feeds O^T = V^T.P^T straight from the S^T accumulators (8 consecutive
//     accumulators are one 16-key MFMA step, V^T read in the matching order).
//     A running offset m (set from the first tile's exact row max, kept
//     bf16-exact) rides in Q' column 3 against 1.0 in K' column 3, so the MFMA
//     emits u = t - m and p = exp2(u) needs no max or subtraction.  Row sums
//     use v_dot2 on the bf16 P that the P.V MFMA consumes; a block whose sum
//     exceeds 2^62 (some p very large) takes a rare path that raises m to the
//     block max and rescales O and l (the result is exact either way).  Each
//     64-key tile is two 32-key blocks: block 0's exponentials overlap block
//     1's QK MFMAs, and block 1's overlap the previous tile's P.V MFMAs.
//     All q heads of a KV group that fit in the workgroup share each K/V tile.
//     Causality uses the kept order (positions increase within a sequence, so
//     pos_j <= pos_i  <=>  j <= i).  Blocks are ordered head-fastest so that,
//     with workgroups dealt round-robin to the 8 XCDs, each KV head keeps to
//     one XCD's L2.
#include <math.h>

#include "tg_common.hpp"

namespace tg {

// Rows of the padded K'/V^T layout: sequence s starts at padded_seq_start();
// the last sequence's final tile may reach 63 rows past its end.
int64_t attn_padded_rows(int n_seqs, int64_t m_tot) {
    return (((m_tot + 16 * (int64_t)n_seqs + 16) + 63) & ~(int64_t)63) + 64;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t attn_workspace_layout(int n_seqs, int64_t m_tot, int hkv, int d, size_t* off_k,
                             size_t* off_vt, size_t* off_cs) {
    const int64_t mp = attn_padded_rows(n_seqs, m_tot);
    const size_t kb = align256((size_t)hkv * mp * (d + 16) * 2);
    const size_t vb = align256((size_t)hkv * mp * d * 2);
    const size_t cb = align256((size_t)(m_tot > 0 ? m_tot : 1) * (d / 2) * sizeof(float2));
    if (off_k) *off_k = 0;
    if (off_vt) *off_vt = kb;
    if (off_cs) *off_cs = kb + vb;
    return kb + vb + cb;
}

namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kExtra = 16;  // extra K'/Q' columns carrying the key bias

struct RopeFreqs {
    double inv_freq[64];   // base^(-2f/D), f < D/2
};

__device__ __forceinline__ void split_bf16(float x, bf16* hi, bf16* lo) {
    const bf16 h = (bf16)x;
    *hi = h;
    *lo = (bf16)(x - (float)h);
}

// Smallest bf16-representable value >= x (x finite).
__device__ __forceinline__ float bf16_ceil(float x) {
    const uint32_t u = __float_as_uint(x);
    const float t = __uint_as_float(u & 0xffff0000u);   // truncation toward zero
    return t >= x ? t : __uint_as_float((u & 0xffff0000u) + 0x10000u);
}

// ---------------------------------------------------------------- pre-pass --
// One workgroup per (64 kept tokens, kv head); lane = token.  Head-0 groups
// also store the (cos, sin) table the queries use.  A last group row zero-fills
// the padding rows (below).
template <int D>
__global__ __launch_bounds__(256) void attn_prep_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, int64_t kv_stride,
    const float* __restrict__ key_score, const int* __restrict__ pos, const int* __restrict__ cu_kept,
    int n_seqs, int64_t m_tot, int hkv, int64_t mp, RopeFreqs fr, int rope, bf16* __restrict__ ws_k,
    bf16* __restrict__ ws_vt, float2* __restrict__ ws_cs) {
    constexpr int HALF = D / 2, KD = D + kExtra, FPW = HALF / 4, VLD = D + 2;
    __shared__ __attribute__((aligned(16))) bf16 vs[64 * VLD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    if (h == hkv) {
        // Zero the padding rows between sequences (and after the last one), so
        // that key tiles can be loaded whole: rows past a sequence's end are then
        // either zeros or other sequences' finite data, and their probabilities
        // are 0.  Grid-stride over (padded row, kv head); a row is padding iff it
        // lies past the end of the sequence whose padded start precedes it.
        const int64_t nthreads = (int64_t)gridDim.x * 256;
        for (int64_t idx = (int64_t)blockIdx.x * 256 + tid; idx < mp * hkv; idx += nthreads) {
            const int64_t r = idx / hkv;
            const int hh = (int)(idx % hkv);
            int lo = 0, hi = n_seqs;   // last sequence whose padded start is <= r (or 0)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (padded_seq_start(cu_kept[mid], mid) <= r) lo = mid; else hi = mid;
            }
            const int64_t p0 = padded_seq_start(cu_kept[lo], lo);
            if (r >= p0 && r < p0 + (cu_kept[lo + 1] - cu_kept[lo])) continue;   // a token row
            bf16* kr = ws_k + ((int64_t)hh * mp + r) * KD;
#pragma unroll
            for (int c = 0; c < KD; c += 8) *(bf16x8*)(kr + c) = bf16x8{};
            bf16* vr = ws_vt + (int64_t)hh * D * mp + vt_col(r);
            for (int d = 0; d < D; ++d) vr[(int64_t)d * mp] = (bf16)0.0f;
        }
        return;
    }
    const int64_t m0 = (int64_t)blockIdx.x * 64;
    const int64_t m = m0 + lane;
    const bool valid = m < m_tot;
    int64_t prow = 0;
    if (valid) {
        const int s = find_seq(cu_kept, n_seqs, m);
        prow = padded_seq_start(cu_kept[s], s) + (m - cu_kept[s]);
    }
    // V^T through LDS: coalesced row loads first (their latency overlaps the
    // rotary work), then per channel d the 64 lanes store 64 consecutive rows.
    constexpr int VCH = 64 * (D / 8) / 256;
    bf16x8 vx[VCH];
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
        const int ch = tid + 256 * i;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        vx[i] = (m0 + r < m_tot) ? *(const bf16x8*)(v + (m0 + r) * kv_stride + (int64_t)h * D + c8 * 8) : bf16x8{};
    }
    // K' row: rotated key + bias columns
    const int f0 = wave * FPW;
    if (valid) {
        float cn[FPW], sn[FPW];
        if (rope) {
            const double p = (double)pos[m];
            const double two_pi = 6.283185307179586;
#pragma unroll
            for (int e = 0; e < FPW; ++e) {
                const double ang = p * fr.inv_freq[f0 + e];
                const double red = ang - two_pi * rint(ang * (1.0 / two_pi));
                sincosf((float)red, &sn[e], &cn[e]);
            }
            if (h == 0) {
                float4* dst = (float4*)(ws_cs + m * HALF + f0);
#pragma unroll
                for (int e = 0; e < FPW; e += 2) dst[e / 2] = make_float4(cn[e], sn[e], cn[e + 1], sn[e + 1]);
            }
        }
        const bf16* src = k + m * kv_stride + (int64_t)h * D;
        bf16* dst = ws_k + ((int64_t)h * mp + prow) * KD;
#pragma unroll
        for (int c = 0; c < FPW / 8; ++c) {
            bf16x8 x1 = *(const bf16x8*)(src + f0 + c * 8);
            bf16x8 x2 = *(const bf16x8*)(src + HALF + f0 + c * 8);
            if (rope) {
                bf16x8 y1, y2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = (float)x1[e], b = (float)x2[e];
                    const float cc = cn[c * 8 + e], ss = sn[c * 8 + e];
                    y1[e] = (bf16)(a * cc - b * ss);
                    y2[e] = (bf16)(b * cc + a * ss);
                }
                x1 = y1;
                x2 = y2;
            }
            *(bf16x8*)(dst + f0 + c * 8) = x1;
            *(bf16x8*)(dst + HALF + f0 + c * 8) = x2;
        }
        if (wave == 0) {
            bf16x8 extra[2] = {bf16x8{}, bf16x8{}};
            bf16 sh, sl;
            split_bf16(key_score[m], &sh, &sl);
            extra[0][0] = sh;
            extra[0][1] = sl;
            extra[0][2] = sh;
            extra[0][3] = (bf16)1.0f;
            *(bf16x8*)(dst + D) = extra[0];
            *(bf16x8*)(dst + D + 8) = extra[1];
        }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
        const int ch = tid + 256 * i;
        const int r = ch / (D / 8), c8 = ch % (D / 8);
        uint32_t* d32 = (uint32_t*)(vs + r * VLD + c8 * 8);   // VLD rows are 4-byte aligned
        const uint32_t* xs = (const uint32_t*)&vx[i];
#pragma unroll
        for (int u = 0; u < 4; ++u) d32[u] = xs[u];
    }
    __syncthreads();
    if (valid) {
        bf16* dst = ws_vt + ((int64_t)h * D) * mp + vt_col(prow);
#pragma unroll 8
        for (int dd = 0; dd < D / 4; ++dd) {
            const int d = wave * (D / 4) + dd;
            dst[(int64_t)d * mp] = vs[lane * VLD + d];
        }
    }
}

template <int D>
struct AttnLds {
    // K' and V^T tiles arrive by global_load_lds_dwordx4: every load
    // instruction copies 64 lanes x 16 B into 1 KiB of consecutive LDS, so rows
    // are padded by one 16-B chunk (pad slots hold a duplicate, never read).
    // The odd row pitch (19 / 9 chunks) keeps the 16-B MFMA operand reads of
    // 8 consecutive lanes on 8 distinct 4-bank groups.
    static constexpr int KD = D + kExtra;
    static constexpr int KCHUNK = KD / 8;          // 16-B chunks per K' row (18 / 10)
    static constexpr int KROW = KCHUNK + 1;        // padded row, in chunks
    static constexpr int KLD = KROW * 8;           // ... in elements (152 / 88)
    static constexpr int VCHUNK = kBN / 8;         // 16-B chunks per V^T row (8)
    static constexpr int VROW = VCHUNK + 1;
    static constexpr int VLD = VROW * 8;           // V^T row pitch in elements (72: 144 B)
    static constexpr int K_INSTR = kBN * KROW / 64;    // load instructions per K' tile (19 / 11)
    static constexpr int V_INSTR = D * VROW / 64;      // ... per V^T tile (18 / 9)
    static_assert(kBN * KROW % 64 == 0 && D * VROW % 64 == 0, "tiles must be whole load instructions");
    static constexpr int KPW = (K_INSTR + 3) / 4;      // per wave
    static constexpr int VPW = (V_INSTR + 3) / 4;
    static constexpr int K_BYTES = kBN * KLD * 2;
    static constexpr int V_BYTES = D * VLD * 2;
    static constexpr int SMEM = 2 * K_BYTES + 2 * V_BYTES;   // two K' and two V^T buffers
};

// HW q heads per workgroup (1, 2 or 4); each of the 4 waves owns QW = 32 QB
// query tokens of one head (QB blocks of 32); WB = 4 / HW waves per head;
// BMT = QW WB tokens per workgroup.  Every K'/V^T fragment read from LDS feeds
// QB MFMAs, so LDS traffic per flop falls as 1/QB; QB = 2 needs one wave per
// SIMD (about 400 registers).
//
// Software pipeline per wave, iteration j (K' runs one tile ahead of V^T):
//   R1  QK MFMAs of tile j+1, key block 0 (K' fragments of block 1 read);
//   R2  QK MFMAs of tile j+1, key block 1  ||  exponentials of key block 0;
//   R3  P.V MFMAs of tile j                ||  exponentials of key block 1;
//       (rare) offset refresh if tile j+1 produced a huge probability;
//   K'(j+2) goes straight to LDS and V^T(j+1) through registers meanwhile.
// Masks are applied between the regions on the (at most two) tiles that reach
// a wave's diagonal; tiles wholly past it are masked to zero probability.
template <int D, int HW, int QB>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void attn_fwd_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const bf16* __restrict__ ws_k,
    const bf16* __restrict__ ws_vt, const float2* __restrict__ ws_cs, int rope,
    const float* __restrict__ gain, float qk_scale_log2, const int* __restrict__ cu_kept, int n_seqs,
    int64_t m_tot, int64_t mp, int hq, int grp, int n_qtiles, int n_hblk, bf16* __restrict__ out,
    float* __restrict__ lse) {
    using L = AttnLds<D>;
    constexpr int WB = 4 / HW;
    constexpr int QW = 32 * QB;
    constexpr int BMT = QW * WB;
    constexpr int KS = D / 16;      // MFMA k-steps over head_dim (+1 for the extra columns)
    constexpr int KD = L::KD;
    constexpr int DB = D / 32;      // 32-row blocks of O^T
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int il = lane & 31, half = lane >> 5;

    // head-fastest block order; largest query tiles first
    const int b = blockIdx.x;
    const int hidx = b % n_hblk;
    const int rest = b / n_hblk;
    const int s = rest % n_seqs;
    const int qt = n_qtiles - 1 - rest / n_seqs;
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int q0 = qt * BMT;
    if (q0 >= ms) return;

    const int nsub = grp / HW;
    const int hk = hidx / nsub;
    const int h = hk * grp + (hidx % nsub) * HW + wave / WB;
    const int qb = q0 + (wave % WB) * QW;    // first query (sequence-local) of this wave
    int qi[QB];                              // this lane's query in block c
#pragma unroll
    for (int c = 0; c < QB; ++c) qi[c] = qb + 32 * c + il;
    const int64_t prow0 = padded_seq_start(cs0, s);
    const int kend = min(ms, q0 + BMT);
    const int n_kt = (kend + kBN - 1) / kBN;

    // ---- Q' fragments (B operand of S^T = K' Q'^T): rotated, scaled, + extra columns
    bf16x8 qf[QB][KS + 1];
#pragma unroll
    for (int c = 0; c < QB; ++c) {
        const bool qvalid = qi[c] < ms;
        const bf16* qrow = q + (int64_t)(cs0 + (qvalid ? qi[c] : 0)) * q_stride + (int64_t)h * D;
        float xf[KS][8];
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const bf16x8 raw = qvalid ? *(const bf16x8*)(qrow + t * 16 + half * 8) : bf16x8{};
#pragma unroll
            for (int e = 0; e < 8; ++e) xf[t][e] = (float)raw[e];
        }
        if (rope && qvalid) {
            const float2* csr = ws_cs + (int64_t)(cs0 + qi[c]) * (D / 2);
#pragma unroll
            for (int t = 0; t < KS / 2; ++t) {
                const float4* c4 = (const float4*)(csr + t * 16 + half * 8);
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float4 cc = c4[e2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = e2 * 2 + u;
                        const float cn = u ? cc.z : cc.x, sn = u ? cc.w : cc.y;
                        const float a = xf[t][e], bb = xf[t + KS / 2][e];
                        xf[t][e] = a * cn - bb * sn;
                        xf[t + KS / 2][e] = bb * cn + a * sn;
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < KS; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[c][t][e] = (bf16)(xf[t][e] * qk_scale_log2);
        qf[c][KS] = bf16x8{};
        if (half == 0) {
            bf16 gh, glo;
            split_bf16(gain[h] * kLog2e, &gh, &glo);
            qf[c][KS][0] = gh;
            qf[c][KS][1] = gh;
            qf[c][KS][2] = glo;
        }
    }

    // ---- LDS-direct tile loads.  Load instruction g of a tile is issued by
    // wave g % 4 and copies one 16-B chunk per lane; the per-lane source
    // offsets are fixed for the whole kernel.
    int koff[L::KPW], voff[L::VPW];
#pragma unroll
    for (int i = 0; i < L::KPW; ++i) {
        const int slot = (wave + 4 * i) * 64 + lane;
        const int r = slot / L::KROW, c = slot % L::KROW;
        koff[i] = r * KD + (c < L::KCHUNK ? c : 0) * 8;
    }
#pragma unroll
    for (int i = 0; i < L::VPW; ++i) {
        const int slot = (wave + 4 * i) * 64 + lane;
        const int r = slot / L::VROW, c = slot % L::VROW;
        voff[i] = r * (int)mp + (c < L::VCHUNK ? c : 0) * 8;   // D * mp < 2^31 (checked at launch)
    }
    const bf16* kbase = ws_k + ((int64_t)hk * mp + prow0) * KD;
    const bf16* vbase = ws_vt + (int64_t)hk * D * mp + prow0;
    char* const kbufs = smem;
    char* const vbufs = smem + 2 * L::K_BYTES;
    auto load_k = [&](int t, int buf) {
        const bf16* src = kbase + (int64_t)t * kBN * KD;
        char* dst = kbufs + buf * L::K_BYTES;
#pragma unroll
        for (int i = 0; i < L::KPW; ++i)
            if (wave + 4 * i < L::K_INSTR) lds_load16(src + koff[i], dst + (wave + 4 * i) * 1024);
    };
    auto load_v = [&](int t, int buf) {
        const bf16* src = vbase + t * kBN;
        char* dst = vbufs + buf * L::V_BYTES;
#pragma unroll
        for (int i = 0; i < L::VPW; ++i)
            if (wave + 4 * i < L::V_INSTR) lds_load16(src + voff[i], dst + (wave + 4 * i) * 1024);
    };

    f32x16 o[QB][DB];
#pragma unroll
    for (int c = 0; c < QB; ++c)
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) o[c][bb] = f32x16{};
    // Running offset m per query block (log2 units), bf16-exact because Q'
    // carries -m in its extra column 3 against a 1.0 in K', so the MFMA emits
    // u = t - m directly.
    float m_run[QB], l_run[QB];
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    // A tile whose row sum exceeds this had some p > ~2^57: refresh the offset.
    constexpr float kSumLimit = 0x1p62f;

    auto set_offset = [&](int c, float m) {
        m_run[c] = m;
        if (half == 0) qf[c][KS][3] = (bf16)(-m);
    };
    // acc[r] <-> key j0 + blk*32 + (r/4)*8 + half*4 + r%4, query qv: one
    // per-lane threshold against compile-time key offsets
    auto mask = [&](f32x16& acc, int j0, int blk, int qv) {
        const int thr = qv - j0 - blk * 32 - half * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r >> 2) * 8 + (r & 3) > thr) acc[r] = -INFINITY;
    };
    auto expo = [&](const f32x16& acc, bf16x8* pbk) {
        float l = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) pbk[r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(acc[r]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 pr = {pbk[u][e], pbk[u][e + 1]};
                l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
            }
        return l;
    };
    auto row_max = [&](float mx) {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    auto tile_max = [&](const f32x16& a0, const f32x16& a1) {
        float mx = a0[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, a0[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, a1[r]);
        return row_max(mx);
    };
    // QK of one 64-key tile for query block c only (prologue and refresh).
    auto qk_block = [&](const bf16* ks, int c, f32x16& a0, f32x16& a1) {
        const bf16* kr0 = ks + il * L::KLD + half * 8;
        const bf16* kr1 = kr0 + 32 * L::KLD;
        a0 = f32x16{};
        a1 = f32x16{};
#pragma unroll
        for (int t = 0; t <= KS; ++t) {
            const bf16x8 f0 = *(const bf16x8*)(kr0 + t * 16);
            const bf16x8 f1 = *(const bf16x8*)(kr1 + t * 16);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, qf[c][t], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[c][t], a1, 0, 0, 0);
        }
    };
    // key block kb of tile j0/64 reaches query block c's diagonal
    auto needs_mask = [&](int j0, int kb) { return j0 + kb * 32 + 31 > qb; };

    bf16x8 pb[QB][2][2];   // bf16 probabilities of the tile whose P.V is next
    // Rare: tile t's probabilities were huge for query block c.  Raise the
    // offset to the tile's row max, rescale what is accumulated, recompute.
    auto refresh = [&](const bf16* ks, int t, int c, float& lt) {
        f32x16 a0, a1;
        qk_block(ks, c, a0, a1);
        if (needs_mask(t * kBN, 0)) mask(a0, t * kBN, 0, qi[c]);
        if (needs_mask(t * kBN, 1)) mask(a1, t * kBN, 1, qi[c]);
        const float target = bf16_ceil(m_run[c] + fmaxf(tile_max(a0, a1), 0.0f));
        const float delta = target - m_run[c];
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        l_run[c] *= alpha;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[c][bb][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            a0[r] -= delta;
            a1[r] -= delta;
        }
        set_offset(c, target);
        lt = expo(a0, pb[c][0]) + expo(a1, pb[c][1]);
    };

    // ---- prologue: K'(0), K'(1), V^T(0); tile 0's logits set the offsets
    load_k(0, 0);
    if (n_kt > 1) load_k(1, 1);
    load_v(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < QB; ++c) {
        f32x16 s0, s1;
        qk_block((const bf16*)kbufs, c, s0, s1);
        if (needs_mask(0, 0)) mask(s0, 0, 0, qi[c]);
        if (needs_mask(0, 1)) mask(s1, 0, 1, qi[c]);
        const float m0 = bf16_ceil(tile_max(s0, s1));   // key 0 is visible to every query
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] -= m0;
            s1[r] -= m0;
        }
        set_offset(c, m0);
        l_run[c] = expo(s0, pb[c][0]) + expo(s1, pb[c][1]);
    }
    __syncthreads();   // K' buffer 0 is reloaded in iteration 0

    for (int j = 0; j < n_kt; ++j) {
        if (j + 2 < n_kt) load_k(j + 2, j & 1);
        if (j + 1 < n_kt) load_v(j + 1, (j + 1) & 1);
        const bf16* ksn = (const bf16*)(kbufs + ((j + 1) & 1) * L::K_BYTES);   // K'(j+1); stale past the end
        const bf16* vs = (const bf16*)(vbufs + (j & 1) * L::V_BYTES);
        const bool more = j + 1 < n_kt;
        const int j1 = (j + 1) * kBN;

        // R1: QK of key block 0 of tile j+1
        f32x16 n[QB][2];
        const bf16* kr0 = ksn + il * L::KLD + half * 8;
        const bf16* kr1 = kr0 + 32 * L::KLD;
        {
            bf16x8 f0[KS + 1];
#pragma unroll
            for (int t = 0; t <= KS; ++t) f0[t] = *(const bf16x8*)(kr0 + t * 16);
#pragma unroll
            for (int c = 0; c < QB; ++c) n[c][0] = f32x16{};
#pragma unroll
            for (int t = 0; t <= KS; ++t)
#pragma unroll
                for (int c = 0; c < QB; ++c)
                    n[c][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[t], qf[c][t], n[c][0], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int t = 0; t <= KS; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);
            }
        }
        if (more && needs_mask(j1, 0)) {
#pragma unroll
            for (int c = 0; c < QB; ++c) mask(n[c][0], j1, 0, qi[c]);
        }

        // R2: QK of key block 1 || exponentials of key block 0
        bf16x8 nb[QB][2][2];
        float ln[QB];
#pragma unroll
        for (int c = 0; c < QB; ++c) n[c][1] = f32x16{};
#pragma unroll
        for (int t = 0; t <= KS; ++t) {
            const bf16x8 f1 = *(const bf16x8*)(kr1 + t * 16);
#pragma unroll
            for (int c = 0; c < QB; ++c)
                n[c][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[c][t], n[c][1], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < QB; ++c) ln[c] = expo(n[c][0], nb[c][0]);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 2);
#pragma unroll
        for (int t = 0; t <= KS; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
#pragma unroll
            for (int c = 0; c < QB; ++c) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
                __builtin_amdgcn_sched_group_barrier(0x400, 2, 2);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 2);
            }
        }
        if (more && needs_mask(j1, 1)) {
#pragma unroll
            for (int c = 0; c < QB; ++c) mask(n[c][1], j1, 1, qi[c]);
        }

        // R3: P.V of tile j || exponentials of key block 1
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) {
                // keys of this 16-key step, in the P^T operand's order (vt_col)
                const bf16x8 a = *(const bf16x8*)(vs + (bb * 32 + il) * L::VLD + u * 16 + half * 8);
#pragma unroll
                for (int c = 0; c < QB; ++c)
                    o[c][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c][u >> 1][u & 1], o[c][bb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < QB; ++c) ln[c] += expo(n[c][1], nb[c][1]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
#pragma unroll
        for (int i = 0; i < 4 * DB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
#pragma unroll
            for (int c = 0; c < QB; ++c) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
                __builtin_amdgcn_sched_group_barrier(0x400, 2 / QB, 3);
                __builtin_amdgcn_sched_group_barrier(0x002, 2 / QB, 3);
            }
        }
        // unconditional uses keep the exponentials in R2/R3 (past the end they are unused)
#pragma unroll
        for (int c = 0; c < QB; ++c)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) pb[c][kb][u] = nb[c][kb][u];
#pragma unroll
        for (int c = 0; c < QB; ++c) {
            if (more && __builtin_amdgcn_ballot_w64(!(ln[c] <= kSumLimit))) refresh(ksn, j + 1, c, ln[c]);
            l_run[c] = more ? l_run[c] + ln[c] : l_run[c];
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's K'/V^T loads have landed in LDS
        __syncthreads();
    }

    // ---- epilogue: combine the two halves' partial sums, normalise, store
#pragma unroll
    for (int c = 0; c < QB; ++c) {
        float l_tot;
        {
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[c]), __float_as_uint(l_run[c]), false,
                                                       false);
            l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        if (qi[c] >= ms) continue;
        const float inv = 1.0f / l_tot;
        bf16* orow = out + ((int64_t)(cs0 + qi[c]) * hq + h) * D;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[c][bb][g * 4 + e] * inv);
                *(bf16x4*)(orow + bb * 32 + g * 8 + half * 4) = v4;
            }
        }
        if (lse && half == 0) lse[(int64_t)h * m_tot + cs0 + qi[c]] = (m_run[c] + __log2f(l_tot)) * kLn2;
    }
}

template <int D, int HW, int QB>
int launch_fwd(const AttnArgs& a, hipStream_t st) {
    constexpr int BMT = 32 * QB * (4 / HW);
    const int grp = a.hq / a.hkv;
    const int n_qtiles = (a.max_kept_seqlen + BMT - 1) / BMT;
    const int n_hblk = a.hkv * (grp / HW);
    const int64_t nblk = (int64_t)n_qtiles * a.n_seqs * n_hblk;
    if (nblk > 0x7fffffff || (int64_t)D * a.mp >= ((int64_t)1 << 31)) return TG_ERR_UNSUPPORTED;
    const size_t shm = (size_t)AttnLds<D>::SMEM;
    static bool attr_set = false;   // idempotent; racing first calls set the same value
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)attn_fwd_kernel<D, HW, QB>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
            return TG_ERR_HIP;
        attr_set = true;
    }
    hipLaunchKernelGGL((attn_fwd_kernel<D, HW, QB>), dim3((unsigned)nblk), dim3(256), shm, st, a.q,
                       a.q_stride, a.ws_k, a.ws_vt, a.ws_cs, (int)a.rope, a.gain, a.qk_scale_log2,
                       a.cu_kept, a.n_seqs, a.m_tot, a.mp, a.hq, grp, n_qtiles, n_hblk, a.out, a.lse);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

// One query block per wave: two query blocks (QB = 2) halve LDS traffic per
// flop but need one wave per SIMD, and measured slower on every workload here
// (128k kept 8448: 469 vs 421 us), so only QB = 1 is instantiated.
template <int D, int HW>
int launch_fwd_qb(const AttnArgs& a, hipStream_t st) {
    return launch_fwd<D, HW, 1>(a, st);
}

template <int D>
int launch_prep(const AttnArgs& a, hipStream_t st) {
    RopeFreqs fr;
    for (int f = 0; f < 64; ++f) fr.inv_freq[f] = f < D / 2 ? exp2(-(2.0 * f / D) * a.rope_log2_base) : 0.0;
    // grid.y = kv heads, plus one extra row of groups for the padding fill
    hipLaunchKernelGGL(attn_prep_kernel<D>, dim3((unsigned)((a.m_tot + 63) / 64), a.hkv + 1), dim3(256), 0, st, a.k,
                       a.v, a.kv_stride, a.key_score, a.pos, a.cu_kept, a.n_seqs, a.m_tot, a.hkv, a.mp, fr,
                       (int)a.rope, a.ws_k, a.ws_vt, a.ws_cs);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

template <int D>
int launch_fwd_grp(const AttnArgs& a, hipStream_t st) {
    const int grp = a.hq / a.hkv;
    switch (grp) {
        case 1: return launch_fwd_qb<D, 1>(a, st);
        case 2: return launch_fwd_qb<D, 2>(a, st);
        case 4:
        case 8: return launch_fwd_qb<D, 4>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace

int launch_attn_prep(const AttnArgs& a, hipStream_t st) {
    if (a.m_tot == 0) return TG_OK;
    switch (a.d) {
        case 64: return launch_prep<64>(a, st);
        case 128: return launch_prep<128>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

int launch_attn_fwd(const AttnArgs& a, hipStream_t st) {
    if (a.m_tot == 0) return TG_OK;
    switch (a.d) {
        case 64: return launch_fwd_grp<64>(a, st);
        case 128: return launch_fwd_grp<128>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace tg
