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
//       and two ones (s_hi, s_lo, s_hi, 1, 1, 0...), so the bias (and a
//       per-query constant) rides inside the QK MFMA;
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
//     accumulators are one 16-key MFMA step, V^T stored in the matching order).
//     A running offset m (set from the first tile's exact row max, kept
//     bf16-exact) rides in Q' column 3 against 1.0 in K' column 3, so the MFMA
//     emits u = t - m and p = exp2(u) needs no max or subtraction.  Row sums
//     add up the bf16 P that the P.V MFMA consumes; a tile whose sum
//     exceeds 2^62 (some p very large) takes a rare path that raises m to the
//     tile max and rescales O and l (the result is exact either way).  The
//     loop is a three-stage pipeline (QK of tile j+2 || exponentials of tile
//     j+1 || P.V of tile j), described at the kernel.
//     Grids of at most two workgroups per CU start whole and pair block k
//     with block n_cu + k on one CU; there the second round runs its query
//     tiles in reverse (largest with smallest), and the longest query tiles
//     may be cut into key chunks (a plan fitted to measured kernel times
//     picks the chunk length): each chunk leaves its unnormalised partial
//     in the workspace's key-split scratch and the last one to finish merges
//     them in chunk order.
//     All q heads of a KV group that fit in the workgroup share each K/V tile.
//     Causality uses the kept order (positions increase within a sequence, so
//     pos_j <= pos_i  <=>  j <= i).  Blocks are ordered head-fastest so that,
//     with workgroups dealt round-robin to the 8 XCDs, each KV head keeps to
//     one XCD's L2; then by sequence, then by query tile, largest first.  The
//     workgroups resident on one XCD thus walk the K'/V^T tiles of one or two
//     sequences at a time, which stay in its L2 (interleaving the sequences
//     made packed batches re-fetch about 4x the read-once bytes).
#include <math.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "tg_common.hpp"


namespace tg {

// Rows of the padded K'/V^T layout: sequence s starts at padded_seq_start();
// the last sequence's final tile may reach 63 rows past its end.
int64_t attn_padded_rows(int n_seqs, int64_t m_tot) {
    return (((m_tot + 16 * (int64_t)n_seqs + 16) + 63) & ~(int64_t)63) + 64;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Partial of one key-split forward workgroup: per lane its O^T accumulators
// (D / 2 floats), then its offset and sum, lane-fastest so that stores and
// loads are whole 256-B rows.
static size_t split_slot_floats(int d) { return (size_t)4 * 64 * (d / 2 + 2); }

size_t attn_workspace_layout(int n_seqs, int64_t m_tot, int hkv, int d, size_t* off_k,
                             size_t* off_vt, size_t* off_cs, size_t* off_split, size_t* off_hdr) {
    const int64_t mp = attn_padded_rows(n_seqs, m_tot);
    const size_t kb = align256((size_t)hkv * mp * (d + 16) * 2);
    const size_t vb = align256((size_t)hkv * mp * d * 2);
    const size_t cb = align256((size_t)(m_tot > 0 ? m_tot : 1) * (d / 2) * sizeof(float2));
    if (off_k) *off_k = 0;
    if (off_vt) *off_vt = kb;
    if (off_cs) *off_cs = kb + vb;
    // key-split scratch, only where a forward grid can be small enough to
    // split (at most kSplitCap workgroups even with one per 64 rows and kv
    // head) and long enough for splitting to pay (1024 kept tokens or more)
    const bool split = m_tot >= 1024 && ((m_tot + 63) / 64) * hkv <= kSplitCap;
    const size_t sb = split ? align256((size_t)kSplitCap * 4) + (size_t)kSplitCap * split_slot_floats(d) * 4 : 0;
    if (off_split) *off_split = split ? kb + vb + cb : 0;
    if (off_hdr) *off_hdr = kb + vb + cb + sb;
    static_assert(sizeof(CacheHeader) <= 256, "header fits its slot");
    return kb + vb + cb + sb + 256;
}

namespace {

constexpr int kBN = 64;     // keys per tile
constexpr int kWaves = 4;   // waves per attention workgroup
constexpr int kExtra = 16;  // extra K'/Q' columns carrying the key bias

struct RopeFreqs {
    double rev[64];   // base^(-2f/D) / (2 pi): turns of frequency f per position, f < D/2
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
// One workgroup per (64 padded rows, kv head).  Padded rows are 64-aligned
// tiles of the K'/V^T layout, so every store is a whole coalesced tile: K'
// rows are contiguous, and V^T rows are 128-B runs.  A padded row holds the
// token at its offset in its sequence, or zeros (rows between and after
// sequences, so that key tiles can be loaded whole: their probabilities are
// then 0).  Head-0 groups also store the (cos, sin) table the queries use.
template <int D>
__global__ __launch_bounds__(256) void attn_prep_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, int64_t kv_stride,
    const float* __restrict__ key_score, const int* __restrict__ pos, const int* __restrict__ cu_kept,
    int n_seqs, int64_t m_tot, int hkv, int64_t mp, RopeFreqs fr, int rope, bf16* __restrict__ ws_k,
    bf16* __restrict__ ws_vt, float2* __restrict__ ws_cs, uint32_t* __restrict__ ws_tk,
    CacheHeader* __restrict__ hdr, double rope_base) {
    constexpr int HALF = D / 2, KD = D + kExtra, NPAIR = D / 16, NC8 = D / 8;
    // V^T tile: row d holds the 64 columns vt_col(r) of this tile; 8-column
    // groups are XOR-swizzled by (d / 8) % 8 so the transposing 2-byte writes
    // of 16 lanes spread over the banks, while 16-B reads stay contiguous.
    __shared__ __attribute__((aligned(16))) bf16 vs[D * 64];
    __shared__ int tok[64];
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * 64;
    if (blockIdx.x == 0 && h == 0) {
        if (ws_tk)
            for (int i = tid; i < kSplitCap; i += 256) ws_tk[i] = 0u;   // the forward's split tickets
        // what was prepared, for the readers' checks under TG_DEBUG
        __shared__ unsigned long long hsum[256];
        unsigned long long acc = 0;
        for (int i = tid; i <= n_seqs; i += 256) acc += cu_hash_term(cu_kept[i], i);
        hsum[tid] = acc;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if (tid < o) hsum[tid] += hsum[tid + o];
            __syncthreads();
        }
        if (tid == 0) {
            CacheHeader c;
            c.magic = kCacheMagic;
            c.n_seqs = n_seqs;
            c.hkv = hkv;
            c.d = D;
            c.m_tot = m_tot;
            c.rope_base = rope_base;
            c.cu_hash = hsum[0];
            *hdr = c;
        }
    }
    if (tid < 64) {
        // last sequence whose padded start is <= row (or 0), then the token
        const int64_t r = p0 + tid;
        int lo = 0, hi = n_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (padded_seq_start(cu_kept[mid], mid) <= r) lo = mid; else hi = mid;
        }
        const int c0 = cu_kept[lo], c1 = cu_kept[lo + 1];
        __asm__ volatile("" ::"v"(c0), "v"(c1));   // both loads issued before either is waited for
        const int64_t ps = padded_seq_start(c0, lo);
        tok[tid] = (r >= ps && r < ps + (c1 - c0)) ? c0 + (int)(r - ps) : -1;
    }
    __syncthreads();

    // Every global load of the tile is issued before the first is used (one
    // memory latency per workgroup, not one per loop trip): rows outside the
    // sequences read row 0 and are replaced by zeros afterwards.
    // V rows, coalesced (lanes over 16-B chunks of a row); K' items (row,
    // chunk pair p) take chunks p and p + D/16 (the rotate-half partners),
    // lanes over p so loads and stores are coalesced.
    constexpr int VIT = 64 * NC8 / 256;
    constexpr int KIT = 64 * NPAIR / 256;
    constexpr int KIT1 = KIT > 0 ? KIT : 1;
    const bool any_rows = m_tot > 0;   // else there is no row 0 to read
    bf16x8 vx[VIT], kx1[KIT1], kx2[KIT1];
    int kpos[KIT1];
    float kscore[KIT1];
    if (any_rows) {
#pragma unroll
        for (int i = 0; i < VIT; ++i) {
            const int item = tid + 256 * i;
            const int r = item / NC8, c8 = item % NC8;
            const int64_t m = max(tok[r], 0);
            vx[i] = *(const bf16x8*)(v + m * kv_stride + (int64_t)h * D + c8 * 8);
        }
#pragma unroll
        for (int i = 0; i < KIT1; ++i) {
            const int item = min(tid + 256 * i, 64 * NPAIR - 1);
            const int r = item / NPAIR, p = item % NPAIR;
            const int64_t m = max(tok[r], 0);
            const bf16* src = k + m * kv_stride + (int64_t)h * D;
            kx1[i] = *(const bf16x8*)(src + p * 8);
            kx2[i] = *(const bf16x8*)(src + HALF + p * 8);
            kpos[i] = pos[m];
            kscore[i] = key_score[m];
        }
    }

    // V rows transposed into LDS
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
        const int item = tid + 256 * i;
        const int r = item / NC8, c8 = item % NC8;
        const bf16x8 x = tok[r] >= 0 ? vx[i] : bf16x8{};
        const int col = (int)vt_col(r) ^ ((c8 & 7) * 8);   // d / 8 == c8 for all 8 values
#pragma unroll
        for (int e = 0; e < 8; ++e) vs[(c8 * 8 + e) * 64 + col] = x[e];
    }

    // K' rows, rotated
#pragma unroll
    for (int i = 0; i < KIT1; ++i) {
        const int item = tid + 256 * i;
        if (KIT == 0 && item >= 64 * NPAIR) break;
        const int r = item / NPAIR, p = item % NPAIR;
        const int m = tok[r];
        bf16x8 x1 = bf16x8{}, x2 = bf16x8{};
        if (m >= 0) {
            x1 = kx1[i];
            x2 = kx2[i];
            if (rope) {
                // angle in turns, reduced in fp64 to [-1/2, 1/2]; the hardware
                // sine and cosine take turns
                float cn[8], sn[8];
                const double ppos = (double)kpos[i];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double t = ppos * fr.rev[p * 8 + e];
                    const float tr = (float)(t - rint(t));
                    sn[e] = __builtin_amdgcn_sinf(tr);
                    cn[e] = __builtin_amdgcn_cosf(tr);
                }
                if (h == 0) {
                    float4* dst = (float4*)(ws_cs + (int64_t)m * HALF + p * 8);
#pragma unroll
                    for (int e = 0; e < 8; e += 2) dst[e / 2] = make_float4(cn[e], sn[e], cn[e + 1], sn[e + 1]);
                }
                bf16x8 y1, y2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = (float)x1[e], b = (float)x2[e];
                    y1[e] = (bf16)(a * cn[e] - b * sn[e]);
                    y2[e] = (bf16)(b * cn[e] + a * sn[e]);
                }
                x1 = y1;
                x2 = y2;
            }
        }
        bf16* dst = ws_k + ((int64_t)h * mp + p0 + r) * KD;
        *(bf16x8*)(dst + p * 8) = x1;
        *(bf16x8*)(dst + HALF + p * 8) = x2;
        if (p == 0) {
            // bias columns: (s_hi, s_lo, s_hi, 1, 1) against Q' (g_hi, g_hi, g_lo,
            // -m, 0); a query-side constant split in two bf16 halves can ride
            // in columns 3 and 4
            bf16x8 extra = bf16x8{};
            if (m >= 0) {
                bf16 sh, sl;
                split_bf16(kscore[i], &sh, &sl);
                extra[0] = sh;
                extra[1] = sl;
                extra[2] = sh;
                extra[3] = (bf16)1.0f;
                extra[4] = (bf16)1.0f;
            }
            *(bf16x8*)(dst + D) = extra;
            *(bf16x8*)(dst + D + 8) = bf16x8{};
        }
    }
    __syncthreads();

    // V^T stores: lanes over the 8 16-B column groups of a d row
    constexpr int TIT = D * 8 / 256;
#pragma unroll
    for (int i = 0; i < TIT; ++i) {
        const int item = tid + 256 * i;
        const int d = item / 8, q = item % 8;
        const bf16x8 x = *(const bf16x8*)(vs + d * 64 + ((q ^ ((d >> 3) & 7)) * 8));
        *(bf16x8*)(ws_vt + ((int64_t)h * D + d) * mp + p0 + q * 8) = x;
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
    static constexpr int K_BYTES = kBN * KLD * 2;
    static constexpr int V_BYTES = D * VLD * 2;
    static constexpr int SMEM = 2 * K_BYTES + 2 * V_BYTES;   // two K' and two V^T buffers
};

// HW q heads per workgroup (1, 2 or 4); each of the NW waves owns 32 query
// tokens of one head; WB = NW / HW waves per head; BMT = 32 WB tokens per
// workgroup, all reading the same K'/V^T tiles.
//
// Three-stage software pipeline.  Iteration j is one scheduling region of
// 34 MFMAs (D = 128): the P.V MFMAs of tile j, then the QK MFMAs of tile j+2,
// with the 32 exponentials of tile j+1 (whose logits are already in
// registers) spread over them, one pair per MFMA or two.  No MFMA waits on an
// exponential of the same iteration and no exponential waits on an MFMA.
// Every operand fragment is read from LDS four MFMAs ahead of its use; empty
// volatile asm statements pin the reads, the MFMAs and the exponentials to
// their slots (the scheduler would otherwise pull each MFMA up against its
// read, exposing the LDS latency on every MFMA).  Steps run in pairs with the
// two sets of logits / probabilities swapped, so nothing is copied.
template <int D, int HW, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const bf16* __restrict__ ws_k,
    const bf16* __restrict__ ws_vt, const float2* __restrict__ ws_cs, int rope,
    const float* __restrict__ gain, float qk_scale_log2, const int* __restrict__ cu_kept, int n_seqs,
    int64_t m_tot, int64_t mp, int hq, int grp, int n_qtiles, int n_hblk, int round2, int split_c,
    int units_per_seq, int max_kept, uint32_t* __restrict__ tk, float* __restrict__ part, bf16* __restrict__ out,
    float* __restrict__ lse) {
    using L = AttnLds<D>;
    constexpr int WB = NW / HW;
    constexpr int BMT = 32 * WB;
    constexpr int KS = D / 16;
    constexpr int KD = L::KD;
    constexpr int DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: every test on it is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 31, half = lane >> 5;

    // With round2 > 0 the whole grid is resident at once, two workgroups per
    // CU, and the dispatcher gives block round2 + k the CU of block k: the
    // second round takes its query tiles in reverse, so the CU with the
    // largest tile of the first round gets the smallest of the second.
    int b = blockIdx.x;
    if (round2 > 0 && b >= round2) {
        const int nu = (int)(gridDim.x - round2) / n_hblk;
        const int u = (b - round2) / n_hblk;
        b = round2 + (nu - 1 - u) * n_hblk + (b - round2) % n_hblk;
    }
    const int hidx = b % n_hblk;
    const int rest = b / n_hblk;
    // Unit `rest` of the grid: a query tile, or with split_c > 0 one key chunk
    // of it.  Per sequence the query tiles come largest first, each with the
    // chunks the longest sequence needs there (its n key tiles cut into
    // ceil(n / split_c) nearly equal runs); r0 is the tile's first unit.
    int s, qt, chunk = 0, r0 = rest;
    if (split_c == 0) {
        s = rest / n_qtiles;
        qt = n_qtiles - 1 - rest % n_qtiles;
    } else {
        s = rest / units_per_seq;
        int u = rest % units_per_seq;
        qt = n_qtiles - 1;
        for (;;) {
            const int nkf = (min((qt + 1) * BMT, max_kept) + kBN - 1) / kBN;
            const int ncf = (nkf + split_c - 1) / split_c;
            if (u < ncf) break;
            u -= ncf;
            --qt;
        }
        chunk = u;
        r0 = rest - u;
    }
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int q0 = qt * BMT;
    if (q0 >= ms) return;

    const int nsub = grp / HW;
    const int hk = hidx / nsub;
    const int h = hk * grp + (hidx % nsub) * HW + wave / WB;
    const int qb = q0 + (wave % WB) * 32;
    const int qi = qb + il;
    const bool qvalid = qi < ms;
    const int64_t prow0 = padded_seq_start(cs0, s);
    const int kend = min(ms, q0 + BMT);
    const int n_kt_all = (kend + kBN - 1) / kBN;
    // this workgroup's key tiles [kt0, kt0 + n_kt), keys from jb; with
    // split_c >= 2 every chunk starts at or before the tile of the query
    // tile's first row, so every row sees key jb (it sets the offset)
    int kt0 = 0, n_kt = n_kt_all, nc = 1;
    if (split_c > 0) {
        nc = (n_kt_all + split_c - 1) / split_c;
        if (chunk >= nc) return;
        kt0 = chunk * n_kt_all / nc;
        n_kt = (chunk + 1) * n_kt_all / nc - kt0;
    }
    const int jb = kt0 * kBN;

    bf16x8 qf[KS + 1];
    {
        const bf16* qrow = q + (int64_t)(cs0 + (qvalid ? qi : 0)) * q_stride + (int64_t)h * D;
        float xf[KS][8];
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const bf16x8 raw = qvalid ? *(const bf16x8*)(qrow + t * 16 + half * 8) : bf16x8{};
#pragma unroll
            for (int e = 0; e < 8; ++e) xf[t][e] = (float)raw[e];
        }
        if (rope && qvalid) {
            const float2* csr = ws_cs + (int64_t)(cs0 + qi) * (D / 2);
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
            for (int e = 0; e < 8; ++e) qf[t][e] = (bf16)(xf[t][e] * qk_scale_log2);
        qf[KS] = bf16x8{};
        if (half == 0) {
            bf16 gh, glo;
            split_bf16(gain[h] * kLog2e, &gh, &glo);
            qf[KS][0] = gh;
            qf[KS][1] = gh;
            qf[KS][2] = glo;
        }
    }

    constexpr int KPW = (L::K_INSTR + NW - 1) / NW;
    constexpr int VPW = (L::V_INSTR + NW - 1) / NW;
    uint32_t koff[KPW], voff[VPW];   // element offsets, then bytes
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int slot = (wave + NW * i) * 64 + lane;
        const int r = slot / L::KROW, c = slot % L::KROW;
        koff[i] = r * KD + (c < L::KCHUNK ? c : 0) * 8;
    }
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
        const int slot = (wave + NW * i) * 64 + lane;
        const int r = slot / L::VROW, c = slot % L::VROW;
        voff[i] = (uint32_t)r * (uint32_t)mp + (c < L::VCHUNK ? c : 0) * 8;
    }
    // this head's K' rows and V^T columns from the sequence start, as buffer
    // resources: 32-bit per-lane offsets, the tile offset in a scalar register
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc(ws_k + ((int64_t)hk * mp + prow0 + jb) * KD, (uint32_t)((mp - prow0 - jb) * KD * 2));
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(ws_vt + (int64_t)hk * D * mp + prow0 + jb, (uint32_t)(((int64_t)D * mp - prow0 - jb) * 2));
#pragma unroll
    for (int i = 0; i < KPW; ++i) koff[i] *= 2;   // bytes
#pragma unroll
    for (int i = 0; i < VPW; ++i) voff[i] *= 2;
    char* const kbufs = smem;
    char* const vbufs = smem + 2 * L::K_BYTES;
    auto load_k = [&](int t, int buf) {
        const uint32_t so = (uint32_t)t * (kBN * KD * 2);
        char* dst = kbufs + buf * L::K_BYTES;
#pragma unroll
        for (int i = 0; i < KPW; ++i)
            if (wave + NW * i < L::K_INSTR) lds_load16_buf(krs, koff[i], so, dst + (wave + NW * i) * 1024);
    };
    auto load_v = [&](int t, int buf) {
        const uint32_t so = (uint32_t)t * (kBN * 2);
        char* dst = vbufs + buf * L::V_BYTES;
#pragma unroll
        for (int i = 0; i < VPW; ++i)
            if (wave + NW * i < L::V_INSTR) lds_load16_buf(vrs, voff[i], so, dst + (wave + NW * i) * 1024);
    };

    f32x16 o[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) o[bb] = f32x16{};
    float m_run = 0.0f, l_run = 0.0f;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    constexpr float kSumLimit = 0x1p62f;

    auto set_offset = [&](float m) {
        m_run = m;
        if (half == 0) qf[KS][3] = (bf16)(-m);
    };
    auto mask = [&](f32x16& acc, int j0, int blk) {
        const int thr = qi - j0 - blk * 32 - half * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if ((r >> 2) * 8 + (r & 3) > thr) acc[r] = -INFINITY;
    };
    auto needs_mask = [&](int j0) { return j0 + kBN - 1 > qb; };   // j0: the tile's first key
    auto mask_tile = [&](f32x16& a0, f32x16& a1, int j0) {
        mask(a0, j0, 0);
        mask(a1, j0, 1);
    };
    auto expo = [&](const f32x16& acc, bf16x8* pbk) {
        float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const bf16x2 pr = {(bf16)__builtin_amdgcn_exp2f(acc[r]), (bf16)__builtin_amdgcn_exp2f(acc[r + 1])};
            pbk[r >> 3][r & 7] = pr[0];
            pbk[r >> 3][(r & 7) + 1] = pr[1];
            const uint32_t pw = __builtin_bit_cast(uint32_t, pr);
            l0 += __uint_as_float(pw << 16);
            l1 += __uint_as_float(pw & 0xffff0000u);
        }
        return l0 + l1;
    };
    auto tile_max = [&](const f32x16& a0, const f32x16& a1) {
        float mx = a0[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, a0[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, a1[r]);
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    auto qk_tile = [&](const bf16* ks, f32x16& a0, f32x16& a1) {
        const bf16* kr0 = ks + il * L::KLD + half * 8;
        const bf16* kr1 = kr0 + 32 * L::KLD;
        a0 = f32x16{};
        a1 = f32x16{};
#pragma unroll
        for (int t = 0; t <= KS; ++t) {
            const bf16x8 f0 = *(const bf16x8*)(kr0 + t * 16);
            const bf16x8 f1 = *(const bf16x8*)(kr1 + t * 16);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, qf[t], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[t], a1, 0, 0, 0);
        }
    };

    // ---- prologue: S(0) sets the offset and gives P(0); S(1) is left in registers
    load_k(0, 0);
    if (n_kt > 1) load_k(1, 1);
    load_v(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8 pb[2][2];
    f32x16 s1a, s1b;   // logits of the tile whose exponentials are next
    {
        f32x16 s0, s1;
        qk_tile((const bf16*)kbufs, s0, s1);
        if (needs_mask(jb)) mask_tile(s0, s1, jb);
        const float m0 = bf16_ceil(tile_max(s0, s1));   // key jb is visible to every query
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s0[r] -= m0;
            s1[r] -= m0;
        }
        set_offset(m0);
        l_run = expo(s0, pb[0]) + expo(s1, pb[1]);
        qk_tile((const bf16*)(kbufs + L::K_BYTES), s1a, s1b);   // stale if n_kt == 1 (unused)
        if (n_kt > 1 && needs_mask(jb + kBN)) mask_tile(s1a, s1b, jb + kBN);
    }
    __syncthreads();   // every wave is done with K'(0) before K'(2) replaces it
    if (n_kt > 2) load_k(2, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // One tile step.  (sa, sb, pc) hold the logits of tile j+1 and the
    // probabilities of tile j; the step writes the logits of tile j+2 into
    // (ta, tb) and the probabilities of tile j+1 into pn.  The loop below runs
    // steps in pairs with the two sets swapped, so nothing is copied.
    auto step = [&](int j, f32x16& sa, f32x16& sb, bf16x8 (&pc)[2][2], f32x16& ta, f32x16& tb,
                    bf16x8 (&pn)[2][2]) {
        if (j + 3 < n_kt) load_k(j + 3, (j + 1) & 1);
        if (j + 1 < n_kt) load_v(j + 1, (j + 1) & 1);
        const bf16* ks2 = (const bf16*)(kbufs + (j & 1) * L::K_BYTES);   // K'(j+2); stale past the end
        const bf16* vs = (const bf16*)(vbufs + (j & 1) * L::V_BYTES);
        const bool more1 = j + 1 < n_kt, more2 = j + 2 < n_kt;
        const int j2 = jb + (j + 2) * kBN;
        const bf16* kr0 = ks2 + il * L::KLD + half * 8;
        const bf16* kr1 = kr0 + 32 * L::KLD;

        // MFMA i < 4 DB: P.V k-step i / DB of O^T block i % DB (with the
        // exponentials of key block 0 of tile j+1); then QK k-step (i - 4 DB)/2
        // of key block (i - 4 DB) % 2 of tile j+2 (with those of key block 1).
        constexpr int NP = 4 * DB, NI = NP + 2 * (KS + 1), PF = 4;
        auto frag = [&](int i) -> bf16x8 {
            if (i < NP) return *(const bf16x8*)(vs + ((i % DB) * 32 + il) * L::VLD + (i / DB) * 16 + half * 8);
            const int k = i - NP;
            return *(const bf16x8*)(((k & 1) ? kr1 : kr0) + (k >> 1) * 16);
        };
        bf16x8 ring[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) ring[i] = frag(i);
        ta = f32x16{};
        tb = f32x16{};
        float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bf16x8 a = ring[i % PF];
            if (i + PF < NI) ring[i % PF] = frag(i + PF);
            // The memory clobber keeps the read above from sinking toward its
            // use; re-defining this MFMA's register operand here keeps the
            // MFMA from rising toward its read.  Together they hold every
            // LDS read PF MFMAs ahead of the MFMA that consumes it.
            __asm__ volatile("" ::: "memory");
            if (i < NP) {
                const int u = i / DB;
                __asm__ volatile("" : "+v"(pc[u >> 1][u & 1]));
                o[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pc[u >> 1][u & 1], o[i % DB], 0, 0, 0);
            } else {
                const int k = i - NP;
                __asm__ volatile("" : "+v"(qf[k >> 1]));
                if (k & 1) tb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k >> 1], tb, 0, 0, 0);
                else ta = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k >> 1], ta, 0, 0, 0);
            }
            // exponentials of tile j+1: 16 pairs spread evenly over the NI
            // MFMAs (key block 0 with the P.V ones, block 1 with the QK ones),
            // packed to bf16 and summed a pair at a time
#pragma unroll
            for (int pr_i = 0; pr_i < 16; ++pr_i) {
                if (pr_i * NI / 16 != i) continue;
                const int kb = pr_i >> 3, r = (pr_i & 7) * 2;
                // not before this step's MFMA (these logits are dead after this)
                if (kb) __asm__ volatile("" : "+v"(sb[r]), "+v"(sb[r + 1]));
                else __asm__ volatile("" : "+v"(sa[r]), "+v"(sa[r + 1]));
                const float x0 = kb ? sb[r] : sa[r], x1 = kb ? sb[r + 1] : sa[r + 1];
                const float e0 = __builtin_amdgcn_exp2f(x0);
                const float e1 = __builtin_amdgcn_exp2f(x1);
                const bf16x2 pr = {(bf16)e0, (bf16)e1};
                pn[kb][r >> 3][r & 7] = pr[0];
                pn[kb][r >> 3][(r & 7) + 1] = pr[1];
                // sums of the bf16 values with plain fp32 adds: v_dot2 would
                // stall the matrix pipe, these co-issue with the MFMAs
                const uint32_t pw = __builtin_bit_cast(uint32_t, pr);
                lsum[kb] += __uint_as_float(pw << 16);
                lsum[2 + kb] += __uint_as_float(pw & 0xffff0000u);
                __asm__ volatile("" ::"v"(lsum[kb]), "v"(lsum[2 + kb]));   // and done before the next step
            }
        }
        float ln = (lsum[0] + lsum[2]) + (lsum[1] + lsum[3]);
        // the refresh test consumes the exponentials before any branch
        if (more1 && __builtin_amdgcn_ballot_w64(!(ln <= kSumLimit))) {
            // Rare: tile j+1's probabilities were huge.  Raise the offset to its
            // row max, rescale what is accumulated, redo its exponentials; tile
            // j+2's logits used the old offset and shift with it.  (The empty
            // volatile asm keeps this block a branch: flattened into selects it
            // would cost its whole arithmetic on every tile.)
            __asm__ volatile("");
            const float target = bf16_ceil(m_run + fmaxf(tile_max(sa, sb), 0.0f));
            const float delta = target - m_run;
            const float alpha = __builtin_amdgcn_exp2f(-delta);
            l_run *= alpha;
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[bb][r] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sa[r] -= delta;
                sb[r] -= delta;
                ta[r] -= delta;
                tb[r] -= delta;
            }
            set_offset(target);
            ln = expo(sa, pn[0]) + expo(sb, pn[1]);
        }
        l_run = more1 ? l_run + ln : l_run;
        if (more2 && needs_mask(j2)) mask_tile(ta, tb, j2);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's K'/V^T loads have landed in LDS
        __syncthreads();
    };
    f32x16 s2a, s2b;
    bf16x8 pb2[2][2];
    for (int j = 0; j < n_kt; j += 2) {
        step(j, s1a, s1b, pb, s2a, s2b, pb2);
        if (j + 1 < n_kt) step(j + 1, s2a, s2b, pb2, s1a, s1b, pb);
    }

    if (nc > 1) {
        // Key chunk of a split query tile: leave the partial (unnormalised
        // O^T accumulators, offset, sum) in this unit's slot; the last chunk
        // of the tile to finish (a ticket taken with release order; the others
        // just leave) merges all of them and writes the tile.  The partials
        // move as device-scope atomic stores and loads, which go past the
        // CU's and XCD's caches to the coherent level, so no acquire fence is
        // needed: one would invalidate the whole XCD L2, and with it the
        // K'/V^T tiles every other workgroup there is reading.
        constexpr int PW = D / 2 + 2;   // floats per lane
        const size_t slot_floats = (size_t)NW * 64 * PW;
        auto lane_ptr = [&](int unit) { return part + (size_t)unit * slot_floats + (size_t)wave * 64 * PW + lane; };
        auto put = [&](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        auto get = [&](const float* p) {
            return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        float* mine = lane_ptr(b);
#pragma unroll
        for (int bb = 0; bb < DB; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) put(mine + (bb * 16 + r) * 64, o[bb][r]);
        put(mine + (D / 2) * 64, m_run);
        put(mine + (D / 2 + 1) * 64, l_run);
        __shared__ int sh_last;
        __syncthreads();   // every wave's stores are done
        if (tid == 0) {
            uint32_t* t = tk + r0 * n_hblk + hidx;
            const bool last = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                              (uint32_t)nc - 1u;
            if (last) __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // for the next forward
            sh_last = last;
        }
        __syncthreads();
        if (!sh_last) return;
        if (nc == 2) {
            // Two chunks: this one's partial is still in registers; every load of
            // the other's is issued before the first is used.  Summed in chunk
            // order, so the result does not depend on which chunk finished last.
            const float* src = lane_ptr((r0 + 1 - chunk) * n_hblk + hidx);
            const float mo = get(src + (D / 2) * 64), lo = get(src + (D / 2 + 1) * 64);
            f32x16 ox[DB];
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) ox[bb][r] = get(src + (bb * 16 + r) * 64);
            const float mx = fmaxf(m_run, mo);
            const float fs = __builtin_amdgcn_exp2f(m_run - mx), fo = __builtin_amdgcn_exp2f(mo - mx);
            const bool first = chunk == 0;
            const float f0 = first ? fs : fo, f1 = first ? fo : fs;
            l_run = fmaf(f1, first ? lo : l_run, f0 * (first ? l_run : lo));
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x0 = first ? o[bb][r] : ox[bb][r], x1 = first ? ox[bb][r] : o[bb][r];
                    o[bb][r] = fmaf(f1, x1, f0 * x0);
                }
            m_run = mx;
        } else {
            // every chunk, this one included, from its slot and in chunk order, so
            // the result does not depend on which chunk finished last
            float mx = -INFINITY;
            for (int c = 0; c < nc; ++c) mx = fmaxf(mx, get(lane_ptr((r0 + c) * n_hblk + hidx) + (D / 2) * 64));
            l_run = 0.0f;
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) o[bb] = f32x16{};
            for (int c = 0; c < nc; ++c) {
                const float* src = lane_ptr((r0 + c) * n_hblk + hidx);
                const float f = __builtin_amdgcn_exp2f(get(src + (D / 2) * 64) - mx);
                l_run += f * get(src + (D / 2 + 1) * 64);
#pragma unroll
                for (int bb = 0; bb < DB; ++bb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[bb][r] += f * get(src + (bb * 16 + r) * 64);
            }
            m_run = mx;
        }
    }
    float l_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!qvalid) return;
    const float inv = 1.0f / l_tot;
    bf16* orow = out + ((int64_t)(cs0 + qi) * hq + h) * D;
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[bb][g * 4 + e] * inv);
            *(bf16x4*)(orow + bb * 32 + g * 8 + half * 4) = v4;
        }
    }
    if (lse && half == 0) lse[(int64_t)h * m_tot + cs0 + qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// Grid plan of the forward.  A grid of at most two workgroups per CU starts
// whole, and the dispatcher gives block n_cu + k the CU of block k (round 2),
// so the CU's time is that of its two units run side by side.  For such small
// grids, cutting the long query tiles into key chunks evens out the CUs'
// work, at the price of each chunk's own prologue and of the partials that
// split tiles write and merge.  The plan compares the modelled longest CU
// time, in key-tile steps, of the unsplit grid and of every chunk length,
// with every sequence taken as long as the longest.  The model's constants
// are fitted to kernel times measured on MI355X at 16k and 32k@5% with chunk
// lengths from 8 to 26 tiles (RMS error 1.9 us; its choice lands within
// 1.6 us of the best measured one): two workgroups on a CU each run 1.5x
// slower, a unit's prologue costs 4 steps, and every unit of a split tile
// adds 0.04 steps.
struct FwdPlan {
    int split_c = 0;        // key tiles per chunk, 0: no split
    int units_per_seq = 0;  // grid units per sequence (query tiles or chunks)
    int64_t nblk = 0;
    int round2 = 0;         // first block of round 2, 0: no pairing
};

static FwdPlan plan_fwd_uncached(int n_seqs, int max_kept, int bmt, int n_hblk, int n_cu, bool can_split) {
    constexpr double kShare = 1.5, kPrologue = 4.0, kSplitUnit = 0.04;
    const int n_qtiles = (max_kept + bmt - 1) / bmt;
    auto nkf = [&](int qt) { return (std::min((qt + 1) * bmt, max_kept) + kBN - 1) / kBN; };
    auto finish = [&](FwdPlan p) {
        p.round2 = p.nblk > n_cu && p.nblk <= 2 * (int64_t)n_cu && n_cu % n_hblk == 0 ? n_cu : 0;
        return p;
    };
    FwdPlan base;
    base.units_per_seq = n_qtiles;
    base.nblk = (int64_t)n_qtiles * n_seqs * n_hblk;
    if (!can_split || n_cu <= 0 || n_cu % n_hblk != 0 || base.nblk >= 2 * (int64_t)n_cu) return finish(base);
    const int cap = std::min(2 * n_cu, kSplitCap);
    std::vector<double> sz;
    auto cost = [&](int c, int* units) -> double {
        sz.clear();
        int per_seq = 0, split_units = 0;
        for (int qt = n_qtiles - 1; qt >= 0; --qt) {
            const int nk = nkf(qt), nc = c > 0 ? (nk + c - 1) / c : 1;
            if (nc > 1) split_units += nc;
            per_seq += nc;
            for (int ch = 0; ch < nc; ++ch) {
                const int len = (ch + 1) * nk / nc - ch * nk / nc;
                for (int h = 0; h < n_hblk; ++h) sz.push_back(len + kPrologue);
            }
        }
        *units = per_seq;
        const int64_t nblk = (int64_t)per_seq * n_seqs * n_hblk;
        if (nblk > cap) return 1e30;
        const int per = (int)sz.size();   // one sequence; the others repeat it
        auto size_of = [&](int64_t lb) { return sz[lb % per]; };
        const bool paired = nblk > n_cu;
        const int64_t nu = paired ? (nblk - n_cu) / n_hblk : 0;
        double worst = 0.0;
        for (int64_t k = 0; k < std::min<int64_t>(nblk, n_cu); ++k) {
            const double a = size_of(k);
            double t = a;
            if (paired && n_cu + k < nblk) {
                const int64_t lb = n_cu + (nu - 1 - k / n_hblk) * n_hblk + k % n_hblk;
                const double b = size_of(lb);
                t = kShare * std::min(a, b) + std::fabs(a - b);
            }
            worst = std::max(worst, t);
        }
        return worst + kSplitUnit * split_units * n_seqs * n_hblk;
    };
    int units = 0;
    double best = cost(0, &units);
    FwdPlan p = base;
    for (int c = 2; c < nkf(n_qtiles - 1); ++c) {
        const double t = cost(c, &units);
        if (t < best) {
            best = t;
            p.split_c = c;
            p.units_per_seq = units;
            p.nblk = (int64_t)units * n_seqs * n_hblk;
        }
    }
    return finish(p);
}

// Plans are cached (a serving loop repeats the same shapes): the search
// above takes tens of microseconds of host time.
static FwdPlan plan_fwd(int n_seqs, int max_kept, int bmt, int n_hblk, int n_cu, bool can_split) {
    struct Entry {
        int key[6];
        FwdPlan plan;
    };
    constexpr int kEntries = 16;
    static std::mutex mu;
    static Entry cache[kEntries];
    static int n_used = 0, next = 0;
    const int key[6] = {n_seqs, max_kept, bmt, n_hblk, n_cu, (int)can_split};
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < n_used; ++i)
            if (std::equal(key, key + 6, cache[i].key)) return cache[i].plan;
    }
    const FwdPlan p = plan_fwd_uncached(n_seqs, max_kept, bmt, n_hblk, n_cu, can_split);
    std::lock_guard<std::mutex> g(mu);
    Entry& e = cache[next];
    std::copy(key, key + 6, e.key);
    e.plan = p;
    next = (next + 1) % kEntries;
    n_used = std::min(n_used + 1, kEntries);
    return p;
}

template <int D, int HW, int NW>
int launch_fwd(const AttnArgs& a, hipStream_t st) {
    constexpr int BMT = 32 * (NW / HW);
    static_assert(NW == 4, "the key-split slots hold four waves");
    const int grp = a.hq / a.hkv;
    const int n_qtiles = (a.max_kept_seqlen + BMT - 1) / BMT;
    const int n_hblk = a.hkv * (grp / HW);
    int n_cu = 0;
    if (const int e = device_cu_count(&n_cu)) return e;
    const FwdPlan plan = plan_fwd(a.n_seqs, a.max_kept_seqlen, BMT, n_hblk, n_cu, a.ws_tk != nullptr);
    const int64_t nblk = plan.nblk;
    // buffer offsets into one head's K' rows ((D+16)*2 B each) stay 32-bit
    if (nblk > 0x7fffffff || (int64_t)(D + kExtra) * 2 * a.mp >= ((int64_t)1 << 32)) return TG_ERR_UNSUPPORTED;
    const size_t shm = (size_t)AttnLds<D>::SMEM;
    static std::atomic<uint64_t> lds_set{0};
    if (const int e = set_dyn_lds_once((const void*)attn_fwd_kernel<D, HW, NW>, (int)shm, lds_set)) return e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, HW, NW>), dim3((unsigned)nblk), dim3(NW * 64), shm, st, a.q,
                       a.q_stride, a.ws_k, a.ws_vt, a.ws_cs, (int)a.rope, a.gain, a.qk_scale_log2,
                       a.cu_kept, a.n_seqs, a.m_tot, a.mp, a.hq, grp, n_qtiles, n_hblk, plan.round2,
                       plan.split_c, plan.units_per_seq, a.max_kept_seqlen, a.ws_tk, a.ws_part, a.out, a.lse);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

template <int D>
int launch_prep(const AttnArgs& a, hipStream_t st) {
    RopeFreqs fr;
    for (int f = 0; f < 64; ++f)
        fr.rev[f] = f < D / 2 ? exp2(-(2.0 * f / D) * a.rope_log2_base) / 6.283185307179586 : 0.0;
    // one group per (64 padded rows, kv head); a.mp is a multiple of 64
    hipLaunchKernelGGL(attn_prep_kernel<D>, dim3((unsigned)(a.mp / 64), a.hkv), dim3(256), 0, st, a.k,
                       a.v, a.kv_stride, a.key_score, a.pos, a.cu_kept, a.n_seqs, a.m_tot, a.hkv, a.mp, fr,
                       (int)a.rope, a.ws_k, a.ws_vt, a.ws_cs, a.ws_tk, a.ws_hdr, a.rope_base);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

template <int D>
int launch_fwd_grp(const AttnArgs& a, hipStream_t st) {
    const int grp = a.hq / a.hkv;
    switch (grp) {
        case 1: return launch_fwd<D, 1, kWaves>(a, st);
        case 2: return launch_fwd<D, 2, kWaves>(a, st);
        case 4:
        case 8: return launch_fwd<D, 4, kWaves>(a, st);
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
