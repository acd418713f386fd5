// Gate-side gradients of token-gated attention: dL/ds_j, dL/dg_h, dL/dtau.
//
// TokenGate ([ES] "¿Qué es la atención con control de acceso por tokens…?"):
// the per-head gain and the temperature are learned, and the bias on the
// attention logits is the path by which the loss reaches the gate's scores.
// With l_ij = <q~_i, k~_j> / (sqrt(D) tau) + g_h s_j and dO = dL/dO:
//     P = softmax_j(l),  dP_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>,
//     dS_ij = P_ij (dP_ij - Delta_i)                          (= dL/dl_ij)
//     dL/ds_j = sum_h g_h C_hj,   dL/dg_h = sum_j s_j C_hj,   C_hj = sum_i dS_hij
//     dL/dtau = -(1/tau) sum_h (ln 2 * A_h - g_h dL/dg_h),    A_h = sum_ij dS_hij S_hij
// where S = l log2(e) is what the MFMA produces, so ln 2 * S - g_h s_j is the
// q.k part of the logit.  (Delta_i = sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.)
//
// Kernels:
//   prep    rotated, scaled queries Q' in the layout of the prepared key cache
//           (bias columns (g_hi, g_hi, g_lo, 0) against K' (s_hi, s_lo, s_hi, 1)),
//           plus the log2-domain LSE and Delta of every (q head, kept token);
//   main    key-outer: a workgroup owns 128 keys (32 per wave) of one q head,
//           keeps their K' and V operand fragments in registers and streams
//           every query tile at or after its keys (Q' and dO, 64 rows) through
//           a two-slot LDS ring.  S = Q'.K'^T and dP = dO.V^T run on 32x32x16
//           bf16 MFMA; the accumulator layout puts one key per lane, so C_hj is
//           an in-lane sum over the query rows (no atomics, deterministic), and
//           the workgroup leaves C_hj plus its partial sums of s_j C_hj and of
//           dS S;
//   reduce  dL/ds over heads; per head dL/dg and its share of dL/dtau; tau.
#include <math.h>

#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdWaves = 4;
constexpr int kBwdKeys = 32 * kBwdWaves;   // keys per main workgroup
constexpr int kBwdQ = 64;                  // query rows per tile
constexpr int kBwdExtra = 16;              // bias columns, as in K'

template <int D>
struct BwdLds {
    // tiles arrive by 16-B LDS-direct loads (64 lanes x 16 B per instruction);
    // rows are padded by one chunk so that the 16-B operand reads of eight
    // consecutive rows fall on distinct bank groups (pad slots hold a
    // duplicate, never read)
    static constexpr int KD = D + kBwdExtra;
    static constexpr int QCH = KD / 8;            // 16-B chunks per Q' row
    static constexpr int QROW = QCH + 1;
    static constexpr int OCH = D / 8;             // 16-B chunks per dO row
    static constexpr int OROW = OCH + 1;
    static constexpr int Q_INSTR = kBwdQ * QROW / 64;
    static constexpr int O_INSTR = kBwdQ * OROW / 64;
    static_assert(kBwdQ * QROW % 64 == 0 && kBwdQ * OROW % 64 == 0, "tiles must be whole load instructions");
    static constexpr int QT = kBwdQ * QROW * 8;   // elements per Q' tile
    static constexpr int OT = kBwdQ * OROW * 8;   // elements per dO tile
    static constexpr size_t SMEM = (size_t)2 * (QT + OT) * 2 + (size_t)2 * 2 * kBwdQ * 4;   // + LSE2, Delta rows
    // load instructions one wave issues per tile: its share of the Q' and dO
    // instructions, plus the LSE2 row (wave 3) or the Delta row (wave 2)
    __device__ static int per_wave(int w) {
        return (Q_INSTR - w + kBwdWaves - 1) / kBwdWaves + (O_INSTR - w + kBwdWaves - 1) / kBwdWaves + (w >= 2);
    }
};

// ---------------------------------------------------------------- prep ----
// One workgroup per (64 padded rows, q head).  Padded rows follow the key
// cache's per-sequence layout; rows without a token are zero.  Items (row,
// rotate-half chunk pair) as in the key pre-pass, lanes over chunk pairs; the
// (cos, sin) table of the key pre-pass supplies the rotation.  Threads 0..63
// also compute Delta and LSE2 for their row.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const bf16* __restrict__ o, const bf16* __restrict__ dout,
    int64_t do_stride, const float* __restrict__ lse, const float* __restrict__ gain, float qk_scale_log2,
    const float2* __restrict__ ws_cs, int rope, const int* __restrict__ cu_kept, int n_seqs, int64_t m_tot,
    int hq, int64_t mp, bf16* __restrict__ qc, float* __restrict__ l2, float* __restrict__ delta) {
    constexpr int HALF = D / 2, KD = D + kBwdExtra, NPAIR = D / 16;
    __shared__ int tok[64];
    const int tid = threadIdx.x;
    const int h = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * 64;
    if (tid < 64) {
        const int64_t r = p0 + tid;
        int lo = 0, hi = n_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (padded_seq_start(cu_kept[mid], mid) <= r) lo = mid; else hi = mid;
        }
        const int64_t ps = padded_seq_start(cu_kept[lo], lo);
        const int len = cu_kept[lo + 1] - cu_kept[lo];
        const int m = (r >= ps && r < ps + len) ? cu_kept[lo] + (int)(r - ps) : -1;
        tok[tid] = m;
        if (m >= 0) {
            const bf16* dr = dout + (int64_t)m * do_stride + (int64_t)h * D;
            const bf16* orr = o + ((int64_t)m * hq + h) * D;
            float acc = 0.0f;
#pragma unroll 4
            for (int c = 0; c < D / 8; ++c) {
                const bf16x8 a = *(const bf16x8*)(dr + c * 8);
                const bf16x8 b = *(const bf16x8*)(orr + c * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
            }
            delta[(int64_t)h * m_tot + m] = acc;
            l2[(int64_t)h * m_tot + m] = lse[(int64_t)h * m_tot + m] * kLog2e;
        }
    }
    __syncthreads();
    constexpr int KIT = 64 * NPAIR / 256;
#pragma unroll
    for (int i = 0; i < (KIT > 0 ? KIT : 1); ++i) {
        const int item = tid + 256 * i;
        if (KIT == 0 && item >= 64 * NPAIR) break;
        const int r = item / NPAIR, p = item % NPAIR;
        const int m = tok[r];
        bf16x8 x1 = bf16x8{}, x2 = bf16x8{};
        if (m >= 0) {
            const bf16* src = q + (int64_t)m * q_stride + (int64_t)h * D;
            const bf16x8 a1 = *(const bf16x8*)(src + p * 8);
            const bf16x8 a2 = *(const bf16x8*)(src + HALF + p * 8);
            const float4* cs = (const float4*)(ws_cs + (int64_t)m * HALF + p * 8);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float4 c = make_float4(1.0f, 0.0f, 1.0f, 0.0f);
                if (rope) c = cs[e2];   // (cos, sin) of frequencies 2 e2 and 2 e2 + 1 of this chunk
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * e2 + u;
                    const float cn = u ? c.z : c.x, sn = u ? c.w : c.y;
                    const float a = (float)a1[e], b = (float)a2[e];
                    x1[e] = (bf16)((a * cn - b * sn) * qk_scale_log2);
                    x2[e] = (bf16)((b * cn + a * sn) * qk_scale_log2);
                }
            }
        }
        bf16* dst = qc + ((int64_t)h * mp + p0 + r) * KD;
        *(bf16x8*)(dst + p * 8) = x1;
        *(bf16x8*)(dst + HALF + p * 8) = x2;
        if (p == 0) {
            bf16x8 extra = bf16x8{};
            if (m >= 0) {
                const float g = gain[h] * kLog2e;
                const bf16 gh = (bf16)g;
                extra[0] = gh;
                extra[1] = gh;
                extra[2] = (bf16)(g - (float)gh);
            }
            *(bf16x8*)(dst + D) = extra;
            *(bf16x8*)(dst + D + 8) = bf16x8{};
        }
    }
}

// ---------------------------------------------------------------- main ----
// Block b: q head b % hq (fastest, so that the workgroups of one head sit on
// one XCD's L2 and follow each other down the same Q'/dO rows), then the
// sequence, then the key tile (tile 0, with the most query rows, first).
template <int D>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_main_kernel(
    const bf16* __restrict__ qc, const bf16* __restrict__ ws_k, const bf16* __restrict__ v, int64_t kv_stride,
    const bf16* __restrict__ dout, int64_t do_stride, const float* __restrict__ l2g,
    const float* __restrict__ deltag, const float* __restrict__ key_score, const int* __restrict__ cu_kept,
    int n_seqs, int64_t m_tot, int hq, int grp, int64_t mp, int n_kt, float* __restrict__ colsum,
    float2* __restrict__ part) {
    using L = BwdLds<D>;
    constexpr int KD = L::KD;
    constexpr int KS = D / 16;   // k-steps of the q.k part; one more for the bias columns
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* const qs = (bf16*)smem;                       // [2][QT]
    bf16* const os = qs + 2 * L::QT;                    // [2][OT]
    float* const ls = (float*)(os + 2 * L::OT);         // [2][64] LSE2
    float* const dls = ls + 2 * kBwdQ;                  // [2][64] Delta
    __shared__ float2 wsum[kBwdWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 31, half = lane >> 5;

    const int b = blockIdx.x;
    const int h = b % hq;
    const int rest = b / hq;
    const int s = rest % n_seqs;
    const int kt = rest / n_seqs;
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int key0 = kt * kBwdKeys;
    float2* const pout = part + ((int64_t)h * n_seqs + s) * n_kt + kt;
    if (key0 >= ms) {
        if (tid == 0) *pout = make_float2(0.0f, 0.0f);
        return;
    }
    const int hk = h / grp;
    const int64_t prow0 = padded_seq_start(cs0, s);
    const int kb0 = key0 + 32 * wave;   // this wave's first key
    const int kj = kb0 + il;            // this lane's key
    const bool kvalid = kj < ms;

    // this wave's K' and V fragments as B operands (lane j + 32 (k / 8) holds
    // B[k..k+7][j]); keys past the sequence end are zero and masked
    bf16x8 kf[KS + 1], vf[KS];
    {
        const bf16* kr = ws_k + ((int64_t)hk * mp + prow0 + (kvalid ? kj : 0)) * KD + half * 8;
        const bf16* vr = v + (int64_t)(cs0 + (kvalid ? kj : 0)) * kv_stride + (int64_t)hk * D + half * 8;
#pragma unroll
        for (int t = 0; t <= KS; ++t) kf[t] = kvalid ? *(const bf16x8*)(kr + t * 16) : bf16x8{};
#pragma unroll
        for (int t = 0; t < KS; ++t) vf[t] = kvalid ? *(const bf16x8*)(vr + t * 16) : bf16x8{};
    }

    // query tiles from the one holding key0 to the end of the sequence
    const int q_begin = key0 & ~(kBwdQ - 1);
    const int n_qt = (ms - q_begin + kBwdQ - 1) / kBwdQ;
    // buffer resources over this head's rows from the sequence start: reads
    // past the end return zero
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(qc + ((int64_t)h * mp + prow0) * KD, (uint32_t)((mp - prow0) * KD * 2));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(dout + (int64_t)cs0 * do_stride + (int64_t)h * D,
                                                 (uint32_t)(((m_tot - cs0 - 1) * do_stride + D) * 2));
    const __amdgpu_buffer_rsrc_t lrs = make_rsrc(l2g + (int64_t)h * m_tot + cs0, (uint32_t)((m_tot - cs0) * 4));
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(deltag + (int64_t)h * m_tot + cs0, (uint32_t)((m_tot - cs0) * 4));
    const int n_per_tile = L::per_wave(wave);
    auto load_tile = [&](int t, int slot) {
        const uint32_t q0 = (uint32_t)(q_begin + t * kBwdQ);
        for (int i = wave; i < L::Q_INSTR; i += kBwdWaves) {
            const int sl = i * 64 + lane;
            const int r = sl / L::QROW, c = sl % L::QROW;
            const uint32_t off = (uint32_t)((r * KD + (c < L::QCH ? c : 0) * 8) * 2);
            lds_load16_buf(qrs, off, q0 * (KD * 2), qs + slot * L::QT + i * 512);
        }
        // rows of dO, LSE2 and Delta can run past the last token: their row
        // offset goes into the per-lane offset, which the bounds check covers
        for (int i = wave; i < L::O_INSTR; i += kBwdWaves) {
            const int sl = i * 64 + lane;
            const int r = sl / L::OROW, c = sl % L::OROW;
            const uint32_t off = (uint32_t)(((q0 + r) * do_stride + (c < L::OCH ? c : 0) * 8) * 2);
            lds_load16_buf(ors, off, 0u, os + slot * L::OT + i * 512);
        }
        if (wave == 3)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                lrs, (__attribute__((address_space(3))) void*)(ls + slot * kBwdQ), 4, (q0 + lane) * 4, 0, 0, 0);
        if (wave == 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                drs, (__attribute__((address_space(3))) void*)(dls + slot * kBwdQ), 4, (q0 + lane) * 4, 0, 0, 0);
    };
    load_tile(0, 0);
    if (n_qt > 1) load_tile(1, 1);

    float csum = 0.0f, asum = 0.0f;
    for (int t = 0; t < n_qt; ++t) {
        const int slot = t & 1;
        // tile t has landed once at most the next tile's loads are outstanding
        if (t + 1 < n_qt) wait_vm_le(n_per_tile);
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int q0 = q_begin + t * kBwdQ;
        const bf16* qt = qs + slot * L::QT;
        const bf16* ot = os + slot * L::OT;
        const float* lt = ls + slot * kBwdQ;
        const float* dt = dls + slot * kBwdQ;
        // one 32-query x 32-key block; masked: causal diagonal or the
        // sequence's last rows (keys past the end need no test: every query
        // at or after them is past the end too)
        auto block = [&](int qb, bool masked) {
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            const bf16* qrow = qt + (qb * 32 + il) * (L::QROW * 8) + half * 8;
            const bf16* orow = ot + (qb * 32 + il) * (L::OROW * 8) + half * 8;
#pragma unroll
            for (int k = 0; k <= KS; ++k)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qrow + k * 16), kf[k], sacc, 0, 0, 0);
#pragma unroll
            for (int k = 0; k < KS; ++k)
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(orow + k * 16), vf[k], pacc, 0, 0, 0);
            // accumulator register 4a + e is query row 8a + 4 half + e of the block
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int rb = qb * 32 + 8 * a + 4 * half;
                const f32x4 lv = *(const f32x4*)(lt + rb);
                const f32x4 dv = *(const f32x4*)(dt + rb);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    const float sv = sacc[r];
                    float p = __builtin_amdgcn_exp2f(sv - lv[e]);
                    if (masked) {
                        const int qi = q0 + rb + e;
                        p = (qi >= kj && qi < ms) ? p : 0.0f;
                    }
                    const float ds = p * (pacc[r] - dv[e]);
                    csum += ds;
                    asum = fmaf(ds, sv, asum);
                }
            }
        };
#pragma unroll
        for (int qb = 0; qb < kBwdQ / 32; ++qb) {
            const int qr0 = q0 + qb * 32;                       // first query row of the block
            if (qr0 + 31 < kb0 || qr0 >= ms) continue;          // every query before this wave's keys, or past the end
            if (qr0 < kb0 + 31 || qr0 + 31 >= ms) block(qb, true);
            else block(qb, false);
        }
        __syncthreads();   // every wave is done with this slot
        if (t + 2 < n_qt) load_tile(t + 2, slot);
    }
    // the two lane halves hold the same key over different query rows
    float cs_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(csum), __float_as_uint(csum), false, false);
        cs_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    float dgl = 0.0f;
    if (half == 0 && kvalid) {
        colsum[(int64_t)h * m_tot + cs0 + kj] = cs_tot;
        dgl = key_score[cs0 + kj] * cs_tot;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        asum += __shfl_xor(asum, o, 64);
        dgl += __shfl_xor(dgl, o, 64);
    }
    if (lane == 0) wsum[wave] = make_float2(dgl, asum);
    __syncthreads();
    if (tid == 0) {
        float2 t = wsum[0];
#pragma unroll
        for (int w = 1; w < kBwdWaves; ++w) {
            t.x += wsum[w].x;
            t.y += wsum[w].y;
        }
        *pout = t;
    }
}

// -------------------------------------------------------------- reduce ----
// dL/ds_j = sum_h g_h C_hj (every q head sees every key of its sequence)
__global__ __launch_bounds__(256) void bwd_ds_kernel(const float* __restrict__ colsum, const float* __restrict__ gain,
                                                     int hq, int64_t m_tot, float* __restrict__ ds) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= m_tot) return;
    float t = 0.0f;
    for (int h = 0; h < hq; ++h) t = fmaf(gain[h], colsum[(int64_t)h * m_tot + j], t);
    ds[j] = t;
}

// per head: dL/dg_h = sum of the (s C) partials; T_h = ln 2 * A_h - g_h dL/dg_h
__global__ __launch_bounds__(256) void bwd_head_kernel(const float2* __restrict__ part, const float* __restrict__ gain,
                                                       int n_part, float* __restrict__ dg, float* __restrict__ th) {
    __shared__ float2 red[4];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float a = 0.0f, c = 0.0f;
    for (int i = tid; i < n_part; i += 256) {
        const float2 x = part[(int64_t)h * n_part + i];
        a += x.x;
        c += x.y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o, 64);
        c += __shfl_xor(c, o, 64);
    }
    if (lane == 0) red[w] = make_float2(a, c);
    __syncthreads();
    if (tid == 0) {
        const float dgh = (red[0].x + red[1].x) + (red[2].x + red[3].x);
        const float ah = (red[0].y + red[1].y) + (red[2].y + red[3].y);
        dg[h] = dgh;
        th[h] = kLn2 * ah - gain[h] * dgh;
    }
}

__global__ __launch_bounds__(64) void bwd_tau_kernel(const float* __restrict__ th, int hq, float tau,
                                                     float* __restrict__ dtau) {
    float t = 0.0f;
    for (int h = threadIdx.x; h < hq; h += 64) t += th[h];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
    if (threadIdx.x == 0) dtau[0] = -t / tau;
}

__global__ __launch_bounds__(64) void bwd_zero_kernel(float* __restrict__ dg, int hq, float* __restrict__ dtau) {
    for (int h = threadIdx.x; h < hq; h += 64) dg[h] = 0.0f;
    if (threadIdx.x == 0) dtau[0] = 0.0f;
}

struct BwdLayout {
    size_t qc, l2, delta, colsum, part, th, total;
};

BwdLayout bwd_layout(int n_seqs, int64_t m_tot, int max_kept, int hq, int d) {
    const int64_t mp = attn_padded_rows(n_seqs, m_tot);
    const int n_kt = (max_kept + kBwdKeys - 1) / kBwdKeys;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdLayout L;
    size_t o = 0;
    L.qc = o;     o += al((size_t)hq * mp * (d + kBwdExtra) * 2);
    L.l2 = o;     o += al((size_t)hq * m_tot * 4);
    L.delta = o;  o += al((size_t)hq * m_tot * 4);
    L.colsum = o; o += al((size_t)hq * m_tot * 4);
    L.part = o;   o += al((size_t)hq * n_seqs * (n_kt > 0 ? n_kt : 1) * 8);
    L.th = o;     o += al((size_t)hq * 4);
    L.total = o;
    return L;
}

template <int D>
int launch_bwd_d(const BwdArgs& a, hipStream_t st) {
    using L = BwdLds<D>;
    const BwdLayout W = bwd_layout(a.n_seqs, a.m_tot, a.max_kept_seqlen, a.hq, D);
    char* w = (char*)a.ws;
    bf16* qc = (bf16*)(w + W.qc);
    float* l2 = (float*)(w + W.l2);
    float* delta = (float*)(w + W.delta);
    float* colsum = (float*)(w + W.colsum);
    float2* part = (float2*)(w + W.part);
    float* th = (float*)(w + W.th);
    const int grp = a.hq / a.hkv;
    const int n_kt = (a.max_kept_seqlen + kBwdKeys - 1) / kBwdKeys;
    const int64_t nblk = (int64_t)n_kt * a.n_seqs * a.hq;
    if (nblk > 0x7fffffff) return TG_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)(a.mp / 64), a.hq), dim3(256), 0, st, a.q, a.q_stride,
                       a.o, a.dout, a.do_stride, a.lse, a.gain, a.qk_scale_log2, a.ws_cs, (int)a.rope, a.cu_kept,
                       a.n_seqs, a.m_tot, a.hq, a.mp, qc, l2, delta);
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)bwd_main_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)L::SMEM) != hipSuccess)
            return TG_ERR_HIP;
        attr_set = true;
    }
    hipLaunchKernelGGL(bwd_main_kernel<D>, dim3((unsigned)nblk), dim3(kBwdThreads), L::SMEM, st, (const bf16*)qc,
                       a.ws_k, a.v, a.kv_stride, a.dout, a.do_stride, (const float*)l2, (const float*)delta,
                       a.key_score, a.cu_kept, a.n_seqs, a.m_tot, a.hq, grp, a.mp, n_kt, colsum, part);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3((unsigned)((a.m_tot + 255) / 256)), dim3(256), 0, st, (const float*)colsum,
                       a.gain, a.hq, a.m_tot, a.d_score);
    hipLaunchKernelGGL(bwd_head_kernel, dim3((unsigned)a.hq), dim3(256), 0, st, (const float2*)part, a.gain,
                       a.n_seqs * n_kt, a.d_gain, th);
    hipLaunchKernelGGL(bwd_tau_kernel, dim3(1), dim3(64), 0, st, (const float*)th, a.hq, a.tau, a.d_tau);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace

size_t bwd_workspace_bytes(int n_seqs, int64_t m_tot, int max_kept, int hq, int d) {
    return bwd_layout(n_seqs, m_tot, max_kept, hq, d).total;
}

int launch_gate_grads_zero(int hq, float* d_gain, float* d_tau, hipStream_t st) {
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), dim3(64), 0, st, d_gain, hq, d_tau);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

int launch_attn_gate_grads(const BwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 64: return launch_bwd_d<64>(a, st);
        case 128: return launch_bwd_d<128>(a, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

}  // namespace tg
