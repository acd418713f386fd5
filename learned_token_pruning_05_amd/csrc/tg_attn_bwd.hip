// Gate-side gradients of token-gated attention: dL/ds_j, dL/dg_h, dL/dtau.
//
// TokenGate ([ES] "¿Qué es la atención con control de acceso por tokens…?"):
// the per-head gain and the temperature are learned, and the bias on the
// attention logits is the path by which the loss reaches the gate's scores.
// With l_ij = <q~_i, k~_j> / (sqrt(D) tau) + g_h s_j and dO = dL/dO:
//     P = softmax_j(l),  dP_ij = <dO_i, v_j>,  Delta_i = <dO_i, O_i>,
//     dS_ij = P_ij (dP_ij - Delta_i)                          (= dL/dl_ij)
//     dL/ds_j = sum_h g_h C_hj,   dL/dg_h = sum_j s_j C_hj,   C_hj = sum_i dS_hij
//     dL/dtau = -(ln 2 / tau) sum_h A_h,    A_h = sum_ij dS_hij Z_hij
// where Z = <q~_i, k~_j> log2(e) / (sqrt(D) tau) is the q.k part of the logit
// in the log2 units the MFMAs work in.  (Delta_i = sum_j P_ij dP_ij because
// O_i = sum_j P_ij v_j.)
//
// Z comes out of the data k-steps of the q.k MFMA chain; its last k-step
// (the extra columns) continues from Z into S' = Z + g_h s_j log2(e) - LSE2_i,
// and dP' = dP - Delta_i comes out of the dO.V MFMAs: the prepared queries
// carry (g_hi, g_hi, g_lo, -LSE2_hi, -LSE2_lo) against the key cache's
// (s_hi, s_lo, s_hi, 1, 1), and the prepared dO rows carry (-Delta_hi,
// -Delta_lo) against a (1, 1) key fragment, so per element the VALU does
// P = exp2(S'), dS = P dP', two sums.  The temperature sum takes Z itself, not
// S': with the stored bf16 O the rows of dS do not sum exactly to zero, and a
// per-row constant such as LSE2_i would then leak into the sum.
//
// Kernels:
//   prep    Q' and dO' rows [Hq][padded row][D+16] in the key cache's padded
//           per-sequence layout (rows without a token are zero): queries
//           rotated on their positions and scaled by log2(e)/(sqrt(D) tau);
//   main    key-outer: a workgroup owns 256 keys (32 per wave) of one q head,
//           keeps their K' and V operand fragments in registers and streams
//           every query tile at or after its keys (Q' and dO', 64 rows) through
//           a four-slot LDS ring, loaded three tiles ahead.  S' = Q'.K'^T and dP' = dO'.V'^T run on
//           32x32x16 bf16 MFMA; the accumulator layout puts one key per lane,
//           so C_hj is an in-lane sum over the query rows (no atomics,
//           deterministic), and the workgroup leaves C_hj plus its partial
//           sums of s_j C_hj and of dS Z.  When the key blocks are fewer than
//           the CUs, each block's query tiles are cut into up to four ranges,
//           one workgroup each, so no workgroup walks all of them;
//   reduce  one launch: dL/ds over heads (and query ranges, in order), and
//           per head dL/dg and dL/dtau.
#include <math.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <type_traits>
#include <vector>

#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBwdThreads = 512;
constexpr int kBwdWaves = 8;
constexpr int kBwdKeys = 32 * kBwdWaves;   // keys per main workgroup
constexpr int kBwdSlots = 4;               // LDS ring slots (tiles loaded 3 ahead)
constexpr int kBwdQ = 64;                  // query rows per tile
constexpr int kBwdExtra = 16;              // bias columns, as in K'
constexpr int kBwdMaxSplit = 4;            // query ranges per key block, at most

template <int D>
struct BwdLds {
    // Q' and dO' tiles arrive by 16-B LDS-direct loads (64 lanes x 16 B per
    // instruction); rows are padded by one chunk so that the 16-B operand
    // reads of eight consecutive rows fall on distinct bank groups (pad slots
    // hold a duplicate, never read)
    static constexpr int KD = D + kBwdExtra;
    static constexpr int CH = KD / 8;             // 16-B chunks per row
    static constexpr int ROW = CH + 1;
    static constexpr int INSTR = kBwdQ * ROW / 64;   // load instructions per tile
    static_assert(kBwdQ * ROW % 64 == 0, "tiles must be whole load instructions");
    static constexpr int T = kBwdQ * ROW * 8;     // elements per tile
    static constexpr size_t SMEM = (size_t)kBwdSlots * 2 * T * 2;   // Q' and dO' per slot
    // load instructions one wave issues per tile (at most 6: two tiles ahead
    // stay within the 12 outstanding loads wait_vm_le handles)
    __device__ static int per_wave(int w) { return 2 * ((INSTR - w + kBwdWaves - 1) / kBwdWaves); }
    static_assert(2 * 2 * ((INSTR + kBwdWaves - 1) / kBwdWaves) <= 12, "too many loads in flight per wave");
};

// ---------------------------------------------------------------- prep ----
// One workgroup per (q head, 64 padded rows).  Four threads per row copy dO
// into dO' while computing Delta = <dO, O>, and LSE2 = LSE log2(e); then the
// Q' items (row, rotate-half chunk pair), lanes over chunk pairs, with the
// (cos, sin) table of the key pre-pass, and the extra columns.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const bf16* __restrict__ q, int64_t q_stride, const bf16* __restrict__ o, const bf16* __restrict__ dout,
    int64_t do_stride, const float* __restrict__ lse, const float* __restrict__ gain, float qk_scale_log2,
    const float2* __restrict__ ws_cs, int rope, const int* __restrict__ cu_kept, int n_seqs, int64_t m_tot,
    int hq, int64_t mp, bf16* __restrict__ qc, bf16* __restrict__ oc) {
    constexpr int HALF = D / 2, KD = D + kBwdExtra, NPAIR = D / 16, NC8 = D / 8;
    __shared__ int tok[64];
    __shared__ float rowc[2][64];   // Delta, LSE2
    const int tid = threadIdx.x;
    // head fastest: the heads of a row block run side by side and share the
    // (cos, sin) rows and the O / dO row segments through the caches
    const int h = blockIdx.x;
    const int64_t p0 = (int64_t)blockIdx.y * 64;
    if (tid < 64) {
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
    // Every load of the workgroup is issued before the first is used (one
    // memory round trip after the token lookup): the dO and O row segments,
    // the LSE, and the Q' items' q chunks and (cos, sin) rows.  The loads take
    // no branch: a padding row reads row 0 (m_tot > 0 here), whose values are
    // not used.
    constexpr int KIT = 64 * NPAIR / 256;
    constexpr int KIT1 = KIT > 0 ? KIT : 1;
    const int r = tid >> 2, part = tid & 3;   // four threads per dO / O row
    const int m = tok[r];
    const int64_t mr = max(m, 0);
    bf16x8 dx[NC8 / 4], oy[NC8 / 4];
    {
        // instruction i of the row's threads covers chunks 4i..4i+3 (64 contiguous bytes)
        const bf16* dr = dout + mr * do_stride + (int64_t)h * D;
        const bf16* orr = o + (mr * hq + h) * D;
#pragma unroll
        for (int i = 0; i < NC8 / 4; ++i) {
            dx[i] = *(const bf16x8*)(dr + (4 * i + part) * 8);
            oy[i] = *(const bf16x8*)(orr + (4 * i + part) * 8);
        }
    }
    const float lse_r = lse[(int64_t)h * m_tot + mr];
    bf16x8 qa1[KIT1], qa2[KIT1];
    float4 csv[KIT1][4];
#pragma unroll
    for (int i = 0; i < KIT1; ++i) {
        const int item = min(tid + 256 * i, 64 * NPAIR - 1);
        const int r2 = item / NPAIR, p = item % NPAIR;
        const int64_t m2 = max(tok[r2], 0);
        const bf16* src = q + m2 * q_stride + (int64_t)h * D;
        qa1[i] = *(const bf16x8*)(src + p * 8);
        qa2[i] = *(const bf16x8*)(src + HALF + p * 8);
        const float4* cs = (const float4*)(ws_cs + m2 * HALF + p * 8);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)   // (cos, sin) of frequencies 2 e2, 2 e2 + 1
            csv[i][e2] = rope ? cs[e2] : make_float4(1.0f, 0.0f, 1.0f, 0.0f);
    }
    {
        // dO is copied into the data columns of dO' as it is used for Delta
        bf16* odst = oc + ((int64_t)h * mp + p0 + r) * KD;
        float acc = 0.0f;
        if (m >= 0) {
#pragma unroll
            for (int i = 0; i < NC8 / 4; ++i) {
                *(bf16x8*)(odst + (4 * i + part) * 8) = dx[i];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)dx[i][e], (float)oy[i][e], acc);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NC8 / 4; ++i) *(bf16x8*)(odst + (4 * i + part) * 8) = bf16x8{};
        }
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        if (part == 0) {
            rowc[0][r] = acc;
            rowc[1][r] = m >= 0 ? lse_r * kLog2e : 0.0f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KIT1; ++i) {
        const int item = tid + 256 * i;
        if (KIT == 0 && item >= 64 * NPAIR) break;
        const int r2 = item / NPAIR, p = item % NPAIR;
        const int m2 = tok[r2];
        bf16x8 x1 = bf16x8{}, x2 = bf16x8{};
        if (m2 >= 0) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float4 c = csv[i][e2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = 2 * e2 + u;
                    const float cn = u ? c.z : c.x, sn = u ? c.w : c.y;
                    const float a = (float)qa1[i][e], b = (float)qa2[i][e];
                    x1[e] = (bf16)((a * cn - b * sn) * qk_scale_log2);
                    x2[e] = (bf16)((b * cn + a * sn) * qk_scale_log2);
                }
            }
        }
        const int64_t row = (int64_t)h * mp + p0 + r2;
        bf16* dst = qc + row * KD;
        *(bf16x8*)(dst + p * 8) = x1;
        *(bf16x8*)(dst + HALF + p * 8) = x2;
        if (p == 0) {
            // Q' (g_hi, g_hi, g_lo, -LSE2_hi, -LSE2_lo), dO' (-Delta_hi, -Delta_lo)
            bf16x8 qx = bf16x8{}, ox = bf16x8{};
            if (m2 >= 0) {
                const float g = gain[h] * kLog2e;
                const bf16 gh = (bf16)g;
                qx[0] = gh;
                qx[1] = gh;
                qx[2] = (bf16)(g - (float)gh);
                const float l2 = -rowc[1][r2];
                const bf16 lh = (bf16)l2;
                qx[3] = lh;
                qx[4] = (bf16)(l2 - (float)lh);
                const float dl = -rowc[0][r2];
                const bf16 dh = (bf16)dl;
                ox[0] = dh;
                ox[1] = (bf16)(dl - (float)dh);
            }
            *(bf16x8*)(dst + D) = qx;
            *(bf16x8*)(dst + D + 8) = bf16x8{};
            bf16* odst = oc + row * KD;
            *(bf16x8*)(odst + D) = ox;
            *(bf16x8*)(odst + D + 8) = bf16x8{};
        }
    }
}

// ---------------------------------------------------------------- main ----
// Block b: q head b % hq (fastest, so that the workgroups of one head sit on
// one XCD's L2 and follow each other down the same Q'/dO' rows), then the
// sequence, then the key tile (tile 0, with the most query rows, first).
template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_main_kernel(
    const bf16* __restrict__ qc, const bf16* __restrict__ oc, const bf16* __restrict__ ws_k,
    const bf16* __restrict__ v, int64_t kv_stride, const float* __restrict__ key_score,
    const int* __restrict__ cu_kept, int n_seqs, int64_t m_tot, int hq, int grp, int64_t mp, int n_kt,
    int nsplit, float* __restrict__ colsum, float2* __restrict__ part) {
    using L = BwdLds<D>;
    constexpr int KD = L::KD;
    constexpr int KS = D / 16;   // k-steps of the data columns; one more for the extra columns
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* const qs = (bf16*)smem;                   // [slots][T] Q'
    bf16* const os = qs + kBwdSlots * L::T;         // [slots][T] dO'
    __shared__ float2 wsum[kBwdWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 31, half = lane >> 5;

    // block = ((s * n_kt + kt) * nsplit + split) * hq + h: query range
    // `split` of the key block kt of sequence s, for q head h (heads fastest)
    const int b = blockIdx.x;
    const int h = b % hq;
    const int rest = b / hq;
    const int split = rest % nsplit;
    const int s = rest / nsplit / n_kt;
    const int kt = rest / nsplit % n_kt;
    const int cs0 = cu_kept[s];
    const int ms = cu_kept[s + 1] - cs0;
    const int key0 = kt * kBwdKeys;
    // partials split-major: part[h][split][s][kt], colsum[split][h][key]
    float2* const pout = part + (((int64_t)h * nsplit + split) * n_seqs + s) * n_kt + kt;
    float* const cout = colsum + ((int64_t)split * hq + h) * m_tot + cs0;
    if (key0 >= ms) {
        if (tid == 0) *pout = make_float2(0.0f, 0.0f);
        return;
    }
    const int hk = h / grp;
    const int64_t prow0 = padded_seq_start(cs0, s);
    const int kb0 = key0 + 32 * wave;   // this wave's first key
    const int kj = kb0 + il;            // this lane's key
    const bool kvalid = kj < ms;

    // this wave's K' and V' fragments as B operands (lane j + 32 (k / 8) holds
    // B[k..k+7][j]); V' is V with the columns (1, 1, 0...) appended; keys past
    // the sequence end are zero and masked
    bf16x8 kf[KS + 1], vf[KS + 1];
    {
        const bf16* kr = ws_k + ((int64_t)hk * mp + prow0 + (kvalid ? kj : 0)) * KD + half * 8;
        const bf16* vr = v + (int64_t)(cs0 + (kvalid ? kj : 0)) * kv_stride + (int64_t)hk * D + half * 8;
#pragma unroll
        for (int t = 0; t <= KS; ++t) kf[t] = kvalid ? *(const bf16x8*)(kr + t * 16) : bf16x8{};
#pragma unroll
        for (int t = 0; t < KS; ++t) vf[t] = kvalid ? *(const bf16x8*)(vr + t * 16) : bf16x8{};
        vf[KS] = bf16x8{};
        if (kvalid && half == 0) {
            vf[KS][0] = (bf16)1.0f;
            vf[KS][1] = (bf16)1.0f;
        }
    }

    // query tiles from the one holding key0 to the end of the sequence; the
    // padded layout keeps every tile row inside this head's rows
    const int q_begin = key0 & ~(kBwdQ - 1);
    const int n_qt_all = (ms - q_begin + kBwdQ - 1) / kBwdQ;
    // this split's tiles [t_lo, t_lo + n_qt), relative to q_begin; a split
    // with none leaves zero partials
    const int t_lo = (int)((int64_t)split * n_qt_all / nsplit);
    const int n_qt = (int)((int64_t)(split + 1) * n_qt_all / nsplit) - t_lo;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc(qc + ((int64_t)h * mp + prow0) * KD, (uint32_t)((mp - prow0) * KD * 2));
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(oc + ((int64_t)h * mp + prow0) * KD, (uint32_t)((mp - prow0) * KD * 2));
    const int n_per_tile = L::per_wave(wave);
    auto load_tile = [&](int t, int slot) {
        const uint32_t so = (uint32_t)(q_begin + (t_lo + t) * kBwdQ) * (KD * 2);
        for (int i = wave; i < L::INSTR; i += kBwdWaves) {
            const int sl = i * 64 + lane;
            const int r = sl / L::ROW, c = sl % L::ROW;
            const uint32_t off = (uint32_t)((r * KD + (c < L::CH ? c : 0) * 8) * 2);
            lds_load16_buf(qrs, off, so, qs + slot * L::T + i * 512);
            lds_load16_buf(ors, off, so, os + slot * L::T + i * 512);
        }
    };
#pragma unroll
    for (int t = 0; t < kBwdSlots - 1; ++t)
        if (t < n_qt) load_tile(t, t);

    float csum = 0.0f, asum = 0.0f;
    // Software pipeline over this wave's 32-query blocks.  Block qb of a tile
    // accumulates into set qb (sA/pA or sB/pB); each step issues the 18 MFMAs
    // of one block (D = 128) with the element work of the block before it,
    // whose accumulators are the other set, spread over them.  A block's
    // element work may thus run after its tile's slot is released: it needs
    // only registers.  The wave's active blocks are consecutive: the first is
    // its diagonal block (query rows kb0..kb0+31), the last holds the
    // sequence's last row.  So inside the loop only the diagonal block needs
    // a mask: right after its MFMAs its causally hidden logits are set to
    // -1e30 (exp2 gives 0, so dS = 0 there).  The
    // last block's element work, after the loop, masks rows past the end.
    // Sets start at zero, so the element work of the step before the first
    // block adds exactly 0 (P = 1, dP' = 0).
    f32x16 sA = f32x16{}, pA = f32x16{}, zA = f32x16{}, sB = f32x16{}, pB = f32x16{}, zB = f32x16{};
    constexpr int NI = 2 * (KS + 1);   // MFMAs per block
    constexpr int PF = 4;              // operand reads ahead of their MFMA
    auto elem = [&](const f32x16& sv, const f32x16& pv, const f32x16& zv, int r, float& cs, float& as) {
        const float p = __builtin_amdgcn_exp2f(sv[r]);
        const float ds = p * pv[r];
        cs += ds;
        as = fmaf(ds, zv[r], as);
    };
    auto step = [&](auto QB, const bf16* qt, const bf16* ot) {
        constexpr int qb = decltype(QB)::value;
        f32x16& sc = qb ? sB : sA;
        f32x16& pc = qb ? pB : pA;
        f32x16& zc = qb ? zB : zA;
        f32x16& sp = qb ? sA : sB;
        f32x16& pp = qb ? pA : pB;
        f32x16& zp = qb ? zA : zB;
        float& cs = csum;   // named here so that the generic lambda captures them
        float& as = asum;
        const bf16* qrow = qt + (qb * 32 + il) * (L::ROW * 8) + half * 8;
        const bf16* orow = ot + (qb * 32 + il) * (L::ROW * 8) + half * 8;
        auto frag = [&](int i) -> bf16x8 {
            return i <= KS ? *(const bf16x8*)(qrow + i * 16) : *(const bf16x8*)(orow + (i - KS - 1) * 16);
        };
        bf16x8 ring[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) ring[i] = frag(i);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bf16x8 x = ring[i % PF];
            if (i + PF < NI) ring[i % PF] = frag(i + PF);
            // the memory clobber keeps the read above from sinking toward its
            // use; re-defining the MFMA's LDS operand here keeps the MFMA from
            // rising toward its read
            __asm__ volatile("" ::: "memory");
            __asm__ volatile("" : "+v"(x));
            if (i == 0) zc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, kf[0], f32x16{}, 0, 0, 0);
            else if (i < KS) zc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, kf[i], zc, 0, 0, 0);
            else if (i == KS) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, kf[KS], zc, 0, 0, 0);
            else if (i == KS + 1) pc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, vf[0], f32x16{}, 0, 0, 0);
            else pc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, vf[i - KS - 1], pc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r * NI / 16 != i) continue;
                __asm__ volatile("" : "+v"(sp[r]), "+v"(pp[r]), "+v"(zp[r]));   // not before this MFMA
                elem(sp, pp, zp, r, cs, as);
                __asm__ volatile("" ::"v"(cs), "v"(as));           // and done before the next
            }
        }
    };
    // the diagonal block: hide key j from query rows before it
    auto diag_mask = [&](f32x16& sv) {
        const int lo = il - 4 * half;   // row k of the block (minus 4 half) sees key il iff k >= lo
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + (r & 3);
            sv[r] = k >= lo ? sv[r] : -1e30f;
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int last_set = -1, last_qr0 = 0;
    for (int t = 0; t < n_qt; ++t) {
        const int slot = t % kBwdSlots;
        // tile t has landed once at most the later tiles' loads (up to two)
        // are outstanding; after the barrier every wave's part of it has
        // landed and every wave is past tile t-1, whose slot takes tile t+3
        wait_vm_le(min(kBwdSlots - 2, n_qt - 1 - t) * n_per_tile);
        __syncthreads();
        if (t + kBwdSlots - 1 < n_qt) load_tile(t + kBwdSlots - 1, (t + kBwdSlots - 1) % kBwdSlots);
        const int q0 = q_begin + (t_lo + t) * kBwdQ;
        const bf16* qt = qs + slot * L::T;
        const bf16* ot = os + slot * L::T;
        if (q0 + 31 >= kb0 && q0 < ms) {
            step(I0{}, qt, ot);
            if (q0 == kb0) diag_mask(sA);
            last_set = 0;
            last_qr0 = q0;
        }
        if (q0 + 63 >= kb0 && q0 + 32 < ms) {
            step(I1{}, qt, ot);
            if (q0 + 32 == kb0) diag_mask(sB);
            last_set = 1;
            last_qr0 = q0 + 32;
        }
    }
    // element work of the last block: rows past the sequence end are hidden
    if (last_set >= 0) {
        const int hi = ms - last_qr0 - 4 * half;
        const f32x16& sv = last_set ? sB : sA;
        const f32x16& pv = last_set ? pB : pA;
        const f32x16& zv = last_set ? zB : zA;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int k = 8 * (r >> 2) + (r & 3);
            const float p = k < hi ? __builtin_amdgcn_exp2f(sv[r]) : 0.0f;
            const float ds = p * pv[r];
            csum += ds;
            asum = fmaf(ds, zv[r], asum);
        }
    }
    // the two lane halves hold the same key over different query rows
    float cs_tot;
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(csum), __float_as_uint(csum), false, false);
        cs_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    float dgl = 0.0f;
    if (half == 0 && kvalid) {
        cout[kj] = cs_tot;
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
// One launch: blocks 0..n_ds-1 write dL/ds_j = sum_h g_h C_hj (every q head
// sees every key of its sequence; C_hj summed over the query ranges in
// order); block n_ds reduces the per-block partials of each head to dL/dg_h
// and A_h, then dL/dtau = -(ln 2 / tau) sum_h A_h.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ colsum,
                                                         const float2* __restrict__ part,
                                                         const float* __restrict__ gain, int hq, int64_t m_tot,
                                                         int nsplit, int n_part, float tau, float* __restrict__ ds,
                                                         float* __restrict__ dg, float* __restrict__ dtau) {
    const int tid = threadIdx.x;
    if (blockIdx.x + 1 < gridDim.x) {
        const int64_t j = (int64_t)blockIdx.x * 256 + tid;
        if (j >= m_tot) return;
        // every column sum of a group of 16 heads is loaded before the first is
        // used; the sums run in head order, each head's ranges in range order
        constexpr int HB = 16;
        float t = 0.0f;
        for (int h0 = 0; h0 < hq; h0 += HB) {
            float x[kBwdMaxSplit][HB];
#pragma unroll
            for (int sp = 0; sp < kBwdMaxSplit; ++sp)
#pragma unroll
                for (int u = 0; u < HB; ++u)
                    x[sp][u] = sp < nsplit && h0 + u < hq ? colsum[((int64_t)sp * hq + h0 + u) * m_tot + j] : 0.0f;
#pragma unroll
            for (int u = 0; u < HB; ++u) {
                if (h0 + u >= hq) break;
                float c = x[0][u];
#pragma unroll
                for (int sp = 1; sp < kBwdMaxSplit; ++sp)
                    if (sp < nsplit) c += x[sp][u];
                t = fmaf(gain[h0 + u], c, t);
            }
        }
        ds[j] = t;
        return;
    }
    // heads spread over the four waves, partials over the lanes
    __shared__ float tw[4];
    const int lane = tid & 63, w = tid >> 6;
    float tsum = 0.0f;
    for (int h = w; h < hq; h += 4) {
        float a = 0.0f, c = 0.0f;
        for (int i = lane; i < n_part; i += 64) {
            const float2 x = part[(int64_t)h * n_part + i];
            a += x.x;
            c += x.y;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            a += __shfl_xor(a, o, 64);
            c += __shfl_xor(c, o, 64);
        }
        if (lane == 0) dg[h] = a;
        tsum += kLn2 * c;
    }
    if (lane == 0) tw[w] = tsum;
    __syncthreads();
    if (tid == 0) dtau[0] = -((tw[0] + tw[1]) + (tw[2] + tw[3])) / tau;
}

__global__ __launch_bounds__(64) void bwd_zero_kernel(float* __restrict__ dg, int hq, float* __restrict__ dtau) {
    for (int h = threadIdx.x; h < hq; h += 64) dg[h] = 0.0f;
    if (threadIdx.x == 0) dtau[0] = 0.0f;
}

struct BwdLayout {
    size_t qc, oc, colsum, part, total;
};

BwdLayout bwd_layout(int n_seqs, int64_t m_tot, int max_kept, int hq, int d) {
    const int64_t mp = attn_padded_rows(n_seqs, m_tot);
    const int n_kt = (max_kept + kBwdKeys - 1) / kBwdKeys;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdLayout L;
    size_t o = 0;
    L.qc = o;     o += al((size_t)hq * mp * (d + kBwdExtra) * 2);
    L.oc = o;     o += al((size_t)hq * mp * (d + kBwdExtra) * 2);
    L.colsum = o; o += al((size_t)kBwdMaxSplit * hq * m_tot * 4);
    L.part = o;   o += al((size_t)kBwdMaxSplit * hq * n_seqs * (n_kt > 0 ? n_kt : 1) * 8);
    L.total = o;
    return L;
}

// Query ranges per key block.  A main workgroup fills its CU's LDS, so a
// grid runs one workgroup per CU and later workgroups take the CUs that free
// first, in block order.  The plan simulates that dispatch for 1..4 ranges
// (every sequence taken as long as the longest; a workgroup costs its query
// tiles plus 6 tiles of start-up) and keeps the count with the shortest
// modelled finish, the smallest on a tie.  The start-up constant is fitted to
// the gradient call measured on MI355X at 16k, 32k@5% and 32k@10% with 1-4
// ranges (RMS error 1.7 us; the model picks the measured best in each case).
// Grids of 2 n_cu key blocks or more are not cut.
static int plan_bwd_uncached(int n_seqs, int max_kept, int hq, int n_cu) {
    constexpr int kStartup = 6;
    const int n_kt = (max_kept + kBwdKeys - 1) / kBwdKeys;
    const int64_t nblk1 = (int64_t)n_kt * n_seqs * hq;
    if (n_cu <= 0 || nblk1 == 0 || nblk1 >= 2 * (int64_t)n_cu) return 1;
    int best = 1;
    int64_t best_t = INT64_MAX;
    std::vector<int64_t> slot;
    for (int ns = 1; ns <= kBwdMaxSplit; ++ns) {
        slot.assign(n_cu, 0);   // min-heap of the CUs' finish times
        int64_t finish = 0;
        for (int s = 0; s < n_seqs; ++s)
            for (int kt = 0; kt < n_kt; ++kt) {
                const int nq = (max_kept - kt * kBwdKeys + kBwdQ - 1) / kBwdQ;
                for (int sp = 0; sp < ns; ++sp) {
                    const int len = (sp + 1) * nq / ns - sp * nq / ns + kStartup;
                    for (int h = 0; h < hq; ++h) {
                        std::pop_heap(slot.begin(), slot.end(), std::greater<int64_t>());
                        slot.back() += len;
                        finish = std::max(finish, slot.back());
                        std::push_heap(slot.begin(), slot.end(), std::greater<int64_t>());
                    }
                }
            }
        if (finish < best_t) {
            best_t = finish;
            best = ns;
        }
    }
    return best;
}

static int plan_bwd(int n_seqs, int max_kept, int hq, int n_cu) {
    struct Entry {
        int key[4];
        int nsplit;
    };
    constexpr int kEntries = 16;
    static std::mutex mu;
    static Entry cache[kEntries];
    static int n_used = 0, next = 0;
    const int key[4] = {n_seqs, max_kept, hq, n_cu};
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < n_used; ++i)
            if (std::equal(key, key + 4, cache[i].key)) return cache[i].nsplit;
    }
    const int ns = plan_bwd_uncached(n_seqs, max_kept, hq, n_cu);
    std::lock_guard<std::mutex> g(mu);
    Entry& e = cache[next];
    std::copy(key, key + 4, e.key);
    e.nsplit = ns;
    next = (next + 1) % kEntries;
    n_used = std::min(n_used + 1, kEntries);
    return ns;
}

template <int D>
int launch_bwd_d(const BwdArgs& a, hipStream_t st) {
    using L = BwdLds<D>;
    const BwdLayout W = bwd_layout(a.n_seqs, a.m_tot, a.max_kept_seqlen, a.hq, D);
    char* w = (char*)a.ws;
    bf16* qc = (bf16*)(w + W.qc);
    bf16* oc = (bf16*)(w + W.oc);
    float* colsum = (float*)(w + W.colsum);
    float2* part = (float2*)(w + W.part);
    const int grp = a.hq / a.hkv;
    const int n_kt = (a.max_kept_seqlen + kBwdKeys - 1) / kBwdKeys;
    // small grids cut every key block's query tiles into ranges (plan_bwd);
    // the reduce kernel adds the ranges' column sums and partials in order
    int n_cu = 0;
    if (const int e = device_cu_count(&n_cu)) return e;
    const int nsplit = plan_bwd(a.n_seqs, a.max_kept_seqlen, a.hq, n_cu);
    const int64_t nblk = (int64_t)n_kt * a.n_seqs * a.hq * nsplit;
    if (nblk > 0x7fffffff) return TG_ERR_UNSUPPORTED;
    static std::atomic<uint64_t> lds_set{0};   // before the first launch of the call
    if (const int e = set_dyn_lds_once((const void*)bwd_main_kernel<D>, (int)L::SMEM, lds_set)) return e;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(a.hq, (unsigned)(a.mp / 64)), dim3(256), 0, st, a.q, a.q_stride,
                       a.o, a.dout, a.do_stride, a.lse, a.gain, a.qk_scale_log2, a.ws_cs, (int)a.rope, a.cu_kept,
                       a.n_seqs, a.m_tot, a.hq, a.mp, qc, oc);
    hipLaunchKernelGGL(bwd_main_kernel<D>, dim3((unsigned)nblk), dim3(kBwdThreads), L::SMEM, st, (const bf16*)qc,
                       (const bf16*)oc, a.ws_k, a.v, a.kv_stride, a.key_score, a.cu_kept, a.n_seqs, a.m_tot, a.hq,
                       grp, a.mp, n_kt, nsplit, colsum, part);
    const unsigned n_ds = (unsigned)((a.m_tot + 255) / 256);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(n_ds + 1), dim3(256), 0, st, (const float*)colsum,
                       (const float2*)part, a.gain, a.hq, a.m_tot, nsplit, nsplit * a.n_seqs * n_kt, a.tau,
                       a.d_score, a.d_gain, a.d_tau);
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
