// Gate MLP score of every token.
//
// TokenGate (spke.com article, gate-module phase): a small MLP scores each
// token from its post-attention residual at the gate layer.  Computed here as
//     s_t = w2 . SiLU(W1 x_t + b1) + b2.
//
// bf16 path: one workgroup owns 256 tokens and the whole hidden layer, so the
// hidden activations never leave registers: X.W1^T on 32x32x16 bf16 MFMA with
// fp32 accumulation, then b1 + SiLU + w2-dot in fp32 in the epilogue, reduced
// to one score per token.  Both operands are K-contiguous; 64-column slabs (a
// whole 128-B line of every row) go straight from memory into double-buffered
// LDS.  With
// enough tokens, 256 tokens per workgroup keeps the W1 re-reads (all of W1 per
// workgroup, from L2) equal to the X stream; smaller inputs use 128, and
// inputs too small to give every CU a 128-token tile use 64-token tiles whose
// four waves each take a quarter of the hidden layer.
//
// In tg_gated_select the bf16 kernel also zeroes the counters the top-K's
// four-launch form needs (the workgroups share the sequences out, after their
// scores are stored), so that form launches no clear kernel of its own.
//
// fp32 path: plain FMA (no rounding of the residual), for fp32 residuals.
#include "tg_common.hpp"

namespace tg {
namespace {

// Slab geometry: BK reduction columns per slab; rows padded by one 16-B chunk.
template <int BK>
struct Slab {
    static constexpr int ROW_CHUNKS = BK / 8 + 1;   // 16-B chunks per padded LDS row
    static constexpr int LDK = ROW_CHUNKS * 8;      // padded row (elements): 80 B / 144 B
};
constexpr int kBK = 64;      // reduction slab (a full 128-B line of every X row)
constexpr int kStages = 2;   // slabs in LDS: one in use, one in flight
constexpr int kRowChunks = Slab<kBK>::ROW_CHUNKS;
constexpr int kLdk = Slab<kBK>::LDK;

__device__ __forceinline__ float silu_f32(float a) {
    // a * sigmoid(a) with the hardware reciprocal (1 ulp): a / (1 + 2^(-a log2 e)).
    // For a -> -inf the denominator overflows to +inf and the product is -0.
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
}


// BM tokens per workgroup (BM / 64 row groups of waves x NCG hidden-column
// groups); d_hid = 64 * CB, so a wave holds CBW = 2 CB / NCG 32-wide hidden
// blocks.  Both operands
// are K-contiguous, in two LDS slab buffers (one multiplied while the next
// fills; rows padded by one 16-B chunk).  W1 slabs arrive by
// global_load_lds_dwordx4 (1 KiB of consecutive LDS per instruction, the pad
// slot reloading chunk 0).  With 256-token tiles X comes through registers,
// loaded two slabs ahead and stored to LDS one slab ahead; with 128-token
// tiles X takes the LDS-direct path as well, one slab ahead.
template <int CB, int BM, int NCG>
__global__ __launch_bounds__(BM * NCG, 1) void gate_bf16_kernel(
    const bf16* __restrict__ x, int64_t n, int d_model, int64_t x_stride,
    const bf16* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, float* __restrict__ scores, SelZero sz) {
    constexpr int NT = BM * NCG;                       // threads
    constexpr int CBW = 2 * CB / NCG;                  // 32-wide hidden blocks per wave
    static_assert(CBW * NCG == 2 * CB, "hidden blocks split evenly over the column groups");
    constexpr int NW = NT / 64;                        // waves
    constexpr int NH = 64 * CB;
    constexpr int XI = BM * kRowChunks / 64;           // load instructions per X slab
    constexpr int WI = NH * kRowChunks / 64;           // ... per W1 slab
    constexpr int SLAB = (BM + NH) * kLdk;             // elements per slab buffer
    constexpr int RED_LD = NCG * 32 + 1;               // epilogue partial sums: per token, one per lane
    constexpr int RED_BYTES = BM * RED_LD * 4;
    constexpr int LDS_BYTES = kStages * SLAB * 2 > RED_BYTES ? kStages * SLAB * 2 : RED_BYTES;
    static_assert(BM * kRowChunks % 64 == 0 && NH * kRowChunks % 64 == 0, "whole load instructions");
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    bf16* const lds0 = (bf16*)lds_raw;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: wave tests branch on SCC
    const int wr = wave / NCG, wc = wave % NCG;
    const int il = lane & 31, half = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * BM;
    const int rows = (int)min((int64_t)BM, n - row0);

    // W1 slabs: LDS-direct, instruction g = wave + NW i (g < WI), one 16-B
    // chunk per lane; the pad chunk of each padded row reloads chunk 0.
    constexpr int WPW = (WI + NW - 1) / NW;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w1, (uint32_t)((int64_t)NH * d_model * 2));
    uint32_t woff[WPW];
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
        const int slot = (wave + NW * i) * 64 + lane;
        const int r = slot / kRowChunks, c = slot % kRowChunks;
        woff[i] = (uint32_t)((r * d_model + (c < kBK / 8 ? c : 0) * 8) * 2);
    }
    auto issue_w = [&](int kb, int buf) {
        bf16* dst = lds0 + buf * SLAB + BM * kLdk;
#pragma unroll
        for (int i = 0; i < WPW; ++i)
            if (wave + NW * i < WI) lds_load16_buf(wrs, woff[i], (uint32_t)kb * (kBK * 2), dst + (wave + NW * i) * 512);
    };
    // X slabs: coalesced 16-B loads into registers (8 lanes per 128-B row
    // slice), written to the slab's LDS buffer one iteration later.  With the
    // LDS buffer in flight as well, two X slabs are in flight per workgroup.
    constexpr int XPT = BM * (kBK / 8) / NT;   // 16-B chunks per thread per slab (4)
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(x + row0 * x_stride, (uint32_t)(((int64_t)(rows - 1) * x_stride + d_model) * 2));
    uint32_t xoff[XPT];
    int xlds[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + NT * i;
        const int r = c / (kBK / 8), ch = c % (kBK / 8);
        xoff[i] = (uint32_t)(((int64_t)min(r, rows - 1) * x_stride + ch * 8) * 2);   // rows past the end: clamped
        xlds[i] = r * kLdk + ch * 8;
    }
    // 128-token tiles (one wave per SIMD) keep X on the LDS-direct path,
    // which measured faster there
    constexpr bool XREG = BM == 256;
    const __amdgpu_buffer_rsrc_t xrs_lds = xrs;
    constexpr int XI_W = (XI + NW - 1) / NW;
    uint32_t xloff[XREG ? 1 : XI_W];
#pragma unroll
    for (int i = 0; i < (XREG ? 1 : XI_W); ++i) {
        const int slot = (wave + NW * i) * 64 + lane;
        const int r = slot / kRowChunks, c = slot % kRowChunks;
        xloff[i] = (uint32_t)(((int64_t)min(r, rows - 1) * x_stride + (c < kBK / 8 ? c : 0) * 8) * 2);
    }
    auto issue_x_lds = [&](int kb, int buf) {
        bf16* dst = lds0 + buf * SLAB;
#pragma unroll
        for (int i = 0; i < XI_W; ++i)
            if (wave + NW * i < XI) lds_load16_buf(xrs_lds, xloff[i], (uint32_t)kb * (kBK * 2), dst + (wave + NW * i) * 512);
    };
    auto load_x = [&](int kb, u32x4 (&xr)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) xr[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], kb * (kBK * 2), 0);
    };
    auto store_x = [&](const u32x4 (&xr)[XPT], int buf) {
        bf16* dst = lds0 + buf * SLAB;
#pragma unroll
        for (int i = 0; i < XPT; ++i) *(u32x4*)(dst + xlds[i]) = xr[i];
    };

    f32x16 acc[2][CBW];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) acc[rb][cb] = f32x16{};

    const int nk = d_model / kBK;
    // One slab: 4 k-steps of 2 x CBW MFMAs.  Fragments of k-step ks+1 are read
    // while k-step ks multiplies (two fragment sets); empty volatile asm
    // statements keep those reads ahead of the MFMAs and each MFMA in its
    // slot, so no MFMA waits on a read issued just before it.
    auto mma_slab = [&](int buf) {
        const bf16* xs = lds0 + buf * SLAB + (wr * 64 + il) * kLdk + half * 8;
        const bf16* ws = lds0 + buf * SLAB + BM * kLdk + (wc * CBW * 32 + il) * kLdk + half * 8;
        constexpr int NF = 2 + CBW;   // fragments per k-step: 2 of X, CBW of W1
        auto frag = [&](int ks, int f) -> bf16x8 {
            return f < 2 ? *(const bf16x8*)(xs + f * 32 * kLdk + ks * 16)
                         : *(const bf16x8*)(ws + (f - 2) * 32 * kLdk + ks * 16);
        };
        bf16x8 fr[2][NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) fr[0][f] = frag(0, f);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int c = ks & 1;
#pragma unroll
            for (int m = 0; m < 2 * CBW; ++m) {
                if (ks + 1 < kBK / 16 && m < NF) {
                    fr[c ^ 1][m] = frag(ks + 1, m);
                    __asm__ volatile("" ::: "memory");
                }
                const int rb = m / CBW, cb = m % CBW;
                __asm__ volatile("" : "+v"(fr[c][rb]), "+v"(fr[c][2 + cb]));
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[c][rb], fr[c][2 + cb], acc[rb][cb], 0, 0, 0);
            }
            // fewer MFMAs than fragments (CBW = 1): read the rest now
#pragma unroll
            for (int f = 2 * CBW; f < NF; ++f)
                if (ks + 1 < kBK / 16) fr[c ^ 1][f] = frag(ks + 1, f);
        }
    };
    // Iteration kb computes slab kb from LDS buffer kb % 2 while W1(kb+1)
    // lands in the other buffer and X(kb+2) loads into the registers X(kb)
    // came through; at its end X(kb+1), loaded since the previous iteration,
    // is stored from registers into the other buffer.  Each X slab thus has
    // two iterations to arrive.
    auto step = [&](int kb, u32x4 (&xcur)[XPT], u32x4 (&xnext)[XPT]) {
        const int buf = kb & 1;
        if (kb + 1 < nk) issue_w(kb + 1, buf ^ 1);
        if (kb + 2 < nk) load_x(kb + 2, xcur);
        mma_slab(buf);
        if (kb + 1 < nk) store_x(xnext, buf ^ 1);
        // W1(kb+1) (issued before X(kb+2)) must land; X(kb+2) may stay in flight
        if (kb + 2 < nk) wait_vm_le(XPT);
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if constexpr (XREG) {
        u32x4 xa[XPT], xb[XPT];
        load_x(0, xa);
        if (nk > 1) load_x(1, xb);
        issue_w(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        store_x(xa, 0);
        __syncthreads();
        for (int kb = 0; kb < nk; kb += 2) {
            step(kb, xa, xb);
            if (kb + 1 < nk) step(kb + 1, xb, xa);
        }
    } else {
        // both operands LDS-direct, one slab in flight while one is consumed
        issue_x_lds(0, 0);
        issue_w(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int kb = 0; kb < nk; ++kb) {
            if (kb + 1 < nk) {
                issue_x_lds(kb + 1, (kb + 1) & 1);
                issue_w(kb + 1, (kb + 1) & 1);
            }
            mma_slab(kb & 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // Epilogue: per token, sum over this wave's hidden units of SiLU(a + b1) * w2.
    // acc[rb][cb][r] = hidden unit n = wc*CBW*32 + cb*32 + il of token
    // wr*64 + rb*32 + (r/4)*8 + half*4 + r%4.
    float bias1[CBW], wout[CBW];
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
        const int nidx = wc * CBW * 32 + cb * 32 + il;
        bias1[cb] = b1 ? b1[nidx] : 0.0f;
        wout[cb] = w2[nidx];
    }
    float* red = (float*)lds_raw;   // [BM][RED_LD] partial sums, aliases the slab buffers
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) p += silu_f32(acc[rb][cb][r] + bias1[cb]) * wout[cb];
            const int tok = wr * 64 + rb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            red[tok * RED_LD + wc * 32 + il] = p;
        }
    }
    __syncthreads();
    // NCG threads per token, 32 partials each, then shuffles
    {
        const int tok = tid / NCG, part = tid % NCG;
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) sum += red[tok * RED_LD + part * 32 + j];
#pragma unroll
        for (int o = 1; o < NCG; o <<= 1) sum += __shfl_xor(sum, o, 64);
        if (part == 0 && row0 + tok < n) scores[row0 + tok] = sum + b2;
    }
    // the selector's counters (the selector's kernels all run after this one)
    if (sz.base)
        for (int s = blockIdx.x; s < sz.n_seqs; s += gridDim.x)
            if (seq_selects(sz.db[s], sz.de[s], sz.kd[s])) {
                u32x4* p = (u32x4*)(sz.base + (int64_t)s * sz.stride);
                for (int i = tid; i < sz.words / 4; i += NT) p[i] = u32x4{0u, 0u, 0u, 0u};
            }
}

template <int CB, int BM, int NCG>
int launch_gate_tile(const bf16* x, int64_t n, int d_model, int64_t x_stride, const bf16* w1,
                     const float* b1, const float* w2, float b2, float* scores, const SelZero& sz,
                     hipStream_t st) {
    constexpr int NH = 64 * CB;
    constexpr size_t slab = (size_t)(BM + NH) * kLdk * 2;
    constexpr size_t red = (size_t)BM * (NCG * 32 + 1) * 4;
    constexpr size_t shm = kStages * slab > red ? kStages * slab : red;
    static std::atomic<uint64_t> lds_set{0};
    if (const int e = set_dyn_lds_once((const void*)gate_bf16_kernel<CB, BM, NCG>, (int)shm, lds_set)) return e;
    const dim3 grid((unsigned)((n + BM - 1) / BM));
    hipLaunchKernelGGL((gate_bf16_kernel<CB, BM, NCG>), grid, dim3(BM * NCG), shm, st, x, n, d_model, x_stride,
                       w1, b1, w2, b2, scores, sz);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

template <int CB>
int launch_gate_cb(const bf16* x, int64_t n, int d_model, int64_t x_stride, const bf16* w1,
                   const float* b1, const float* w2, float b2, float* scores, const SelZero& sz,
                   hipStream_t st) {
    // 256-token tiles once there are at least two per CU (256 CUs); 64-token
    // tiles of four waves (each 64 tokens x a quarter of the hidden layer)
    // while 128-token tiles would leave CUs idle; else 128
    if (n >= (int64_t)256 * 256 * 2)
        return launch_gate_tile<CB, 256, 2>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
    if constexpr (CB % 2 == 0)
        if (n < (int64_t)128 * 256)
            return launch_gate_tile<CB, 64, 4>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
    return launch_gate_tile<CB, 128, 2>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
}

// fp32 residuals: 4 tokens per workgroup staged in LDS, threads stride over
// hidden units, fp32 FMA throughout.
constexpr int kF32Tok = 4;
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float* __restrict__ x, int64_t n, int d_model, int64_t x_stride,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, int d_hid, float* __restrict__ scores) {
    extern __shared__ float xs[];   // [kF32Tok][d_model]
    __shared__ float red[kF32Tok][256];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kF32Tok;
    for (int i = tid; i < kF32Tok * d_model; i += 256) {
        const int tt = i / d_model, c = i % d_model;
        const int64_t row = t0 + tt < n ? t0 + tt : n - 1;
        xs[i] = x[row * x_stride + c];
    }
    __syncthreads();
    float part[kF32Tok] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int h = tid; h < d_hid; h += 256) {
        const float* __restrict__ wr = w1 + (int64_t)h * d_model;
        float a[kF32Tok] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = 0; c < d_model; c += 4) {
            const float4 wv = *(const float4*)(wr + c);
#pragma unroll
            for (int tt = 0; tt < kF32Tok; ++tt) {
                const float* xr = xs + tt * d_model + c;
                a[tt] = fmaf(wv.x, xr[0], a[tt]);
                a[tt] = fmaf(wv.y, xr[1], a[tt]);
                a[tt] = fmaf(wv.z, xr[2], a[tt]);
                a[tt] = fmaf(wv.w, xr[3], a[tt]);
            }
        }
        const float bb = b1 ? b1[h] : 0.0f, ww = w2[h];
#pragma unroll
        for (int tt = 0; tt < kF32Tok; ++tt) part[tt] += silu_f32(a[tt] + bb) * ww;
    }
#pragma unroll
    for (int tt = 0; tt < kF32Tok; ++tt) red[tt][tid] = part[tt];
    __syncthreads();
    if (tid < 64 * kF32Tok) {
        const int tt = tid >> 6, l = tid & 63;
        float s = red[tt][l] + red[tt][l + 64] + red[tt][l + 128] + red[tt][l + 192];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
        if (l == 0 && t0 + tt < n) scores[t0 + tt] = s + b2;
    }
}

}  // namespace

int launch_gate_bf16(const bf16* x, int64_t n, int d_model, int64_t x_stride, const bf16* w1,
                     const float* b1, const float* w2, float b2, int d_hid, float* scores,
                     hipStream_t st, const SelZero* zero) {
    if (n == 0) return TG_OK;
    const SelZero sz = zero ? *zero : SelZero{};
    switch (d_hid) {
        case 64: return launch_gate_cb<1>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
        case 128: return launch_gate_cb<2>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
        case 192: return launch_gate_cb<3>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
        case 256: return launch_gate_cb<4>(x, n, d_model, x_stride, w1, b1, w2, b2, scores, sz, st);
        default: return TG_ERR_UNSUPPORTED;
    }
}

int launch_gate_f32(const float* x, int64_t n, int d_model, int64_t x_stride, const float* w1,
                    const float* b1, const float* w2, float b2, int d_hid, float* scores,
                    hipStream_t st) {
    if (n == 0) return TG_OK;
    const dim3 grid((unsigned)((n + kF32Tok - 1) / kF32Tok));
    const size_t shm = (size_t)kF32Tok * d_model * sizeof(float);
    hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(256), shm, st, x, n, d_model, x_stride, w1, b1,
                       w2, b2, d_hid, scores);
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
}

}  // namespace tg
