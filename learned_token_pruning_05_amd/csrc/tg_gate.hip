// Gate MLP score of every token.
//
// TokenGate (spke.com article, gate-module phase): a small MLP scores each
// token from its post-attention residual at the gate layer.  Computed here as
//     s_t = w2 . SiLU(W1 x_t + b1) + b2.
//
// bf16 path: one workgroup owns 128 tokens and the whole hidden layer, so the
// hidden activations never leave registers: X.W1^T on 32x32x16 bf16 MFMA with
// fp32 accumulation, then b1 + SiLU + w2-dot in fp32 in the epilogue, reduced
// to one score per token.  Both operands are K-contiguous and staged through
// double-buffered LDS in 32-column slabs.
//
// fp32 path: plain FMA (no rounding of the residual), for fp32 residuals.
#include "tg_common.hpp"

namespace tg {
namespace {

constexpr int kBM = 128;   // tokens per workgroup
constexpr int kBK = 32;    // reduction slab
constexpr int kLdk = kBK + 8;  // padded LDS row (elements): 80 B, conflict-free 16-B reads

__device__ __forceinline__ float silu_f32(float a) {
    // a * sigmoid(a); exp2 of a finite argument, saturating correctly at +-inf.
    return a / (1.0f + __builtin_amdgcn_exp2f(-a * kLog2e));
}

// CB = hidden units per wave / 32; d_hid = 64 * CB; waves arranged 2 (rows) x 2 (cols).
template <int CB>
__global__ __launch_bounds__(256, 2) void gate_bf16_kernel(
    const bf16* __restrict__ x, int64_t n, int d_model, int64_t x_stride,
    const bf16* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    float b2, float* __restrict__ scores) {
    constexpr int NH = 64 * CB;
    constexpr int XCH = kBM * kBK / 8 / 256;   // 16-B chunks of the X slab per thread (2)
    constexpr int WCH = NH * kBK / 8 / 256;    // ... of the W1 slab (CB)
    constexpr int SLAB = (kBM + NH) * kLdk;            // elements per slab buffer
    constexpr int RED_BYTES = kBM * 65 * 4;            // epilogue partial sums
    constexpr int LDS_BYTES = 2 * SLAB * 2 > RED_BYTES ? 2 * SLAB * 2 : RED_BYTES;
    __shared__ __attribute__((aligned(16))) char lds_raw[LDS_BYTES];
    bf16* const lds0 = (bf16*)lds_raw;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int il = lane & 31, half = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * kBM;

    // global -> register staging of one slab
    u32x4 xr[XCH], wreg[WCH];
    auto load_slab = [&](int kb) {
        const int k0 = kb * kBK;
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int ch = tid + 256 * c;
            const int r = ch >> 2, cc = ch & 3;
            int64_t gr = row0 + r;
            gr = gr < n ? gr : n - 1;
            xr[c] = *(const u32x4*)(x + gr * x_stride + k0 + cc * 8);
        }
#pragma unroll
        for (int c = 0; c < WCH; ++c) {
            const int ch = tid + 256 * c;
            const int r = ch >> 2, cc = ch & 3;
            wreg[c] = *(const u32x4*)(w1 + (int64_t)r * d_model + k0 + cc * 8);
        }
    };
    auto store_slab = [&](int buf) {
        bf16* xs = lds0 + buf * SLAB;
        bf16* ws = xs + kBM * kLdk;
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int ch = tid + 256 * c;
            *(u32x4*)(xs + (ch >> 2) * kLdk + (ch & 3) * 8) = xr[c];
        }
#pragma unroll
        for (int c = 0; c < WCH; ++c) {
            const int ch = tid + 256 * c;
            *(u32x4*)(ws + (ch >> 2) * kLdk + (ch & 3) * 8) = wreg[c];
        }
    };

    f32x16 acc[2][CB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x16{};

    const int nk = d_model / kBK;
    load_slab(0);
    store_slab(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nk) load_slab(kb + 1);
        const bf16* xs = lds0 + buf * SLAB;
        const bf16* ws = xs + kBM * kLdk;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            bf16x8 a[2], b[CB];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                a[rb] = *(const bf16x8*)(xs + (wr * 64 + rb * 32 + il) * kLdk + ks * 16 + half * 8);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                b[cb] = *(const bf16x8*)(ws + (wc * CB * 32 + cb * 32 + il) * kLdk + ks * 16 + half * 8);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
        }
        if (kb + 1 < nk) store_slab(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: per token, sum over this wave's hidden units of SiLU(a + b1) * w2.
    // acc[rb][cb][r] = hidden unit n = wc*CB*32 + cb*32 + il of token
    // wr*64 + rb*32 + (r/4)*8 + half*4 + r%4.
    float bias1[CB], wout[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int nidx = wc * CB * 32 + cb * 32 + il;
        bias1[cb] = b1 ? b1[nidx] : 0.0f;
        wout[cb] = w2[nidx];
    }
    float* red = (float*)lds_raw;   // [kBM][65] partial sums, aliases the slab buffers
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) p += silu_f32(acc[rb][cb][r] + bias1[cb]) * wout[cb];
            const int tok = wr * 64 + rb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            red[tok * 65 + wc * 32 + il] = p;
        }
    }
    __syncthreads();
    // two threads per token, 32 partials each, then one shuffle
    {
        const int tok = tid >> 1, part = tid & 1;
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) sum += red[tok * 65 + part * 32 + j];
        sum += __shfl_xor(sum, 1, 64);
        if (part == 0 && row0 + tok < n) scores[row0 + tok] = sum + b2;
    }
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
                     hipStream_t st) {
    if (n == 0) return TG_OK;
    const dim3 grid((unsigned)((n + kBM - 1) / kBM));
    switch (d_hid) {
        case 64:  hipLaunchKernelGGL(gate_bf16_kernel<1>, grid, dim3(256), 0, st, x, n, d_model, x_stride, w1, b1, w2, b2, scores); break;
        case 128: hipLaunchKernelGGL(gate_bf16_kernel<2>, grid, dim3(256), 0, st, x, n, d_model, x_stride, w1, b1, w2, b2, scores); break;
        case 192: hipLaunchKernelGGL(gate_bf16_kernel<3>, grid, dim3(256), 0, st, x, n, d_model, x_stride, w1, b1, w2, b2, scores); break;
        case 256: hipLaunchKernelGGL(gate_bf16_kernel<4>, grid, dim3(256), 0, st, x, n, d_model, x_stride, w1, b1, w2, b2, scores); break;
        default: return TG_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_HIP;
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
