// k_small.hip -- the BatchNorm fold and the classifier tail (pool + fc).
#include "cvx_internal.h"

namespace cvx {

// scale = gamma / sqrt(var + eps), bias = beta - mean * scale: the BatchNorm
// inference form ("Как я свертки ускорял", "А теперь — хардкор на Metal",
// step 4) rewritten as one multiply-add per output.
__global__ void __launch_bounds__(256) k_fold_bn(const float* __restrict__ gamma,
                                                 const float* __restrict__ beta,
                                                 const float* __restrict__ mean,
                                                 const float* __restrict__ var, float eps, int c,
                                                 float* __restrict__ scale,
                                                 float* __restrict__ bias)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= c) return;
    float sc = gamma[i] / sqrtf(var[i] + eps);
    scale[i] = sc;
    bias[i] = fmaf(-mean[i], sc, beta[i]);
}

hipError_t launch_fold_bn(const float* gamma, const float* beta, const float* mean,
                          const float* var, float eps, int c, float* scale, float* bias,
                          hipStream_t s)
{
    dim3 grid((c + 255) / 256);
    hipLaunchKernelGGL(k_fold_bn, grid, dim3(256), 0, s, gamma, beta, mean, var, eps, c, scale,
                       bias);
    return hipGetLastError();
}

// Global average pool over each [hw] plane, optionally followed by an fc layer
// ("Как я свертки ускорял", "Пациента на стол": pool to 1x1, flatten, Linear).
// One workgroup per image.  With fc_w == nullptr the pooled vector is the
// output ([n][c]); with hw == 1 the pool is the identity and this is a plain fc.
// The pooled vector lives in LDS (c <= kTailMaxC, checked by the host).
// When the image fits (c*hw <= kTailStage floats, 16-byte aligned and a
// multiple of 4), it is first copied to LDS with independent 16-byte loads --
// one memory round trip for the image rather than one per plane -- and each
// thread then sums a plane from LDS.
constexpr int kTailMaxC = 4096;
constexpr int kTailStage = 12288;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_gap_fc(const float* __restrict__ x, int c, int hw,
                                                const float* __restrict__ fc_w,
                                                const float* __restrict__ fc_b, int out_f,
                                                float* __restrict__ out, int staged)
{
    __shared__ float pooled[kTailMaxC];
    __shared__ __attribute__((aligned(16))) float img[kTailStage];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const float* xb = x + (long)b * c * hw;
    const float inv = 1.0f / (float)hw;
    if (staged) {
        const int n4 = c * hw / 4;
        const f32x4* x4 = reinterpret_cast<const f32x4*>(xb);
#pragma unroll 4
        for (int e = threadIdx.x; e < n4; e += 256) reinterpret_cast<f32x4*>(img)[e] = x4[e];
        __syncthreads();
        for (int ch = threadIdx.x; ch < c; ch += 256) {
            const float* p = img + ch * hw;
            float s = 0.0f;
            for (int q = 0; q < hw; ++q) s += p[q];
            pooled[ch] = s * inv;
        }
    } else {
        // each wave pools whole planes: lanes stride over the plane, then reduce
        for (int ch = wave; ch < c; ch += 4) {
            const float* p = xb + (long)ch * hw;
            float s = 0.0f;
            for (int q = lane; q < hw; q += 64) s += p[q];
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
            if (lane == 0) pooled[ch] = s * inv;
        }
    }
    __syncthreads();
    if (fc_w == nullptr) {
        for (int ch = threadIdx.x; ch < c; ch += 256) out[(long)b * c + ch] = pooled[ch];
        return;
    }
    for (int o = wave; o < out_f; o += 4) {
        const float* wr = fc_w + (long)o * c;
        float s = 0.0f;
        for (int ch = lane; ch < c; ch += 64) s = fmaf(wr[ch], pooled[ch], s);
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) out[(long)b * out_f + o] = s + fc_b[o];
    }
}

hipError_t launch_gap_fc(const float* x, int n, int c, int hw, const float* fc_w,
                         const float* fc_b, int out_f, float* out, hipStream_t s)
{
    const int staged = (long)c * hw <= kTailStage && (c * hw) % 4 == 0 &&
                       (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    hipLaunchKernelGGL(k_gap_fc, dim3(n), dim3(256), 0, s, x, c, hw, fc_w, fc_b, out_f, out, staged);
    return hipGetLastError();
}

// Plain copy (the packed form of weights that the direct kernels read as OIHW).
__global__ void __launch_bounds__(256) k_copy(const float* __restrict__ src, float* __restrict__ dst,
                                              long n)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

hipError_t launch_copy(const float* src, float* dst, long n, hipStream_t s)
{
    dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(k_copy, grid, dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace cvx
