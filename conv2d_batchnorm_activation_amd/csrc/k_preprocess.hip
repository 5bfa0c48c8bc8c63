// k_preprocess.hip -- stem prologue: u8 HWC RGB frame -> half-pixel bilinear
// resize -> /255 -> per-channel normalise -> fp32 CHW, in one pass over memory.
//
// "A fused Ampere preprocess kernel" ("The theory"): the three passes (resize,
// normalise, layout) move the frame through DRAM three times; fused, the u8 frame
// is read once, the fp32 tensor is written once and the interpolated values stay
// in registers.  "My notes from Day 7": the resize must be the half-pixel
// bilinear function (source coordinate (d + 0.5) * src/dst - 0.5, clamped at 0).
//
// Source coordinates are computed from integers, exactly: with
// num = (2d + 1) * src - dst and den = 2 * dst, s = num / den, so the integer part
// and the fraction come from one integer division and one rounding, for any ratio.
#include "cvx_internal.h"

namespace cvx {

struct Axis {
    int i0, i1;
    float f;
};

__device__ __forceinline__ Axis src_axis(int d, int src, int dst)
{
    long num = (long)(2 * d + 1) * src - dst;
    long den = 2L * dst;
    Axis a;
    if (num <= 0) {  // coordinate clamped at 0
        a.i0 = 0;
        a.f = 0.0f;
    } else {
        long q = num / den;
        a.i0 = (int)q;
        a.f = (float)(num - q * den) / (float)den;
    }
    if (a.i0 > src - 1) a.i0 = src - 1;
    a.i1 = a.i0 + 1 < src ? a.i0 + 1 : src - 1;
    return a;
}

// One thread per destination pixel; a block covers 256 consecutive pixels of one
// destination row band, so the three planar stores of a wave are coalesced.
__global__ void __launch_bounds__(256) k_preprocess(const unsigned char* __restrict__ src,
                                                    int src_h, int src_w, long row_bytes,
                                                    float* __restrict__ dst, int dst_h, int dst_w,
                                                    float m0, float m1, float m2, float s0,
                                                    float s1, float s2)
{
    const int b = blockIdx.y;
    const long plane = (long)dst_h * dst_w;
    const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= plane) return;
    const int dy = (int)(q / dst_w);
    const int dx = (int)(q - (long)dy * dst_w);
    const Axis ay = src_axis(dy, src_h, dst_h);
    const Axis ax = src_axis(dx, src_w, dst_w);
    const unsigned char* img = src + (long)b * src_h * row_bytes;
    const unsigned char* r0 = img + (long)ay.i0 * row_bytes;
    const unsigned char* r1 = img + (long)ay.i1 * row_bytes;
    const int c0 = 3 * ax.i0, c1 = 3 * ax.i1;
    const float mean[3] = {m0, m1, m2};
    const float sd[3] = {s0, s1, s2};
    float* out = dst + (long)b * 3 * plane + q;
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) {
        float p00 = (float)r0[c0 + ch], p01 = (float)r0[c1 + ch];
        float p10 = (float)r1[c0 + ch], p11 = (float)r1[c1 + ch];
        float top = fmaf(ax.f, p01 - p00, p00);
        float bot = fmaf(ax.f, p11 - p10, p10);
        float v = fmaf(ay.f, bot - top, top);
        out[ch * plane] = (v / 255.0f - mean[ch]) / sd[ch];
    }
}

hipError_t launch_preprocess(const unsigned char* src, int n, int src_h, int src_w,
                             long src_row_bytes, float* dst, int dst_h, int dst_w,
                             const float mean[3], const float stdv[3], hipStream_t s)
{
    const long plane = (long)dst_h * dst_w;
    dim3 grid((unsigned)((plane + 255) / 256), (unsigned)n);
    hipLaunchKernelGGL(k_preprocess, grid, dim3(256), 0, s, src, src_h, src_w, src_row_bytes, dst,
                       dst_h, dst_w, mean[0], mean[1], mean[2], stdv[0], stdv[1], stdv[2]);
    return hipGetLastError();
}

}  // namespace cvx
