// k_direct.hip -- direct convolution on the vector ALUs, for layers whose
// reduction is too short to feed the matrix cores: the stems with 1 or 3 input
// channels (K = 9 or 27), grouped convolutions and kernels larger than 3x3.
//
// Each thread owns one output pixel and COB output channels of one group: it
// reads each input tap once and feeds COB accumulators.  The weight index is
// uniform across the workgroup, so weights come through scalar loads and the
// only per-lane memory traffic is the input window and the stores.
// The window arithmetic is the zero-padded cross-correlation of
// "Как я свертки ускорял", "А теперь — хардкор на Metal", steps 2-3.
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

template <int COB>
__global__ void __launch_bounds__(256) k_direct(const float* __restrict__ x,
                                                const float* __restrict__ w,
                                                const float* __restrict__ scale,
                                                const float* __restrict__ bias,
                                                const float* __restrict__ res,
                                                float* __restrict__ y, int cin, int h, int wd,
                                                int cout, int kh, int kw, int stride, int pad,
                                                int groups, int oh, int ow, int act, int res_mode)
{
    const int q = blockIdx.x * blockDim.x + threadIdx.x;  // output pixel in the plane
    const int cout_g = cout / groups;
    const int cob_per_group = (cout_g + COB - 1) / COB;
    const int grp = blockIdx.y / cob_per_group;
    const int co0 = grp * cout_g + (blockIdx.y % cob_per_group) * COB;
    const int co_end = min(co0 + COB, (grp + 1) * cout_g);
    const int b = blockIdx.z;
    const int cin_g = cin / groups;
    const int ohw = oh * ow;
    const bool live = q < ohw;
    const int qq = live ? q : 0;
    const int oy = qq / ow;
    const int ox = qq - oy * ow;
    const int iy0 = oy * stride - pad;
    const int ix0 = ox * stride - pad;
    const float* xb = x + ((long)b * cin + (long)grp * cin_g) * h * wd;
    const int ksz = kh * kw;

    float acc[COB];
#pragma unroll
    for (int c = 0; c < COB; ++c) acc[c] = 0.0f;

    for (int ci = 0; ci < cin_g; ++ci) {
        const float* xp = xb + (long)ci * h * wd;
        for (int i = 0; i < kh; ++i) {
            const int iy = iy0 + i;
            const bool row_ok = iy >= 0 && iy < h;
            for (int j = 0; j < kw; ++j) {
                const int ix = ix0 + j;
                const float v = (row_ok && ix >= 0 && ix < wd) ? xp[iy * wd + ix] : 0.0f;
                const int widx = ci * ksz + i * kw + j;
#pragma unroll
                for (int c = 0; c < COB; ++c) {
                    // channels past the group end reuse the last valid row (result discarded)
                    const int co = min(co0 + c, co_end - 1);
                    acc[c] = fmaf(v, w[(long)co * cin_g * ksz + widx], acc[c]);
                }
            }
        }
    }
    if (!live) return;
#pragma unroll
    for (int c = 0; c < COB; ++c) {
        const int co = co0 + c;
        if (co < co_end) {
            const long idx = ((long)b * cout + co) * ohw + q;
            y[idx] = epilogue(acc[c], scale[co], bias[co], act, res_mode, res, idx);
        }
    }
}

hipError_t launch_direct(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                         const float* scale, const float* bias, const float* res, float* y,
                         hipStream_t s)
{
    const int cout_g = g.cout / g.groups;
    const int ohw = g.oh * g.ow;
    const int cob = p.direct_cob;
    dim3 grid((ohw + 255) / 256, g.groups * ((cout_g + cob - 1) / cob), g.n);
#define CVX_DIRECT(C)                                                                          \
    hipLaunchKernelGGL(k_direct<C>, grid, dim3(256), 0, s, x, w, scale, bias, res, y, g.cin, g.h, \
                       g.w, g.cout, g.k, g.k, g.stride, g.pad, g.groups, g.oh, g.ow, g.act,      \
                       g.res_mode)
    switch (cob) {
    case 1: CVX_DIRECT(1); break;
    case 4: CVX_DIRECT(4); break;
    case 8: CVX_DIRECT(8); break;
    case 16: CVX_DIRECT(16); break;
    default: return hipErrorInvalidValue;
    }
#undef CVX_DIRECT
    return hipGetLastError();
}

}  // namespace cvx
