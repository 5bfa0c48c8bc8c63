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
#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// Stem layers (3x3, pad 1, stride 1 or 2, a handful of input channels, widths a
// multiple of 4): each thread computes 4 adjacent output pixels of one row for
// COB output channels, fully unrolled.  Per input channel and window row it
// loads the row's pixels as 16-byte vectors plus the one or two edge pixels
// (out-of-range offsets read zero: image borders are the padding), and it
// stores 16 bytes per output channel.  ("YOLO26N Inference Optimisation",
// "Baseline benchmark": the detector's stem convolutions; "Как я свертки
// ускорял", "Пациента на стол": the MNIST net's first convolution.)
template <int CIN, int COB, int S>
__global__ void __launch_bounds__(256) k_stem(const float* __restrict__ x,
                                              const float* __restrict__ w,
                                              const float* __restrict__ scale,
                                              const float* __restrict__ bias,
                                              const float* __restrict__ res,
                                              float* __restrict__ y, int h, int wd, int cout,
                                              int oh, int ow, int act, int res_mode)
{
    constexpr int NCOL = S == 2 ? 9 : 6;  // input columns under 4 outputs
    const int qw = ow >> 2;                // quads per output row
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.z;
    const int co0 = blockIdx.y * COB;
    const bool live = t < oh * qw;
    const int tt = live ? t : 0;
    const int oy = tt / qw;
    const int ox0 = (tt - oy * qw) * 4;
    const int hw = h * wd;
    const rsrc_t rx = make_rsrc(x + (long)b * CIN * hw, 4u * (unsigned)(CIN * hw));
    const int cx = ox0 * S - 1;  // first input column

    float acc[COB][4];
#pragma unroll
    for (int c = 0; c < COB; ++c)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[c][p] = 0.0f;

#pragma unroll
    for (int ci = 0; ci < CIN; ++ci)
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int iy = oy * S - 1 + i;
            const bool rok = iy >= 0 && iy < h;
            const unsigned row = 4u * (unsigned)(ci * hw + iy * wd);
            float col[NCOL];
            // column cx (left edge), then 16-byte vectors from cx + 1
            col[0] = bload(rx, rok && cx >= 0 ? row + 4u * (unsigned)cx : kOOB);
            const unsigned v0 = rok ? row + 4u * (unsigned)(cx + 1) : kOOB;
            const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)v0, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) col[1 + e] = a[e];
            if constexpr (S == 2) {
                const f32x4 bq = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(rok ? v0 + 16u : kOOB), 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) col[5 + e] = bq[e];
            } else {
                col[5] = bload(rx, rok && cx + 5 < wd ? row + 4u * (unsigned)(cx + 5) : kOOB);
            }
#pragma unroll
            for (int c = 0; c < COB; ++c) {
                const int co = min(co0 + c, cout - 1);
                const float* wr = w + ((long)co * CIN + ci) * 9 + i * 3;
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const float wv = wr[j];
#pragma unroll
                    for (int p = 0; p < 4; ++p) acc[c][p] = fmaf(wv, col[p * S + j], acc[c][p]);
                }
            }
        }
    if (!live) return;
    const int ohw = oh * ow;
    const rsrc_t ry = make_rsrc(y, 4u * (unsigned)((long)gridDim.z * cout * ohw));
    const rsrc_t rr = make_rsrc(res, res ? 4u * (unsigned)((long)gridDim.z * cout * ohw) : 0u);
#pragma unroll
    for (int c = 0; c < COB; ++c) {
        const int co = co0 + c;
        if (co >= cout) break;
        const unsigned off = 4u * (unsigned)(((long)b * cout + co) * ohw + oy * ow + ox0);
        f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
        if (res_mode != CVX_RES_NONE)
            r = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)off, 0, 0));
        const float sc = scale[co], bi = bias[co];
        f32x4 z;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float v = fmaf(sc, acc[c][p], bi);
            if (res_mode == CVX_RES_BEFORE_ACT) v += r[p];
            v = apply_act_fast(v, act);
            if (res_mode == CVX_RES_AFTER_ACT) v += r[p];
            z[p] = v;
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z), ry, (int)off, 0, 0);
    }
}

bool stem_shape(const ConvGeom& g)
{
    return g.groups == 1 && g.k == 3 && g.pad == 1 && (g.stride == 1 || g.stride == 2) &&
           (g.cin == 1 || g.cin == 3) && g.w % 4 == 0 && g.ow % 4 == 0 && g.w == g.ow * g.stride;
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int CIN>
static void launch_stem_cin(const ConvGeom& g, dim3 grid, hipStream_t s, const float* x,
                            const float* w, const float* scale, const float* bias, const float* res,
                            float* y)
{
    if (g.stride == 2)
        hipLaunchKernelGGL((k_stem<CIN, 8, 2>), grid, dim3(256), 0, s, x, w, scale, bias, res, y, g.h,
                           g.w, g.cout, g.oh, g.ow, g.act, g.res_mode);
    else
        hipLaunchKernelGGL((k_stem<CIN, 8, 1>), grid, dim3(256), 0, s, x, w, scale, bias, res, y, g.h,
                           g.w, g.cout, g.oh, g.ow, g.act, g.res_mode);
}

hipError_t launch_direct(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                         const float* scale, const float* bias, const float* res, float* y,
                         hipStream_t s)
{
    const int cout_g = g.cout / g.groups;
    const int ohw = g.oh * g.ow;
    if (p.direct_stem && al16(x) && al16(y) && (res == nullptr || al16(res))) {
        dim3 grid((unsigned)((g.oh * (g.ow / 4) + 255) / 256), (unsigned)((g.cout + 7) / 8),
                  (unsigned)g.n);
        if (g.cin == 1)
            launch_stem_cin<1>(g, grid, s, x, w, scale, bias, res, y);
        else
            launch_stem_cin<3>(g, grid, s, x, w, scale, bias, res, y);
        return hipGetLastError();
    }
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
