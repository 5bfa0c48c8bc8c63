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

// Stem layers (3x3, pad 1, stride 1 or 2, one or three input channels, widths a
// multiple of 4): the detector's stem convolutions ("YOLO26N Inference
// Optimisation", "Baseline benchmark") and the MNIST net's first convolution
// ("Как я свертки ускорял", "Пациента на стол").  Their reduction (9 or 27
// taps) is too short for the matrix cores and they are bound by the output
// stores, so:
//   * a thread computes a quad of four consecutive output pixels (a quad never
//     leaves its row) for COB output channels, and stores each channel's quad
//     with one 16-byte store, coalesced across the wave;
//   * its input window (3 rows x 6 columns at stride 1, 3 x 9 at stride 2, per
//     input channel) comes straight to registers, one 16-byte load per aligned
//     group of four columns and single loads for the edge columns; rows and
//     columns outside the image read through out-of-range offsets as zeros (the
//     padding), and neighbouring quads share their rows in the caches;
//   * the workgroup's weights, scale and bias are read with lane-uniform
//     addresses, through the scalar cache;
//   * a workgroup is one wave, and quads are numbered over batch x rows x
//     columns, so even a single image gives hundreds of workgroups.
constexpr int kStemThreads = 64;

template <int CIN, int COB, int S>
__global__ void __launch_bounds__(kStemThreads) k_stem(const float* __restrict__ x,
                                              const float* __restrict__ w,
                                              const float* __restrict__ scale,
                                              const float* __restrict__ bias,
                                              const float* __restrict__ res,
                                              float* __restrict__ y, int nquads, int h, int wd,
                                              int cout, int ohw, int qrow, int Q, unsigned m_q,
                                              unsigned l_q, unsigned m_r, unsigned l_r,
                                              unsigned x_bytes, unsigned y_bytes, int act,
                                              int res_mode)
{
    constexpr int KT = CIN * 9;         // taps per output channel
    constexpr int WC = S == 1 ? 6 : 9;  // window columns of a quad
    const int t = threadIdx.x;
    const int co0 = blockIdx.y * COB;

    const int g = blockIdx.x * kStemThreads + t;
    if (g >= nquads) return;
    const int img = (int)((__umulhi((unsigned)g, m_q) + (unsigned)g) >> l_q);
    const int qi = g - img * Q;
    const int oy = (int)((__umulhi((unsigned)qi, m_r) + (unsigned)qi) >> l_r);
    const int ox = 4 * (qi - oy * qrow);
    const int c0 = ox * S;  // first column of the aligned group (16-byte aligned)

    const rsrc_t rx = make_rsrc(x, x_bytes);
    float win[CIN][3][WC];
#pragma unroll
    for (int ci = 0; ci < CIN; ++ci)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int iy = oy * S - 1 + kh;
            const bool rok = (unsigned)iy < (unsigned)h;
            const unsigned row = rok ? (unsigned)(((img * CIN + ci) * h + iy) * wd) : 0u;
            win[ci][kh][0] = bload(rx, rok && c0 > 0 ? 4u * (row + c0 - 1) : kOOB);
            const f32x4 m0 = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(rok ? 4u * (row + c0) : kOOB), 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) win[ci][kh][1 + e] = m0[e];
            if constexpr (S == 1) {
                win[ci][kh][5] = bload(rx, rok && c0 + 4 < wd ? 4u * (row + c0 + 4) : kOOB);
            } else {
                // columns c0+4 .. c0+7 stay inside the row: wd = 2*ow
                const f32x4 m1 = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(rok ? 4u * (row + c0 + 4) : kOOB), 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) win[ci][kh][5 + e] = m1[e];
            }
        }

    // A channel past c_out gets an out-of-range offset: its store is dropped.
    // Vector-memory stores and loads share one completion counter, so any load
    // after the first store would wait for the stores before it: the residual
    // quads of all COB channels are loaded first.
    const rsrc_t ry = make_rsrc(y, y_bytes);
    const unsigned obase = (unsigned)(img * cout * ohw + oy * (4 * qrow) + ox);
    auto offset = [&](int c) { return co0 + c < cout ? 4u * (obase + (unsigned)((co0 + c) * ohw)) : kOOB; };
    f32x4 r[COB];
    if (res_mode != CVX_RES_NONE) {
        const rsrc_t rr = make_rsrc(res, y_bytes);
#pragma unroll
        for (int c = 0; c < COB; ++c)
            r[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)offset(c), 0, 0));
    } else {
#pragma unroll
        for (int c = 0; c < COB; ++c) r[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // One loop per activation, so the epilogue has no branches.  The
    // workgroup is one wave and its channels are the same for every lane, so
    // weights, scale and bias come through the scalar cache (no LDS copy and
    // no barrier in front of the window loads, which are already in flight).
    auto channels = [&](auto act_fn) {
#pragma unroll
        for (int c = 0; c < COB; ++c) {
            const int cw = min(co0 + c, cout - 1);  // channels past c_out: results dropped
            const float* wc = w + (long)cw * KT;
            float wv[KT];
#pragma unroll
            for (int k = 0; k < KT; ++k) wv[k] = wc[k];
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ci = 0; ci < CIN; ++ci)
#pragma unroll
                for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) {
                        const float wt = wv[ci * 9 + kh * 3 + kw];
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[j] = fmaf(wt, win[ci][kh][j * S + kw], acc[j]);
                    }
            const float sc = scale[cw], bi = bias[cw];
            f32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = fmaf(sc, acc[j], bi);
                v = res_mode == CVX_RES_BEFORE_ACT ? v + r[c][j] : v;
                v = act_fn(v);
                o[j] = res_mode == CVX_RES_AFTER_ACT ? v + r[c][j] : v;
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ry, (int)offset(c), 0, 0);
        }
    };
    if (act == CVX_ACT_SILU)
        channels([](float v) { return apply_act_fast(v, CVX_ACT_SILU); });
    else if (act == CVX_ACT_RELU)
        channels([](float v) { return fmaxf(v, 0.0f); });
    else
        channels([](float v) { return v; });
}

// Output channels per stem workgroup: the most (16, 8, 4) that still gives
// the layer about six waves per compute unit (1536), so that a small image's
// few quads still keep the units busy; each wave's FMA chain is COB x taps
// long, and fewer channels per wave shortens it at the price of reading the
// window again for every group (from the caches).
int stem_cob(const ConvGeom& g)
{
    const long waves_per_group = ((long)g.n * g.oh * (g.ow / 4) + kStemThreads - 1) / kStemThreads;
    for (int cob : {16, 8}) {
        if (cob > 8 && g.cout < 32) continue;  // a 16-channel group needs 32+ channels to pay off
        if (waves_per_group * ((g.cout + cob - 1) / cob) >= 1536) return cob;
    }
    return 4;
}

bool stem_shape(const ConvGeom& g)
{
    return g.groups == 1 && g.k == 3 && g.pad == 1 && (g.stride == 1 || g.stride == 2) &&
           (g.cin == 1 || g.cin == 3) && g.w % 4 == 0 && g.ow % 4 == 0 && g.w == g.ow * g.stride &&
           (long)g.n * g.cin * g.h * g.w * 4 < 0x7fffffffL && (long)g.n * g.cout * g.oh * g.ow * 4 < 0x7fffffffL;
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void fastdiv_params(int d, unsigned* m, unsigned* l);

template <int CIN, int COB>
static void launch_stem_cin(const ConvGeom& g, hipStream_t s, const float* x, const float* w,
                            const float* scale, const float* bias, const float* res, float* y)
{
    const int qrow = g.ow / 4;
    const int Q = g.oh * qrow;
    const int nquads = g.n * Q;
    unsigned m_q, l_q, m_r, l_r;
    fastdiv_params(Q, &m_q, &l_q);
    fastdiv_params(qrow, &m_r, &l_r);
    const unsigned xb = (unsigned)((long)g.n * g.cin * g.h * g.w * 4);
    const unsigned yb = (unsigned)((long)g.n * g.cout * g.oh * g.ow * 4);
    dim3 grid((unsigned)((nquads + kStemThreads - 1) / kStemThreads), (unsigned)((g.cout + COB - 1) / COB));
    if (g.stride == 2)
        hipLaunchKernelGGL((k_stem<CIN, COB, 2>), grid, dim3(kStemThreads), 0, s, x, w, scale, bias, res, y,
                           nquads, g.h, g.w, g.cout, g.oh * g.ow, qrow, Q, m_q, l_q, m_r, l_r, xb, yb, g.act,
                           g.res_mode);
    else
        hipLaunchKernelGGL((k_stem<CIN, COB, 1>), grid, dim3(kStemThreads), 0, s, x, w, scale, bias, res, y,
                           nquads, g.h, g.w, g.cout, g.oh * g.ow, qrow, Q, m_q, l_q, m_r, l_r, xb, yb, g.act,
                           g.res_mode);
}

hipError_t launch_direct(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                         const float* scale, const float* bias, const float* res, float* y,
                         hipStream_t s)
{
    const int cout_g = g.cout / g.groups;
    const int ohw = g.oh * g.ow;
    if (p.direct_stem && al16(x) && al16(y) && (res == nullptr || al16(res))) {
        const int cob = stem_cob(g);
        if (g.cin == 1) {
            if (cob == 16) launch_stem_cin<1, 16>(g, s, x, w, scale, bias, res, y);
            else if (cob == 8) launch_stem_cin<1, 8>(g, s, x, w, scale, bias, res, y);
            else launch_stem_cin<1, 4>(g, s, x, w, scale, bias, res, y);
        } else {
            if (cob == 16) launch_stem_cin<3, 16>(g, s, x, w, scale, bias, res, y);
            else if (cob == 8) launch_stem_cin<3, 8>(g, s, x, w, scale, bias, res, y);
            else launch_stem_cin<3, 4>(g, s, x, w, scale, bias, res, y);
        }
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
