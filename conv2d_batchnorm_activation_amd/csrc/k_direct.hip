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
// multiple of 4).  A workgroup takes 256 consecutive output pixels of one image
// (flattened over rows) and COB output channels.  It stages the input rows those
// pixels touch (every input channel, whole rows; each wave takes whole rows,
// at a pitch of 64 quads so a partial last load zero-fills its own row) in LDS
// with 16-byte LDS-direct loads, all in flight at once.  The workgroup has two
// threads per pixel (8 waves, so latency has other waves to hide behind, and
// three workgroups still fit a compute unit's LDS); each holds its pixel's
// CIN x 9 window in registers (the pad column reads as zero) and computes half
// of the COB channels, two at a time, storing each pair as soon as it is done so
// that the stores overlap the rest of the arithmetic.  The weights
// are the same for every lane: scalar loads straight into the multiply-adds'
// scalar operand (read per lane from LDS, every wave would pull a kilobyte per
// read through LDS).  Stores are one float per channel, coalesced across the
// wave.  ("YOLO26N Inference Optimisation", "Baseline benchmark": the
// detector's stem convolutions; "Как я свертки ускорял", "Пациента на стол":
// the MNIST net's first convolution.)
constexpr int kStemCob = 16;      // output channels per workgroup
constexpr int kStemSplit = 2;     // threads per output pixel
constexpr int kStemThreads = 256 * kStemSplit;

__device__ __forceinline__ void stem_lds_load16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}

template <int CIN, int COB, int S>
__global__ void __launch_bounds__(kStemThreads) k_stem(const float* __restrict__ x,
                                              const float* __restrict__ w,
                                              const float* __restrict__ scale,
                                              const float* __restrict__ bias,
                                              const float* __restrict__ res,
                                              float* __restrict__ y, int h, int wd, int cout,
                                              int oh, int ow, int nrows, int act, int res_mode)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int b = blockIdx.z;
    const int co0 = blockIdx.y * COB;
    const int ohw = oh * ow;
    const int p0 = blockIdx.x * 256;
    const int oy_first = p0 / ow;
    const int iy_first = oy_first * S - 1;  // staged row 0
    const int hw = h * wd;
    const int qpr = wd >> 2;                // 16-byte quads per row
    const int nq = (qpr + 63) >> 6;         // loads per row
    const int pitch = 256 * nq;             // LDS floats per staged row
    const int srows = CIN * nrows;          // staged rows: [channel][row]

    // Staging: wave w takes staged rows w, w+8, ...; rows outside the image and
    // quads past the row's end read through out-of-range offsets as zeros.
    {
        const int lane = t & 63;
        const rsrc_t rx = make_rsrc(x + (long)b * CIN * hw, 4u * (unsigned)(CIN * hw));
        for (int r = wave; r < srows; r += kStemThreads / 64) {
            const int ci = r / nrows;  // uniform
            const int iy = iy_first + (r - ci * nrows);
            const bool rok = iy >= 0 && iy < h;
            for (int j = 0; j < nq; ++j) {
                const int qx = 64 * j + lane;
                const unsigned off = rok && qx < qpr ? 4u * (unsigned)(ci * hw + iy * wd + 4 * qx) : kOOB;
                int base = r * pitch + 256 * j;
                asm volatile("" : "+s"(base));
                stem_lds_load16(rx, (__attribute__((address_space(3))) void*)(lds + base), off);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int p = p0 + (t & 255);
    const int part = __builtin_amdgcn_readfirstlane(t >> 8);  // channels COB / kStemSplit * part ...
    if (p >= ohw) return;
    const int oy = p / ow;
    const int ox = p - oy * ow;
    const int rrow = (oy - oy_first) * S;  // staged row of window row 0

    float win[CIN * 9];
#pragma unroll
    for (int ci = 0; ci < CIN; ++ci)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int col = ox * S - 1 + kw;
                const bool ok = col >= 0 && col < wd;
                const int idx = ok ? (ci * nrows + rrow + kh) * pitch + col : 0;
                const float v = lds[idx];
                win[ci * 9 + kh * 3 + kw] = ok ? v : 0.0f;
            }

    // Stores through a descriptor over the output: a channel past c_out gets an
    // out-of-range offset and is dropped, so the epilogue has no branches and the
    // pair's two accumulation chains interleave.
    const unsigned out_bytes = 4u * (unsigned)(gridDim.z * cout * ohw);
    const rsrc_t ry = make_rsrc(y, out_bytes);
    const rsrc_t rr = make_rsrc(res, res_mode != CVX_RES_NONE ? out_bytes : 0u);
    const unsigned obase = (unsigned)(b * cout * ohw + p);
#pragma unroll 1
    for (int g = part * (COB / kStemSplit / 2); g < (part + 1) * (COB / kStemSplit / 2); ++g) {
        const int c0 = min(co0 + 2 * g, cout - 1), c1 = min(co0 + 2 * g + 1, cout - 1);  // uniform
        const float* w0 = w + (long)c0 * CIN * 9;
        const float* w1 = w + (long)c1 * CIN * 9;
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int tap = 0; tap < CIN * 9; ++tap) {
            a0 = fmaf(w0[tap], win[tap], a0);
            a1 = fmaf(w1[tap], win[tap], a1);
        }
        const float acc[2] = {a0, a1};
        const float scs[2] = {scale[c0], scale[c1]}, bis[2] = {bias[c0], bias[c1]};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int co = co0 + 2 * g + e;
            const unsigned o = co < cout ? 4u * (obase + (unsigned)(co * ohw)) : kOOB;
            const float r = bload(rr, o);
            float v = fmaf(scs[e], acc[e], bis[e]);
            if (res_mode == CVX_RES_BEFORE_ACT) v += r;
            v = apply_act_fast(v, act);
            if (res_mode == CVX_RES_AFTER_ACT) v += r;
            bstore(ry, o, v);
        }
    }
}

// Staged input rows of the stem kernel's largest workgroup: 256 consecutive
// output pixels span at most ceil(255 / ow) + 1 output rows.
static int stem_rows(const ConvGeom& g)
{
    int rows_out = (255 + g.ow - 1) / g.ow + 1;
    rows_out = rows_out < g.oh ? rows_out : g.oh;
    return (rows_out - 1) * g.stride + 3;
}

// Staged rows at a pitch of whole 64-quad loads.
static size_t stem_lds(const ConvGeom& g)
{
    const long pitch = 256L * ((g.w / 4 + 63) / 64);
    return (size_t)g.cin * stem_rows(g) * pitch * sizeof(float);
}

bool stem_shape(const ConvGeom& g)
{
    return g.groups == 1 && g.k == 3 && g.pad == 1 && (g.stride == 1 || g.stride == 2) &&
           (g.cin == 1 || g.cin == 3) && g.w % 4 == 0 && g.ow % 4 == 0 && g.w == g.ow * g.stride &&
           stem_lds(g) <= kMaxLdsBytes;
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int CIN>
static void launch_stem_cin(const ConvGeom& g, dim3 grid, hipStream_t s, const float* x,
                            const float* w, const float* scale, const float* bias, const float* res,
                            float* y)
{
    const size_t lds = stem_lds(g);
    const int nrows = stem_rows(g);
    if (g.stride == 2)
        hipLaunchKernelGGL((k_stem<CIN, kStemCob, 2>), grid, dim3(kStemThreads), lds, s, x, w, scale, bias, res,
                           y, g.h, g.w, g.cout, g.oh, g.ow, nrows, g.act, g.res_mode);
    else
        hipLaunchKernelGGL((k_stem<CIN, kStemCob, 1>), grid, dim3(kStemThreads), lds, s, x, w, scale, bias, res,
                           y, g.h, g.w, g.cout, g.oh, g.ow, nrows, g.act, g.res_mode);
}

hipError_t launch_direct(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                         const float* scale, const float* bias, const float* res, float* y,
                         hipStream_t s)
{
    const int cout_g = g.cout / g.groups;
    const int ohw = g.oh * g.ow;
    if (p.direct_stem && al16(x) && al16(y) && (res == nullptr || al16(res))) {
        dim3 grid((unsigned)((g.oh * g.ow + 255) / 256), (unsigned)((g.cout + kStemCob - 1) / kStemCob),
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
