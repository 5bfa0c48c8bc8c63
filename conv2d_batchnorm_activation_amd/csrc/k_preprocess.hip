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
#include "bufio.h"
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

// The same coordinates in 32-bit arithmetic, for sizes where (2d + 1) * src
// stays below 2^31 (the host checks).
__device__ __forceinline__ Axis src_axis32(int d, int src, int dst)
{
    const int num = (2 * d + 1) * src - dst;
    const int den = 2 * dst;
    Axis a;
    if (num <= 0) {
        a.i0 = 0;
        a.f = 0.0f;
    } else {
        const int q = (int)((unsigned)num / (unsigned)den);
        a.i0 = q;
        a.f = (float)(num - q * den) / (float)den;
    }
    if (a.i0 > src - 1) a.i0 = src - 1;
    a.i1 = a.i0 + 1 < src ? a.i0 + 1 : src - 1;
    return a;
}

__device__ __forceinline__ void pre_lds_load16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}

// Row kernel, for frames whose base and row pitch are 16-byte aligned: one
// workgroup per destination row.  Its two source rows go global -> LDS with
// 16-byte LDS-direct loads (one round trip, every byte read once per
// workgroup); then each thread interpolates a quad of four consecutive
// destination pixels from LDS and stores each plane's quad with one 16-byte
// store (when the destination rows are whole 16-byte runs), coalesced.  The
// horizontal source coordinate divides by 2*dst_w through a host-computed
// multiplier, and /255 and the normalisation fold into one multiply-add per
// channel: out = v * (1 / (255 * std)) - mean / std.
__global__ void __launch_bounds__(256) k_preprocess_rows(const unsigned char* __restrict__ src,
                                                         int src_h, int src_w, unsigned row_bytes,
                                                         float* __restrict__ dst, int dst_h,
                                                         int dst_w, int pitch, unsigned m_den,
                                                         unsigned l_den, float inv_den, int vec4,
                                                         float a0, float a1, float a2, float b0,
                                                         float b1, float b2)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lrow[];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int dy = blockIdx.x, b = blockIdx.y;
    const Axis ay = src_axis32(dy, src_h, dst_h);
    const unsigned img_bytes = (unsigned)src_h * row_bytes;
    const rsrc_t r = make_rsrc(src + (long)b * img_bytes, img_bytes);
    const int len = 3 * src_w;             // bytes of a row's pixels
    const int chunks = (len + 1023) >> 10;  // 64 quads of 16 bytes each
    for (int k = 0; k < 2; ++k) {
        const unsigned row = (unsigned)(k ? ay.i1 : ay.i0) * row_bytes;
        for (int j = wave; j < chunks; j += 4) {
            const int q = 64 * j + lane;
            const unsigned off = 16 * q < len ? row + 16u * (unsigned)q : kOOB;
            int base = k * pitch + 1024 * j;
            asm volatile("" : "+s"(base));
            pre_lds_load16(r, (__attribute__((address_space(3))) void*)(lrow + base), off);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const float ca[3] = {a0, a1, a2};
    const float cb[3] = {b0, b1, b2};
    const long plane = (long)dst_h * dst_w;
    float* out = dst + (long)b * 3 * plane + (long)dy * dst_w;
    const unsigned char* r0 = lrow;
    const unsigned char* r1 = lrow + pitch;
    const unsigned den = 2u * (unsigned)dst_w;
    // source column pair and weight of destination column dx (exact integers:
    // (2dx + 1) * src_w - dst_w over 2 * dst_w, clamped like src_axis32)
    auto axis = [&](int dx) {
        const int num = (2 * dx + 1) * src_w - dst_w;
        Axis a;
        if (num <= 0) {
            a.i0 = 0;
            a.f = 0.0f;
        } else {
            const unsigned q = (__umulhi((unsigned)num, m_den) + (unsigned)num) >> l_den;
            a.i0 = (int)q;
            a.f = (float)((unsigned)num - q * den) * inv_den;
        }
        if (a.i0 > src_w - 1) a.i0 = src_w - 1;
        a.i1 = a.i0 + 1 < src_w ? a.i0 + 1 : src_w - 1;
        return a;
    };
    auto pixel = [&](int dx, float (&v)[3]) {
        const Axis ax = axis(dx);
        const int c0 = 3 * ax.i0, c1 = 3 * ax.i1;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            const float p00 = (float)r0[c0 + ch], p01 = (float)r0[c1 + ch];
            const float p10 = (float)r1[c0 + ch], p11 = (float)r1[c1 + ch];
            const float top = fmaf(ax.f, p01 - p00, p00);
            const float bot = fmaf(ax.f, p11 - p10, p10);
            v[ch] = fmaf(fmaf(ay.f, bot - top, top), ca[ch], cb[ch]);
        }
    };
    if (vec4) {
        for (int dx = 4 * t; dx < dst_w; dx += 1024) {
            float v[4][3];
#pragma unroll
            for (int e = 0; e < 4; ++e) pixel(dx + e, v[e]);
#pragma unroll
            for (int ch = 0; ch < 3; ++ch)
                *reinterpret_cast<float4*>(out + ch * plane + dx) = make_float4(v[0][ch], v[1][ch], v[2][ch], v[3][ch]);
        }
    } else {
        for (int dx = t; dx < dst_w; dx += 256) {
            float v[3];
            pixel(dx, v);
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) out[ch * plane + dx] = v[ch];
        }
    }
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

void fastdiv_params(int d, unsigned* m, unsigned* l);

hipError_t launch_preprocess(const unsigned char* src, int n, int src_h, int src_w,
                             long src_row_bytes, float* dst, int dst_h, int dst_w,
                             const float mean[3], const float stdv[3], hipStream_t s)
{
    const long plane = (long)dst_h * dst_w;
    const long len = 3L * src_w;
    const long pitch = (len + 1023) / 1024 * 1024;
    const bool rows = (reinterpret_cast<uintptr_t>(src) & 15u) == 0 && src_row_bytes % 16 == 0 &&
                      2 * pitch <= (long)kMaxLdsBytes && (long)src_h * src_row_bytes < 0x7fffffffL &&
                      (2L * dst_w + 1) * src_w < 0x7fffffffL && (2L * dst_h + 1) * src_h < 0x7fffffffL;
    if (rows) {
        dim3 grid((unsigned)dst_h, (unsigned)n);
        unsigned m_den, l_den;
        fastdiv_params(2 * dst_w, &m_den, &l_den);
        const int vec4 = dst_w % 4 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0 ? 1 : 0;
        float ca[3], cb[3];
        for (int c = 0; c < 3; ++c) {
            ca[c] = (float)(1.0 / (255.0 * (double)stdv[c]));
            cb[c] = (float)(-(double)mean[c] / (double)stdv[c]);
        }
        hipLaunchKernelGGL(k_preprocess_rows, grid, dim3(256), (size_t)(2 * pitch), s, src, src_h,
                           src_w, (unsigned)src_row_bytes, dst, dst_h, dst_w, (int)pitch, m_den, l_den,
                           (float)(1.0 / (2.0 * dst_w)), vec4, ca[0], ca[1], ca[2], cb[0], cb[1], cb[2]);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((plane + 255) / 256), (unsigned)n);
    hipLaunchKernelGGL(k_preprocess, grid, dim3(256), 0, s, src, src_h, src_w, src_row_bytes, dst,
                       dst_h, dst_w, mean[0], mean[1], mean[2], stdv[0], stdv[1], stdv[2]);
    return hipGetLastError();
}

}  // namespace cvx
