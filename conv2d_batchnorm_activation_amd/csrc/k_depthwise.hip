// k_depthwise.hip -- depthwise 3x3 convolution + folded BN + activation
// (+ residual), a memory-bound direct kernel with an LDS halo tile.
//
// The operation is the one of "Как я свертки ускорял", "А теперь — хардкор на
// Metal", steps 1-5: each output channel sees only its own input plane, the 3x3
// window starts at output position * stride - 1 (pad 1 there; any pad here),
// out-of-image taps are zero, BN and the activation are applied in registers and
// each output is stored once.  Its arithmetic intensity is 0.9-2.2 FLOP/byte
// ("Ускоряем скорость", problem 3), far below the MI355X fp32 ridge, so the
// kernel is built around moving bytes:
//   * NCHW planes of consecutive (n, c) pairs are contiguous, so a workgroup
//     stages `ppb` whole planes (or a band of `toh` output rows of one large
//     plane) into LDS with one linear, coalesced sweep over global memory and
//     reads every input element from HBM exactly once;
//   * the zero padding is written into the LDS tile, so the 9-tap loop has no
//     bounds checks;
//   * outputs are written as dense NCHW rows: no tile ever writes past a row
//     end, whatever OW is (the edge-tile overrun of "YOLO26N Inference
//     Optimisation", "Bug fixed: TMA overflow", cannot happen by construction).
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

template <int S>
__global__ void __launch_bounds__(256) k_depthwise3x3(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, const float* __restrict__ res, float* __restrict__ y,
    int planes, int C, int H, int W, int OH, int OW, int pad, int ppb, int toh, int bands,
    int act, int res_mode)
{
    extern __shared__ float tile[];
    const int task = blockIdx.x;
    const int band = task % bands;
    const int plane0 = (task / bands) * ppb;
    const int np = min(ppb, planes - plane0);
    const int oh0 = band * toh;
    const int nrows = min(toh, OH - oh0);
    const int PR = (toh - 1) * S + 3;        // input rows staged per plane
    const int PW = W + 2 * pad;              // staged row width incl. zero padding
    const int iy0 = oh0 * S - pad;
    const int tile_elems = np * PR * PW;

    // stage: element e = (pl, r, c) of the halo tile, zero outside the image
    for (int e = threadIdx.x; e < tile_elems; e += 256) {
        const int pl = e / (PR * PW);
        const int rem = e - pl * PR * PW;
        const int r = rem / PW;
        const int c = rem - r * PW;
        const int iy = iy0 + r;
        const int ix = c - pad;
        float v = 0.0f;
        if (iy >= 0 && iy < H && ix >= 0 && ix < W)
            v = x[((long)(plane0 + pl) * H + iy) * W + ix];
        tile[e] = v;
    }
    __syncthreads();

    const int outs = np * nrows * OW;
    for (int e = threadIdx.x; e < outs; e += 256) {
        const int pl = e / (nrows * OW);
        const int rem = e - pl * nrows * OW;
        const int r = rem / OW;
        const int c = rem - r * OW;
        const int plane = plane0 + pl;
        const int ch = plane % C;
        const float* wp = w + ch * 9;
        const float* t = tile + (pl * PR + r * S) * PW + c * S;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) acc = fmaf(t[i * PW + j], wp[i * 3 + j], acc);
        const long idx = ((long)plane * OH + oh0 + r) * OW + c;
        y[idx] = epilogue(acc, scale[ch], bias[ch], act, res_mode, res, idx);
    }
}

hipError_t launch_depthwise(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                            const float* scale, const float* bias, const float* res, float* y,
                            hipStream_t s)
{
    const int planes = g.n * g.cout;
    const int bands = (g.oh + p.dw_toh - 1) / p.dw_toh;
    const int groups_of_planes = (planes + p.dw_ppb - 1) / p.dw_ppb;
    const int PR = (p.dw_toh - 1) * g.stride + 3;
    const size_t lds = (size_t)p.dw_ppb * PR * (g.w + 2 * g.pad) * sizeof(float);
    dim3 grid((unsigned)(groups_of_planes * bands));
    if (g.stride == 1)
        hipLaunchKernelGGL(k_depthwise3x3<1>, grid, dim3(256), lds, s, x, w, scale, bias, res, y,
                           planes, g.cout, g.h, g.w, g.oh, g.ow, g.pad, p.dw_ppb, p.dw_toh, bands,
                           g.act, g.res_mode);
    else if (g.stride == 2)
        hipLaunchKernelGGL(k_depthwise3x3<2>, grid, dim3(256), lds, s, x, w, scale, bias, res, y,
                           planes, g.cout, g.h, g.w, g.oh, g.ow, g.pad, p.dw_ppb, p.dw_toh, bands,
                           g.act, g.res_mode);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace cvx
