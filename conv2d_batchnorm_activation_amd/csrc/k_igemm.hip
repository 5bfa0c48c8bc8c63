// k_igemm.hip -- dense KxK (K = 1 or 3) convolution + folded BN + activation
// (+ residual) as an implicit GEMM on the fp32 matrix cores of gfx950.
//
// GEMM view ("YOLO26N Inference Optimisation", "NHWC migration", "What NHWC
// is": the reduction dimension of a convolution cast as a matrix product is
// c_in * kh * kw):
//     M = c_out,  N = output pixels of one image,  K = c_in * kh * kw
//     Y[co][q] = sum_k W[co][k] * X_im2col[k][q]
// The page's reason for NHWC was that its tensor-core instructions needed the
// reduction dimension contiguous in global memory.  The MI355X matrix cores
// read their operands from VGPRs, which we fill from LDS, so NCHW stays: the
// output pixels (the N dimension) are contiguous, global loads and stores stay
// coalesced, and the im2col matrix is never materialised.
//
// Per workgroup (256 threads = 4 wave64s) one BM x BN output tile:
//   * the weight block W[co0 .. co0+BM)[chunk] is staged in LDS as
//     sW[(ci*KK + tap)][m] (m contiguous), zero-filled past c_out / c_in;
//   * the input rows the tile's pixels need, for `ck` input channels, are staged
//     as full zero-padded rows sX[ci][r][c] (c = input column + pad), read with
//     one coalesced sweep per row; every staged element feeds up to KK taps;
//   * each wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks
//     (v_mfma_f32_32x32x2_f32, true fp32, no reduced-precision emulation);
//     the two K values of one MFMA are two adjacent input channels at one tap;
//   * the epilogue (folded BN, residual, activation) runs on the accumulators
//     and each output is stored once, masked to the real pixel count, so rows
//     of any width are never overrun ("Bug fixed: TMA overflow").
// When the tile count alone cannot fill the chip, the channel chunks are split
// over blockIdx.z; each slice stores raw partial sums in the workspace and a
// finishing kernel adds the slices in a fixed order (deterministic) and applies
// the epilogue.
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM, int BN, int WM, int WN, int K>
__global__ void __launch_bounds__(256) k_igemm(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, const float* __restrict__ res, float* __restrict__ y,
    float* __restrict__ partial, int cin, int H, int W, int cout, int stride, int pad, int OH,
    int OW, int ck, int rows_max, int tiles_per_img, int chunks_per_split, int act, int res_mode)
{
    static_assert(WM * WN == 4, "four waves per workgroup");
    constexpr int TM = BM / WM, TN = BN / WN;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is made of 32x32 blocks");
    constexpr int MT = TM / 32, NT = TN / 32;
    constexpr int KK = K * K;
    constexpr int BMP = BM + 1;  // odd row pitch: transposed LDS writes hit distinct banks

    extern __shared__ float smem[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hi = lane >> 5;   // which of the two K values of an MFMA this lane carries
    const int l32 = lane & 31;
    const int wm0 = (wave / WN) * TM;
    const int wn0 = (wave % WN) * TN;

    const int OHW = OH * OW;
    const int b = blockIdx.x / tiles_per_img;
    const int q0 = (blockIdx.x - b * tiles_per_img) * BN;
    const int q_end = min(q0 + BN, OHW);
    const int co0 = blockIdx.y * BM;
    const int oh_a = q0 / OW;
    const int oh_b = (q_end - 1) / OW;
    const int PR = (oh_b - oh_a) * stride + K;      // staged rows for this tile
    const int PW = W + 2 * pad;                     // staged row width
    const int PRW = ((rows_max - 1) * stride + K) * PW;  // per-channel pitch in sX
    const int iy0 = oh_a * stride - pad;

    float* sW = smem;
    float* sX = smem + ck * KK * BMP;

    // LDS offset of each lane's output pixel inside a staged channel; lanes past
    // the tile end point at the last real pixel (their results are not stored)
    int loff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int q = min(q0 + wn0 + nt * 32 + l32, q_end - 1);
        int oh = q / OW;
        int ow = q - oh * OW;
        loff[nt] = (oh - oh_a) * stride * PW + ow * stride;
    }

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

    const int nchunks = (cin + ck - 1) / ck;
    const int c_begin = blockIdx.z * chunks_per_split;
    const int c_end = min(nchunks, c_begin + chunks_per_split);
    const float* xb = x + (long)b * cin * H * W;

    for (int chunk = c_begin; chunk < c_end; ++chunk) {
        const int ci0 = chunk * ck;
        __syncthreads();  // the previous chunk's reads are done
        // weights: wave-strided rows m, lanes over the contiguous (ci, tap) run
        for (int m = wave; m < BM; m += 4) {
            const int co = co0 + m;
            const float* wr = w + ((long)co * cin + ci0) * KK;
            for (int t = lane; t < ck * KK; t += 64) {
                const int ci = t / KK;
                float v = 0.0f;
                if (co < cout && ci0 + ci < cin) v = wr[t];
                sW[t * BMP + m] = v;
            }
        }
        // input rows: wave-strided (channel, row) pairs, lanes over columns
        for (int row = wave; row < ck * PR; row += 4) {
            const int ci = row / PR;
            const int r = row - ci * PR;
            const int cig = ci0 + ci;
            const int iy = iy0 + r;
            const bool ok = cig < cin && iy >= 0 && iy < H;
            const float* src = xb + ((long)cig * H + iy) * W;
            float* dst = sX + ci * PRW + r * PW;
            for (int c = lane; c < PW; c += 64) {
                const int ix = c - pad;
                dst[c] = (ok && ix >= 0 && ix < W) ? src[ix] : 0.0f;
            }
        }
        __syncthreads();

        for (int ci = 0; ci < ck; ci += 2) {
            const float* wa = sW + ((ci + hi) * KK) * BMP + wm0 + l32;
            const float* xa = sX + (ci + hi) * PRW;
#pragma unroll
            for (int tap = 0; tap < KK; ++tap) {
                const int toff = (tap / K) * PW + (tap % K);
                float av[MT], bv[NT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = wa[tap * BMP + mt * 32];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bv[nt] = xa[loff[nt] + toff];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] =
                            __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
            }
        }
    }

    // D layout of the 32x32 block: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32.
    const long total = (long)gridDim.x / tiles_per_img * cout * OHW;  // n * cout * OHW
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int q = q0 + wn0 + nt * 32 + l32;
            if (q >= q_end) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + wm0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (co >= cout) continue;
                const long idx = ((long)b * cout + co) * OHW + q;
                if (partial != nullptr)
                    partial[blockIdx.z * total + idx] = acc[mt][nt][r];
                else
                    y[idx] = epilogue(acc[mt][nt][r], scale[co], bias[co], act, res_mode, res, idx);
            }
        }
    }
}

// Adds the split-K slices in slice order and applies the epilogue.
__global__ void __launch_bounds__(256) k_splitk_finish(const float* __restrict__ partial,
                                                       int splitk, long total, int cout, int ohw,
                                                       const float* __restrict__ scale,
                                                       const float* __restrict__ bias,
                                                       const float* __restrict__ res,
                                                       float* __restrict__ y, int act,
                                                       int res_mode)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    float s = partial[idx];
    for (int z = 1; z < splitk; ++z) s += partial[z * total + idx];
    const int co = (int)((idx / ohw) % cout);
    y[idx] = epilogue(s, scale[co], bias[co], act, res_mode, res, idx);
}

int igemm_rows_max(const ConvGeom& g, int bn)
{
    int rows = (bn - 1) / g.ow + 2;
    return rows < g.oh ? rows : g.oh;
}

size_t igemm_lds_bytes(const ConvGeom& g, const GemmTile& t)
{
    const int kk = g.k * g.k;
    const size_t sw = (size_t)t.ck * kk * (t.bm + 1);
    const size_t prw = (size_t)((igemm_rows_max(g, t.bn) - 1) * g.stride + g.k) * (g.w + 2 * g.pad);
    return (sw + (size_t)t.ck * prw) * sizeof(float);
}

bool igemm_tile_supported(const GemmTile& t)
{
    return (t.bm == 64 && t.bn == 64) || (t.bm == 32 && t.bn == 128) ||
           (t.bm == 128 && t.bn == 64) || (t.bm == 64 && t.bn == 128);
}

template <int K>
static hipError_t launch_igemm_k(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                                 const float* scale, const float* bias, const float* res, float* y,
                                 float* partial, hipStream_t s)
{
    const GemmTile& t = p.tile;
    const int ohw = g.oh * g.ow;
    const int tiles = (ohw + t.bn - 1) / t.bn;
    const int nchunks = (g.cin + t.ck - 1) / t.ck;
    const int per_split = (nchunks + t.splitk - 1) / t.splitk;
    const int rows_max = igemm_rows_max(g, t.bn);
    const size_t lds = igemm_lds_bytes(g, t);
    dim3 grid((unsigned)(g.n * tiles), (unsigned)((g.cout + t.bm - 1) / t.bm), (unsigned)t.splitk);
#define CVX_IGEMM(BM_, BN_, WM_, WN_)                                                            \
    hipLaunchKernelGGL((k_igemm<BM_, BN_, WM_, WN_, K>), grid, dim3(256), lds, s, x, w, scale,   \
                       bias, res, y, partial, g.cin, g.h, g.w, g.cout, g.stride, g.pad, g.oh,     \
                       g.ow, t.ck, rows_max, tiles, per_split, g.act, g.res_mode)
    if (t.bm == 64 && t.bn == 64)
        CVX_IGEMM(64, 64, 2, 2);
    else if (t.bm == 32 && t.bn == 128)
        CVX_IGEMM(32, 128, 1, 4);
    else if (t.bm == 128 && t.bn == 64)
        CVX_IGEMM(128, 64, 2, 2);
    else if (t.bm == 64 && t.bn == 128)
        CVX_IGEMM(64, 128, 2, 2);
    else
        return hipErrorInvalidValue;
#undef CVX_IGEMM
    return hipGetLastError();
}

hipError_t launch_igemm(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                        const float* scale, const float* bias, const float* res, float* y,
                        void* ws, hipStream_t s)
{
    float* partial = p.tile.splitk > 1 ? static_cast<float*>(ws) : nullptr;
    hipError_t e;
    if (g.k == 1)
        e = launch_igemm_k<1>(g, p, x, w, scale, bias, res, y, partial, s);
    else if (g.k == 3)
        e = launch_igemm_k<3>(g, p, x, w, scale, bias, res, y, partial, s);
    else
        return hipErrorInvalidValue;
    if (e != hipSuccess || partial == nullptr) return e;
    const long total = (long)g.n * g.cout * g.oh * g.ow;
    dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(k_splitk_finish, grid, dim3(256), 0, s, partial, p.tile.splitk, total,
                       g.cout, g.oh * g.ow, scale, bias, res, y, g.act, g.res_mode);
    return hipGetLastError();
}

}  // namespace cvx
