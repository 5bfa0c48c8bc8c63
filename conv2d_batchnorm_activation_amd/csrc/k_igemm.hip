// k_igemm.hip -- dense KxK (K = 1 or 3) convolution + folded BN + activation
// (+ residual) as an implicit GEMM on the fp32 matrix cores of gfx950.
//
// GEMM view ("YOLO26N Inference Optimisation", "NHWC migration", "What NHWC
// is": the reduction dimension of a convolution cast as a matrix product is
// c_in * kh * kw):
//     M = c_out,  N = output pixels of one image,  K = c_in * kh * kw
//     Y[co][q] = sum_k W[co][k] * X_im2col[k][q]
// The page moved to NHWC because its tensor-core instructions needed the
// reduction dimension contiguous in global memory.  The MI355X matrix cores
// take their operands from VGPRs, which we fill from LDS, so NCHW stays: output
// pixels (N) are contiguous, global loads and stores stay coalesced, and the
// im2col matrix is never materialised.
//
// Per workgroup (256 threads = 4 wave64s), one BM x BN output tile:
//   * the reduction runs over chunks of CK input channels.  For each chunk the
//     weight block W[co0 .. co0+BM)[ci0*KK .. (ci0+CK)*KK) goes to LDS as
//     sW[t][m] (t = ci*KK + tap, odd row pitch BM+1: conflict-free transposed
//     writes and contiguous MFMA reads), and the input region the tile's pixels
//     read (PR rows x PC columns per channel, zero outside the image, so the
//     padding costs nothing in the inner loop) goes to sX[ci][r][c];
//   * every thread owns a fixed set of load slots (NW weight floats, NPX input
//     floats per chunk), computed once; the loads of chunk i+1 are issued into
//     registers before the MFMAs of chunk i, so global latency hides behind the
//     matrix work, and only the LDS writes sit between the two barriers;
//   * the four waves split the tile (WM x WN) and/or the chunk's channel pairs
//     (WK); each wave computes 32x32 blocks with v_mfma_f32_32x32x2_f32 (true
//     fp32), the two K values of one MFMA being two adjacent input channels at
//     one tap; WK > 1 partial tiles are summed through LDS in wave order;
//   * the epilogue (folded BN, residual, activation) runs on the accumulators and
//     each output is stored once, masked to the real pixel count, so rows of any
//     width are never overrun ("Bug fixed: TMA overflow").
// When the tiles alone cannot fill the chip, chunks are also split over
// blockIdx.z; each slice stores raw partial sums in the workspace and a
// finishing kernel adds the slices in slice order (deterministic) and applies
// the epilogue.
#include <stdio.h>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// n / d for 0 <= n < 2^31 with a precomputed multiplier (round-up method):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, q = (umulhi(n, m) + n) >> l.
__device__ __forceinline__ int fdiv(int n, unsigned m, unsigned l)
{
    unsigned hi = __umulhi((unsigned)n, m);
    return (int)((hi + (unsigned)n) >> l);
}

void fastdiv_params(int d, unsigned* m, unsigned* l)
{
    unsigned s = 0;
    while ((1ull << s) < (unsigned long long)d) ++s;
    *l = s;
    *m = (unsigned)(((1ull << 32) * ((1ull << s) - (unsigned long long)d)) / (unsigned long long)d + 1);
}

struct IgemmArgs {
    const float* x;
    const float* w;
    const float* scale;
    const float* bias;
    const float* res;
    float* y;
    float* partial;
    int cin, H, W, cout, stride, pad, OH, OW;
    int tiles_per_img, chunks_per_split;
    int tc;                 // 0: tiles are runs of BN consecutive pixels; else TR x tc blocks
    int tiles_w;            // 2-D tiles: tiles across one band of rows
    unsigned m_tc, l_tc;    // fast division by tc
    int PR, PC;             // staged region per channel (launch constants)
    unsigned m_rc, l_rc;    // fast division by PR*PC
    unsigned m_c, l_c;      // fast division by PC
    unsigned m_ow, l_ow;    // fast division by OW
    int act, res_mode;
};

template <int BM, int BN, int WM, int WN, int WK, int K, int CK, int NPX>
__global__ void __launch_bounds__(256) k_igemm(IgemmArgs a)
{
    static_assert(WM * WN * WK == 4, "four waves per workgroup");
    constexpr int TM = BM / WM, TN = BN / WN;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is made of 32x32 blocks");
    constexpr int MT = TM / 32, NT = TN / 32;
    constexpr int KK = K * K;
    constexpr int BMP = BM + 1;
    constexpr int CKK = CK * KK;
    static_assert((BM * CKK) % 256 == 0, "weight block splits evenly over the threads");
    constexpr int NW = BM * CKK / 256;
    constexpr int PAIRS = CK / 2;
    static_assert(CK % 2 == 0 && PAIRS % WK == 0, "channel pairs split evenly over WK waves");

    extern __shared__ float smem[];
    float* sW = smem;
    float* sX = smem + CKK * BMP;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hi = lane >> 5;
    const int l32 = lane & 31;
    const int wk = wave % WK;
    const int wmn = wave / WK;
    const int wm0 = (wmn / WN) * TM;
    const int wn0 = (wmn % WN) * TN;

    const int OHW = a.OH * a.OW;
    const int HW = a.H * a.W;
    const int b = blockIdx.x / a.tiles_per_img;
    const int tile = blockIdx.x - b * a.tiles_per_img;
    const int co0 = blockIdx.y * BM;
    // Tile origin.  Runs of pixels: q0 .. q0+BN-1 in row-major order; the staged
    // region spans the rows they touch (from column ow_a*s - pad when they stay in
    // one row, else whole rows).  2-D tiles: TR rows x tc columns from (oh0, ow0).
    int q0 = 0, q_end = 0, oh_ref, ix0;
    if (a.tc == 0) {
        q0 = tile * BN;
        q_end = min(q0 + BN, OHW);
        oh_ref = fdiv(q0, a.m_ow, a.l_ow);
        const int ow_a = q0 - oh_ref * a.OW;
        const int oh_b = fdiv(q_end - 1, a.m_ow, a.l_ow);
        ix0 = (oh_ref == oh_b ? ow_a * a.stride : 0) - a.pad;
    } else {
        const int band = tile / a.tiles_w;
        const int tw = tile - band * a.tiles_w;
        oh_ref = band * (BN / a.tc);
        ix0 = tw * a.tc * a.stride - a.pad;
        q0 = tw * a.tc;  // ow0
    }
    const int iy0 = oh_ref * a.stride - a.pad;
    const int RC = a.PR * a.PC;
    const int RE = CK * RC;  // staged input floats per chunk

    // Each lane's output pixel per 32-column block: LDS offset within one staged
    // channel (B operand), and output index (-1: outside the tile or the image,
    // computed on a clamped in-region pixel and not stored).
    int loff[NT], qout[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = wn0 + nt * 32 + l32;
        int oh, ow;
        bool ok;
        if (a.tc == 0) {
            const int q = q0 + j;
            ok = q < q_end;
            const int qc = ok ? q : q_end - 1;
            oh = fdiv(qc, a.m_ow, a.l_ow);
            ow = qc - oh * a.OW;
        } else {
            const int jr = fdiv(j, a.m_tc, a.l_tc);
            oh = oh_ref + jr;
            ow = q0 + (j - jr * a.tc);
            ok = oh < a.OH && ow < a.OW;
            oh = min(oh, a.OH - 1);
            ow = min(ow, a.OW - 1);
        }
        loff[nt] = (oh - oh_ref) * a.stride * a.PC + ow * a.stride - a.pad - ix0;
        qout[nt] = ok ? oh * a.OW + ow : -1;
    }

    // Input load slots: element e = tid + 256*i of the staged region, as a byte
    // offset from the chunk's first channel plane within this image; kOOB (reads
    // as 0) outside the image or past the region.  Channels past c_in fall
    // outside the image's descriptor and read as 0 too.
    unsigned goff[NPX];
#pragma unroll
    for (int i = 0; i < NPX; ++i) {
        const int e = tid + 256 * i;
        const int ci = fdiv(e, a.m_rc, a.l_rc);
        const int rem = e - ci * RC;
        const int r = fdiv(rem, a.m_c, a.l_c);
        const int c = rem - r * a.PC;
        const int iy = iy0 + r, ix = ix0 + c;
        goff[i] = (e < RE && iy >= 0 && iy < a.H && ix >= 0 && ix < a.W)
                      ? 4u * (unsigned)(ci * HW + iy * a.W + ix) : kOOB;
    }
    // Weight load slots: float f = tid + 256*j of the BM x CK*KK block.  Rows past
    // c_out fall outside the descriptor (read 0); in a last, partial chunk the
    // columns past c_in read the next row's weights, which multiply inputs that
    // read as 0.
    unsigned woff[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int f = tid + 256 * j;
        const int m = f / CKK, t = f - m * CKK;
        woff[j] = co0 + m < a.cout ? 4u * (unsigned)((co0 + m) * a.cin * KK + t) : kOOB;
    }
    const rsrc_t rx = make_rsrc(a.x + (long)b * a.cin * HW, 4u * (unsigned)(a.cin * HW));
    const rsrc_t rw = make_rsrc(a.w, 4u * (unsigned)(a.cout * a.cin * KK));
    float pw[NW], px[NPX];

    auto load_chunk = [&](int chunk) {
        const unsigned wb = 4u * (unsigned)(chunk * CK * KK);
#pragma unroll
        for (int j = 0; j < NW; ++j) pw[j] = bload(rw, woff[j] + wb);
        const unsigned xb = 4u * (unsigned)(chunk * CK * HW);
#pragma unroll
        for (int i = 0; i < NPX; ++i) px[i] = bload(rx, goff[i] + xb);
    };
    auto store_chunk = [&]() {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const int f = tid + 256 * j;
            const int m = f / CKK, t = f - m * CKK;
            sW[t * BMP + m] = pw[j];
        }
        // slots past the region store into LDS that is allocated but never read
#pragma unroll
        for (int i = 0; i < NPX; ++i) sX[tid + 256 * i] = px[i];
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.0f;

    const int nchunks = (a.cin + CK - 1) / CK;
    const int c_begin = blockIdx.z * a.chunks_per_split;
    const int c_end = min(nchunks, c_begin + a.chunks_per_split);

    if (c_begin < c_end) load_chunk(c_begin);
    for (int chunk = c_begin; chunk < c_end; ++chunk) {
        __syncthreads();  // every wave is done reading the previous chunk
        store_chunk();
        __syncthreads();
        if (chunk + 1 < c_end) load_chunk(chunk + 1);  // lands while the MFMAs run
#pragma unroll
        for (int jp = 0; jp < PAIRS / WK; ++jp) {
            const int ci = 2 * (wk + WK * jp) + hi;
            const float* wa = sW + ci * KK * BMP + wm0 + l32;
            const float* xa = sX + ci * RC;
#pragma unroll
            for (int tap = 0; tap < KK; ++tap) {
                const int toff = (tap / K) * a.PC + (tap % K);
                float av[MT], bv[NT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) av[mt] = wa[tap * BMP + mt * 32];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bv[nt] = xa[loff[nt] + toff];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mt], bv[nt],
                                                                           acc[mt][nt], 0, 0, 0);
            }
        }
    }

    if constexpr (WK > 1) {
        // sum the WK partial tiles of each (wm, wn) group through LDS, in wave order
        __syncthreads();
        float* red = smem;
        constexpr int SLAB = MT * NT * 16 * 64;
        if (wk > 0) {
            float* dst = red + (wmn * (WK - 1) + wk - 1) * SLAB;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dst[((mt * NT + nt) * 16 + r) * 64 + lane] = acc[mt][nt][r];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int k = 1; k < WK; ++k) {
            const float* src = red + (wmn * (WK - 1) + k - 1) * SLAB;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[mt][nt][r] += src[((mt * NT + nt) * 16 + r) * 64 + lane];
        }
    }

    // D layout of a 32x32 block: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32.  The epilogue issues every load it
    // needs (scale, bias, residual) as one batch, then computes and stores; rows
    // past c_out and pixels outside the tile get kOOB offsets (loads read 0,
    // stores are dropped).
    const unsigned plane_b = 4u * (unsigned)OHW;
    unsigned rowoff[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int co = co0 + wm0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            rowoff[mt][r] = co < a.cout ? (unsigned)(b * a.cout + co) * plane_b : kOOB;
        }
    unsigned qb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qb[nt] = qout[nt] >= 0 ? 4u * (unsigned)qout[nt] : kOOB;
    const unsigned out_bytes = 4u * (unsigned)((gridDim.x / a.tiles_per_img) * a.cout * OHW);
    if (a.partial != nullptr) {
        const rsrc_t rp = make_rsrc(a.partial + (long)blockIdx.z * (out_bytes / 4), out_bytes);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    bstore(rp, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB),
                           acc[mt][nt][r]);
        return;
    }
    const rsrc_t rsb = make_rsrc(a.scale, 4u * (unsigned)a.cout);
    const rsrc_t rbb = make_rsrc(a.bias, 4u * (unsigned)a.cout);
    float sc[MT][16], bi[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int co = co0 + wm0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const unsigned o = co < a.cout ? 4u * (unsigned)co : kOOB;
            sc[mt][r] = bload(rsb, o);
            bi[mt][r] = bload(rbb, o);
        }
    const rsrc_t ry = make_rsrc(a.y, out_bytes);
    float rv[MT][NT][16];
    if (a.res_mode != CVX_RES_NONE) {
        const rsrc_t rr = make_rsrc(a.res, out_bytes);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    rv[mt][nt][r] = bload(rr, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float z = fmaf(sc[mt][r], acc[mt][nt][r], bi[mt][r]);
                if (a.res_mode == CVX_RES_BEFORE_ACT) z += rv[mt][nt][r];
                z = apply_act_fast(z, a.act);
                if (a.res_mode == CVX_RES_AFTER_ACT) z += rv[mt][nt][r];
                bstore(ry, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB), z);
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

// ------------------------------------------------------------------ host side
// The compiled tile configurations.  ck = 16 channels per chunk throughout.
struct TileKind {
    int bm, bn, wm, wn, wk, npx;
};
static constexpr TileKind kTiles[] = {
    {32, 32, 1, 1, 4, 24},   // T0: small tiles, four waves split the reduction
    {32, 64, 1, 2, 2, 24},   // T1
    {64, 64, 2, 2, 1, 24},   // T2
    {64, 128, 2, 2, 1, 24},  // T3: wide tiles for large maps / batches
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kCK = 16;

int igemm_num_tiles() { return kNumTiles; }

// Staged region per channel (rows x columns) for tile kind `tile` with layout tc
// (0 = runs of pixels, else 2-D tiles of BN/tc rows x tc columns).
void igemm_region(const ConvGeom& g, int bn, int tc, int* pr, int* pc)
{
    if (tc > 0) {
        *pr = (bn / tc - 1) * g.stride + g.k;
        *pc = (tc - 1) * g.stride + g.k;
        return;
    }
    if (g.ow % bn == 0) {  // runs never leave their output row
        *pr = g.k;
        *pc = (bn - 1) * g.stride + g.k;
    } else if (bn % g.ow == 0 && bn / g.ow <= g.oh) {  // whole rows per tile
        *pr = (bn / g.ow - 1) * g.stride + g.k;
        *pc = g.w + 2 * g.pad;
    } else {
        int rows = (bn - 1) / g.ow + 2;
        rows = rows < g.oh ? rows : g.oh;
        *pr = (rows - 1) * g.stride + g.k;
        *pc = g.w + 2 * g.pad;
    }
}

long igemm_tiles_per_image(const ConvGeom& g, int tile, int tc)
{
    const int bn = kTiles[tile].bn;
    if (tc == 0) return (g.oh * g.ow + bn - 1) / bn;
    const int tr = bn / tc;
    return (long)((g.oh + tr - 1) / tr) * ((g.ow + tc - 1) / tc);
}

long igemm_stage_floats(const ConvGeom& g, int tile, int tc)
{
    int pr, pc;
    igemm_region(g, kTiles[tile].bn, tc, &pr, &pc);
    return (long)kCK * pr * pc + (long)kTiles[tile].bm * kCK * g.k * g.k;
}

bool igemm_tile_fits(const ConvGeom& g, int tile, int tc, size_t* lds_bytes)
{
    const TileKind& t = kTiles[tile];
    // every buffer the kernel addresses must stay below 2^31 bytes (32-bit offsets)
    const long lim = 0x7fffffffL;
    if ((long)g.cin * g.h * g.w * 4 >= lim || (long)g.cout * g.cin * g.k * g.k * 4 >= lim ||
        (long)g.n * g.cout * g.oh * g.ow * 4 >= lim)
        return false;
    if (tc < 0 || (tc > 0 && (t.bn % tc != 0 || (tc & (tc - 1)) != 0))) return false;
    int pr, pc;
    igemm_region(g, t.bn, tc, &pr, &pc);
    const long re = (long)kCK * pr * pc;
    if (re > 256L * t.npx) return false;
    const int kk = g.k * g.k;
    const size_t stage = ((size_t)kCK * kk * (t.bm + 1) + 256 * (size_t)t.npx) * sizeof(float);
    const size_t red = t.wk > 1 ? (size_t)(4 / t.wk) * (t.wk - 1) * (t.bm / t.wm / 32) *
                                      (t.bn / t.wn / 32) * 16 * 64 * sizeof(float)
                                : 0;
    const size_t lds = stage > red ? stage : red;
    if (lds > kMaxLdsBytes) return false;
    if (lds_bytes) *lds_bytes = lds;
    return true;
}

void igemm_tile_shape(int tile, int* bm, int* bn)
{
    *bm = kTiles[tile].bm;
    *bn = kTiles[tile].bn;
}

int igemm_chunk_channels() { return kCK; }

template <int K, int TILE>
static void launch_tile(dim3 grid, size_t lds, hipStream_t s, const IgemmArgs& a)
{
    constexpr TileKind t = kTiles[TILE];
    hipLaunchKernelGGL((k_igemm<t.bm, t.bn, t.wm, t.wn, t.wk, K, kCK, t.npx>), grid, dim3(256), lds,
                       s, a);
}

template <int K>
static void launch_k(int tile, dim3 grid, size_t lds, hipStream_t s, const IgemmArgs& a)
{
    switch (tile) {
    case 0: launch_tile<K, 0>(grid, lds, s, a); break;
    case 1: launch_tile<K, 1>(grid, lds, s, a); break;
    case 2: launch_tile<K, 2>(grid, lds, s, a); break;
    case 3: launch_tile<K, 3>(grid, lds, s, a); break;
    }
}

hipError_t launch_igemm(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                        const float* scale, const float* bias, const float* res, float* y,
                        void* ws, hipStream_t s)
{
    const int tile = p.tile.kind;
    if (tile < 0 || tile >= kNumTiles || (g.k != 1 && g.k != 3)) return hipErrorInvalidValue;
    size_t lds = 0;
    if (!igemm_tile_fits(g, tile, p.tile.tc, &lds)) return hipErrorInvalidValue;
    const TileKind& t = kTiles[tile];
    IgemmArgs a;
    a.x = x;
    a.w = w;
    a.scale = scale;
    a.bias = bias;
    a.res = res;
    a.y = y;
    a.partial = p.tile.splitk > 1 ? static_cast<float*>(ws) : nullptr;
    a.cin = g.cin;
    a.H = g.h;
    a.W = g.w;
    a.cout = g.cout;
    a.stride = g.stride;
    a.pad = g.pad;
    a.OH = g.oh;
    a.OW = g.ow;
    a.tc = p.tile.tc;
    a.tiles_per_img = (int)igemm_tiles_per_image(g, tile, a.tc);
    a.tiles_w = a.tc > 0 ? (g.ow + a.tc - 1) / a.tc : 0;
    fastdiv_params(a.tc > 0 ? a.tc : 1, &a.m_tc, &a.l_tc);
    const int nchunks = (g.cin + kCK - 1) / kCK;
    a.chunks_per_split = (nchunks + p.tile.splitk - 1) / p.tile.splitk;
    igemm_region(g, t.bn, a.tc, &a.PR, &a.PC);
    fastdiv_params(a.PR * a.PC, &a.m_rc, &a.l_rc);
    fastdiv_params(a.PC, &a.m_c, &a.l_c);
    fastdiv_params(g.ow, &a.m_ow, &a.l_ow);
    a.act = g.act;
    a.res_mode = g.res_mode;
    dim3 grid((unsigned)(g.n * a.tiles_per_img), (unsigned)((g.cout + t.bm - 1) / t.bm),
              (unsigned)p.tile.splitk);
    if (g.k == 1)
        launch_k<1>(tile, grid, lds, s, a);
    else
        launch_k<3>(tile, grid, lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.partial == nullptr) return e;
    return launch_splitk_finish(g, p.tile.splitk, a.partial, scale, bias, res, y, s);
}

void igemm_kernel_name(const ConvGeom& g, int tile, char* buf, int len)
{
    const TileKind& t = kTiles[tile];
    snprintf(buf, len, "cvx::k_igemm<%d, %d, %d, %d, %d, %d, %d, %d>", t.bm, t.bn, t.wm, t.wn, t.wk,
             g.k, kCK, t.npx);
}

hipError_t launch_splitk_finish(const ConvGeom& g, int splitk, const float* partial,
                                const float* scale, const float* bias, const float* res, float* y,
                                hipStream_t s)
{
    const long total = (long)g.n * g.cout * g.oh * g.ow;
    dim3 fgrid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(k_splitk_finish, fgrid, dim3(256), 0, s, partial, splitk, total, g.cout,
                       g.oh * g.ow, scale, bias, res, y, g.act, g.res_mode);
    return hipGetLastError();
}

}  // namespace cvx
