// k_stem_pair.hip -- the first two convolutions of a detector stem as one
// kernel: a direct 3x3 convolution of a few input channels into 16 channels
// (folded BN, activation), whose output only the next layer reads, and that
// next layer, a dense 3x3 convolution on fp32 matrix cores (folded BN,
// residual, activation) -- "YOLO26N Inference Optimisation", "Baseline
// benchmark" (the stem's two Conv2d+BN+SiLU blocks) and "Improvements"
// (fusing what a layer writes into what the next one reads).
//
// Run apart, the two layers are each one round of workgroups whose latency
// (argument fetch, first loads, store drain) nothing overlaps, and the 16
// channels in between go through memory.  Here a workgroup computes one tile of
// the second layer (32 output channels x 32*NT pixels, a block of TR rows x TC
// columns) and makes its input itself:
//   1. all eight waves copy the first layer's input window (every channel, the
//      rows and columns the tile's 3x3 windows of 3x3 windows reach) to LDS
//      with 16-byte LDS-direct loads; outside the image they read zeros (the
//      first layer's padding).  With U8 the input is a u8 frame instead: the
//      two frame rows each window row interpolates between are staged, then
//      resized (half-pixel bilinear) and normalised into the window, so the
//      normalised image is never written ("A fused Ampere preprocess kernel",
//      "The theory");
//   2. all eight waves compute the first layer's 16 output channels over the
//      region the tile's 3x3 windows cover, on matrix cores
//      (v_mfma_f32_16x16x4_f32: 16 pixels x 16 channels a block, the taps
//      read from the LDS window), apply its BN and activation and store them
//      to LDS in the layout the matrix loop reads, writing zeros outside the
//      image (the second layer's padding);
//   3. four consumer waves run the second layer's reduction (16 channels x 9
//      taps) on v_mfma_f32_32x32x2_f32, as k_igemm_packed does for one chunk,
//      sum their partial tiles through LDS and apply the epilogue.
// The first layer's outputs are recomputed where the regions of neighbouring
// tiles overlap (about a quarter more of them), which costs less than writing
// and reading the 16 channels and running a second round of workgroups.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSPThreads = 512;
constexpr int kC1 = 16;              // channels between the two layers: one chunk
constexpr int kWinRounds = 6;        // 512-lane rounds of 16-byte window loads, at most
constexpr int kSrcRounds = 6;        // 512-lane rounds of 16-byte frame loads (u8 source), at most
constexpr int kMaxCin1 = 4;
constexpr int kBCFloats = 4 * 5 * 256;  // packed 3x3 floats per (32-row block, chunk)

__device__ __forceinline__ int sp_div(int n, unsigned m, unsigned l)
{
    return (int)((__umulhi((unsigned)n, m) + (unsigned)n) >> l);
}

__device__ __forceinline__ void sp_lds_load16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}

}  // namespace

struct StemPairArgs {
    const float* x;       // layer 1 input [n][cin1][H1][W1]
    const float* w1;      // layer 1 weights [16][cin1][3][3]
    const float* scale1;
    const float* bias1;
    const float* wp;      // layer 2 packed 3x3 weights (c_in 16: one chunk per row block)
    const float* scale2;
    const float* bias2;
    const float* res;
    float* y;
    int n, cin1, H1, W1, S1;  // layer 1
    int H2, W2;               // layer 1 output = layer 2 input
    int S2, OH, OW, cout;     // layer 2
    int act1, act2, res_mode;
    int tc, tr, tiles_w, tiles_per_img, nmb;
    unsigned m_tc, l_tc, m_tw, l_tw, m_tpi, l_tpi, m_nb, l_nb;
    int PR, PCW;              // staged layer-1 output region per channel: PR rows x PCW floats
    unsigned m_pcw, l_pcw;    // divide by PCW
    int WR, WCW;              // layer-1 input window per channel: WR rows x WCW floats
    int win_elems, win_rounds;  // 16-byte elements of the window, 512-lane rounds
    unsigned m_we, l_we;      // divide by WCW / 4
    unsigned m_wc, l_wc;      // divide by WR * WCW / 4 (elements per channel)
    unsigned x_bytes, wp_bytes;
    int vout;
    // u8 source: layer 1's input is a u8 HWC frame, resized (half-pixel
    // bilinear) and normalised here, as the stem prologue does
    const unsigned char* src;
    int src_h, src_w;
    unsigned row_bytes, img_bytes;
    unsigned m_dh, l_dh, m_dw, l_dw;  // divide by 2 * H1, 2 * W1
    float inv_dh, inv_dw;             // 1 / (2 * H1), 1 / (2 * W1)
    float na[3], nb[3];               // /255 and the normalisation: v * na + nb
    int SRB;                          // bytes of a staged frame row segment (multiple of 16)
    int src_elems, src_rounds;        // 16-byte elements staged, 512-lane rounds
    unsigned m_srb, l_srb;            // divide by SRB / 16
    unsigned m_wcw, l_wcw;            // divide by WCW
};

// Source row (or column) pair and weight of destination index d for the
// half-pixel bilinear resize, from integers: (2d + 1) * src - dst over 2 * dst,
// clamped at 0 and at the last row (the prologue's arithmetic).
struct SrcAxis {
    int i0, i1;
    float f;
};
__device__ __forceinline__ SrcAxis sp_axis(int d, int src, int dst, unsigned m, unsigned l, float inv)
{
    const int num = (2 * d + 1) * src - dst;
    SrcAxis a;
    if (num <= 0) {
        a.i0 = 0;
        a.f = 0.0f;
    } else {
        const unsigned q = (__umulhi((unsigned)num, m) + (unsigned)num) >> l;
        a.i0 = (int)q;
        a.f = (float)((unsigned)num - q * (2u * (unsigned)dst)) * inv;
    }
    if (a.i0 > src - 1) a.i0 = src - 1;
    a.i1 = a.i0 + 1 < src ? a.i0 + 1 : src - 1;
    return a;
}

template <int NT, int S1, int C1, bool U8>
__global__ void __launch_bounds__(kSPThreads) k_stem_pair(StemPairArgs a)
{
    // the first layer's reduction: C1 channels x 9 taps, four per matrix
    // instruction (a compile-time count, so that its operands sit in fixed
    // registers and every LDS read of a block can be issued ahead)
    constexpr int KT = C1 * 9;
    constexpr int STEPS = (KT + 3) / 4;
    constexpr int BN = 32 * NT;
    constexpr int PITCH = BN + 4;
    extern __shared__ __attribute__((aligned(16))) float smem[];
    warm_kernargs<sizeof(StemPairArgs)>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // workgroup -> (row block, image, tile), dealt to the XCDs in turn
    int mb, b, tile;
    {
        const unsigned h = blockIdx.x, G8 = gridDim.x;
        const unsigned xcd = h & 7u, i8 = h >> 3, base = G8 >> 3, rem = G8 & 7u;
        const int L = (int)(xcd * base + min(xcd, rem) + i8);
        mb = sp_div(L, a.m_nb, a.l_nb);
        const int bt = L - mb * (a.n * a.tiles_per_img);
        b = sp_div(bt, a.m_tpi, a.l_tpi);
        tile = bt - b * a.tiles_per_img;
    }
    const int band = sp_div(tile, a.m_tw, a.l_tw);
    const int tw = tile - band * a.tiles_w;
    const int oh_ref = band * a.tr;
    const int ow0 = tw * a.tc;
    const int gx0 = (ow0 * a.S2 - 1) & ~3;   // first staged column of the region (16-byte aligned)
    const int iy0 = oh_ref * a.S2 - 1;       // first staged row of the region
    // LDS: the first layer's input window from 0, its output region after it
    // (the staged frame rows, dead once resized, share the region's space),
    // and the consumers' exchange from 0 again once the region has been read
    const int RS = a.PR * a.PCW;             // LDS floats per region channel
    constexpr int WIN = 0;                   // the window
    const int REG = a.cin1 * a.WR * a.WCW;   // the region (a multiple of 4 floats)
    constexpr int XO = 0;                    // the exchange
    const int wx0 = S1 * gx0 - 4;            // first window column (16-byte aligned)
    const int wy0 = S1 * iy0 - 1;            // first window row

    // ---- 1. the first layer's input window -> LDS (all waves).  From a u8
    // frame: the frame rows the window rows interpolate between (each once,
    // from the first window row's upper one on), over the window's span of
    // frame columns, go to LDS (16-byte LDS-direct loads), then are resized
    // and normalised into the window below.
    const int SRC = 4 * REG;                              // byte offset of the staged frame rows
    int sb0 = 0;                                          // first staged frame byte of a row
    if constexpr (U8) {
        const int x_lo = max(wx0, 0);
        sb0 = (3 * sp_axis(x_lo, a.src_w, a.W1, a.m_dw, a.l_dw, a.inv_dw).i0) & ~15;
        const int sy0 = sp_axis(max(wy0, 0), a.src_h, a.H1, a.m_dh, a.l_dh, a.inv_dh).i0;  // first staged row
        const rsrc_t rs = make_rsrc(a.src + (long)b * a.img_bytes, a.img_bytes);
        const int epr = a.SRB >> 4;
        unsigned char* sm = reinterpret_cast<unsigned char*>(smem);
#pragma unroll
        for (int i = 0; i < kSrcRounds; ++i) {
            if (i >= a.src_rounds) break;
            const int e = tid + kSPThreads * i;
            const int rr = sp_div(e, a.m_srb, a.l_srb);  // staged row: frame row sy0 + rr
            const int j = e - rr * epr;
            const int srow = sy0 + rr;
            const bool ok = e < a.src_elems && srow < a.src_h;
            const unsigned off = ok ? (unsigned)srow * a.row_bytes + (unsigned)(sb0 + 16 * j) : kOOB;
            // lane l of the wave writes 16 bytes at d + 16 l: element e lands at SRC + 16 e
            sp_lds_load16(rs, (__attribute__((address_space(3))) void*)(sm + SRC + 16 * (kSPThreads * i + 64 * wave)), off);
        }
        // while the rows are in flight: the resize's column and row terms, once
        // per window column and row (the interpolation below then looks them
        // up): column -> {first and second source byte in a staged row,
        // weight, inside the image}; row -> {weight, inside the image, byte
        // offsets of its two staged rows}
        const int TB = SRC + 16 * kSPThreads * a.src_rounds;
        if (tid < a.WCW) {
            const int x = wx0 + tid;
            const bool ok = (unsigned)x < (unsigned)a.W1;
            const SrcAxis ax = sp_axis(ok ? x : 0, a.src_w, a.W1, a.m_dw, a.l_dw, a.inv_dw);
            *reinterpret_cast<int4*>(sm + TB + 16 * tid) =
                int4{ok ? 3 * ax.i0 - sb0 : 0, ok ? 3 * ax.i1 - sb0 : 0, __float_as_int(ax.f), ok ? 1 : 0};
        } else if (tid - a.WCW < a.WR) {
            const int r = tid - a.WCW;
            const int y = wy0 + r;
            const bool ok = (unsigned)y < (unsigned)a.H1;
            const SrcAxis ay = sp_axis(ok ? y : 0, a.src_h, a.H1, a.m_dh, a.l_dh, a.inv_dh);
            *reinterpret_cast<int4*>(sm + TB + 16 * a.WCW + 16 * r) =
                int4{__float_as_int(ay.f), ok ? 1 : 0, ok ? (ay.i0 - sy0) * a.SRB : 0, ok ? (ay.i1 - sy0) * a.SRB : 0};
        }
    } else {
        const rsrc_t rx = make_rsrc(a.x, a.x_bytes);
        const int epr = a.WCW >> 2;  // 16-byte elements per window row
#pragma unroll
        for (int i = 0; i < kWinRounds; ++i) {
            if (i >= a.win_rounds) break;
            const int e = tid + kSPThreads * i;
            const int ci = sp_div(e, a.m_wc, a.l_wc);
            const int rem = e - ci * (a.WR * epr);
            const int r = sp_div(rem, a.m_we, a.l_we);
            const int c4 = rem - r * epr;
            const int iy = wy0 + r, ix = wx0 + 4 * c4;
            const bool ok = e < a.win_elems && (unsigned)iy < (unsigned)a.H1 && ix >= 0 && ix + 4 <= a.W1;
            const unsigned off = ok ? 4u * (unsigned)(((b * a.cin1 + ci) * a.H1 + iy) * a.W1 + ix) : kOOB;
            // lane l of the wave writes 16 bytes at d + 16 l: element e lands at WIN + 4 e
            // (a round's lanes past the window write zeros into the region, which
            // the first layer rewrites whole)
            sp_lds_load16(rx, (__attribute__((address_space(3))) void*)(smem + WIN + 4 * (kSPThreads * i + 64 * wave)), off);
        }
    }

    // the first layer's operands of this lane for phase 2 (all waves): its
    // weight of each step (channel l%16, tap 4s + l/16; zero past c_in x 9),
    // where that tap sits in the window, and its channel's scale and bias --
    // loaded now, so that their latency hides under the window's
    const int co1 = lane & 15;
    const int kg = lane >> 4;
    float bw[STEPS];
    int aoff[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int k = 4 * st + kg;
        const bool live = k < KT;
        bw[st] = live ? a.w1[co1 * KT + k] : 0.0f;
        const int ci = k / 9, t = k - 9 * (k / 9);
        aoff[st] = live ? (ci * a.WR + t / 3) * a.WCW + t % 3 + 3 : 0;
    }
    const float s1 = a.scale1[co1], b1 = a.bias1[co1];

    // consumers: the second layer's weights (one chunk of row block mb, this
    // wave's quarter, in the operand's lane order), scale, bias and residual
    const bool consumer = wave < 4;
    const int erow = 8 * (wave & 3) + (lane >> 3);
    const int eco = mb * 32 + erow;
    const bool row_ok = eco < a.cout;
    f32x4 wq[4];
    f32x2 wt;
    float sc2 = 0.0f, bi2 = 0.0f;
    f32x4 rv[NT];
    const unsigned plane_b = 4u * (unsigned)(a.OH * a.OW);
    const unsigned out_bytes = 4u * (unsigned)(a.n * a.cout * a.OH * a.OW);
    // output offset of pixel e of this lane's quad k, or kOOB
    auto at = [&](int k, int e) {
        const int p = 32 * k + 4 * (lane & 7) + e;
        const int jr = sp_div(p, a.m_tc, a.l_tc);
        const int oh = oh_ref + jr, ow = ow0 + (p - jr * a.tc);
        const bool ok = oh < a.OH && ow < a.OW && row_ok;
        return ok ? (unsigned)(b * a.cout + eco) * plane_b + 4u * (unsigned)(oh * a.OW + ow) : kOOB;
    };
    if (consumer) {
        const rsrc_t rw = make_rsrc(a.wp, a.wp_bytes);
        const unsigned wo = 4u * (unsigned)(mb * kBCFloats + (wave & 3) * (kBCFloats / 4)) + 16u * (unsigned)lane;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            wq[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wo + 1024u * s), 0, 0));
        wt = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(wo + 4096u), 0, 0));
        const unsigned o = row_ok ? 4u * (unsigned)eco : kOOB;
        sc2 = bload(make_rsrc(a.scale2, 4u * (unsigned)a.cout), o);
        bi2 = bload(make_rsrc(a.bias2, 4u * (unsigned)a.cout), o);
        const rsrc_t rr = make_rsrc(a.res, a.res_mode != CVX_RES_NONE ? out_bytes : 0u);
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            if (a.vout) {
                rv[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)at(k, 0), 0, 0));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[k][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, (int)at(k, e), 0, 0));
            }
        }
    }
    // the window (or the frame rows) has landed, and with it every operand load above
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if constexpr (U8) {
        // resize and normalise the frame rows into the window: a thread takes
        // a window pixel (row r, column col) and its three channels; outside the
        // resized image, zeros (the first layer's padding)
        const unsigned char* sm = reinterpret_cast<const unsigned char*>(smem) + SRC;
        const unsigned char* tb = reinterpret_cast<const unsigned char*>(smem) + SRC + 16 * kSPThreads * a.src_rounds;
        const int n_px = a.WR * a.WCW;
        for (int idx = tid; idx < n_px; idx += kSPThreads) {
            const int r = sp_div(idx, a.m_wcw, a.l_wcw);
            const int col = idx - r * a.WCW;
            const int4 cx = *reinterpret_cast<const int4*>(tb + 16 * col);
            const int4 cy = *reinterpret_cast<const int4*>(tb + 16 * a.WCW + 16 * r);
            const bool ok = (cx.w & cy.y) != 0;
            const SrcAxis ax{0, 0, __int_as_float(cx.z)}, ay{0, 0, __int_as_float(cy.x)};
            const unsigned char* r0 = sm + cy.z;
            const unsigned char* r1 = sm + cy.w;
            const int c0 = ok ? cx.x : 0, c1 = ok ? cx.y : 0;
            // all twelve bytes first: the window stores below could alias them
            // as far as the compiler knows, and would otherwise wait on each
            unsigned char px[4][3];
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                px[0][ch] = r0[c0 + ch];
                px[1][ch] = r0[c1 + ch];
                px[2][ch] = r1[c0 + ch];
                px[3][ch] = r1[c1 + ch];
            }
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) {
                const float p00 = (float)px[0][ch], p01 = (float)px[1][ch];
                const float p10 = (float)px[2][ch], p11 = (float)px[3][ch];
                const float top = fmaf(ax.f, p01 - p00, p00);
                const float bot = fmaf(ax.f, p11 - p10, p10);
                const float v = fmaf(fmaf(ay.f, bot - top, top), a.na[ch], a.nb[ch]);
                smem[WIN + (ch * a.WR + r) * a.WCW + col] = ok ? v : 0.0f;
            }
        }
        lds_barrier();
    }

    // ---- 2. the first layer over the region (all waves), on matrix cores:
    // v_mfma_f32_16x16x4_f32 with the region's pixels as rows (16 consecutive
    // of its flat [row][column] order per block), the 16 channels as columns
    // and K = c_in x 9 taps, four per instruction (lane l: pixel l%16 of the
    // block, tap 4s + l/16 of step s; the weights' lane: channel l%16, same
    // tap).  A lane's four sums are four consecutive pixels of channel l%16,
    // which go to the region as one 16-byte store.  Taps past c_in x 9 have
    // zero weights.  Wave w takes blocks w, w+8, ...
    {
        const int nblk = (RS + 15) >> 4;
        for (int blk = wave; blk < nblk; blk += 8) {
            // the A operand's pixel of this lane: flat index, clamped into the region
            const int f = min(16 * blk + (lane & 15), RS - 1);
            const int r = sp_div(f, a.m_pcw, a.l_pcw);
            const int x = f - r * a.PCW;
            const float* wb = smem + WIN + S1 * r * a.WCW + S1 * x;
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            float av[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) av[st] = wb[aoff[st]];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bw[st], acc, 0, 0, 0);
            // sums: channel co1, flat pixels fo .. fo+3 (one region row: PCW % 4 == 0)
            const int fo = 16 * blk + 4 * kg;
            if (fo < RS) {
                const int ro = sp_div(fo, a.m_pcw, a.l_pcw);
                const int xo = fo - ro * a.PCW;
                const bool rok = (unsigned)(iy0 + ro) < (unsigned)a.H2;
                f32x4 o;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float t = apply_act_fast(fmaf(s1, acc[v], b1), a.act1);
                    o[v] = rok && (unsigned)(gx0 + xo + v) < (unsigned)a.W2 ? t : 0.0f;
                }
                *reinterpret_cast<f32x4*>(smem + REG + co1 * RS + fo) = o;
            }
        }
    }
    lds_barrier();

    if (!consumer) {
        __syncthreads();  // the region read: the exchange overwrites it
        __syncthreads();  // the consumers' exchange
        return;
    }

    // ---- 3. the second layer: one chunk of 16 channels x 9 taps; wave h takes
    // channel pairs 2h and 2h+1 (lane: channel 2 (2h + pp) + hi)
    int loff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int j = nt * 32 + l32;
        const int jr = sp_div(j, a.m_tc, a.l_tc);
        const int oh = min(oh_ref + jr, a.OH - 1);
        const int ow = min(ow0 + (j - jr * a.tc), a.OW - 1);
        loff[nt] = (oh - oh_ref) * a.S2 * a.PCW + ow * a.S2 - 1 - gx0;
    }
    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
    auto wsel = [&](int f) { return f < 16 ? wq[f / 4][f % 4] : wt[f - 16]; };
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const float* xa = smem + REG + (2 * (2 * wave + pp) + hi) * RS;
        float bv[9][NT];
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const int toff = (tap / 3) * a.PCW + (tap % 3);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[tap][nt] = xa[loff[nt] + toff];
        }
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const float wv = wsel(9 * pp + tap);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[tap][nt], wv, acc[nt], 0, 0, 0);
        }
    }

    // partial tiles of the four waves through LDS (over the window and the
    // region, once every wave has read its part of the region), then wave w
    // sums channels 8w .. 8w+7 of the tile
    __syncthreads();
    {
        float* red = smem + XO + wave * 32 * PITCH + l32 * PITCH + 4 * hi;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4*>(red + 32 * nt + 8 * g) =
                    f32x4{acc[nt][4 * g], acc[nt][4 * g + 1], acc[nt][4 * g + 2], acc[nt][4 * g + 3]};
    }
    __syncthreads();
    const rsrc_t ry = make_rsrc(a.y, out_bytes);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int off = XO + erow * PITCH + 32 * k + 4 * (lane & 7);
        f32x4 v = *reinterpret_cast<const f32x4*>(smem + off);
#pragma unroll
        for (int s = 1; s < 4; ++s) v += *reinterpret_cast<const f32x4*>(smem + s * 32 * PITCH + off);
        f32x4 z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = fmaf(sc2, v[e], bi2);
            if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[k][e];
            t = apply_act_fast(t, a.act2);
            if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[k][e];
            z[e] = t;
        }
        if (a.vout) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z), ry, (int)at(k, 0), 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = z[e];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, f), ry, (int)at(k, e), 0, 0);
            }
        }
    }
}

// ------------------------------------------------------------------ host side
void fastdiv_params(int d, unsigned* m, unsigned* l);

namespace {

struct PairGeom {
    int nt, tc, tr, tiles_w, tiles_per_img, nmb;
    int PR, PCW, WR, WCW, win_elems, win_rounds;
    int SRB, src_elems, src_rounds;  // u8 source only
    size_t lds;
};

// Source column index pair of destination column d (host copy of sp_axis's
// integer part).
int host_axis_i0(int d, int src, int dst)
{
    const long num = (long)(2 * d + 1) * src - dst;
    long q = num <= 0 ? 0 : num / (2L * dst);
    return (int)std::min<long>(q, src - 1);
}

// The region of layer-1 outputs a tile of layer 2 reads, and the window of
// layer-1 inputs that region needs; with a u8 source (pre != null), the frame
// rows the window interpolates from, their widest byte span over the tiles.
bool pair_geom(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre, int nt, int tc, PairGeom* pg)
{
    const int bn = 32 * nt;
    if (tc <= 0 || bn % tc != 0 || (tc * g2.stride) % 4 != 0) return false;
    pg->nt = nt;
    pg->tc = tc;
    pg->tr = bn / tc;
    pg->tiles_w = (g2.ow + tc - 1) / tc;
    pg->tiles_per_img = ((g2.oh + pg->tr - 1) / pg->tr) * pg->tiles_w;
    pg->nmb = (g2.cout + 31) / 32;
    pg->PR = (pg->tr - 1) * g2.stride + 3;
    // columns from gx0 = (ow0*S2 - 1) & ~3 = ow0*S2 - 4 to ow0*S2 - 1 + (tc-1)*S2 + 2
    pg->PCW = ((3 + (tc - 1) * g2.stride + 3) + 3) & ~3;
    pg->WR = g1.stride * (pg->PR - 1) + 3;
    pg->WCW = (g1.stride * pg->PCW - g1.stride + 6 + 3) & ~3;
    pg->win_elems = g1.cin * pg->WR * (pg->WCW / 4);
    pg->win_rounds = (pg->win_elems + kSPThreads - 1) / kSPThreads;
    pg->SRB = pg->src_elems = pg->src_rounds = 0;
    // floats: the window from 0, the region after it, the exchange from 0
    const size_t region = (size_t)kC1 * pg->PR * pg->PCW;
    const size_t xch = (size_t)4 * 32 * (bn + 4);
    const size_t win = (size_t)g1.cin * pg->WR * pg->WCW;
    size_t total;
    if (pre == nullptr) {
        if (pg->win_rounds > kWinRounds) return false;
        // every lane of a window round writes its 16 bytes (zeros past the window)
        total = std::max(std::max(win + region, (size_t)4 * kSPThreads * pg->win_rounds), xch);
    } else {
        // widest frame byte span of a window's columns, from its 16-byte aligned start
        int srb = 16;
        for (int tw = 0; tw < pg->tiles_w; ++tw) {
            const int gx0 = (tw * tc * g2.stride - 1) & ~3;
            const int wx0 = g1.stride * gx0 - 4;
            const int x_lo = std::max(wx0, 0), x_hi = std::min(wx0 + pg->WCW - 1, g1.w - 1);
            if (x_hi < x_lo) continue;
            const int b0 = (3 * host_axis_i0(x_lo, pre->src_w, g1.w)) & ~15;
            const int i1 = std::min(host_axis_i0(x_hi, pre->src_w, g1.w) + 1, pre->src_w - 1);
            srb = std::max(srb, ((3 * i1 + 3 + 15) & ~15) - b0);
        }
        pg->SRB = srb;
        // frame rows a tile's window interpolates between, widest over the
        // bands of tiles: from the first in-image window row's upper row to the
        // last one's lower row
        int nr = 1;
        const int tiles_h = (g2.oh + pg->tr - 1) / pg->tr;
        for (int band = 0; band < tiles_h; ++band) {
            const int wy0 = g1.stride * (band * pg->tr * g2.stride - 1) - 1;
            const int y_lo = std::max(wy0, 0), y_hi = std::min(wy0 + pg->WR - 1, g1.h - 1);
            if (y_hi < y_lo) continue;
            const int r0 = host_axis_i0(y_lo, pre->src_h, g1.h);
            const int r1 = std::min(host_axis_i0(y_hi, pre->src_h, g1.h) + 1, pre->src_h - 1);
            nr = std::max(nr, r1 - r0 + 1);
        }
        pg->src_elems = nr * (srb / 16);
        pg->src_rounds = (pg->src_elems + kSPThreads - 1) / kSPThreads;
        if (pg->src_rounds > kSrcRounds) return false;
        // the staged frame rows share the region's space (every lane of a
        // round writes its 16 bytes), then the resize's column and row tables
        // (16 bytes a column or row, filled by one thread each)
        if (pg->WCW + pg->WR > kSPThreads) return false;
        const size_t src = (size_t)4 * kSPThreads * pg->src_rounds + 4 * pg->WCW + 4 * pg->WR;  // floats
        total = std::max(win + std::max(region, src), xch);
    }
    pg->lds = total * sizeof(float);
    return pg->lds + 256 <= kMaxLdsBytes;
}

bool pair_choose(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre, PairGeom* pg)
{
    // 64-pixel tiles of 4 rows x 16 columns recompute the fewest layer-1
    // outputs per layer-2 output; then 2 x 32, 8 x 8, and 32-pixel tiles
    const char* env = getenv("CVX_STEM_PAIR_TILE");
    const int forced_nt = env ? atoi(env) / 100 : 0;
    const int forced_tc = env ? atoi(env) % 100 : 0;
    if (forced_nt > 0 && pair_geom(g1, g2, pre, forced_nt, forced_tc, pg)) return true;
    const int cand[][2] = {{2, 16}, {2, 32}, {2, 8}, {1, 16}, {1, 8}, {1, 32}};
    for (const auto& c : cand)
        if (pair_geom(g1, g2, pre, c[0], c[1], pg)) return true;
    return false;
}

bool pair_shapes(const ConvGeom& g1, const ConvGeom& g2)
{
    if (!stem_shape(g1) || g1.cout != kC1 || g1.cin > kMaxCin1 || g1.res_mode != CVX_RES_NONE) return false;
    if (g2.groups != 1 || g2.k != 3 || g2.pad != 1 || (g2.stride != 1 && g2.stride != 2)) return false;
    if (g2.cin != kC1 || g2.n != g1.n || g2.h != g1.oh || g2.w != g1.ow) return false;
    if (g2.w_layout != CVX_W_PACKED) return false;
    return (long)g2.n * g2.cout * g2.oh * g2.ow * 4 < 0x7fffffffL;
}

}  // namespace

bool stem_pair_fits(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre)
{
    if (!pair_shapes(g1, g2)) return false;
    if (pre != nullptr) {
        if (g1.cin != 3 || pre->src_h < 1 || pre->src_w < 1) return false;
        if ((3L * pre->src_w) % 16 != 0) return false;  // whole 16-byte frame rows
        if ((long)g1.n * pre->src_h * pre->src_w * 3 >= 0x7fffffffL) return false;
        if ((2L * g1.h + 1) * pre->src_h >= 0x7fffffffL || (2L * g1.w + 1) * pre->src_w >= 0x7fffffffL) return false;
    }
    PairGeom pg;
    return pair_choose(g1, g2, pre, &pg);
}

void stem_pair_describe(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre, char* buf, int len)
{
    PairGeom pg;
    if (!pair_choose(g1, g2, pre, &pg)) {
        snprintf(buf, len, "unsupported");
        return;
    }
    snprintf(buf, len, "stem_pair k3 s%d+s%d bn=%d tc=%d%s kernel=cvx::k_stem_pair<%d, %d, %d, %s>", g1.stride,
             g2.stride, 32 * pg.nt, pg.tc, pre ? " from=u8" : "", pg.nt, g1.stride, g1.cin, pre ? "true" : "false");
}

template <int NT, int S1>
static void launch_pair_u8(bool u8, int cin1, dim3 grid, size_t lds, hipStream_t s, const StemPairArgs& a)
{
    if (u8) {  // a u8 frame has three channels
        hipLaunchKernelGGL((k_stem_pair<NT, S1, 3, true>), grid, dim3(kSPThreads), lds, s, a);
        return;
    }
    switch (cin1) {
    case 1: hipLaunchKernelGGL((k_stem_pair<NT, S1, 1, false>), grid, dim3(kSPThreads), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_stem_pair<NT, S1, 2, false>), grid, dim3(kSPThreads), lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_stem_pair<NT, S1, 3, false>), grid, dim3(kSPThreads), lds, s, a); break;
    default: hipLaunchKernelGGL((k_stem_pair<NT, S1, 4, false>), grid, dim3(kSPThreads), lds, s, a); break;
    }
}

hipError_t launch_stem_pair(const ConvGeom& g1, const float* x, const StemPrologue* pre, const float* w1,
                            const float* scale1, const float* bias1, const ConvGeom& g2, const float* wp,
                            const float* scale2, const float* bias2, const float* res, float* y, hipStream_t s)
{
    PairGeom pg;
    if (!pair_choose(g1, g2, pre, &pg)) return hipErrorInvalidValue;
    if (pre == nullptr && (reinterpret_cast<uintptr_t>(x) & 15u) != 0) return hipErrorInvalidValue;
    if (pre != nullptr && ((reinterpret_cast<uintptr_t>(pre->src) & 15u) != 0 || pre->row_bytes % 16 != 0))
        return hipErrorInvalidValue;
    StemPairArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.w1 = w1;
    a.scale1 = scale1;
    a.bias1 = bias1;
    a.wp = wp;
    a.scale2 = scale2;
    a.bias2 = bias2;
    a.res = res;
    a.y = y;
    a.n = g1.n;
    a.cin1 = g1.cin;
    a.H1 = g1.h;
    a.W1 = g1.w;
    a.S1 = g1.stride;
    a.H2 = g1.oh;
    a.W2 = g1.ow;
    a.S2 = g2.stride;
    a.OH = g2.oh;
    a.OW = g2.ow;
    a.cout = g2.cout;
    a.act1 = g1.act;
    a.act2 = g2.act;
    a.res_mode = g2.res_mode;
    a.tc = pg.tc;
    a.tr = pg.tr;
    a.tiles_w = pg.tiles_w;
    a.tiles_per_img = pg.tiles_per_img;
    a.nmb = pg.nmb;
    fastdiv_params(pg.tc, &a.m_tc, &a.l_tc);
    fastdiv_params(pg.tiles_w, &a.m_tw, &a.l_tw);
    fastdiv_params(pg.tiles_per_img, &a.m_tpi, &a.l_tpi);
    fastdiv_params(g1.n * pg.tiles_per_img, &a.m_nb, &a.l_nb);
    a.PR = pg.PR;
    a.PCW = pg.PCW;
    fastdiv_params(pg.PCW, &a.m_pcw, &a.l_pcw);
    a.WR = pg.WR;
    a.WCW = pg.WCW;
    a.win_elems = pg.win_elems;
    a.win_rounds = pg.win_rounds;
    fastdiv_params(pg.WCW / 4, &a.m_we, &a.l_we);
    fastdiv_params(pg.WR * pg.WCW / 4, &a.m_wc, &a.l_wc);
    fastdiv_params(pg.WCW, &a.m_wcw, &a.l_wcw);
    a.x_bytes = (unsigned)((long)g1.n * g1.cin * g1.h * g1.w * 4);
    a.wp_bytes = (unsigned)(packed_copy_floats(g2) * 4);
    if (pre != nullptr) {
        a.src = pre->src;
        a.src_h = pre->src_h;
        a.src_w = pre->src_w;
        a.row_bytes = (unsigned)pre->row_bytes;
        a.img_bytes = (unsigned)((long)pre->src_h * pre->row_bytes);
        fastdiv_params(2 * g1.h, &a.m_dh, &a.l_dh);
        fastdiv_params(2 * g1.w, &a.m_dw, &a.l_dw);
        a.inv_dh = (float)(1.0 / (2.0 * g1.h));
        a.inv_dw = (float)(1.0 / (2.0 * g1.w));
        for (int c = 0; c < 3; ++c) {
            a.na[c] = (float)(1.0 / (255.0 * (double)pre->stdv[c]));
            a.nb[c] = (float)(-(double)pre->mean[c] / (double)pre->stdv[c]);
        }
        a.SRB = pg.SRB;
        a.src_elems = pg.src_elems;
        a.src_rounds = pg.src_rounds;
        fastdiv_params(pg.SRB / 16, &a.m_srb, &a.l_srb);
    }
    const bool quads = pg.tc % 4 == 0 && g2.ow % 4 == 0;
    const bool al_y = (reinterpret_cast<uintptr_t>(y) & 15u) == 0;
    const bool al_r = res == nullptr || (reinterpret_cast<uintptr_t>(res) & 15u) == 0;
    a.vout = quads && al_y && al_r ? 1 : 0;
    dim3 grid((unsigned)((long)g1.n * pg.tiles_per_img * pg.nmb));
    const bool u8 = pre != nullptr;
    if (pg.nt == 2) {
        if (g1.stride == 2)
            launch_pair_u8<2, 2>(u8, g1.cin, grid, pg.lds, s, a);
        else
            launch_pair_u8<2, 1>(u8, g1.cin, grid, pg.lds, s, a);
    } else {
        if (g1.stride == 2)
            launch_pair_u8<1, 2>(u8, g1.cin, grid, pg.lds, s, a);
        else
            launch_pair_u8<1, 1>(u8, g1.cin, grid, pg.lds, s, a);
    }
    return hipGetLastError();
}

}  // namespace cvx
