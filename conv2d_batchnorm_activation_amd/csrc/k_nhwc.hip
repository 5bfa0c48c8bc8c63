// k_nhwc.hip -- dense 1x1 / 3x3 convolution + folded BatchNorm + activation
// (+ residual) on channels-last tensors, stored as fp32, fp16 or bf16,
// accumulated in fp32.
//
// The pages name two next steps for the convolutions: moving the activations
// to NHWC with the weights reordered to match ("YOLO26N Inference
// Optimisation", "NHWC migration -- detailed scope": "What NHWC is and why it
// matters", "What must change in the kernels", "Weight layout"), and fp16
// arithmetic ("Как я свертки ускорял", "Идеи и следующие шаги", item 1).
// Channels-last is what makes the half-precision matrix instruction cheap to
// feed: v_mfma_f32_32x32x16_f16 takes eight consecutive input channels of one
// pixel per lane, which in NHWC are one 16-byte run.
//
// Implicit GEMM with the weights as the A operand (M = output channels) and
// the staged input as the B operand (N = output pixels), so a lane's
// accumulators hold 16 output channels of one pixel -- four runs of four
// consecutive channels, which NHWC stores contiguously.
//   * fp32: v_mfma_f32_32x32x2_f32, K = 2 channels per instruction (lane l:
//     channel 2p + l/32 of pair p);
//   * fp16 / bf16: v_mfma_f32_32x32x16_f16 / _bf16, K = 16 channels (lane
//     l: channels 8*(l/32) .. +7); the two 16-bit types share the layout,
//     the staging and the tiles, and differ in the instruction and in the
//     conversions (both round to nearest even).
// A workgroup (four waves) computes WM x 32 output pixels (a block of TR rows
// x TC columns) x WN x 32 output channels; wave (wm, wn) one 32 x 32 block.
// Each stage stages KC input channels of the tile's input window in LDS as
// [row][col][piece], a piece being 16 bytes of consecutive channels of one
// pixel (with a fifth, unused piece per pixel so that the 32 pixels a wave
// reads fall in different banks), all four waves loading with 16-byte
// LDS-direct loads; positions outside the image or past c_in read as zero.
// Two stage buffers, one barrier per stage: stage s+1 loads while s computes.
// Weights go global -> registers, a stage ahead, in the operand's lane order
// (cvx_nhwc_pack_weights).  The epilogue (folded BN, residual, activation)
// runs on the fp32 sums and stores 16 or 8 bytes per run of four channels.
#include <stdio.h>

#include <algorithm>
#include <type_traits>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

namespace {

typedef _Float16 half_t;
typedef half_t h8 __attribute__((ext_vector_type(8)));
typedef half_t h4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16_t;
typedef bf16_t b8 __attribute__((ext_vector_type(8)));
typedef bf16_t b4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPPX = 4;        // 16-byte pieces of channels per pixel per stage
constexpr int kPPXP = 5;       // the same with the unused fifth piece (LDS pitch)
constexpr int kMaxRounds = 8;  // 256-piece LDS-direct rounds per stage, at most

}  // namespace

struct NhwcArgs {
    const void* x;
    const void* wp;
    const float* scale;
    const float* bias;
    const void* res;
    void* y;
    int n, cin, H, W, cout, stride, pad, OH, OW;
    int TR, TC;                  // output tile: TR rows x TC columns (TR*TC = 32*WM)
    int tiles_w, tiles_per_img;  // tiles along OW, per image
    int ngroups;                 // output-channel groups of 32*WN
    int nstages;                 // stages of KC input channels
    int PR, PC;                  // staged rows and columns of the input window
    int pieces, rounds;          // staged 16-byte pieces per stage, 256-piece rounds
    unsigned m_pp, l_pp;         // divide by kPPXP
    unsigned m_pc, l_pc;         // divide by PC
    unsigned m_tc, l_tc;         // divide by TC
    unsigned m_tw, l_tw;         // divide by tiles_w
    unsigned m_tpi, l_tpi;       // divide by tiles_per_img
    unsigned x_bytes, y_bytes, w_bytes;
    int act, res_mode;
};

namespace {

__device__ __forceinline__ int pdiv(int n, unsigned m, unsigned l)
{
    unsigned hi = __umulhi((unsigned)n, m);
    return (int)((hi + (unsigned)n) >> l);
}

__device__ __forceinline__ void lds16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}

// Packed weight floats (or 16-bit values) per (32-channel block, stage): KK taps x
// KC input channels x 32 output channels, in the A operand's lane order.
template <typename T, int K>
constexpr int wstage_elems()
{
    return K * K * 32 * (sizeof(T) == 2 ? 32 : 16);
}

template <typename T, int K, int WM, int WN>
__global__ void __launch_bounds__(256) k_conv_nhwc(NhwcArgs a)
{
    constexpr bool F16 = sizeof(T) == 2;       // a 16-bit type: fp16 or bf16
    constexpr bool BF = std::is_same<T, bf16_t>::value;
    typedef typename std::conditional<BF, b8, h8>::type V8;
    typedef typename std::conditional<BF, b4, h4>::type V4;
    constexpr int KC = F16 ? 32 : 16;          // input channels per stage
    constexpr int PER = 16 / (int)sizeof(T);   // channels per 16-byte piece
    constexpr int KK = K * K;
    constexpr int WSE = wstage_elems<T, K>();  // weight elements per (block, stage)

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    warm_kernargs<sizeof(NhwcArgs)>();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // workgroup -> (image, pixel tile, channel group), channel groups fastest
    int g = blockIdx.x;
    const int t2 = g / a.ngroups;
    const int grp = g - t2 * a.ngroups;
    const int b = pdiv(t2, a.m_tpi, a.l_tpi);
    const int tile = t2 - b * a.tiles_per_img;
    const int band = pdiv(tile, a.m_tw, a.l_tw);
    const int oh0 = band * a.TR, ow0 = (tile - band * a.tiles_w) * a.TC;
    const int co = grp * 32 * WN + wn * 32;  // this wave's first output channel
    const int iy0 = oh0 * a.stride - a.pad, ix0 = ow0 * a.stride - a.pad;
    const int BUFB = a.rounds * 4096;        // bytes per stage buffer

    // Staged pieces e = tid + 256*i: (pixel of the window, piece of the pixel)
    // -> byte offset in x without the stage's channel term, or kOOB.
    unsigned goff[kMaxRounds];
    int gch[kMaxRounds];
#pragma unroll
    for (int i = 0; i < kMaxRounds; ++i) {
        goff[i] = kOOB;
        gch[i] = 1 << 30;
        const int e = tid + 256 * i;
        if (i < a.rounds && e < a.pieces) {
            const int px = pdiv(e, a.m_pp, a.l_pp);
            const int q = e - px * kPPXP;
            const int r = pdiv(px, a.m_pc, a.l_pc);
            const int c = px - r * a.PC;
            const int iy = iy0 + r, ix = ix0 + c;
            if (q < kPPX && (unsigned)iy < (unsigned)a.H && (unsigned)ix < (unsigned)a.W) {
                goff[i] = (unsigned)((((long)b * a.H + iy) * a.W + ix) * a.cin + q * PER) * (unsigned)sizeof(T);
                gch[i] = q * PER;
            }
        }
    }
    const rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    auto stage_in = [&](int st, int buf) {
        const int c0 = st * KC;
#pragma unroll
        for (int i = 0; i < kMaxRounds; ++i) {
            if (i >= a.rounds) break;
            const unsigned off = c0 + gch[i] < a.cin ? goff[i] + (unsigned)(c0 * (int)sizeof(T)) : kOOB;
            auto* d = (__attribute__((address_space(3))) void*)(lds + buf * BUFB + 4096 * i + 1024 * wave);
            lds16(rx, d, off);
        }
    };

    // This lane's pixel (B operand column n = lane % 32) in the tile, and its
    // LDS byte offset in a stage buffer for tap (0, 0).
    const int p = 32 * wm + l32;
    const int pr = pdiv(p, a.m_tc, a.l_tc);
    const int pc = p - pr * a.TC;
    const int boff = ((pr * a.stride) * a.PC + pc * a.stride) * (kPPXP * 16);

    // Weights: A operand rows m = lane % 32 (output channel co + m).
    const rsrc_t rw = make_rsrc(a.wp, a.w_bytes);
    const int blk = co / 32;
    typedef typename std::conditional<F16, V8, float>::type AV;
    constexpr int NA = F16 ? KK * 2 : KK * 8;  // A values per lane per stage
    AV w0[NA], w1[NA];
    auto load_w = [&](int st, AV (&wv)[NA]) {
        const bool live = st < a.nstages && co < a.cout;
        const unsigned base = (unsigned)(((long)blk * a.nstages + st) * WSE) * (unsigned)sizeof(T);
#pragma unroll
        for (int j = 0; j < NA; ++j) {
            if constexpr (F16) {
                const unsigned off = live ? base + (unsigned)((j * 64 + lane) * 16) : kOOB;
                wv[j] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0));
            } else if (j % 4 == 0) {
                // a tap's eight pair values are consecutive per lane: two 16-byte loads
                const int tap = j / 8, q = (j / 4) & 1;
                const unsigned off = live ? base + (unsigned)(((tap * 64 + lane) * 8 + 4 * q) * 4) : kOOB;
                const f32x4 v4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[j + e] = v4[e];
            }
        }
    };

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    auto compute = [&](int buf, const AV (&wv)[NA]) {
        const unsigned char* sb = lds + buf * BUFB + boff;
#pragma unroll
        for (int tap = 0; tap < KK; ++tap) {
            const int toff = ((tap / K) * a.PC + (tap % K)) * (kPPXP * 16);
            if constexpr (F16) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {  // two 16-channel halves of the stage
                    const V8 bv = *reinterpret_cast<const V8*>(sb + toff + 32 * h + 16 * hi);
                    if constexpr (BF)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[tap * 2 + h], bv, acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[tap * 2 + h], bv, acc, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {  // eight channel pairs
                    const float bv = *reinterpret_cast<const float*>(sb + toff + 4 * (2 * pp + hi));
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wv[tap * 8 + pp], bv, acc, 0, 0, 0);
                }
            }
        }
    };

    stage_in(0, 0);
    load_w(0, w0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int st = 0; st < a.nstages; st += 2) {
        if (st + 1 < a.nstages) stage_in(st + 1, 1);
        load_w(st + 1, w1);
        compute(0, w0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (st + 1 >= a.nstages) break;
        if (st + 2 < a.nstages) stage_in(st + 2, 0);
        load_w(st + 2, w0);
        compute(1, w1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Epilogue: lane (hi, l32) holds pixel p's channels co + 8j + 4hi + 0..3.
    const int oh = oh0 + pr, ow = ow0 + pc;
    const bool px_ok = pr < a.TR && oh < a.OH && ow < a.OW;
    const long pix = ((long)b * a.OH + oh) * a.OW + ow;
    const rsrc_t ry = make_rsrc(a.y, a.y_bytes);
    const rsrc_t rr = make_rsrc(a.res, a.res_mode != CVX_RES_NONE ? a.y_bytes : 0u);
    const rsrc_t rs = make_rsrc(a.scale, 4u * (unsigned)a.cout);
    const rsrc_t rbias = make_rsrc(a.bias, 4u * (unsigned)a.cout);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = co + 8 * j + 4 * hi;
        const bool ok = px_ok && c < a.cout;
        const unsigned eoff = ok ? (unsigned)((pix * a.cout + c) * (long)sizeof(T)) : kOOB;
        const unsigned coff = c < a.cout ? 4u * (unsigned)c : kOOB;
        const f32x4 sc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)coff, 0, 0));
        const f32x4 bi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rbias, (int)coff, 0, 0));
        f32x4 rv;
        if constexpr (F16) {
            const V4 r4 = __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(rr, (int)eoff, 0, 0));
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[i] = (float)r4[i];
        } else {
            rv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)eoff, 0, 0));
        }
        f32x4 z;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = fmaf(sc[i], acc[4 * j + i], bi[i]);
            if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[i];
            t = apply_act_fast(t, a.act);
            if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[i];
            z[i] = t;
        }
        if constexpr (F16) {
            V4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (T)z[i];
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), ry, (int)eoff, 0, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z), ry, (int)eoff, 0, 0);
        }
    }
}

// OIHW fp32 -> the A operand's lane order per (32-channel block, stage):
// fp16 / bf16: [tap][half h][lane][8] holds output channel 32*blk + lane%32, input
// channels KC*st + 16h + 8*(lane/32) + 0..7; fp32: [tap][lane][pair p] holds
// input channel KC*st + 2p + lane/32.  Zero where the channel does not exist.
template <typename T, int K>
__global__ void __launch_bounds__(256) k_pack_nhwc(const float* __restrict__ w, int cout, int cin, int nstages,
                                                   long total, T* __restrict__ wp)
{
    constexpr bool F16 = sizeof(T) == 2;
    constexpr int KC = F16 ? 32 : 16;
    constexpr int KK = K * K;
    constexpr int WSE = wstage_elems<T, K>();
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const long bs = idx / WSE;
    const int r = (int)(idx - bs * WSE);
    const int st = (int)(bs % nstages);
    const int blk = (int)(bs / nstages);
    int tap, lane, ci;
    if constexpr (F16) {
        const int e = r & 7;
        lane = (r >> 3) & 63;
        const int h = (r >> 9) & 1;
        tap = r >> 10;
        ci = KC * st + 16 * h + 8 * (lane >> 5) + e;
    } else {
        const int pp = r & 7;
        lane = (r >> 3) & 63;
        tap = r >> 9;
        ci = KC * st + 2 * pp + (lane >> 5);
    }
    const int o = blk * 32 + (lane & 31);
    float v = 0.0f;
    if (o < cout && ci < cin && tap < KK) v = w[((long)o * cin + ci) * KK + tap];
    wp[idx] = (T)v;
}

struct NhwcTile {
    int wm, wn, tr, tc;
};

}  // namespace

// ------------------------------------------------------------------ host side
static bool nhwc_dtype_ok(int dt) { return dt == CVX_DT_F32 || dt == CVX_DT_F16 || dt == CVX_DT_BF16; }
static int dt_size(int dt) { return dt == CVX_DT_F32 ? 4 : 2; }
static int dt_kc(int dt) { return dt == CVX_DT_F32 ? 16 : 32; }

long nhwc_packed_weight_elems(const ConvGeom& g, int dt)
{
    const int KC = dt_kc(dt);
    const long blocks = (g.cout + 31) / 32, stages = (g.cin + KC - 1) / KC;
    const long per = (long)g.k * g.k * 32 * KC;
    return blocks * stages * per;
}

bool nhwc_supported(const ConvGeom& g, int dt)
{
    if (!nhwc_dtype_ok(dt)) return false;
    if (g.groups != 1 || (g.k != 1 && g.k != 3) || g.stride > 2) return false;
    if (g.cin % (16 / dt_size(dt)) != 0 || g.cout % 4 != 0) return false;  // whole 16-byte pieces, runs of 4
    const long xb = (long)g.n * g.h * g.w * g.cin * dt_size(dt);
    const long yb = (long)g.n * g.oh * g.ow * g.cout * dt_size(dt);
    return xb < 0x7fffffffL && yb < 0x7fffffffL && nhwc_packed_weight_elems(g, dt) * dt_size(dt) < 0x7fffffffL;
}

// Tile of a layer: the pixel block (TR x TC, TR*TC = 32*WM) and the split of
// the four waves between pixels (WM) and output channels (WN): channels first
// while there are enough output channels, then the widest block whose staged
// window fits kMaxRounds rounds.
static bool nhwc_tile(const ConvGeom& g, NhwcTile* t, int* rounds, int* pieces, int* PR, int* PC)
{
    const int groups32 = (g.cout + 31) / 32;
    for (int wn : {4, 2, 1}) {
        if (wn > 1 && groups32 < wn) continue;
        const int wm = 4 / wn;
        const int px = 32 * wm;
        for (int tc : {32, 16, 64, 8, 128, 4}) {
            if (tc > px || px % tc != 0) continue;
            const int tr = px / tc;
            const int pr = (tr - 1) * g.stride + g.k, pc = (tc - 1) * g.stride + g.k;
            const int pcs = pr * pc * kPPXP;
            const int rd = (pcs + 255) / 256;
            if (rd > kMaxRounds) continue;
            if (tc > 2 * g.ow && tc > 4) continue;  // mostly outside the image
            *t = NhwcTile{wm, wn, tr, tc};
            *rounds = rd;
            *pieces = pcs;
            *PR = pr;
            *PC = pc;
            return true;
        }
    }
    return false;
}

hipError_t launch_pack_nhwc(const ConvGeom& g, int dt, const float* w, void* wp, hipStream_t s)
{
    const long total = nhwc_packed_weight_elems(g, dt);
    const int KC = dt_kc(dt);
    const int nst = (g.cin + KC - 1) / KC;
    dim3 grid((unsigned)((total + 255) / 256));
    if (dt == CVX_DT_F16) {
        if (g.k == 3)
            hipLaunchKernelGGL((k_pack_nhwc<half_t, 3>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<half_t*>(wp));
        else
            hipLaunchKernelGGL((k_pack_nhwc<half_t, 1>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<half_t*>(wp));
    } else if (dt == CVX_DT_BF16) {
        if (g.k == 3)
            hipLaunchKernelGGL((k_pack_nhwc<bf16_t, 3>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<bf16_t*>(wp));
        else
            hipLaunchKernelGGL((k_pack_nhwc<bf16_t, 1>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<bf16_t*>(wp));
    } else {
        if (g.k == 3)
            hipLaunchKernelGGL((k_pack_nhwc<float, 3>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<float*>(wp));
        else
            hipLaunchKernelGGL((k_pack_nhwc<float, 1>), grid, dim3(256), 0, s, w, g.cout, g.cin, nst, total,
                               static_cast<float*>(wp));
    }
    return hipGetLastError();
}

void nhwc_describe(const ConvGeom& g, int dt, char* buf, int len)
{
    NhwcTile t;
    int rd, pcs, pr, pc;
    if (!nhwc_tile(g, &t, &rd, &pcs, &pr, &pc)) {
        snprintf(buf, len, "unsupported");
        return;
    }
    snprintf(buf, len, "nhwc k%d s%d %s wm=%d wn=%d tr=%d tc=%d kernel=cvx::k_conv_nhwc<%s, %d, %d, %d>", g.k,
             g.stride, dt == CVX_DT_F16 ? "f16" : dt == CVX_DT_BF16 ? "bf16" : "f32", t.wm, t.wn, t.tr, t.tc,
             dt == CVX_DT_F16 ? "_Float16" : dt == CVX_DT_BF16 ? "__bf16" : "float", g.k, t.wm, t.wn);
}

template <typename T, int K>
static void launch_nhwc_k(const NhwcTile& t, dim3 grid, size_t lds, hipStream_t s, const NhwcArgs& a)
{
    if (t.wm == 4)
        hipLaunchKernelGGL((k_conv_nhwc<T, K, 4, 1>), grid, dim3(256), lds, s, a);
    else if (t.wm == 2)
        hipLaunchKernelGGL((k_conv_nhwc<T, K, 2, 2>), grid, dim3(256), lds, s, a);
    else
        hipLaunchKernelGGL((k_conv_nhwc<T, K, 1, 4>), grid, dim3(256), lds, s, a);
}

hipError_t launch_conv_nhwc(const ConvGeom& g, int dt, const void* x, const void* wp, const float* scale,
                            const float* bias, const void* res, void* y, hipStream_t s)
{
    NhwcTile t;
    int rounds, pieces, PR, PC;
    if (!nhwc_supported(g, dt) || !nhwc_tile(g, &t, &rounds, &pieces, &PR, &PC)) return hipErrorInvalidValue;
    const int sz = dt_size(dt), KC = dt_kc(dt);
    NhwcArgs a;
    a.x = x;
    a.wp = wp;
    a.scale = scale;
    a.bias = bias;
    a.res = res;
    a.y = y;
    a.n = g.n;
    a.cin = g.cin;
    a.H = g.h;
    a.W = g.w;
    a.cout = g.cout;
    a.stride = g.stride;
    a.pad = g.pad;
    a.OH = g.oh;
    a.OW = g.ow;
    a.TR = t.tr;
    a.TC = t.tc;
    a.tiles_w = (g.ow + t.tc - 1) / t.tc;
    a.tiles_per_img = ((g.oh + t.tr - 1) / t.tr) * a.tiles_w;
    a.ngroups = (g.cout + 32 * t.wn - 1) / (32 * t.wn);
    a.nstages = (g.cin + KC - 1) / KC;
    a.PR = PR;
    a.PC = PC;
    a.pieces = pieces;
    a.rounds = rounds;
    fastdiv_params(kPPXP, &a.m_pp, &a.l_pp);
    fastdiv_params(PC, &a.m_pc, &a.l_pc);
    fastdiv_params(t.tc, &a.m_tc, &a.l_tc);
    fastdiv_params(a.tiles_w, &a.m_tw, &a.l_tw);
    fastdiv_params(a.tiles_per_img, &a.m_tpi, &a.l_tpi);
    a.x_bytes = (unsigned)((long)g.n * g.h * g.w * g.cin * sz);
    a.y_bytes = (unsigned)((long)g.n * g.oh * g.ow * g.cout * sz);
    a.w_bytes = (unsigned)(nhwc_packed_weight_elems(g, dt) * sz);
    a.act = g.act;
    a.res_mode = g.res_mode;
    const long wgs = (long)g.n * a.tiles_per_img * a.ngroups;
    if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs);
    const size_t lds = (size_t)2 * rounds * 4096;
    if (dt == CVX_DT_F16) {
        if (g.k == 3)
            launch_nhwc_k<half_t, 3>(t, grid, lds, s, a);
        else
            launch_nhwc_k<half_t, 1>(t, grid, lds, s, a);
    } else if (dt == CVX_DT_BF16) {
        if (g.k == 3)
            launch_nhwc_k<bf16_t, 3>(t, grid, lds, s, a);
        else
            launch_nhwc_k<bf16_t, 1>(t, grid, lds, s, a);
    } else {
        if (g.k == 3)
            launch_nhwc_k<float, 3>(t, grid, lds, s, a);
        else
            launch_nhwc_k<float, 1>(t, grid, lds, s, a);
    }
    return hipGetLastError();
}

}  // namespace cvx
