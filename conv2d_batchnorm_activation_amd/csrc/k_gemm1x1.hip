// k_gemm1x1.hip -- dense 1x1 convolution (stride 1, no padding) + folded
// BatchNorm + activation (+ residual) on NCHW fp32, as one GEMM per image,
// Y[c_out, pixels] = W[c_out, c_in] . X[c_in, pixels], on fp32 matrix cores.
//
// The pages' detector runs its 1x1 layers as the same fused conv+BN+SiLU as
// its 3x3 ones ("YOLO26N Inference Optimisation", "Baseline benchmark"; the
// per-shape choice of kernel and tile, "Improvements" #1), and the MNIST
// page's pointwise layers are a plain matrix product per image ("Как я
// свертки ускорял", the depthwise-separable block).  In NCHW a 1x1 layer's
// input rows are runs of consecutive pixels, so the input operand of
// v_mfma_f32_32x32x2_f32 (lane l: pixel l%32, channel l/32 of a pair) is two
// 128-byte runs of one channel pair: each wave loads it straight from global
// memory, without staging in LDS.
//
// A wave computes 32 output channels x 32 pixels over the whole reduction, so
// no partial sums cross waves; a workgroup is four waves, four consecutive
// 32-pixel blocks of one 32-channel row block, whose weights (c_in up to 256)
// go to LDS once, with 16-byte LDS-direct loads of the contiguous packed block
// (the 1x1 layout of cvx_pack_weights, where lane l's values for output
// channel l%32 and a chunk's eight channel pairs are four 8-byte pieces).  Per
// 16-channel chunk a wave issues eight input loads, two chunks ahead of the
// matrix instructions, and reads the chunk's weights from LDS; past the last
// chunk the loads read zeros (out-of-range offsets), which keeps every wait
// count exact.  Lane l ends with pixel l%32 of output channels
// 8g + 4*(l/32) + 0..3 (g = 0..3): the epilogue stores 128-byte runs.
#include <stdio.h>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kG1Threads = 256;  // four waves
constexpr int kG1Ch = 16;        // input channels per chunk
constexpr int kG1WF = 512;       // packed weight floats per (32-row block, chunk)
constexpr int kG1MaxChunks = 16;  // c_in <= 256: a row block's weights, 32 KB, in LDS
constexpr int kG1MaxWRounds = kG1MaxChunks / 2;  // 256-lane rounds of 16-byte pieces

__device__ __forceinline__ int g1div(int n, unsigned m, unsigned l)
{
    return (int)((__umulhi((unsigned)n, m) + (unsigned)n) >> l);
}

}  // namespace

struct Gemm1x1Args {
    const float* x;
    const float* wp;
    const float* scale;
    const float* bias;
    const float* res;
    float* y;
    int n, cin, hw, cout;
    int nchunks;          // ceil(c_in / 16)
    int mblocks;          // ceil(c_out / 32)
    int pblocks;          // 32-pixel blocks per image: ceil(hw / 32)
    int total_pblocks;    // n * pblocks
    unsigned m_pb, l_pb;  // divide by pblocks
    unsigned m_mb, l_mb;  // divide by mblocks
    unsigned x_bytes, y_bytes;
    int wrounds;          // rounds of the weights' LDS-direct copy: ceil(nchunks / 2)
    int vsb;              // scale and bias 16-byte aligned (four channels a load)
    int act, res_mode;
};

__global__ void __launch_bounds__(kG1Threads) k_gemm1x1(Gemm1x1Args a)
{
    warm_kernargs<sizeof(Gemm1x1Args)>();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // Workgroup -> (pixel group, row block), row blocks fastest; consecutive
    // workgroups go to the eight XCDs in turn and are numbered XCD by XCD, so
    // each XCD takes one band of pixels (and every row block of it), the band
    // it wrote in a layer before this one.
    int mb, pg;
    {
        const unsigned h = blockIdx.x, G8 = gridDim.x;
        const unsigned xcd = h & 7u, i8 = h >> 3, base = G8 >> 3, rem = G8 & 7u;
        const int L = (int)(xcd * base + min(xcd, rem) + i8);
        pg = g1div(L, a.m_mb, a.l_mb);
        mb = L - pg * a.mblocks;
    }
    const int pbk = 4 * pg + wave;                // this wave's 32-pixel block
    const bool live = pbk < a.total_pblocks;      // past the end: loads read nothing, and the
                                                  // wave leaves after the barrier
    const int img = live ? g1div(pbk, a.m_pb, a.l_pb) : 0;
    const int p = 32 * (pbk - img * a.pblocks) + l32;
    const bool p_ok = live && p < a.hw;

    // The row block's weights, every chunk, go to LDS once for the four waves
    // (16-byte LDS-direct loads of the contiguous packed block: chunk c at
    // float 512 c, lane l's pairs (2h, 2h+1) at + 128 h + 2 l).
    extern __shared__ __attribute__((aligned(16))) float wl[];
    {
        const rsrc_t rw = make_rsrc(a.wp + (long)mb * a.nchunks * kG1WF, 4u * (unsigned)(a.nchunks * kG1WF));
        const int pieces = a.nchunks * (kG1WF / 4);
#pragma unroll
        for (int i = 0; i < kG1MaxWRounds; ++i) {
            if (i >= a.wrounds) break;
            const int e = threadIdx.x + kG1Threads * i;
            const unsigned off = e < pieces ? 16u * (unsigned)e : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(wl + 4 * (kG1Threads * i + 64 * wave)), 16, off, 0,
                0, 0);
        }
    }

    // input: channel ci of this lane's pixel at ((img * cin + ci) * hw + p) * 4
    const rsrc_t rx = make_rsrc(a.x, a.x_bytes);
    const unsigned xrow = 4u * (unsigned)a.hw;
    const unsigned xbase = p_ok ? 4u * (unsigned)(img * a.cin * a.hw + p) + (unsigned)hi * xrow : kOOB;
    // Out-of-range offsets are formed by setting bit 31 (every offset in range
    // is below 2^31), not by selects: the compiler turns a select on the
    // uniform chunk test into branches that wait for all loads in flight.
    typedef float Ops[8];  // inputs of the chunk's pairs 0..7
    auto load = [&](int c, Ops& o) {
        const unsigned dead = (unsigned)(c >= a.nchunks) << 31;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int ci = kG1Ch * c + 2 * q + hi;
            const unsigned xo = (xbase + (unsigned)(kG1Ch * c + 2 * q) * xrow) | dead |
                                ((unsigned)(ci >= a.cin) << 31);
            o[q] = bload(rx, xo);
        }
    };
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    // chunk c's weights from LDS (a chunk past the end reads the last chunk's,
    // against zero inputs)
    auto compute = [&](int c, const Ops& o) {
        const float* wc = wl + kG1WF * min(c, a.nchunks - 1) + 2 * lane;
        float wv[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(wc + 128 * h);
            wv[2 * h] = v[0];
            wv[2 * h + 1] = v[1];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wv[q], o[q], acc, 0, 0, 0);
    };

    // the first two chunks' inputs go out behind the weights; the weights are
    // waited for (the inputs stay in flight), then the epilogue operands
    Ops o0, o1;
    load(0, o0);
    load(1, o1);
    wait_vm_at_most(16);
    lds_barrier();
    if (!live) return;
    const int co0 = 32 * mb + 4 * hi;  // this lane's channels: co0 + 8 g + 0..3
    f32x4 sc[4], bi[4];
    {
        const rsrc_t rs = make_rsrc(a.scale, 4u * (unsigned)a.cout);
        const rsrc_t rb = make_rsrc(a.bias, 4u * (unsigned)a.cout);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = co0 + 8 * g;
            if (a.vsb) {
                const unsigned off = c < a.cout ? 4u * (unsigned)c : kOOB;  // c_out % 4 == 0 here
                sc[g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
                bi[g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, 0));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned off = c + i < a.cout ? 4u * (unsigned)(c + i) : kOOB;
                    sc[g][i] = bload(rs, off);
                    bi[g][i] = bload(rb, off);
                }
            }
        }
    }
    // this lane's output element j: channel co0 + 8 (j / 4) + j % 4, pixel p
    const unsigned ybase = p_ok ? 4u * (unsigned)(img * a.cout * a.hw + p) : kOOB;
    auto yoff = [&](int j) {
        const int c = co0 + 8 * (j >> 2) + (j & 3);
        return c < a.cout && p_ok ? ybase + (unsigned)c * xrow : kOOB;
    };
    float rv[16];
    {
        const rsrc_t rr = make_rsrc(a.res, a.res_mode != CVX_RES_NONE ? a.y_bytes : 0u);
#pragma unroll
        for (int j = 0; j < 16; ++j) rv[j] = bload(rr, yoff(j));
    }

    // two chunks in flight (four measured no faster: the loads are not what
    // the loop waits on)
    for (int c = 0; c < a.nchunks; c += 2) {
        compute(c, o0);
        load(c + 2, o0);
        compute(c + 1, o1);
        load(c + 3, o1);
    }

    const rsrc_t ry = make_rsrc(a.y, a.y_bytes);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float t = fmaf(sc[j >> 2][j & 3], acc[j], bi[j >> 2][j & 3]);
        if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[j];
        t = apply_act_fast(t, a.act);
        if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[j];
        bstore(ry, yoff(j), t);
    }
}

// ------------------------------------------------------------------ host side
void fastdiv_params(int d, unsigned* m, unsigned* l);

bool gemm1x1_fits(const ConvGeom& g)
{
    if (g.groups != 1 || g.k != 1 || g.stride != 1 || g.pad != 0 || g.w_layout != CVX_W_PACKED) return false;
    if (g.cin < 16 || (g.cin + kG1Ch - 1) / kG1Ch > kG1MaxChunks) return false;
    const long hw = (long)g.h * g.w;
    const long xb = (long)g.n * g.cin * hw * 4, yb = (long)g.n * g.cout * hw * 4;
    return xb < 0x7fffffffL && yb < 0x7fffffffL && packed_weight_floats(g) * 4 < 0x7fffffffL &&
           (long)g.n * ((hw + 31) / 32) < (1L << 28);
}

long gemm1x1_waves(const ConvGeom& g)
{
    const long hw = (long)g.h * g.w;
    return (long)((g.cout + 31) / 32) * g.n * ((hw + 31) / 32);
}

void gemm1x1_describe(const ConvGeom& g, char* buf, int len)
{
    snprintf(buf, len, "gemm1x1 k1 s1 waves=%ld splitk=1 kernel=cvx::k_gemm1x1", gemm1x1_waves(g));
}

hipError_t launch_gemm1x1(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                          const float* bias, const float* res, float* y, hipStream_t s)
{
    if (!gemm1x1_fits(g)) return hipErrorInvalidValue;
    Gemm1x1Args a;
    a.x = x;
    a.wp = wp;
    a.scale = scale;
    a.bias = bias;
    a.res = res;
    a.y = y;
    a.n = g.n;
    a.cin = g.cin;
    a.hw = g.h * g.w;
    a.cout = g.cout;
    a.nchunks = (g.cin + kG1Ch - 1) / kG1Ch;
    a.mblocks = (g.cout + 31) / 32;
    a.pblocks = (a.hw + 31) / 32;
    a.total_pblocks = g.n * a.pblocks;
    fastdiv_params(a.pblocks, &a.m_pb, &a.l_pb);
    fastdiv_params(a.mblocks, &a.m_mb, &a.l_mb);
    a.x_bytes = (unsigned)((long)g.n * g.cin * a.hw * 4);
    a.y_bytes = (unsigned)((long)g.n * g.cout * a.hw * 4);
    a.wrounds = (a.nchunks + 1) / 2;
    a.vsb = (reinterpret_cast<uintptr_t>(scale) & 15u) == 0 && (reinterpret_cast<uintptr_t>(bias) & 15u) == 0 &&
                    g.cout % 4 == 0
                ? 1
                : 0;
    a.act = g.act;
    a.res_mode = g.res_mode;
    const long groups = ((long)a.total_pblocks + 3) / 4;
    const long wgs = groups * a.mblocks;
    if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
    const size_t lds = (size_t)a.wrounds * kG1Threads * 16;
    hipLaunchKernelGGL(k_gemm1x1, dim3((unsigned)wgs), dim3(kG1Threads), lds, s, a);
    return hipGetLastError();
}

}  // namespace cvx
