// k_dsblock.hip -- a whole depthwise-separable block as one launch, for small
// batches: depthwise 3x3 (+ BN + act) -> pointwise 1x1 (+ BN) + shortcut ->
// act, where the shortcut is the block input itself or a strided 1x1
// convolution of it (+ BN).  The depthwise output never leaves LDS
// ("Как я свертки ускорял", "А теперь — хардкор на Metal" and "Есть ощутимый
// прирост": one launch in place of three; "Пациента на стол" for the block).
//
// At batch 1 to a few images the MNIST blocks are a few MFLOP each and every
// launch is mostly its fixed cost (start, first loads, drain), so the block's
// three kernels cost about three times one.  Here a workgroup owns a run of
// kPix consecutive output pixels of one image and kCo output channels:
//   0. it issues every global load it needs at once, with in-bounds (clamped)
//      addresses and no branch between them, so they share one round trip:
//      the input rows the run's 3x3 windows touch (a contiguous run of each
//      input plane), the depthwise weights, scales and biases, and its kCo
//      rows of the pointwise (and shortcut) weights, unpacked from the packed
//      1x1 operand order when the layer holds packed weights; all to LDS;
//   1. it computes the depthwise layer for the run's pixels over all input
//      channels from LDS (taps outside the image select zero);
//   2. each thread sums four output channels of one pixel over all input
//      channels from LDS -- the strided shortcut reads its input samples from
//      the same staged rows -- and applies the epilogue (folded BN of both
//      products, the shortcut, the activation) before its single store.
// The depthwise values of a pixel run are recomputed by each of the
// ceil(c_out / kCo) channel groups: cheap next to a launch at these sizes, and
// it keeps every workgroup independent.
#include <hip/hip_runtime.h>

#include "bufio.h"
#include "cvx_internal.h"
#include "dsblock.h"
#include "epilogue.h"

namespace cvx {

namespace {

constexpr int kPix = 32;       // output pixels per workgroup
constexpr int kCo = 32;        // output channels per workgroup
constexpr int kThreads = 256;  // (kPix x kCo) / 4 outputs per thread
constexpr int kMaxCin = 256;
constexpr int kMaxRun = 256;   // floats of one input plane a run's windows touch
constexpr int kChunk = 16;     // input channels per chunk of the packed 1x1 order
constexpr size_t kMaxLds = 160 * 1024;

// Weight (co, ci) of a 1x1 layer: OIHW, or the packed order the 1x1 matrix
// kernels read ([32-row block][16-channel chunk][h][lane][2]: lane l holds
// output channel l % 32 of the block and input channel 4h + 2j + l / 32 of the
// chunk in element j).
__device__ __forceinline__ long w1x1_index(bool packed, int cin, int nchunks, int co, int ci)
{
    if (!packed) return (long)co * cin + ci;
    const int blk = co >> 5, chunk = ci >> 4, c16 = ci & 15;
    const int h = c16 >> 2, j = (c16 >> 1) & 1, lane = (co & 31) + 32 * (c16 & 1);
    return ((((long)blk * nchunks + chunk) * 4 + h) * 64 + lane) * 2 + j;
}

// Input rows the 3x3 windows (pad 1) of output rows [oy0, oy1] read.
__host__ __device__ __forceinline__ void run_rows(int oy0, int oy1, int stride, int h, int* r0, int* r1)
{
    *r0 = oy0 * stride - 1 < 0 ? 0 : oy0 * stride - 1;
    *r1 = oy1 * stride + 1 > h - 1 ? h - 1 : oy1 * stride + 1;
}

// Largest staged run over the workgroups' pixel runs (floats per plane).
int max_run(int h, int w, int oh, int ow, int stride)
{
    int most = 0;
    for (int p0 = 0; p0 < oh * ow; p0 += kPix) {
        const int last = (p0 + kPix < oh * ow ? p0 + kPix : oh * ow) - 1;
        int r0, r1;
        run_rows(p0 / ow, last / ow, stride, h, &r0, &r1);
        most = most > (r1 - r0 + 1) * w ? most : (r1 - r0 + 1) * w;
    }
    return most;
}

__host__ __device__ __forceinline__ int round256(int v) { return (v + 255) & ~255; }

// Staged floats per plane: the largest run rounded up to a power of two >= 64
// (each wave instruction fills 64 consecutive floats of one channel).
int run_pitch(int run)
{
    int p = 64;
    while (p < run) p *= 2;
    return p;
}

size_t lds_bytes(int cin, int runp, bool proj)
{
    const size_t floats = (size_t)(proj ? 2 : 1) * round256(cin * kCo) + (size_t)cin * kPix + round256(cin * 9) +
                          2 * (size_t)round256(cin) + (size_t)cin * runp;
    return floats * sizeof(float);
}

}  // namespace

__global__ void __launch_bounds__(kThreads) k_dsblock(DsBlockArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int cin = a.cin, runp = a.runp;
    const bool proj = a.skip_w != nullptr;
    // LDS regions (floats); those filled by whole rounds of 256 are rounded up
    const int wpn = round256(cin * kCo);
    const int o_ws = wpn;                             // [cin][kCo] shortcut weights (projection)
    const int o_d = o_ws + (proj ? wpn : 0);          // [cin][kPix] depthwise output
    const int o_pw = o_d + cin * kPix;                // [cin][9] depthwise taps
    const int o_psc = o_pw + round256(cin * 9);       // [cin] depthwise scales
    const int o_pbi = o_psc + round256(cin);          // [cin] depthwise biases
    const int o_s = o_pbi + round256(cin);            // [cin][runp] staged input rows
    const int t = threadIdx.x, lane = t & 63;
    const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const int ohw = a.oh * a.ow;
    const int p0 = blockIdx.x * kPix;
    const int co0 = blockIdx.y * kCo;
    const int n = blockIdx.z;
    const int last = (p0 + kPix < ohw ? p0 + kPix : ohw) - 1;
    int r0, r1;
    run_rows(p0 / a.ow, last / a.ow, a.stride, a.h, &r0, &r1);
    const int run = (r1 - r0 + 1) * a.w;  // <= runp (host)
    const int plane = a.h * a.w;

    // 0. every load at once, global -> LDS directly (no registers, no wait
    // before the barrier); out-of-range lanes read zero
    const rsrc_t rx = make_rsrc(a.x + (long)n * cin * plane, (unsigned)(cin * plane * 4));
    for (int ci = wv; ci < cin; ci += kThreads / 64) {
        for (int m = 0; m < runp; m += 64) {
            const int j = m + lane;
            int d = o_s + ci * runp + m;
            asm volatile("" : "+s"(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                     j < run ? (unsigned)(ci * plane + r0 * a.w + j) * 4u : kOOB, 0, 0,
                                                     0);
        }
    }
    {
        const rsrc_t rw = make_rsrc(a.dw_w, (unsigned)(cin * 9 * 4));
        const rsrc_t rs = make_rsrc(a.dw_scale, (unsigned)(cin * 4));
        const rsrc_t rb = make_rsrc(a.dw_bias, (unsigned)(cin * 4));
        for (int e0 = 0; e0 < cin * 9; e0 += kThreads) {
            int d = o_pw + e0 + 64 * wv;
            asm volatile("" : "+s"(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                     (unsigned)(e0 + t) * 4u, 0, 0, 0);
        }
        for (int e0 = 0; e0 < cin; e0 += kThreads) {
            int d = o_psc + e0 + 64 * wv;
            int d2 = o_pbi + e0 + 64 * wv;
            asm volatile("" : "+s"(d), "+s"(d2));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                     (unsigned)(e0 + t) * 4u, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(lds + d2), 4,
                                                     (unsigned)(e0 + t) * 4u, 0, 0, 0);
        }
    }
    {
        // weight (co0 + c, ci) to Wp[ci][c]: round e0 covers entries e0 .. e0 + 255
        const int nchunks = (cin + kChunk - 1) / kChunk;
        const rsrc_t rp = make_rsrc(a.pw_w, (unsigned)(a.pw_elems * 4));
        const rsrc_t rk = make_rsrc(proj ? a.skip_w : a.pw_w, (unsigned)((proj ? a.skip_elems : a.pw_elems) * 4));
        for (int e0 = 0; e0 < cin * kCo; e0 += kThreads) {
            const int e = e0 + t;
            const int ci = e / kCo, co = co0 + e % kCo;
            const bool live = co < a.cout && ci < cin;
            int d = e0 + 64 * wv;
            asm volatile("" : "+s"(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rp, (__attribute__((address_space(3))) void*)(lds + d), 4,
                live ? (unsigned)w1x1_index(a.pw_packed, cin, nchunks, co, ci) * 4u : kOOB, 0, 0, 0);
            if (proj) {
                int d2 = o_ws + e0 + 64 * wv;
                asm volatile("" : "+s"(d2));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (__attribute__((address_space(3))) void*)(lds + d2), 4,
                    live ? (unsigned)w1x1_index(a.skip_packed, cin, nchunks, co, ci) * 4u : kOOB, 0, 0, 0);
            }
        }
    }
    __syncthreads();
    const float* Wp = lds;
    const float* Ws = lds + o_ws;
    float* D = lds + o_d;
    const float* S = lds + o_s;

    // 1. depthwise 3x3 (pad 1) for the run's pixels, every input channel
    const int p = t % kPix;
    const int cq = t / kPix;  // 0..7
    const int pix = min(p0 + p, ohw - 1);
    const int oy = pix / a.ow, ox = pix - oy * a.ow;
    int off[9];
    bool ok[9];
#pragma unroll
    for (int ky = 0; ky < 3; ++ky) {
        const int iy = oy * a.stride - 1 + ky;
        const bool oky = iy >= 0 && iy < a.h;
        const int ry = (oky ? iy : r0) - r0;
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) {
            const int ix = ox * a.stride - 1 + kx;
            const bool okx = ix >= 0 && ix < a.w;
            ok[ky * 3 + kx] = oky && okx;
            off[ky * 3 + kx] = ry * a.w + (okx ? ix : 0);
        }
    }
#pragma unroll 2
    for (int ci = cq; ci < cin; ci += kThreads / kPix) {
        const float* __restrict__ sc = S + ci * runp;
        const float* __restrict__ pc = lds + o_pw + ci * 9;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < 9; ++k) acc = fmaf(pc[k], ok[k] ? sc[off[k]] : 0.0f, acc);
        D[ci * kPix + p] = apply_act(fmaf(lds[o_psc + ci], acc, lds[o_pbi + ci]), a.dw_act);
    }
    __syncthreads();

    // 2. four output channels of one pixel per thread
    const int xoff = (oy * a.stride - r0) * a.w + ox * a.stride;  // the strided shortcut's sample
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float acs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int ci = 0; ci < cin; ++ci) {
        const float d = D[ci * kPix + p];
        const float4 w4 = *reinterpret_cast<const float4*>(Wp + ci * kCo + 4 * cq);
        acc[0] = fmaf(w4.x, d, acc[0]);
        acc[1] = fmaf(w4.y, d, acc[1]);
        acc[2] = fmaf(w4.z, d, acc[2]);
        acc[3] = fmaf(w4.w, d, acc[3]);
        if (proj) {
            const float xs = S[ci * runp + xoff];
            const float4 s4 = *reinterpret_cast<const float4*>(Ws + ci * kCo + 4 * cq);
            acs[0] = fmaf(s4.x, xs, acs[0]);
            acs[1] = fmaf(s4.y, xs, acs[1]);
            acs[2] = fmaf(s4.z, xs, acs[2]);
            acs[3] = fmaf(s4.w, xs, acs[3]);
        }
    }
    if (p0 + p >= ohw) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int co = co0 + 4 * cq + k;
        if (co >= a.cout) break;
        const long o = ((long)n * a.cout + co) * ohw + pix;
        float z = fmaf(a.pw_scale[co], acc[k], a.pw_bias[co]);
        if (proj) z += fmaf(a.skip_scale[co], acs[k], a.skip_bias[co]);
        float y;
        if (a.res_mode == CVX_RES_BEFORE_ACT && !proj)
            y = apply_act(z + a.res[o], a.pw_act);
        else if (a.res_mode == CVX_RES_AFTER_ACT)
            y = apply_act(z, a.pw_act) + a.res[o];
        else
            y = apply_act(z, a.pw_act);
        a.y[o] = y;
    }
}

// The planner's test for a block: a depthwise 3x3 layer (pad 1, stride 1 or
// 2, no residual) whose one reader is a 1x1 stride-1 layer, with a shortcut
// that is absent, an identity tensor of the output's shape, or a 1x1 layer
// of the block input at the depthwise stride (BN, no activation) added before
// the pointwise activation; input channels up to kMaxCin; small enough that
// launches, not bytes, decide its time.
bool dsblock_fits(const ConvGeom& dw, const ConvGeom& pw, const ConvGeom* skip)
{
    if (!(dw.groups == dw.cin && dw.cout == dw.cin && dw.k == 3 && dw.pad == 1)) return false;
    if (dw.stride != 1 && dw.stride != 2) return false;
    if (dw.res_mode != CVX_RES_NONE) return false;
    if (pw.k != 1 || pw.stride != 1 || pw.pad != 0 || pw.groups != 1) return false;
    if (pw.cin != dw.cout || pw.n != dw.n || pw.h != dw.oh || pw.w != dw.ow) return false;
    if (dw.cin > kMaxCin) return false;
    const int run = max_run(dw.h, dw.w, dw.oh, dw.ow, dw.stride);
    if (run > kMaxRun || lds_bytes(dw.cin, run_pitch(run), skip != nullptr) > kMaxLds) return false;
    if ((long)dw.n * dw.cin * dw.h * dw.w >= (1L << 29)) return false;  // 32-bit buffer offsets
    if (skip) {
        if (skip->k != 1 || skip->pad != 0 || skip->groups != 1 || skip->stride != dw.stride) return false;
        if (skip->act != CVX_ACT_NONE || skip->res_mode != CVX_RES_NONE) return false;
        if (skip->n != dw.n || skip->cin != dw.cin || skip->h != dw.h || skip->w != dw.w) return false;
        if (skip->cout != pw.cout || skip->oh != pw.oh || skip->ow != pw.ow) return false;
        if (pw.res_mode != CVX_RES_BEFORE_ACT) return false;
    }
    // the small-batch regime: at most a few workgroups per compute unit
    const long groups = (long)((pw.oh * pw.ow + kPix - 1) / kPix) * ((pw.cout + kCo - 1) / kCo) * pw.n;
    return groups <= kDsBlockMaxGroups && pw.n <= 65535;
}

void dsblock_describe(const ConvGeom& dw, const ConvGeom& pw, bool proj, char* buf, int len)
{
    snprintf(buf, len, "dsblock dw s%d + pw k1%s pix=%d co=%d kernel=cvx::k_dsblock", dw.stride,
             proj ? " + shortcut k1" : "", kPix, kCo);
}

hipError_t launch_dsblock(DsBlockArgs a, hipStream_t s)
{
    a.runp = run_pitch(max_run(a.h, a.w, a.oh, a.ow, a.stride));
    const long nchunks = (a.cin + kChunk - 1) / kChunk;
    const long packed = (a.cout + 31) / 32 * nchunks * 512;  // one lane order of the packed 1x1 weights
    a.pw_elems = a.pw_packed ? packed : (long)a.cout * a.cin;
    a.skip_elems = a.skip_packed ? packed : (long)a.cout * a.cin;
    const int ohw = a.oh * a.ow;
    dim3 grid((unsigned)((ohw + kPix - 1) / kPix), (unsigned)((a.cout + kCo - 1) / kCo), (unsigned)a.n);
    const size_t lds = lds_bytes(a.cin, a.runp, a.skip_w != nullptr);
    hipLaunchKernelGGL(k_dsblock, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace cvx
