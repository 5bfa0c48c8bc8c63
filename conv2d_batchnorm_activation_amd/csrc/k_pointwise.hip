// k_pointwise.hip -- 1x1 convolution (stride 1 or 2, no padding) + folded
// BatchNorm + residual + activation on fp32 matrix cores, for batches of small
// planes; optionally with a second 1x1 convolution (a block's shortcut) summed
// into the same output ahead of the activation.
//
// A 1x1 layer is one matrix product per image, Y[c_out][OH*OW] =
// W[c_out][c_in] X[c_in][OH*OW] (the pointwise and shortcut layers of the
// depthwise-separable MNIST net, "Как я свертки ускорял"; the 1x1 layers of
// "YOLO26N Inference Optimisation").  When a plane holds at most a few hundred
// pixels, one workgroup takes one whole image and a group of CO output
// channels (all of them, or an equal share), so that
//   * a chunk of 16 input channels of the image is one contiguous run (stride
//     1) or 16 x OH input rows (stride s: rows s*oh), copied to LDS with
//     16-byte LDS-direct loads whatever the plane's width;
//   * the input is read once, however many output channels there are;
//   * the image's CO output planes are one contiguous run of CO*OH*OW floats:
//     the tile is written to LDS in exactly that order, then every residual
//     load and output store moves 16 contiguous bytes per lane.
// The reduction runs over the chunks of one or two sources, each with its own
// input, packed weights and BatchNorm scale: a block's last 1x1 layer and its
// shortcut convolution, whose sum the block's activation takes, are one
// product over the channels of both.  Each source's scale multiplies its
// weights as they are read (one multiply per weight and lane), so the sums are
// already scaled and the epilogue only adds the biases.
// Roles as in the packed implicit GEMM: four producer waves stage chunk st+2
// while four consumer waves compute chunk st (three LDS buffers, one barrier
// per chunk).  The tile's 32x32 blocks (pixel block x channel block) are split
// over the consumer waves in a wpx x (4 / wpx) grid; each block is a chain of
// v_mfma_f32_32x32x2_f32 with the input as the A operand (lane l: pixel l%32,
// channel 2k + l/32) and the weights, in the packed 1x1 order, as B (lane l:
// output channel l%32, same channel), so a lane's sums cover runs of four
// consecutive pixels of one output channel.
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPwThreads = 512;    // four producer and four consumer waves
constexpr int kPwMaxRounds = 8;    // input staging rounds (256 16-byte elements) per chunk
constexpr int kPwWRounds = 3;      // weight staging rounds per chunk: up to six channel blocks
constexpr int kPwMaxCB = 6;
constexpr int kPwResQ = 20;        // output quads per producer thread: tiles of up to 20480 floats
constexpr int kPwChunkW = 512;     // packed 1x1 weight floats per (32-channel block, chunk)

__device__ __forceinline__ int pw_div(int n, unsigned m, unsigned l)
{
    return (int)((__umulhi((unsigned)n, m) + (unsigned)n) >> l);
}

// Keeps the compiler from moving memory operations across this point (the
// waits count loads in issue order).
__device__ __forceinline__ void pw_order()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// 16-byte LDS-direct load (lane i writes d + 16 i); outside the kernel template
// so the host pass, which cannot check this gfx950 form, still emits the stubs.
__device__ __forceinline__ void pw_lds_load16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}

// One source of the reduction: its input, packed weights and BatchNorm scale,
// and how a chunk of it is staged and read.
struct PwSrc {
    const float* x;
    const float* wp;
    const float* scale;
    int cin, HW, nchunks;
    // Staging of one chunk: element e (16 bytes) -> row r = e / RQ and quad e % RQ;
    // row r -> channel r / RPC, first float (r % RPC) * RSTR of that channel.
    int rounds, RE, RQ, RPC, RSTR;
    unsigned m_rq, l_rq, m_rpc, l_rpc;
    // A staged chunk in LDS: pixel q -> (oh, ow) = divmod(q, OWD) at float
    // oh*WS + S*ow + channel*CS.
    int OWD, WS, S, CS;
    unsigned m_owd, l_owd;
    unsigned wp_bytes;
};

struct PwArgs {
    PwSrc src[2];               // chunks n1 .. nchunks-1 come from src[1]
    const float* bias;
    const float* bias2;         // the second source's bias, or null
    const float* res;
    float* y;
    int cout, OHW;
    int groups_co;              // channel groups per image: c_out / CO
    int CO, CB, PB;             // channels of a tile, its 32-channel blocks, its 32-pixel blocks
    int nchunks, n1;            // chunks of both sources; chunks of src[0]
    unsigned m_g, l_g;          // divide by groups_co
    int wrounds;
    int wpx, pb_per, cb_per;    // consumer grid: waves along pixels, blocks per wave
    int BUF, WOFF;              // floats per stage buffer, weights' offset within it
    int SPARE;                  // LDS float offset of a 16-byte slot that takes dropped sums
    int rq, rq_per;             // output quads per producer thread, residual quads loaded per chunk
    int act, res_mode;
};

// TWO: a second source follows the first (compiled apart, so a one-source
// layer carries none of its arguments, registers or branches).
template <int MP, int MC, bool TWO>
__global__ void __launch_bounds__(kPwThreads) k_pointwise(PwArgs a)
{
    extern __shared__ __attribute__((aligned(16))) float smem[];
    warm_kernargs<sizeof(PwArgs)>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: addresses stay scalar
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // Workgroup -> (image, channel group), numbered XCD by XCD so the groups of
    // one image share an L2.
    int img, grp;
    {
        const unsigned h = blockIdx.x, G8 = gridDim.x;
        const unsigned xcd = h & 7u, i8 = h >> 3, base = G8 >> 3, rem = G8 & 7u;
        const int L = (int)(xcd * base + min(xcd, rem) + i8);
        img = pw_div(L, a.m_g, a.l_g);
        grp = L - img * a.groups_co;
    }
    const int nst = a.nchunks;
    const int n1 = TWO ? a.n1 : a.nchunks;
    const int BUF = a.BUF;

    if (wave >= 4) {
        // ---------------------------------------------------------- producers
        const int ptid = tid - 256;
        const int pw = wave - 4;
        // byte offsets of this lane's staged elements within a chunk of each
        // source, the same for every chunk of it (a stride-1 chunk is one run);
        // past the chunk's elements an out-of-range offset
        unsigned goff[2][kPwMaxRounds];
        unsigned woff[2][kPwWRounds];
        auto setup_src = [&](auto S) {
            constexpr int s = decltype(S)::value;
            const PwSrc& sr = a.src[s];
            if (sr.RPC > 1) {
                const int HW = sr.HW, RPC = sr.RPC, RSTR = sr.RSTR, RQ = sr.RQ, RE = sr.RE;
#pragma unroll
                for (int i = 0; i < kPwMaxRounds; ++i) {
                    const int e = ptid + 256 * i;
                    const int r = pw_div(e, sr.m_rq, sr.l_rq);
                    const int c = pw_div(r, sr.m_rpc, sr.l_rpc);
                    const int f = c * HW + (r - c * RPC) * RSTR + 4 * (e - r * RQ);
                    goff[s][i] = e < RE ? 4u * (unsigned)f : kOOB;
                }
            } else {
#pragma unroll
                for (int i = 0; i < kPwMaxRounds; ++i) {
                    const int e = ptid + 256 * i;
                    goff[s][i] = e < sr.RE ? 16u * (unsigned)e : kOOB;
                }
            }
            // the group's weights of a chunk: CB blocks of 2 KB, kPwChunkW floats
            // apart per chunk and nchunks * kPwChunkW apart per block
#pragma unroll
            for (int j = 0; j < kPwWRounds; ++j) {
                const int e = ptid + 256 * j;
                const int blk = e >> 7;
                woff[s][j] = blk < a.CB ? 4u * ((unsigned)((grp * a.CB + blk) * sr.nchunks) * kPwChunkW +
                                                4u * (unsigned)(e & 127))
                                        : kOOB;
            }
        };
        // the second source's offsets are worked out while the first chunks
        // load, unless those chunks already need them
        setup_src(std::integral_constant<int, 0>{});
        if constexpr (TWO) {
            if (n1 < 3) setup_src(std::integral_constant<int, 1>{});
        }
        // chunk c of source sr into stage buffer sb: sr.rounds + a.wrounds loads
        // per wave
        auto issue_src = [&](const PwSrc& sr, const unsigned* go, const unsigned* wo, int c, int sb) {
            const float* xim = sr.x + (long)img * sr.cin * sr.HW;
            const rsrc_t rx = make_rsrc(xim + (long)c * 16 * sr.HW, 64u * (unsigned)sr.HW);
            const rsrc_t rw = make_rsrc(sr.wp + (long)c * kPwChunkW, sr.wp_bytes - 4u * kPwChunkW * (unsigned)c);
#pragma unroll
            for (int i = 0; i < kPwMaxRounds; ++i) {
                if (i >= sr.rounds) break;
                pw_lds_load16(rx, (__attribute__((address_space(3))) void*)(smem + sb + 1024 * i + 256 * pw), go[i]);
            }
#pragma unroll
            for (int j = 0; j < kPwWRounds; ++j) {
                if (j >= a.wrounds) break;
                pw_lds_load16(rw, (__attribute__((address_space(3))) void*)(smem + sb + a.WOFF + 1024 * j + 256 * pw),
                              wo[j]);
            }
        };
        auto issue = [&](int st, int sb) {
            if (!TWO || st < n1)
                issue_src(a.src[0], goff[0], woff[0], st, sb);
            else
                issue_src(a.src[1], goff[1], woff[1], st - n1, sb);
        };
        // loads per wave of chunk st
        auto nld = [&](int st) { return (!TWO || st < n1 ? a.src[0].rounds : a.src[1].rounds) + a.wrounds; };
        // This thread's output quads e = ptid + 256 j of the tile's run; their
        // residual comes to registers, a share per chunk while the consumers
        // compute.
        const long obase = ((long)img * a.cout + (long)grp * a.CO) * a.OHW;
        const int tq = a.CO * a.OHW / 4;
        const unsigned run_b = 16u * (unsigned)tq;
        const bool want_res = a.res_mode != CVX_RES_NONE;
        const rsrc_t rres = make_rsrc(want_res ? a.res + obase : a.y, want_res ? run_b : 0u);
        f32x4 rv[kPwResQ];  // only the first a.rq are loaded, and only those are read
        auto load_res = [&](int lo, int hi_) {
#pragma unroll
            for (int j = 0; j < kPwResQ; ++j) {
                if (j >= lo && j < hi_) {
                    const int e = ptid + 256 * j;
                    rv[j] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rres, (int)(e < tq ? 16u * (unsigned)e : kOOB), 0, 0));
                }
            }
        };

        // Stage buffers: chunk s is in buffer s % 3.  The consumers read chunk s
        // between barriers s-1 and s (chunk 0 between an opening barrier and
        // barrier 0), so its buffer takes chunk s+3 right after barrier s;
        // barrier s needs chunk s+1 landed.  Chunks are thus issued two barriers
        // before they are needed.
        auto bufof = [&](int s3) { return (s3 % 3) * BUF; };
        pw_order();
        issue(0, 0);
        if (nst > 1) issue(1, BUF);
        if (nst > 2) issue(2, 2 * BUF);
        pw_order();
        if constexpr (TWO) {
            if (n1 >= 3) setup_src(std::integral_constant<int, 1>{});
        }
        wait_vm_at_most((nst > 1 ? nld(1) : 0) + (nst > 2 ? nld(2) : 0));  // chunk 0
        lds_barrier();                                                     // opening barrier
        wait_vm_at_most(nst > 2 ? nld(2) : 0);                             // chunk 1
        lds_barrier();                                                     // barrier 0
        int rdone = 0;
        for (int st = 1; st < nst; ++st) {
            // after barrier st-1: the buffer of chunk st-1 is free
            int piece = 0;
            if (want_res) {
                const int upto = min(a.rq, st * a.rq_per);
                piece = upto - rdone;
                load_res(rdone, upto);
                rdone = upto;
            }
            pw_order();
            const bool more = st + 2 < nst;
            if (more) issue(st + 2, bufof(st + 2));
            pw_order();
            wait_vm_at_most(piece + (more ? nld(st + 2) : 0));  // chunk st+1 (and every earlier load)
            lds_barrier();
        }
        if (want_res) load_res(rdone, a.rq);
        __syncthreads();  // the consumers' exchange

        // ------------------------------------------------------------ copy-out
        // The tile's finished run, 16 bytes a lane: residual and activation
        // applied on the way.
        __syncthreads();
        const rsrc_t ry = make_rsrc(a.y + obase, run_b);
        auto copy_out = [&](auto act_fn) {
#pragma unroll
            for (int j = 0; j < kPwResQ; ++j) {
                if (j >= a.rq) break;
                const int e = ptid + 256 * j;
                const f32x4 v = reinterpret_cast<const f32x4*>(smem)[min(e, tq - 1)];
                f32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    float t = v[k];
                    t = a.res_mode == CVX_RES_BEFORE_ACT ? t + rv[j][k] : t;
                    t = act_fn(t);
                    o[k] = a.res_mode == CVX_RES_AFTER_ACT ? t + rv[j][k] : t;
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ry,
                                                       (int)(e < tq ? 16u * (unsigned)e : kOOB), 0, 0);
            }
        };
        if (a.act == CVX_ACT_RELU)
            copy_out([](float t) { return fmaxf(t, 0.0f); });
        else if (a.act == CVX_ACT_SILU)
            copy_out([](float t) { return t * __builtin_amdgcn_rcpf(1.0f + __expf(-t)); });
        else
            copy_out([](float t) { return t; });
        return;
    }

    // -------------------------------------------------------------- consumers
    const int wx = wave % a.wpx;
    const int wc = wave / a.wpx;
    const int pb0 = wx * a.pb_per;
    const int cb0 = wc * a.cb_per;
    // A wave owns pixel blocks pb0 .. pb0+MP-1 and channel blocks cb0 ..
    // cb0+MC-1 of the tile.  Blocks past the tile (the template covers the
    // largest share) compute on clamped, in-range operands and are dropped.
    // Per source: this lane's LDS offset of its pixel in a staged chunk, and the
    // BatchNorm scale of its output channel, which multiplies the weights.
    int abase[2][MP];
    int cs2[2];
    float bsc[2][MC];
    int boff[MC];
    float bi[MC];
    {
#pragma unroll
        for (int s = 0; s < (TWO ? 2 : 1); ++s) {
            const PwSrc& sr = a.src[s];
            cs2[s] = 2 * sr.CS;
#pragma unroll
            for (int mp = 0; mp < MP; ++mp) {
                const int q = min(32 * (pb0 + mp) + l32, a.OHW - 1);
                const int oh = pw_div(q, sr.m_owd, sr.l_owd);
                abase[s][mp] = hi * sr.CS + oh * sr.WS + sr.S * (q - oh * sr.OWD);
            }
            const rsrc_t rs = make_rsrc(sr.scale, 4u * (unsigned)a.cout);
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                const int cb = min(cb0 + mc, a.CB - 1);
                bsc[s][mc] = bload(rs, 4u * (unsigned)(grp * a.CO + 32 * cb + l32));
            }
        }
        const rsrc_t rb = make_rsrc(a.bias, 4u * (unsigned)a.cout);
        // a null second bias reads as zeros (a range of 0 bytes)
        const rsrc_t rb2 = make_rsrc(a.bias2 ? a.bias2 : a.bias, a.bias2 ? 4u * (unsigned)a.cout : 0u);
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            const int cb = min(cb0 + mc, a.CB - 1);
            boff[mc] = a.WOFF + cb * kPwChunkW + 2 * lane;
            const unsigned co = (unsigned)(grp * a.CO + 32 * cb + l32);
            bi[mc] = TWO ? bload(rb, 4u * co) + bload(rb2, 4u * co) : bload(rb, 4u * co);
        }
    }
    f32x16 acc[MP][MC];
#pragma unroll
    for (int mp = 0; mp < MP; ++mp)
#pragma unroll
        for (int mc = 0; mc < MC; ++mc)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mp][mc][r] = 0.0f;

    // A chunk's operands: input of eight channel pairs for MP pixel blocks,
    // weights of the pairs for MC channel blocks.  Those of chunk st+1 are read
    // (between barriers st and st+1) while chunk st's matrix instructions run,
    // pair by pair: a wave may have only 15 LDS reads in flight, so issuing a
    // whole chunk's reads at once would stall in front of the matrix work.
    struct Ops {
        float x[8][MP];
        f32x2 w[MC][4];
    };
    // where a chunk of one source is read: pixel offsets and channel-pair stride
    struct View {
        int ab[MP];
        int c2;
    };
    auto view = [&](int ch, View& v) {
        const bool s1 = TWO && ch >= n1;  // uniform
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) v.ab[mp] = s1 ? abase[1][mp] : abase[0][mp];
        v.c2 = s1 ? cs2[1] : cs2[0];
    };
    // reads of pair k: its input, and at even k the weights of pairs k, k+1
    auto read_pair = [&](int sbuf, const View& v, Ops& o, int k) {
        if ((k & 1) == 0) {
#pragma unroll
            for (int mc = 0; mc < MC; ++mc)
                o.w[mc][k >> 1] = *reinterpret_cast<const f32x2*>(smem + sbuf + boff[mc] + 64 * k);
        }
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) o.x[k][mp] = smem[sbuf + v.ab[mp] + k * v.c2];
    };
    // chunk ch (in `o`), and chunk ch+1's operands from buffer `nbuf` into `n`,
    // one pair's reads ahead of each pair's matrix instructions (so the last
    // reads have landed by the barrier's LDS wait).  After the last chunk these
    // reads take whatever a buffer holds, unused: no branch between the matrix
    // instructions.  The first source's sums are scaled once, when the second
    // source starts (or in the epilogue); the second source's weights are
    // scaled as they are used, those of pairs k+2, k+3 among pair k's matrix
    // instructions (a multiply right after the read would wait for it).
    auto compute = [&](const Ops& o, Ops& n, int nbuf, int ch, auto SCALED) {
        constexpr bool scaled = decltype(SCALED)::value;
        View v;
        view(ch + 1, v);
        f32x2 w[MC][4];  // scaled weights (second source only)
        if constexpr (scaled) {
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) w[mc][0] = o.w[mc][0] * bsc[1][mc];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            read_pair(nbuf, v, n, k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mp = 0; mp < MP; ++mp)
#pragma unroll
                for (int mc = 0; mc < MC; ++mc) {
                    if constexpr (scaled)
                        acc[mp][mc] = __builtin_amdgcn_mfma_f32_32x32x2f32(o.x[k][mp], w[mc][k >> 1][k & 1],
                                                                          acc[mp][mc], 0, 0, 0);
                    else
                        acc[mp][mc] = __builtin_amdgcn_mfma_f32_32x32x2f32(o.x[k][mp], o.w[mc][k >> 1][k & 1],
                                                                          acc[mp][mc], 0, 0, 0);
                }
            if constexpr (scaled) {
                if ((k & 1) == 0 && k + 2 < 8) {
#pragma unroll
                    for (int mc = 0; mc < MC; ++mc) w[mc][(k >> 1) + 1] = o.w[mc][(k >> 1) + 1] * bsc[1][mc];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto nextb = [&](int b) { return b == 2 * BUF ? 0 : b + BUF; };
    Ops o0, o1;
    lds_barrier();  // opening barrier: chunk 0 has landed
    {
        View v;
        view(0, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) read_pair(0, v, o0, k);
    }
    lds_barrier();  // barrier 0: chunk 1 has landed, chunk 0's buffer is read
    int sb = 0;     // buffer of chunk st
    int st = 0;
    // chunks st .. end-1, chunk st's operands in o0 (and so again on return)
    auto run = [&](int end, auto SCALED) {
        for (;;) {
            if (st > 0) lds_barrier();
            compute(o0, o1, nextb(sb), st, SCALED);
            sb = nextb(sb);
            if (++st >= end) {
                o0 = o1;
                break;
            }
            lds_barrier();
            compute(o1, o0, nextb(sb), st, SCALED);
            sb = nextb(sb);
            if (++st >= end) break;
        }
    };
    // the first source's chunks plain, then (with a second source) its sums
    // scaled and the second source's chunks with scaled weights: two loops,
    // not a branch per chunk, which would hold two register assignments
    run(n1, std::false_type{});
    if (TWO) {
#pragma unroll
        for (int mp = 0; mp < MP; ++mp)
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) acc[mp][mc] *= bsc[0][mc];
        run(nst, std::true_type{});
    }
    // a single source's sums take their scale here
    float esc[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) esc[mc] = TWO ? 1.0f : bsc[0][mc];

    // Exchange: every scaled sum plus its biases goes to its place in the tile's
    // [channel][pixel] output run (over the stage buffers, free once every wave
    // is past this barrier); pixels past the plane go to a spare slot.
    __syncthreads();
    const bool quads = (a.OHW & 3) == 0;
#pragma unroll
    for (int mp = 0; mp < MP; ++mp) {
        const int pb = pb0 + mp;
        if (pb >= a.PB) break;
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            const int cb = cb0 + mc;
            if (cb >= a.CB) break;
            const int row = (32 * cb + l32) * a.OHW;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int q = 32 * pb + 8 * g + 4 * hi;
                f32x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = fmaf(esc[mc], acc[mp][mc][4 * g + e], bi[mc]);
                if (quads) {
                    // in 16-byte units, so the store is one 16-byte LDS write
                    const int r4 = (32 * cb + l32) * (a.OHW >> 2) + 8 * pb + 2 * g + hi;
                    reinterpret_cast<f32x4*>(smem)[q < a.OHW ? r4 : (a.SPARE >> 2)] = z;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) smem[q + e < a.OHW ? row + q + e : a.SPARE] = z[e];
                }
            }
        }
    }
    __syncthreads();  // the producers copy the run out
}

// ------------------------------------------------------------------ host side
// Compiled shares of a consumer wave: MP pixel blocks x MC channel blocks.
struct PwKind {
    int mp, mc;
};
static constexpr PwKind kPwKinds[] = {{2, 3}, {1, 3}, {2, 2}, {1, 2}};
constexpr int kNumPwKinds = sizeof(kPwKinds) / sizeof(kPwKinds[0]);

void fastdiv_params(int d, unsigned* m, unsigned* l);

// Staging geometry of one chunk: rows of RQ 16-byte elements.
struct PwStage {
    int rq, rpc, rstr, re, rounds;
    int cs, ws, owd;
};

static bool pw_stage(const ConvGeom& g, PwStage* s)
{
    const int hw = g.h * g.w, ohw = g.oh * g.ow;
    if (g.stride == 1) {
        // the chunk is one run of 16*HW floats, 16-byte aligned when c_in*HW and
        // 16*HW are multiples of 4 (c_in is a multiple of 16)
        s->rq = 4 * hw;
        s->rpc = 1;
        s->rstr = 0;
        s->re = 4 * hw;
        s->cs = hw;
        s->ws = 0;
        s->owd = ohw;  // one staged row per channel: (oh, ow) = (0, q)
    } else {
        // rows s*oh of every channel, each widened to whole 16-byte elements
        // (the widening reads at most 12 bytes of the next row, never used)
        if (hw % 4 != 0 || (g.stride * g.w) % 4 != 0) return false;
        const int wq = (g.w + 3) / 4;
        s->rq = wq;
        s->rpc = g.oh;
        s->rstr = g.stride * g.w;
        s->re = 16 * g.oh * wq;
        s->cs = g.oh * 4 * wq;
        s->ws = 4 * wq;
        s->owd = g.ow;
    }
    s->rounds = (s->re + 255) / 256;
    return s->rounds <= kPwMaxRounds;
}

static bool pw_layer_ok(const ConvGeom& g)
{
    if (g.groups != 1 || g.k != 1 || g.pad != 0 || g.cin % 16 != 0 || g.cout % 32 != 0) return false;
    const long lim = 0x7fffffffL;
    return (long)g.n * g.cin * g.h * g.w * 4 < lim && (long)g.n * g.cout * g.oh * g.ow * 4 < lim &&
           packed_weight_floats(g) * 4 < lim;
}

// Channel groups per image, consumer grid and compiled share for a layer, or for
// a layer g and a second source g2 over the same output; false when the
// pointwise kernel does not take it.
struct PwConfig {
    int groups, kind, wpx, pb_per, cb_per;
    size_t lds;
};

static bool pw_config(const ConvGeom& g, const ConvGeom* g2, PwConfig* c)
{
    PwStage s, s2;
    if (!pw_layer_ok(g) || !pw_stage(g, &s)) return false;
    int rounds = s.rounds, cin_all = g.cin;
    if (g2 != nullptr) {
        if (!pw_layer_ok(*g2) || !pw_stage(*g2, &s2)) return false;
        if (g2->n != g.n || g2->cout != g.cout || g2->oh != g.oh || g2->ow != g.ow) return false;
        rounds = std::max(rounds, s2.rounds);
        cin_all += g2->cin;
    }
    const int ohw = g.oh * g.ow;
    const int pb = (ohw + 31) / 32;
    const int cbt = g.cout / 32;
    double best = 1e300;
    bool found = false;
    for (int groups = 1; groups <= cbt; ++groups) {
        if (cbt % groups != 0) continue;
        const int cb = cbt / groups;
        // at most six channel blocks a tile, and enough workgroups to spread
        // over the chip
        if (cb > kPwMaxCB || (long)g.n * groups < 64) continue;
        const int wrounds = (cb * 128 + 255) / 256;
        const size_t buf = (size_t)rounds * 1024 + (size_t)wrounds * 1024;
        const size_t xch = (size_t)32 * cb * ohw;
        // the exchange (plus a spare slot) over the stage buffers; the producers
        // hold the residual of up to kPwResQ output quads each
        const size_t lds = 4 * std::max(3 * buf, xch + 4);
        if (lds > kMaxLdsBytes || xch > (size_t)kPwResQ * 256 * 4) continue;
        for (int wpx = 4; wpx >= 1; wpx /= 2) {
            const int pb_per = (pb + wpx - 1) / wpx;
            const int cb_per = (cb + 4 / wpx - 1) / (4 / wpx);
            for (int kind = 0; kind < kNumPwKinds; ++kind) {
                if (kPwKinds[kind].mp < pb_per || kPwKinds[kind].mc < cb_per) continue;
                // every wave runs MP x MC block chains (clamped ones too): the
                // matrix work per workgroup, times the rounds of workgroups (one
                // per compute unit), plus a start-up per round
                const long wgs = (long)g.n * groups;
                const double wrnds = std::ceil(wgs / 256.0);
                const double units = (double)kPwKinds[kind].mp * kPwKinds[kind].mc;
                const double cost = wrnds * (units * (cin_all / 2) * 64.0 + 5000.0) + 1e-3 * units;
                if (cost < best) {
                    best = cost;
                    *c = PwConfig{groups, kind, wpx, pb_per, cb_per, lds};
                    found = true;
                }
            }
        }
    }
    return found;
}

bool pointwise_fits(const ConvGeom& g)
{
    PwConfig c;
    return pw_config(g, nullptr, &c);
}

bool pointwise_pair_fits(const ConvGeom& g, const ConvGeom& g2)
{
    PwConfig c;
    return pw_config(g, &g2, &c);
}

void pointwise_describe(const ConvGeom& g, const ConvGeom* g2, char* buf, int len)
{
    PwConfig c{};
    pw_config(g, g2, &c);
    if (g2 != nullptr)
        snprintf(buf, len,
                 "pointwise k1 s%d + shortcut k1 s%d groups=%d wpx=%d splitk=1 kernel=cvx::k_pointwise<%d, %d, true>",
                 g.stride, g2->stride, c.groups, c.wpx, kPwKinds[c.kind].mp, kPwKinds[c.kind].mc);
    else
        snprintf(buf, len, "pointwise k1 s%d groups=%d wpx=%d splitk=1 kernel=cvx::k_pointwise<%d, %d, false>",
                 g.stride, c.groups, c.wpx, kPwKinds[c.kind].mp, kPwKinds[c.kind].mc);
}

bool pointwise_aligned(const float* x, const float* res, const float* y)
{
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return al(x) && al(y) && (res == nullptr || al(res));
}

template <int MP, int MC>
static void launch_pw(dim3 grid, size_t lds, hipStream_t s, const PwArgs& a, bool two)
{
    if (two)
        hipLaunchKernelGGL((k_pointwise<MP, MC, true>), grid, dim3(kPwThreads), lds, s, a);
    else
        hipLaunchKernelGGL((k_pointwise<MP, MC, false>), grid, dim3(kPwThreads), lds, s, a);
}

static void fill_src(const ConvGeom& g, const PwStage& st, const float* x, const float* wp,
                     const float* scale, PwSrc* sr)
{
    sr->x = x;
    sr->wp = wp;
    sr->scale = scale;
    sr->cin = g.cin;
    sr->HW = g.h * g.w;
    sr->nchunks = g.cin / 16;
    sr->rounds = st.rounds;
    sr->RE = st.re;
    sr->RQ = st.rq;
    sr->RPC = st.rpc;
    sr->RSTR = st.rstr;
    fastdiv_params(st.rq, &sr->m_rq, &sr->l_rq);
    fastdiv_params(st.rpc, &sr->m_rpc, &sr->l_rpc);
    sr->OWD = st.owd;
    sr->WS = st.ws;
    sr->S = g.stride;
    sr->CS = st.cs;
    fastdiv_params(st.owd, &sr->m_owd, &sr->l_owd);
    sr->wp_bytes = (unsigned)(packed_copy_floats(g) * 4);
}

// One layer (g2 null), or a layer and a second 1x1 source summed into the same
// output ahead of the activation (g's residual mode is then not used).
static hipError_t launch_pw_any(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                                const float* bias, const float* res, const ConvGeom* g2, const float* x2,
                                const float* wp2, const float* scale2, const float* bias2, float* y,
                                hipStream_t s)
{
    PwConfig c;
    PwStage st, st2{};
    if (!pw_config(g, g2, &c) || !pw_stage(g, &st)) return hipErrorInvalidValue;
    if (g2 != nullptr && !pw_stage(*g2, &st2)) return hipErrorInvalidValue;
    if (!pointwise_aligned(x, g2 ? nullptr : res, y) || (g2 != nullptr && !pointwise_aligned(x2, nullptr, y)))
        return hipErrorInvalidValue;
    PwArgs a;
    fill_src(g, st, x, wp, scale, &a.src[0]);
    if (g2 != nullptr)
        fill_src(*g2, st2, x2, wp2, scale2, &a.src[1]);
    else
        a.src[1] = a.src[0];  // never staged: every chunk is the first source's
    a.bias = bias;
    a.bias2 = g2 != nullptr ? bias2 : nullptr;
    a.res = g2 != nullptr ? nullptr : res;
    a.y = y;
    a.cout = g.cout;
    a.OHW = g.oh * g.ow;
    a.groups_co = c.groups;
    a.CO = g.cout / c.groups;
    a.CB = a.CO / 32;
    a.PB = (a.OHW + 31) / 32;
    a.n1 = g.cin / 16;
    a.nchunks = a.n1 + (g2 != nullptr ? g2->cin / 16 : 0);
    fastdiv_params(c.groups, &a.m_g, &a.l_g);
    a.wrounds = (a.CB * 128 + 255) / 256;
    a.wpx = c.wpx;
    a.pb_per = c.pb_per;
    a.cb_per = c.cb_per;
    const int rounds = std::max(st.rounds, g2 != nullptr ? st2.rounds : 0);
    a.BUF = rounds * 1024 + a.wrounds * 1024;
    a.WOFF = rounds * 1024;
    const int tq = a.CO * a.OHW / 4;
    a.SPARE = a.CO * a.OHW;
    a.rq = (tq + 255) / 256;
    // residual loads spread over the chunks' iterations (all but the first)
    a.rq_per = (a.rq + std::max(1, a.nchunks - 1) - 1) / std::max(1, a.nchunks - 1);
    a.act = g.act;
    a.res_mode = g2 != nullptr ? CVX_RES_NONE : g.res_mode;
    dim3 grid((unsigned)((long)g.n * c.groups));
    switch (c.kind) {
    case 0: launch_pw<2, 3>(grid, c.lds, s, a, g2 != nullptr); break;
    case 1: launch_pw<1, 3>(grid, c.lds, s, a, g2 != nullptr); break;
    case 2: launch_pw<2, 2>(grid, c.lds, s, a, g2 != nullptr); break;
    case 3: launch_pw<1, 2>(grid, c.lds, s, a, g2 != nullptr); break;
    }
    return hipGetLastError();
}

hipError_t launch_pointwise(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                            const float* bias, const float* res, float* y, hipStream_t s)
{
    return launch_pw_any(g, x, wp, scale, bias, res, nullptr, nullptr, nullptr, nullptr, nullptr, y, s);
}

hipError_t launch_pointwise_pair(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                                 const float* bias, const ConvGeom& g2, const float* x2, const float* wp2,
                                 const float* scale2, const float* bias2, float* y, hipStream_t s)
{
    return launch_pw_any(g, x, wp, scale, bias, nullptr, &g2, x2, wp2, scale2, bias2, y, s);
}

}  // namespace cvx
