// k_igemm_packed.hip -- the dense 1x1 / 3x3 convolution on fp32 matrix cores,
// reading weights that were packed once, at model load, into the matrix
// instruction's operand order.
//
// Implicit GEMM: M = output pixels, N = c_out, K = c_in*kh*kw, computed with
// v_mfma_f32_32x32x2_f32; the folded BatchNorm, the residual and the activation
// are applied to the sums before the single store of each output
// ("YOLO26N Inference Optimisation", "Improvements" #7; "Как я свертки
// ускорял", "А теперь — хардкор на Metal", steps 4-5).
//
// Work decomposition.  A workgroup computes one tile of 32 output channels x
// 32*NT output pixels with eight waves in two roles:
//   * four producer waves (one per SIMD) only move the input: every stage of
//     CPS 16-channel chunks goes global -> LDS with LDS-direct buffer loads,
//     the chunk's staged region row by row;
//   * four consumer waves (one per SIMD) compute: each takes two of a chunk's
//     eight channel pairs (wave w: pairs 2w, 2w+1), loads its own share of the
//     chunk's packed weights global -> registers two stages ahead, reads the
//     input operands from LDS and issues the matrix instructions; the four
//     partial tiles are summed through LDS at the end.
// A unit's vector-memory path takes ~30 clocks per 64-lane load, so a wave that
// issues loads stalls while the queue drains; with the roles split, only the
// producers wait there and the consumers' matrix pipes stay busy.  Three LDS
// buffers and one barrier per stage: at barrier s the producers have landed
// stage s+1 and the consumers have finished stage s-1, so stage s+2 loads while
// stage s computes, and the consumers read the next stage's first operands
// before the barrier that separates the two.
//
// The pixels of a tile are either a run of consecutive output pixels or a block
// of rows x `tc` columns.  Optionally the reduction is split over `splits`
// workgroups; the last one to finish a tile adds the others' partial sums (in
// split order) and applies the epilogue, so the layer is one launch.
//
// Operand order.  The input is the A operand (lane l: pixel l%32 of a block,
// channel 2*pair + l/32) and the weights the B operand (lane l: output channel
// l%32, same channel), so a lane's accumulators hold four runs of four
// consecutive pixels of one output channel: the exchange and the epilogue move
// them 16 bytes at a time.
//
// The 16-pixel tile (NT = 0) halves a workgroup's work for layers
// whose 32-pixel tiles number fewer than the compute units, which would
// otherwise split the reduction and pay its partial-sum round trip.  It runs
// on v_mfma_f32_16x16x4_f32 (half the work of the 32x32x2 instruction in half
// the clocks): consumer wave h takes channels 4h..4h+3 of every chunk (A lane
// l: pixel l%16, channel 4h + l/16) and issues two instructions per tap, one
// per half of the 32 output channels (B lane l: channel 16*half + l%16), two
// chunks to a stage for 3x3 and four for 1x1.  Its weights are a second copy
// of the block in that lane order, stored after the first.
//
// Layouts:
//   * packed weights: [32-row block][16-channel chunk][pair of channel pairs h
//     (4)][slot (5)][lane][4] for 3x3 -- lane l holds output channel
//     32*block + l%32 and input channels of pairs 2h and 2h+1, its 18 taps (9
//     per pair) in five 16-byte slots; [block][chunk][h][lane][2] for 1x1.
//     A (block, chunk) is one contiguous run of 20 KB (3x3) or 2 KB (1x1);
//     consumer wave h reads its quarter straight into registers, already in
//     the operand's lane order.  The weights then repeat in the 16-pixel
//     tile's order: same shape, lane l holding output channel 32*block +
//     16*half + l%16 and input channel 4h + l/16, its values 9*half + tap
//     (3x3) or half (1x1).  ("YOLO26N Inference Optimisation", "NHWC
//     migration", "Weight layout": weights are reordered once for the layout
//     the kernels read.)
//   * inputs: 16 bytes per lane when rows are 16-byte aligned (VEC), else 4;
//     positions outside the image use out-of-range offsets and read as zero, so
//     padding needs no code.
//   * LDS stage buffer: [chunk j][staged input region] (REP floats per chunk).
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

#include <atomic>
#include <chrono>
#include <mutex>
#include <type_traits>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCh = 16;                        // input channels per chunk
constexpr int kSC1 = 16;                       // cache policy: device-coherent (sc1)
constexpr int kSlots3 = 5;                     // 16-byte weight slots per lane per h (3x3)
constexpr int kBCFloats3 = 4 * kSlots3 * 256;  // floats per (block, chunk), 3x3: 5120
constexpr int kBCFloats1 = 4 * 128;            // floats per (block, chunk), 1x1: 512
constexpr int kThreads = 512;                  // four consumer and four producer waves

__device__ __forceinline__ int pdiv(int n, unsigned m, unsigned l)
{
    unsigned hi = __umulhi((unsigned)n, m);
    return (int)((hi + (unsigned)n) >> l);
}

// LDS-direct loads of 16 and 4 bytes per lane (lane i writes dst + i*size).  The
// 16-byte form is gfx950's; kept out of the kernel template so that the host
// pass, which cannot check that form, still emits the kernels' launch stubs.
__device__ __forceinline__ void lds_load16(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 4, off, 0, 0, 0);
}

struct PackedArgs {
    const float* x;
    const float* wp;
    const float* scale;
    const float* bias;
    const float* res;
    float* y;
    float* partial;             // [splits][n][c_out][oh*ow] when splits > 1
    unsigned long long* ctr;    // one arrival counter per output tile when splits > 1
    unsigned long long epoch;   // tag of this launch's arrivals (never 0)
    int n, cin, H, W, cout, stride, pad, OH, OW;
    int tiles_per_img, splits, chunks_per_split, nchunks;
    int tc, tiles_w;
    int run_in_row;             // flat tiles: output width is a multiple of the tile
    unsigned m_tc, l_tc, m_tw, l_tw, m_ow, l_ow;
    int PR, PCW;                // staged rows, LDS floats per staged row
    int EPR, RE, rounds, REP;   // elements per row, elements per chunk, load rounds, LDS floats per chunk
    unsigned m_rc, l_rc, m_c, l_c;  // divide by staged elements per channel, per row
    int step_ci, step_r, step_c;    // 256 staged elements in mixed radix (channel, row, element)
    unsigned m_nb, l_nb, m_sp, l_sp, m_tpi, l_tpi;  // divide by n*tiles, splits, tiles per image
    int tr;                     // output rows of a 2-D tile (BN / tc)
    int spatial;                // workgroup order: pixel tiles slowest (else row blocks slowest)
    int nms;                    // row blocks x splits (row blocks alone when xsplit)
    unsigned m_ms, l_ms;        // divide by nms
    int nv;                     // tiles x row blocks (the persistent form: the workgroups it stands for)
    int xsplit;                 // the slices of a tile run on one XCD and meet in its L2
    unsigned wp_bytes;
    int vout;                   // 16-byte epilogue accesses
    int act, res_mode;
};

constexpr int kRoundsVec = 8, kRoundsScalar = 24;  // most staging rounds per chunk

template <int K, int NT, int CPS, int VEC>
__global__ void __launch_bounds__(kThreads) k_igemm_packed(PackedArgs a)
{
    constexpr int NR = VEC ? kRoundsVec : kRoundsScalar;
    constexpr int KK = K * K;
    constexpr int G = VEC ? 4 : 1;     // floats per staged element
    constexpr bool H16 = NT == 0;      // the 16-pixel tile
    static_assert(!H16 || CPS % 2 == 0, "16-pixel tile: chunks in pairs");
    constexpr int NB = H16 ? 1 : NT;   // input operands a lane reads per tap
    constexpr int BN = H16 ? 16 : 32 * NT;
    constexpr int PITCH = BN + (NT < 4 ? 4 : 0);  // LDS row pitch of the partial-sum exchange
    constexpr int WF = K == 3 ? kBCFloats3 : kBCFloats1;  // weight floats per chunk

    extern __shared__ __attribute__((aligned(16))) float smem[];
    __shared__ int s_last;
    warm_kernargs<sizeof(PackedArgs)>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: addresses stay scalar
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // Workgroup -> (row block, split, image, tile).  Consecutive workgroups are
    // dealt to the eight XCDs in turn, and the tiles are numbered XCD by XCD, so
    // that one XCD's L2 serves a contiguous range of them: with row blocks
    // slowest, the tiles of one row block (same weights) and neighbouring
    // pixels; with pixel tiles slowest, every row block of a band of pixels
    // (same input rows), for layers whose input outweighs their weights.
    int mb, sp, b, tile;
    {
        const unsigned h = blockIdx.x, G8 = gridDim.x;
        const unsigned xcd = h & 7u, i8 = h >> 3, base = G8 >> 3, rem = G8 & 7u;
        int L = (int)(xcd * base + min(xcd, rem) + i8);
        // XCD-local slices: the grid is a multiple of 8 x splits, so each XCD's
        // range of L holds whole groups of `splits` consecutive values, one
        // group per tile; the last groups are padding
        int sl = 0;
        if (a.xsplit) {
            if (L >= a.nv * a.splits) return;
            const int u = pdiv(L, a.m_sp, a.l_sp);
            sl = L - u * a.splits;
            L = u;
        }
        int ms, bt;
        if (a.spatial) {
            bt = pdiv(L, a.m_ms, a.l_ms);
            ms = L - bt * a.nms;
        } else {
            ms = pdiv(L, a.m_nb, a.l_nb);
            bt = L - ms * (a.n * a.tiles_per_img);
        }
        if (a.xsplit) {
            mb = ms;
            sp = sl;
        } else {
            mb = pdiv(ms, a.m_sp, a.l_sp);
            sp = ms - mb * a.splits;
        }
        b = pdiv(bt, a.m_tpi, a.l_tpi);
        tile = bt - b * a.tiles_per_img;
    }
    const int co0 = mb * 32;
    const int OHW = a.OH * a.OW;
    const int HW = a.H * a.W;

    int q0 = 0, q_end = 0, oh_ref, ix0;
    if (a.tc == 0) {
        q0 = tile * BN;
        q_end = min(q0 + BN, OHW);
        oh_ref = pdiv(q0, a.m_ow, a.l_ow);
        // the staged columns follow the host's region: the run's own columns when
        // runs never leave their row, else whole rows
        ix0 = (a.run_in_row ? (q0 - oh_ref * a.OW) * a.stride : 0) - a.pad;
    } else {
        const int band = pdiv(tile, a.m_tw, a.l_tw);
        const int tw = tile - band * a.tiles_w;
        oh_ref = band * a.tr;
        ix0 = tw * a.tc * a.stride - a.pad;
        q0 = tw * a.tc;  // first output column of the tile
    }
    const int gx0 = VEC ? (ix0 & ~3) : ix0;  // staged columns start on a 16-byte boundary
    const int CHF = a.REP;                   // LDS floats per chunk: its staged input region
    const int BUF = CPS * CHF;               // one of three stage buffers

    const int c_begin = sp * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    const int nstages = (c_end - c_begin + CPS - 1) / CPS;

    if (wave >= 4) {
        // ---------------------------------------------------------- producers
        const int ptid = tid - 256;
        const int pw = wave - 4;
        // Staged input elements e = ptid + 256*i -> (channel, row, element of the
        // row) -> byte offset from the chunk's first channel, or kOOB outside the
        // image (or past the region).  Found once by division, then stepped by 256
        // elements in mixed radix with selects (full-rate operations, no branches).
        const int iy0 = oh_ref * a.stride - a.pad;
        const float* xim = a.x + (long)b * a.cin * HW;
        auto chunk_rsrc = [&](int chunk) {
            const int left = chunk < c_end ? min(kCh, a.cin - chunk * kCh) : 0;
            return make_rsrc(xim + (long)chunk * kCh * HW, 4u * (unsigned)(left * HW));
        };
        auto lds_dst = [&](int cbase, int i) {
            return (__attribute__((address_space(3))) void*)(smem + cbase + 256 * G * i + pw * 64 * G);
        };
        auto load_elem = [&](const rsrc_t& rc, int cbase, int i, unsigned off) {
            if constexpr (VEC)
                lds_load16(rc, lds_dst(cbase, i), off);
            else
                lds_load4(rc, lds_dst(cbase, i), off);
        };
        // Stage 0 goes out round by round as the offsets are found, so the
        // first loads do not wait for all of them.
        rsrc_t rc0[CPS];
#pragma unroll
        for (int j = 0; j < CPS; ++j) rc0[j] = chunk_rsrc(c_begin + j);
        unsigned goff[NR];
        {
            int ci = pdiv(ptid, a.m_rc, a.l_rc);
            const int rem = ptid - ci * (a.PR * a.EPR);
            int r = pdiv(rem, a.m_c, a.l_c);
            int c = rem - r * a.EPR;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                goff[i] = kOOB;
                if (i < a.rounds) {
                    const int iy = iy0 + r, gx = gx0 + G * c;
                    const bool ok = (ptid + 256 * i < a.RE) & ((unsigned)iy < (unsigned)a.H) & (gx >= 0) &
                                    (gx + G <= a.W);
                    // 24-bit products: the host keeps H*W below 2^24
                    const unsigned lin = __umul24((unsigned)ci, (unsigned)HW) +
                                         __umul24((unsigned)iy, (unsigned)a.W) + (unsigned)gx;
                    goff[i] = ok ? 4u * lin : kOOB;
                    if (nstages > 0) {
#pragma unroll
                        for (int j = 0; j < CPS; ++j) load_elem(rc0[j], j * CHF, i, goff[i]);
                    }
                    c += a.step_c;
                    const bool cc = c >= a.EPR;
                    c -= cc ? a.EPR : 0;
                    r += a.step_r + (cc ? 1 : 0);
                    const bool rc = r >= a.PR;
                    r -= rc ? a.PR : 0;
                    ci += a.step_ci + (rc ? 1 : 0);
                }
            }
        }
        auto issue_x = [&](int st, int sb) {
#pragma unroll
            for (int j = 0; j < CPS; ++j) {
                int cbase = sb + j * CHF;
                asm volatile("" : "+s"(cbase));
                const rsrc_t rc = chunk_rsrc(c_begin + st * CPS + j);
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if (i >= a.rounds) break;
                    load_elem(rc, cbase, i, goff[i]);
                }
            }
        };
        // Barrier s (s = 0 .. nstages-1) follows the landing of stage s+1; stage
        // s+2 then goes into the buffer of stage s-1, which the consumers have
        // left by barrier s.  (Stage 0 is in flight already.)
        if (nstages > 1) issue_x(1, BUF);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        int sb = 2 * BUF;
        for (int st = 1; st < nstages; ++st) {
            if (st + 1 < nstages) issue_x(st + 1, sb);
            sb = sb == 2 * BUF ? 0 : sb + BUF;
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        // then the consumers' exchange barriers (and the split's two)
        const int tail = a.partial == nullptr ? 2 : 4;
        for (int i = 0; i < tail; ++i) __syncthreads();
        return;
    }

    // -------------------------------------------------------------- consumers
    // Epilogue rows: after the exchange, wave w owns output channels 8w..8w+7 of
    // the tile; lane -> channel 8w + lane/8 and pixel quads 4*(lane%8) + 32*k.
    const int erow = 8 * wave + (lane >> 3);
    const int eco = co0 + erow;
    const bool row_ok = eco < a.cout;
    // the 16-pixel tile's rows have four quads: lanes 8i+4..8i+7 hold none
    const bool quad_ok = !H16 || (lane & 7) < 4;
    const bool single = a.partial == nullptr;
    float sc = 0.0f, bi = 0.0f;

    // LDS offset of each of this lane's pixels (tap 0) in a staged channel
    const int RS = a.PR * a.PCW;  // LDS floats per staged channel
    int loff[NB];
#pragma unroll
    for (int nt = 0; nt < NB; ++nt) {
        const int j = H16 ? (lane & 15) : nt * 32 + l32;
        int oh, ow;
        if (a.tc == 0) {
            const int qc = min(q0 + j, q_end - 1);
            oh = pdiv(qc, a.m_ow, a.l_ow);
            ow = qc - oh * a.OW;
        } else {
            const int jr = pdiv(j, a.m_tc, a.l_tc);
            oh = min(oh_ref + jr, a.OH - 1);
            ow = min(q0 + (j - jr * a.tc), a.OW - 1);
        }
        loff[nt] = (oh - oh_ref) * a.stride * a.PCW + ow * a.stride - a.pad - gx0;
    }

    // 32x32 blocks: one accumulator per pixel block; 16-pixel tile: one per
    // half of the output channels
    typedef typename std::conditional<H16, f32x4, f32x16>::type AccT;
    constexpr int NACC = H16 ? 2 : NT;
    AccT acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < (H16 ? 4 : 16); ++r) acc[i][r] = 0.0f;

    // Matrix work, pair by pair: for each chunk, this wave's weights (its
    // h = wave block of the chunk) and, for each of its two channel pairs, KK
    // taps x NT pixel blocks.  The input operands of the next pair and the
    // weights of the next chunk are read from LDS before the current pair's
    // instructions, also across a stage boundary: the next stage has landed by
    // the current stage's barrier.
    // This wave's weights of a chunk (its h = wave block) go global -> registers
    // in the operand's lane order: for 3x3 four 16-byte loads and an 8-byte one
    // (the last slot's two live taps; loading its padding too would leave two
    // registers the compiler reuses while the load is in flight), for 1x1 one
    // 8-byte load.  A chunk past the split's end reads zeros.
    struct AT {
        f32x4 q[K == 3 ? 4 : 0 + 1];
        f32x2 t;
        __device__ float operator[](int f) const { return K == 3 ? (f < 16 ? q[f / 4][f % 4] : t[f - 16]) : t[f]; }
    };
    const rsrc_t rw = make_rsrc(a.wp, a.wp_bytes);
    const unsigned wrow = 4u * (unsigned)(mb * a.nchunks * WF + wave * (WF / 4)) +
                          (K == 3 ? 16u : 8u) * (unsigned)lane;
    auto load_a = [&](int st, AT (&av)[CPS]) {
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
            const int chunk = c_begin + st * CPS + j;
            const unsigned wo = chunk < c_end ? wrow + 4u * (unsigned)(chunk * WF) : kOOB;
            if constexpr (K == 3) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    av[j].q[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wo + 1024u * s), 0, 0));
                av[j].t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(wo + 4096u), 0, 0));
            } else {
                av[j].t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)wo, 0, 0));
            }
        }
    };
    // Input operands of step q of a stage: a channel pair (q/2 = chunk, q%2 =
    // pair) or, for the 16-pixel tile, a chunk (this wave's four channels).
    auto read_b = [&](int sb, int q, float (&bv)[KK][NB]) {
        // formed here: hoisting these addresses would hold one register per
        // (chunk, pair, buffer)
        int base = H16 ? sb + q * CHF + (4 * wave + (lane >> 4)) * RS
                       : sb + (q >> 1) * CHF + (2 * (2 * wave + (q & 1)) + hi) * RS;
        asm volatile("" : "+v"(base));
        const float* xa = smem + base;
#pragma unroll
        for (int tap = 0; tap < KK; ++tap) {
            const int toff = (tap / K) * a.PCW + (tap % K);
#pragma unroll
            for (int nt = 0; nt < NB; ++nt) bv[tap][nt] = xa[loff[nt] + toff];
        }
    };
    constexpr int NQ = H16 ? CPS : CPS * 2;
    float b0[KK][NB], b1[KK][NB];
    AT a0[CPS], a1[CPS];
    // One stage at buffer `sb`, the next stage's at `nsb` (when `more`), with
    // weight registers `ac`; once its matrix instructions are issued those
    // registers take the weights of stage st+2.  Pair q uses input registers q&1
    // (NQ is even).
    auto stage = [&](int st, AT (&ac)[CPS], int sb, int nsb, bool more) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float (&cur)[KK][NB] = (q & 1) ? b1 : b0;
            float (&nxt)[KK][NB] = (q & 1) ? b0 : b1;
            if (q + 1 < NQ)
                read_b(sb, q + 1, nxt);
            else if (more)
                read_b(nsb, 0, nxt);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (H16) {
#pragma unroll
                for (int tap = 0; tap < KK; ++tap) {
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[tap][0], ac[q][K == 3 ? tap : 0], acc[0], 0,
                                                                  0, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur[tap][0], ac[q][K == 3 ? 9 + tap : 1], acc[1],
                                                                  0, 0, 0);
                }
            } else {
                const int j = q >> 1, pp = q & 1;
#pragma unroll
                for (int tap = 0; tap < KK; ++tap) {
                    const float wv = ac[j][K == 3 ? 9 * pp + tap : pp];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur[tap][nt], wv, acc[nt], 0, 0, 0);
                }
            }
        }
        load_a(st + 2, ac);  // past the end: zeros, issued anyway (keeps wait counts exact)
    };

    // Epilogue geometry of this lane's quads: byte offset of a pixel within the
    // output tensor, or kOOB outside the tile or past c_out.  With `vout` the
    // quad's four pixels are contiguous and 16-byte aligned and move with one
    // access.  Computed where used, so nothing of it is live during the stages.
    const unsigned plane_b = 4u * (unsigned)OHW;
    const unsigned out_bytes = 4u * (unsigned)(a.n * a.cout * OHW);
    auto at = [&](int k, int e) {
        const int p = 32 * k + 4 * (lane & 7) + e;
        bool ok = quad_ok;
        int q;
        if (a.tc == 0) {
            q = q0 + p;
            ok = ok && q < q_end;
        } else {
            const int jr = pdiv(p, a.m_tc, a.l_tc);
            const int oh = oh_ref + jr, ow = q0 + (p - jr * a.tc);
            ok = ok && oh < a.OH && ow < a.OW;
            q = oh * a.OW + ow;
        }
        return ok && row_ok ? (unsigned)(b * a.cout + eco) * plane_b + 4u * (unsigned)q : kOOB;
    };
    auto load_quad = [&](const rsrc_t& r, int k) {
        f32x4 v;
        if (a.vout) {
            v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)at(k, 0), 0, 0));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)at(k, e), 0, 0));
        }
        return v;
    };
    auto store_quad = [&](const rsrc_t& r, int k, f32x4 v) {
        if (a.vout) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)at(k, 0), 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = v[e];  // a scalar copy: bit_cast of a vector element takes element 0
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, f), r, (int)at(k, e), 0, 0);
            }
        }
    };
    f32x4 rv[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) rv[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const bool want_res = a.res_mode != CVX_RES_NONE;
    // without a residual the descriptor is empty and the loads return zeros
    auto load_res = [&]() {
        const rsrc_t rr = make_rsrc(a.res, want_res ? out_bytes : 0u);
#pragma unroll
        for (int k = 0; k < NB; ++k) rv[k] = load_quad(rr, k);
    };

    // Barrier s: the producers have landed stage s+1, this wave has finished
    // stage s-1 (whose buffer now takes stage s+2).  The barrier orders LDS only,
    // so the weight loads in flight stay in flight.
    // Every global load of the loop is issued unconditionally, in a fixed order
    // (weights of stages 0 and 1, the residual, the scale and bias, then stage
    // st+2's weights at the end of stage st), so each wait for a stage's weights
    // leaves the later loads in flight.
    load_a(0, a0);
    load_a(1, a1);
    load_res();
    if (single) {  // needed only by the epilogue: behind the stages' first loads
        const unsigned o = row_ok ? 4u * (unsigned)eco : kOOB;
        sc = bload(make_rsrc(a.scale, 4u * (unsigned)a.cout), o);
        bi = bload(make_rsrc(a.bias, 4u * (unsigned)a.cout), o);
    }
    lds_barrier();
    if (nstages > 0) read_b(0, 0, b0);
    {
        // stages in pairs (weight registers a0, a1), then an odd last one
        int sb = 0, st = 0;
        for (; st + 1 < nstages; st += 2) {
            if (st > 0) lds_barrier();
            const int sb1 = sb == 2 * BUF ? 0 : sb + BUF;
            stage(st, a0, sb, sb1, true);
            lds_barrier();
            const int sb2 = sb1 == 2 * BUF ? 0 : sb1 + BUF;
            stage(st + 1, a1, sb1, sb2, st + 2 < nstages);
            sb = sb2;
        }
        if (st < nstages) {
            if (st > 0) lds_barrier();
            stage(st, a0, sb, sb, false);
        }
    }

    // Partial-sum exchange (the producers have left): every wave writes its
    // BN x 32 tile as [channel][pixel], then wave w sums channels 8w..8w+7 of the
    // four tiles in wave order.  Lane (hi, l32) holds channel l32 and the pixel
    // runs 32*nt + 8*g + 4*hi + 0..3, g = 0..3.
    // (16-pixel tile: lane l holds channels 16*half + l%16, pixels 4*(l/16) + 0..3.)
    __syncthreads();
    if constexpr (H16) {
        float* red = smem + wave * 32 * PITCH + (lane & 15) * PITCH + 4 * (lane >> 4);
#pragma unroll
        for (int half = 0; half < 2; ++half) *reinterpret_cast<f32x4*>(red + 16 * PITCH * half) = acc[half];
    } else {
        float* red = smem + wave * 32 * PITCH + l32 * PITCH + 4 * hi;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f32x4*>(red + 32 * nt + 8 * g) =
                    f32x4{acc[nt][4 * g], acc[nt][4 * g + 1], acc[nt][4 * g + 2], acc[nt][4 * g + 3]};
    }
    __syncthreads();
    f32x4 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        // (lanes without a quad read their neighbour's: inside the row, unused)
        const int off = erow * PITCH + 32 * k + 4 * (lane & (H16 ? 3 : 7));
        v[k] = *reinterpret_cast<const f32x4*>(smem + off);
#pragma unroll
        for (int s = 1; s < 4; ++s) v[k] += *reinterpret_cast<const f32x4*>(smem + s * 32 * PITCH + off);
    }

    if (!single) {
        // Split reduction: publish this slice's sums, count arrivals at the tile's
        // counter, and let the last arrival finish the tile.  Every wave waits for
        // its stores to complete before the workgroup's arrival is counted, so
        // the last arrival reads every slice.  Each tile owns a region of whole
        // cache lines, [slice][32 rows][BN pixels]: no workgroup ever reads a
        // line holding another tile's sums, so no compute unit's own cache can
        // hold a stale copy of one.  With `xsplit` all slices of the tile run
        // on one XCD and the sums meet in its L2 (plain stores and loads);
        // otherwise they are stored and read with device-coherent accesses.
        // Counters carry the launch's epoch in their upper bits, so whatever a
        // counter held before (another launch's value, or anything at all in a
        // fresh workspace) reads as zero arrivals; the last arrival resets it
        // to 0.
        constexpr int SF = 32 * BN;  // floats of one slice of a tile
        const long tix = (long)(mb * a.n + b) * a.tiles_per_img + tile;
        float* const tp = a.partial + tix * a.splits * SF;
        // + 128 bytes per quad k; lanes without a quad store and load nothing
        const int pofs = quad_ok ? 4 * (erow * BN + 4 * (lane & 7)) : 4 * SF;
        const bool dev = !a.xsplit;
        {
            const rsrc_t rps = make_rsrc(tp + (long)sp * SF, 4u * SF);
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const u32x4 q = __builtin_bit_cast(u32x4, v[k]);
                if (dev)
                    __builtin_amdgcn_raw_buffer_store_b128(q, rps, pofs + 128 * k, 0, kSC1);
                else
                    __builtin_amdgcn_raw_buffer_store_b128(q, rps, pofs + 128 * k, 0, 0);
            }
        }
        // whichever workgroup finishes the tile needs these (and the residual,
        // already here): fetched by all, while the stores drain
        {
            const unsigned o = row_ok ? 4u * (unsigned)eco : kOOB;
            sc = bload(make_rsrc(a.scale, 4u * (unsigned)a.cout), o);
            bi = bload(make_rsrc(a.bias, 4u * (unsigned)a.cout), o);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            unsigned long long* c = a.ctr + tix;
            // a counter left by a finished launch reads 0, so the first attempt
            // assumes that and skips a round trip; anything else (an arrival of
            // this launch, or a stale value) comes back in `cur` for the retry
            unsigned long long cur = 0ull;
            unsigned long long before;
            for (;;) {
                before = (cur >> 8) == a.epoch ? (cur & 0xffull) : 0ull;
                const unsigned long long nv = (a.epoch << 8) | (before + 1);
                if (__hip_atomic_compare_exchange_strong(c, &cur, nv, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    break;
            }
            const int last = before + 1 == (unsigned long long)a.splits;
            if (last) __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        f32x4 tot[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) tot[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s = 0; s < a.splits; ++s) {
            const rsrc_t rps = make_rsrc(tp + (long)s * SF, 4u * SF);
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                f32x4 q;
                if (s == sp)
                    q = v[k];
                else if (dev)
                    q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rps, pofs + 128 * k, 0, kSC1));
                else
                    q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rps, pofs + 128 * k, 0, 0));
                tot[k] += q;
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) v[k] = tot[k];
    }

    const rsrc_t ry = make_rsrc(a.y, out_bytes);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        f32x4 z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float t = fmaf(sc, v[k][e], bi);
            if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[k][e];
            t = apply_act_fast(t, a.act);
            if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[k][e];
            z[e] = t;
        }
        store_quad(ry, k, z);
    }
}

// Persistent form (no split, 16-byte staging).  A layer with more tiles than
// the device holds at once runs as fewer workgroups (a multiple of 8), each
// taking tiles h = blockIdx + k*gridDim numbered as the one-tile-per-workgroup
// launch numbers workgroup h (so a tile still lands on the XCD its neighbours
// use).  The stages of a workgroup's tiles form one stream: the producers stage
// the next tile's first chunks while the consumers finish the current tile, so
// a tile's start-up (argument fetch, address set-up, the first stage's landing)
// is paid once per workgroup instead of once per tile.  The partial-sum
// exchange has its own LDS region past the three stage buffers, and costs one
// barrier per tile: tile k ends at stream stage e = (k+1)*ns - 1, and its
// exchange barrier falls between barriers e and e+1 of the stream.
template <int K, int NT, int CPS>
__global__ void __launch_bounds__(kThreads) k_igemm_persist(PackedArgs a)
{
    constexpr int NR = kRoundsVec;
    constexpr int KK = K * K;
    constexpr int G = 4;  // floats per staged element
    constexpr int BN = 32 * NT;
    constexpr int PITCH = BN + (NT < 4 ? 4 : 0);
    constexpr int WF = K == 3 ? kBCFloats3 : kBCFloats1;

    extern __shared__ __attribute__((aligned(16))) float smem[];
    warm_kernargs<sizeof(PackedArgs)>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    const int NV = a.nv;
    const int GR = (int)gridDim.x;
    const int ntiles = (NV - (int)blockIdx.x + GR - 1) / GR;  // >= 1: the host keeps gridDim <= NV
    const int ns = (a.nchunks + CPS - 1) / CPS;               // stages per tile, >= 2 (host)
    const int S = ntiles * ns;
    const int OHW = a.OH * a.OW;
    const int HW = a.H * a.W;
    const int CHF = a.REP;
    const int BUF = CPS * CHF;
    const int XB = 3 * BUF;  // the exchange region

    struct Tile {
        int mb, b, q0, q_end, oh_ref, gx0;
    };
    auto decode = [&](int k) {
        Tile t;
        const unsigned h = blockIdx.x + (unsigned)(k * GR);
        const unsigned xcd = h & 7u, i8 = h >> 3, base = (unsigned)NV >> 3, rem = (unsigned)NV & 7u;
        const int L = (int)(xcd * base + min(xcd, rem) + i8);
        int bt;
        if (a.spatial) {
            bt = pdiv(L, a.m_ms, a.l_ms);
            t.mb = L - bt * a.nms;
        } else {
            t.mb = pdiv(L, a.m_nb, a.l_nb);
            bt = L - t.mb * (a.n * a.tiles_per_img);
        }
        t.b = pdiv(bt, a.m_tpi, a.l_tpi);
        const int tile = bt - t.b * a.tiles_per_img;
        int ix0;
        if (a.tc == 0) {
            t.q0 = tile * BN;
            t.q_end = min(t.q0 + BN, OHW);
            t.oh_ref = pdiv(t.q0, a.m_ow, a.l_ow);
            ix0 = (a.run_in_row ? (t.q0 - t.oh_ref * a.OW) * a.stride : 0) - a.pad;
        } else {
            const int band = pdiv(tile, a.m_tw, a.l_tw);
            const int tw = tile - band * a.tiles_w;
            t.oh_ref = band * a.tr;
            ix0 = tw * a.tc * a.stride - a.pad;
            t.q0 = tw * a.tc;
            t.q_end = 0;
        }
        t.gx0 = ix0 & ~3;
        return t;
    };

    if (wave >= 4) {
        // ---------------------------------------------------------- producers
        const int ptid = tid - 256;
        const int pw = wave - 4;
        // Staged element e = ptid + 256*i of a chunk: its row r and element c of
        // the region, and its offset from the region's origin (channel 0, row
        // iy0, column gx0) -- the same for every tile; the tile adds its origin.
        int er[NR], ec[NR], elin[NR];
        {
            int ci = pdiv(ptid, a.m_rc, a.l_rc);
            const int rem = ptid - ci * (a.PR * a.EPR);
            int r = pdiv(rem, a.m_c, a.l_c);
            int c = rem - r * a.EPR;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const bool live = i < a.rounds && ptid + 256 * i < a.RE;
                er[i] = live ? r : -0x40000000;  // a row no tile has
                ec[i] = c;
                elin[i] = ci * HW + r * a.W + G * c;
                c += a.step_c;
                const bool cc = c >= a.EPR;
                c -= cc ? a.EPR : 0;
                r += a.step_r + (cc ? 1 : 0);
                const bool rc = r >= a.PR;
                r -= rc ? a.PR : 0;
                ci += a.step_ci + (rc ? 1 : 0);
            }
        }
        unsigned goff[NR];
        const float* xim = a.x;
        auto setup = [&](const Tile& t) {
            const int iy0 = t.oh_ref * a.stride - a.pad;
            const int org = iy0 * a.W + t.gx0;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int iy = iy0 + er[i], gx = t.gx0 + G * ec[i];
                const bool ok = ((unsigned)iy < (unsigned)a.H) & (gx >= 0) & (gx + G <= a.W);
                goff[i] = ok ? 4u * (unsigned)(elin[i] + org) : kOOB;
            }
            xim = a.x + (long)t.b * a.cin * HW;
        };
        int ist = 0, it = 0;  // stage (within its tile) and tile of the next issue
        setup(decode(0));
        auto issue = [&](int sb) {
            if (ist == ns) {
                ist = 0;
                ++it;
                setup(decode(it));
            }
#pragma unroll
            for (int j = 0; j < CPS; ++j) {
                const int chunk = ist * CPS + j;
                int cbase = sb + j * CHF;
                // (no scalar pin here)

                const int left = chunk < a.nchunks ? min(kCh, a.cin - chunk * kCh) : 0;
                const rsrc_t rc = make_rsrc(xim + (long)chunk * kCh * HW, 4u * (unsigned)(left * HW));
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if (i >= a.rounds) break;
                    auto* d = (__attribute__((address_space(3))) void*)(smem + cbase + 256 * G * i + pw * 64 * G);
                    lds_load16(rc, d, goff[i]);
                }
            }
            ++ist;
        };
        // Barrier g of the stream follows the landing of stage g+1; stage g+1 goes
        // into the buffer of stage g-2, which the consumers left by barrier g-1.
        issue(0);
        if (S > 1) issue(BUF);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        int sb = 2 * BUF, in_tile = 1;  // in_tile: stream stage g's index within its tile
        for (int g = 1; g < S; ++g) {
            if (g + 1 < S) issue(sb);
            sb = sb == 2 * BUF ? 0 : sb + BUF;
            if (in_tile == ns) {
                lds_barrier();  // the exchange of the tile that ended at stage g-1
                in_tile = 0;
            }
            ++in_tile;
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
        }
        lds_barrier();  // the last tile's exchange
        return;
    }

    // -------------------------------------------------------------- consumers
    const int erow = 8 * wave + (lane >> 3);  // epilogue: channel of the tile, as in k_igemm_packed
    const int RS = a.PR * a.PCW;
    const rsrc_t rsc = make_rsrc(a.scale, 4u * (unsigned)a.cout);
    const rsrc_t rbi = make_rsrc(a.bias, 4u * (unsigned)a.cout);
    const rsrc_t rw = make_rsrc(a.wp, a.wp_bytes);
    const unsigned plane_b = 4u * (unsigned)OHW;
    const unsigned out_bytes = 4u * (unsigned)(a.n * a.cout * OHW);
    const bool want_res = a.res_mode != CVX_RES_NONE;
    const rsrc_t rr = make_rsrc(a.res, want_res ? out_bytes : 0u);
    const rsrc_t ry = make_rsrc(a.y, out_bytes);
    auto wrow_of = [&](int mb) {
        return 4u * (unsigned)(mb * a.nchunks * WF + wave * (WF / 4)) + (K == 3 ? 16u : 8u) * (unsigned)lane;
    };

    Tile tcur = decode(0);
    int kcur = 0;
    unsigned wr_cur = wrow_of(tcur.mb);
    unsigned wr_nxt = ntiles > 1 ? wrow_of(decode(1).mb) : 0u;

    int loff[NT];
    auto set_loff = [&](const Tile& t) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int j = nt * 32 + l32;
            int oh, ow;
            if (a.tc == 0) {
                const int qc = min(t.q0 + j, t.q_end - 1);
                oh = pdiv(qc, a.m_ow, a.l_ow);
                ow = qc - oh * a.OW;
            } else {
                const int jr = pdiv(j, a.m_tc, a.l_tc);
                oh = min(t.oh_ref + jr, a.OH - 1);
                ow = min(t.q0 + (j - jr * a.tc), a.OW - 1);
            }
            loff[nt] = (oh - t.oh_ref) * a.stride * a.PCW + ow * a.stride - a.pad - t.gx0;
        }
    };
    set_loff(tcur);

    // epilogue offset of pixel e of this lane's quad k in tile t, or kOOB
    auto at = [&](const Tile& t, int k, int e) {
        const int p = 32 * k + 4 * (lane & 7) + e;
        bool ok;
        int q;
        if (a.tc == 0) {
            q = t.q0 + p;
            ok = q < t.q_end;
        } else {
            const int jr = pdiv(p, a.m_tc, a.l_tc);
            const int oh = t.oh_ref + jr, ow = t.q0 + (p - jr * a.tc);
            ok = oh < a.OH && ow < a.OW;
            q = oh * a.OW + ow;
        }
        const int eco = t.mb * 32 + erow;
        return ok && eco < a.cout ? (unsigned)(t.b * a.cout + eco) * plane_b + 4u * (unsigned)q : kOOB;
    };
    auto load_quad = [&](const rsrc_t& r, const Tile& t, int k) {
        f32x4 v;
        if (a.vout) {
            v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)at(t, k, 0), 0, 0));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)at(t, k, e), 0, 0));
        }
        return v;
    };
    auto store_quad = [&](const Tile& t, int k, f32x4 v) {
        if (a.vout) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry, (int)at(t, k, 0), 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = v[e];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, f), ry, (int)at(t, k, e), 0, 0);
            }
        }
    };
    float sc, bi;
    f32x4 rv[NT];
    auto load_tile_consts = [&](const Tile& t) {
        const int eco = t.mb * 32 + erow;
        const unsigned o = eco < a.cout ? 4u * (unsigned)eco : kOOB;
        sc = bload(rsc, o);
        bi = bload(rbi, o);
#pragma unroll
        for (int k = 0; k < NT; ++k) rv[k] = load_quad(rr, t, k);
    };

    struct AT {
        f32x4 q[K == 3 ? 4 : 0 + 1];
        f32x2 t;
        __device__ float operator[](int f) const { return K == 3 ? (f < 16 ? q[f / 4][f % 4] : t[f - 16]) : t[f]; }
    };
    // weights of stage s of the tile whose weight row is `wo_base` (kOOB: none)
    auto load_w = [&](unsigned wo_base, bool valid, int s, AT (&av)[CPS]) {
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
            const int chunk = s * CPS + j;
            const unsigned wo = valid && chunk < a.nchunks ? wo_base + 4u * (unsigned)(chunk * WF) : kOOB;
            if constexpr (K == 3) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    av[j].q[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wo + 1024u * q), 0, 0));
                av[j].t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(wo + 4096u), 0, 0));
            } else {
                av[j].t = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)wo, 0, 0));
            }
        }
    };
    auto read_b = [&](int sb, int q, float (&bv)[KK][NT]) {
        const int j = q >> 1, pp = q & 1;
        int base = sb + j * CHF + (2 * (2 * wave + pp) + hi) * RS;
        asm volatile("" : "+v"(base));
        const float* xa = smem + base;
#pragma unroll
        for (int tap = 0; tap < KK; ++tap) {
            const int toff = (tap / K) * a.PCW + (tap % K);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[tap][nt] = xa[loff[nt] + toff];
        }
    };

    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;

    constexpr int NQ = CPS * 2;
    float b0[KK][NT], b1[KK][NT];
    AT a0[CPS], a1[CPS];
    // Stage st of the current tile at buffer sb (the stream's next stage at nsb,
    // read ahead when it belongs to the same tile), weights `ac`; then `ac` takes
    // the weights of the stream's stage two ahead (this tile's, the next tile's,
    // or zeros past the last).
    auto stage = [&](int st, AT (&ac)[CPS], int sb, int nsb, bool more) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float (&cur)[KK][NT] = (q & 1) ? b1 : b0;
            float (&nxt)[KK][NT] = (q & 1) ? b0 : b1;
            const int j = q >> 1, pp = q & 1;
            if (q + 1 < NQ)
                read_b(sb, q + 1, nxt);
            else if (more)
                read_b(nsb, 0, nxt);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tap = 0; tap < KK; ++tap) {
                const float wv = ac[j][K == 3 ? 9 * pp + tap : pp];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(cur[tap][nt], wv, acc[nt], 0, 0, 0);
            }
        }
        if (st + 2 < ns)
            load_w(wr_cur, true, st + 2, ac);
        else
            load_w(wr_nxt, kcur + 1 < ntiles, st + 2 - ns, ac);
    };
    // After the last stage of the current tile: exchange, read the next tile's
    // first operands (its stage landed at the previous barrier), epilogue and
    // stores, then the next tile's constants and residual.
    auto tile_end = [&](int nsb) {
        {
            float* red = smem + XB + wave * 32 * PITCH + l32 * PITCH + 4 * hi;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<f32x4*>(red + 32 * nt + 8 * g) =
                        f32x4{acc[nt][4 * g], acc[nt][4 * g + 1], acc[nt][4 * g + 2], acc[nt][4 * g + 3]};
        }
        lds_barrier();
        f32x4 v[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const int off = XB + erow * PITCH + 32 * k + 4 * (lane & 7);
            v[k] = *reinterpret_cast<const f32x4*>(smem + off);
#pragma unroll
            for (int s = 1; s < 4; ++s) v[k] += *reinterpret_cast<const f32x4*>(smem + s * 32 * PITCH + off);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;
        const bool has_next = kcur + 1 < ntiles;
        Tile tn = tcur;
        if (has_next) {
            tn = decode(kcur + 1);
            set_loff(tn);
            read_b(nsb, 0, b0);
        }
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            f32x4 z;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float t = fmaf(sc, v[k][e], bi);
                if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[k][e];
                t = apply_act_fast(t, a.act);
                if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[k][e];
                z[e] = t;
            }
            store_quad(tcur, k, z);
        }
        if (has_next) {
            tcur = tn;
            load_tile_consts(tcur);
            wr_cur = wr_nxt;
            if (kcur + 2 < ntiles) wr_nxt = wrow_of(decode(kcur + 2).mb);
        }
        ++kcur;
    };

    load_w(wr_cur, true, 0, a0);
    load_w(wr_cur, true, 1, a1);
    load_tile_consts(tcur);
    lds_barrier();
    read_b(0, 0, b0);
    {
        int sb = 0, st = 0;
        for (int g = 0; g < S; g += 2) {
            if (g > 0) lds_barrier();
            {
                const int nsb = sb == 2 * BUF ? 0 : sb + BUF;
                const bool more = st + 1 < ns;
                stage(st, a0, sb, nsb, more);
                if (more) {
                    ++st;
                } else {
                    tile_end(nsb);
                    st = 0;
                }
                sb = nsb;
            }
            if (g + 1 < S) {
                lds_barrier();
                const int nsb = sb == 2 * BUF ? 0 : sb + BUF;
                const bool more = st + 1 < ns;
                stage(st, a1, sb, nsb, more);
                if (more) {
                    ++st;
                } else {
                    tile_end(nsb);
                    st = 0;
                }
                sb = nsb;
            }
        }
    }
}

// One-time weight transform, OIHW -> the packed order above; zero where the row,
// channel or tap does not exist.  `copy` floats in the 32x32 blocks' lane
// order, then as many in the 16-pixel tile's.
__global__ void __launch_bounds__(256) k_pack_weights(const float* __restrict__ w, int cout, int cin,
                                                      int k, int nchunks, long copy, long total,
                                                      float* __restrict__ wp)
{
    const long at = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (at >= total) return;
    const bool h16 = at >= copy;
    const long idx = h16 ? at - copy : at;
    int co, ci, tap = 0;
    bool live = true;
    if (k == 3) {
        const int j = (int)(idx & 3);
        const int lane = (int)((idx >> 2) & 63);
        const long g = idx >> 8;  // (block, chunk, h, slot)
        const int slot = (int)(g % kSlots3);
        const long g2 = g / kSlots3;
        const int h = (int)(g2 & 3);
        const long g3 = g2 >> 2;
        const int chunk = (int)(g3 % nchunks);
        const int blk = (int)(g3 / nchunks);
        const int f = 4 * slot + j;  // 0..19: 9*(pair within h, or half) + tap; 18 and 19 unused
        live = f < 18;
        const int pp = f / 9;
        tap = f - 9 * pp;
        if (h16) {
            co = blk * 32 + 16 * pp + (lane & 15);
            ci = chunk * kCh + 4 * h + (lane >> 4);
        } else {
            co = blk * 32 + (lane & 31);
            ci = chunk * kCh + 2 * (2 * h + pp) + (lane >> 5);
        }
    } else {
        const int j = (int)(idx & 1);
        const int lane = (int)((idx >> 1) & 63);
        const long g = idx >> 7;  // (block, chunk, h)
        const int h = (int)(g & 3);
        const long g3 = g >> 2;
        const int chunk = (int)(g3 % nchunks);
        const int blk = (int)(g3 / nchunks);
        if (h16) {
            co = blk * 32 + 16 * j + (lane & 15);
            ci = chunk * kCh + 4 * h + (lane >> 4);
        } else {
            co = blk * 32 + (lane & 31);
            ci = chunk * kCh + 2 * (2 * h + j) + (lane >> 5);
        }
    }
    float v = 0.0f;
    if (live && co < cout && ci < cin) v = w[((long)co * cin + ci) * (k * k) + tap];
    wp[at] = v;
}

// ------------------------------------------------------------------ host side
// Compiled configurations: NT pixel blocks per wave, and chunks per pipeline
// stage for 3x3 and 1x1.  The tile is 32 x 32*NT; NT = 0 is the 16-pixel tile.
struct PackedKind {
    int nt, cps3, cps1;
};
static constexpr PackedKind kPacked[] = {{1, 1, 4}, {2, 1, 4}, {4, 1, 2}, {0, 2, 4}};
constexpr int kNumPacked = sizeof(kPacked) / sizeof(kPacked[0]);

int packed_num_kinds() { return kNumPacked; }
int packed_chunks_per_stage(int kind, int k) { return k == 3 ? kPacked[kind].cps3 : kPacked[kind].cps1; }
int packed_tile_n(int kind) { return kPacked[kind].nt > 0 ? 32 * kPacked[kind].nt : 16; }

// One copy of the packed weights (one lane order)
long packed_copy_floats(const ConvGeom& g)
{
    const long blocks = (g.cout + 31) / 32;
    const long nchunks = (g.cin + kCh - 1) / kCh;
    return blocks * nchunks * (g.k == 3 ? kBCFloats3 : kBCFloats1);
}

long packed_weight_floats(const ConvGeom& g) { return 2 * packed_copy_floats(g); }

hipError_t launch_pack_weights(const ConvGeom& g, const float* w, float* wp, hipStream_t s)
{
    const long total = packed_weight_floats(g);
    dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(k_pack_weights, grid, dim3(256), 0, s, w, g.cout, g.cin, g.k,
                       (g.cin + kCh - 1) / kCh, packed_copy_floats(g), total, wp);
    return hipGetLastError();
}

void fastdiv_params(int d, unsigned* m, unsigned* l);

long packed_tiles_per_image(const ConvGeom& g, int kind, int tc)
{
    const int bn = packed_tile_n(kind);
    if (tc == 0) return (g.oh * g.ow + bn - 1) / bn;
    const int tr = bn / tc;
    return (long)((g.oh + tr - 1) / tr) * ((g.ow + tc - 1) / tc);
}

// Staged region of a tile: rows, and columns from the first column a tile can
// touch; `vec` widens each row to whole 16-byte elements aligned to the image.
struct Region {
    int pr, pc, pcw, epr, re, rounds, rep;
};

static Region packed_region(const ConvGeom& g, int kind, int tc, bool vec)
{
    Region r;
    const int bn = packed_tile_n(kind);
    if (tc > 0) {
        r.pr = (bn / tc - 1) * g.stride + g.k;
        r.pc = (tc - 1) * g.stride + g.k;
    } else if (g.ow % bn == 0) {  // runs never leave their output row
        r.pr = g.k;
        r.pc = (bn - 1) * g.stride + g.k;
    } else if (bn % g.ow == 0 && bn / g.ow <= g.oh) {  // whole rows per tile
        r.pr = (bn / g.ow - 1) * g.stride + g.k;
        r.pc = g.w + 2 * g.pad;
    } else {
        int rows = (bn - 1) / g.ow + 2;
        rows = rows < g.oh ? rows : g.oh;
        r.pr = (rows - 1) * g.stride + g.k;
        r.pc = g.w + 2 * g.pad;
    }
    if (vec) {
        // The first staged column ix0 = (first output column)*stride - pad starts
        // (ix0 mod 4) floats into its 16-byte element.  For flat runs (which start
        // at a multiple of 32 pixels of a row, or at column 0) and for 2-D tiles
        // whose column step tc*stride is a multiple of 4, that residue is the
        // same for every tile: (-pad) mod 4; otherwise allow for 3.
        const bool fixed = tc == 0 || (tc * g.stride) % 4 == 0;
        const int shift = fixed ? ((-g.pad) & 3) : 3;
        r.pcw = (r.pc + shift + 3) & ~3;
        r.epr = r.pcw / 4;
    } else {
        r.pcw = r.pc;
        r.epr = r.pc;
    }
    r.re = kCh * r.pr * r.epr;
    r.rounds = (r.re + 255) / 256;
    r.rep = r.rounds * 256 * (vec ? 4 : 1);
    return r;
}

void packed_stage_geometry(const ConvGeom& g, int kind, int tc, bool vec, PackedStage* st)
{
    const Region r = packed_region(g, kind, tc, vec);
    st->pr = r.pr;
    st->pcw = r.pcw;
    st->epr = r.epr;
    st->re = r.re;
    st->rounds = r.rounds;
    st->rep = r.rep;
}

static size_t packed_lds(const ConvGeom& g, int kind, const Region& r)
{
    const int nt = kPacked[kind].nt;
    const size_t stage = 3 * (size_t)packed_chunks_per_stage(kind, g.k) * r.rep * sizeof(float);
    const size_t red = (size_t)4 * 32 * (packed_tile_n(kind) + (nt < 4 ? 4 : 0)) * sizeof(float);
    return stage > red ? stage : red;
}

static size_t packed_persist_lds(const ConvGeom& g, int kind, const Region& r)
{
    const int nt = kPacked[kind].nt;
    const size_t stage = 3 * (size_t)packed_chunks_per_stage(kind, g.k) * r.rep * sizeof(float);
    const size_t red = (size_t)4 * 32 * (32 * nt + (nt < 4 ? 4 : 0)) * sizeof(float);
    return stage + red;
}

long packed_num_tiles(const ConvGeom& g, int kind, int tc)
{
    return (long)g.n * packed_tiles_per_image(g, kind, tc) * ((g.cout + 31) / 32);
}

bool packed_persist_fits(const ConvGeom& g, int kind, int tc, int wgs)
{
    // tiles of 32 or 64 pixels (at 128 the compiler keeps the accumulators in scratch)
    if (kind < 0 || kind >= kNumPacked || kPacked[kind].nt > 2 || kPacked[kind].nt < 1) return false;
    if (!packed_tile_fits(g, kind, tc, nullptr)) return false;
    if (g.w % 4 != 0) return false;  // 16-byte staging only
    const int cps = packed_chunks_per_stage(kind, g.k);
    const int nchunks = (g.cin + kCh - 1) / kCh;
    if ((nchunks + cps - 1) / cps < 2) return false;
    const Region r = packed_region(g, kind, tc, true);
    if (packed_persist_lds(g, kind, r) + 256 > kMaxLdsBytes) return false;
    return wgs >= 8 && wgs % 8 == 0 && wgs <= packed_num_tiles(g, kind, tc);
}

bool packed_tile_fits(const ConvGeom& g, int kind, int tc, size_t* lds_bytes)
{
    if (kind < 0 || kind >= kNumPacked) return false;
    if (g.groups != 1 || (g.k != 1 && g.k != 3)) return false;
    const int bn = packed_tile_n(kind);
    if (tc < 0 || (tc > 0 && (tc > bn || bn % tc != 0 || (tc & (tc - 1)) != 0))) return false;
    const long lim = 0x7fffffffL;
    if ((long)g.h * g.w >= (1L << 24)) return false;  // staging offsets use 24-bit products
    if ((long)g.cin * g.h * g.w * 4 >= lim || packed_weight_floats(g) * 4 >= lim ||
        (long)g.n * g.cout * g.oh * g.ow * 4 >= lim)
        return false;
    // both staging forms must fit: which one runs depends on pointer alignment
    size_t lds = 0;
    for (int vec = 0; vec < 2; ++vec) {
        const Region r = packed_region(g, kind, tc, vec != 0);
        if (r.rounds > (vec ? kRoundsVec : kRoundsScalar)) return false;
        const size_t l = packed_lds(g, kind, r);
        if (l + 256 > kMaxLdsBytes) return false;  // leaves room for the static flag
        lds = l > lds ? l : lds;
    }
    if (lds_bytes) *lds_bytes = lds;
    return true;
}

// Split-K partial sums, then one 8-byte arrival counter per output tile.
// Split partial sums: one region per tile, [slice][32 rows][tile pixels].
static size_t packed_partial_bytes(const ConvGeom& g, int kind, int tc, int splits)
{
    const size_t tiles = (size_t)g.n * packed_tiles_per_image(g, kind, tc) * ((g.cout + 31) / 32);
    return (tiles * splits * 32 * packed_tile_n(kind) * sizeof(float) + 255) & ~(size_t)255;
}

size_t packed_workspace_bytes(const ConvGeom& g, int kind, int tc, int splits)
{
    if (splits <= 1) return 0;
    const size_t tiles = (size_t)g.n * packed_tiles_per_image(g, kind, tc) * ((g.cout + 31) / 32);
    return packed_partial_bytes(g, kind, tc, splits) + tiles * sizeof(unsigned long long);
}

// Workgroups per compute unit the compiled kernels allow: each puts two waves
// on every SIMD, and a SIMD holds 512 registers per lane (VGPRs plus
// accumulation registers, as the compiler reports them for gfx950); capped at
// two (LDS).
int packed_occupancy(int kind, int k)
{
    static constexpr int kRegs[2][kNumPacked] = {{56, 81, 123, 51},    // 1x1: NT = 1, 2, 4, 16-pixel tile
                                                 {87, 127, 207, 118}};  // 3x3
    const int regs = kRegs[k == 3 ? 1 : 0][kind];
    const int occ = 512 / regs / 2;
    return occ < 1 ? 1 : occ > 2 ? 2 : occ;
}

// Vector-memory instructions a workgroup issues per chunk: the consumers'
// weight loads (counted as one per 1 KB of packed weights) and the producers'
// four per input round.
int packed_loads_per_chunk(const ConvGeom& g, int kind, int tc)
{
    const bool vec = g.w % 4 == 0;
    const Region r = packed_region(g, kind, tc, vec);
    return (g.k == 3 ? kBCFloats3 : kBCFloats1) / 256 + 4 * r.rounds;
}

int packed_persist_capacity(const ConvGeom& g, int kind, int tc)
{
    // registers per lane of k_igemm_persist as the compiler reports them for
    // gfx950 (1x1: NT = 1, 2; 3x3: NT = 1, 2); two waves per SIMD per workgroup
    static constexpr int kRegs[2][2] = {{71, 113}, {106, 160}};
    const int nt = kPacked[kind].nt;
    if (nt > 2 || nt < 1) return 0;
    const Region r = packed_region(g, kind, tc, true);
    const size_t lds = packed_persist_lds(g, kind, r) + 256;
    int occ = 512 / kRegs[g.k == 3 ? 1 : 0][nt - 1] / 2;
    occ = std::min<int>(std::min(occ, 2), (int)(kMaxLdsBytes / lds));
    return 256 * std::max(occ, 1);
}

void packed_kernel_name(const ConvGeom& g, int kind, char* buf, int len)
{
    const PackedKind& t = kPacked[kind];
    const bool vec = g.w % 4 == 0;  // as launched on 16-byte aligned tensors
    snprintf(buf, len, "cvx::k_igemm_packed<%d, %d, %d, %d>", g.k, t.nt,
             packed_chunks_per_stage(kind, g.k), vec ? 1 : 0);
}

void packed_persist_kernel_name(const ConvGeom& g, int kind, char* buf, int len)
{
    const PackedKind& t = kPacked[kind];
    snprintf(buf, len, "cvx::k_igemm_persist<%d, %d, %d>", g.k, t.nt, packed_chunks_per_stage(kind, g.k));
}

// A fresh tag per split launch.  The first value mixes the clock and an address,
// so a workspace's earlier contents practically never hold the same tag.
unsigned long long packed_next_epoch()
{
    static std::atomic<unsigned long long> ctr{
        (((unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() *
          0x9E3779B97F4A7C15ull) ^
         (unsigned long long)reinterpret_cast<uintptr_t>(&ctr)) >> 9};
    for (;;) {
        const unsigned long long e = ctr.fetch_add(1) & ((1ull << 56) - 1);
        if (e != 0) return e;
    }
}

template <int K, int NT, int CPS, int VEC>
static void launch_packed_cfg(dim3 grid, size_t lds, hipStream_t s, const PackedArgs& a)
{
    hipLaunchKernelGGL((k_igemm_packed<K, NT, CPS, VEC>), grid, dim3(kThreads), lds, s, a);
}

template <int K, int KIND>
static void launch_packed_kind(bool vec, bool persist, dim3 grid, size_t lds, hipStream_t s, const PackedArgs& a)
{
    constexpr PackedKind t = kPacked[KIND];
    constexpr int cps = K == 3 ? t.cps3 : t.cps1;
    if constexpr (t.nt >= 1 && t.nt <= 2) {
        if (persist) {
            hipLaunchKernelGGL((k_igemm_persist<K, t.nt, cps>), grid, dim3(kThreads), lds, s, a);
            return;
        }
    }
    if (vec)
        launch_packed_cfg<K, t.nt, cps, 1>(grid, lds, s, a);
    else
        launch_packed_cfg<K, t.nt, cps, 0>(grid, lds, s, a);
}

template <int K>
static void launch_packed_k(int kind, bool vec, bool persist, dim3 grid, size_t lds, hipStream_t s,
                            const PackedArgs& a)
{
    switch (kind) {
    case 0: launch_packed_kind<K, 0>(vec, persist, grid, lds, s, a); break;
    case 1: launch_packed_kind<K, 1>(vec, persist, grid, lds, s, a); break;
    case 2: launch_packed_kind<K, 2>(vec, persist, grid, lds, s, a); break;
    case 3: launch_packed_kind<K, 3>(vec, persist, grid, lds, s, a); break;
    }
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Placement report: the XCD each workgroup ran on (the XCC_ID hardware
// register, bits 0..3).
__global__ void __launch_bounds__(64) k_workgroup_xcds(int* __restrict__ xcd, int n)
{
    const int id = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);
    if (threadIdx.x == 0 && (int)blockIdx.x < n) xcd[blockIdx.x] = id;
}

hipError_t launch_workgroup_xcds(int* xcd, int n, hipStream_t s)
{
    hipLaunchKernelGGL(k_workgroup_xcds, dim3((unsigned)n), dim3(64), 0, s, xcd, n);
    return hipGetLastError();
}

// Whether the slices of a split tile run on one XCD and reduce through its L2.
// The device deals consecutive workgroups to its XCDs in turn (workgroup i to
// XCD i mod 8, or mod a divisor of 8 on a partition with fewer XCDs), so a
// launch whose workgroups are numbered as the kernel numbers them puts a
// tile's slices on one XCD and one L2.  The first split launch on a device
// checks this once: 2048 workgroups report their XCD, and every workgroup must
// share it with the workgroup whose index agrees modulo 8.  Until the check
// has run (it needs a synchronisation, so it is skipped while the stream is
// being captured into a graph), and wherever it fails, the reduction goes
// through device-coherent memory.  CVX_SPLIT_XCD=0 selects that path always.
__device__ int g_placement[2048];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_split_xcd[kMaxDevices];  // 0 not checked, 1 holds, 2 does not
std::mutex g_split_mu;
}  // namespace

bool packed_split_xcd(hipStream_t s)
{
    const char* e = getenv("CVX_SPLIT_XCD");
    if (e && e[0] == '0') return false;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    const int st = g_split_xcd[dev].load();
    if (st != 0) return st == 1;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    std::lock_guard<std::mutex> lock(g_split_mu);
    if (g_split_xcd[dev].load() != 0) return g_split_xcd[dev].load() == 1;
    constexpr int n = 2048;
    void* dptr = nullptr;
    static int host[n];
    if (hipGetSymbolAddress(&dptr, HIP_SYMBOL(g_placement)) != hipSuccess || dptr == nullptr) return false;
    if (launch_workgroup_xcds(static_cast<int*>(dptr), n, s) != hipSuccess) return false;
    if (hipMemcpyAsync(host, dptr, sizeof host, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return false;
    bool ok = true;
    for (int i = 8; i < n; ++i) ok = ok && host[i] == host[i & 7];
    g_split_xcd[dev].store(ok ? 1 : 2);
    return ok;
}

// Workgroup order of a layer.  Pixel tiles slowest (the default): each XCD
// takes one band of the image and reads that band of the input and all the
// weights; in a forward, every layer gives each XCD the same band, so the
// rows a workgroup reads were mostly written by its own XCD in the layer
// before.  Row blocks slowest: each row block's tiles fill about 8/nmb XCDs,
// so every XCD group reads the whole input and its row blocks' weights, fewer
// fetches for a layer alone whose weights outweigh its input (the detector's
// d, e and g at batch 1), but the detector forward measured 0.6 us slower
// with those three in that order.  CVX_PACKED_ORDER=blocks|pixels overrides.
bool packed_spatial_order(const ConvGeom& g, int nmb)
{
    (void)g;
    (void)nmb;
    const char* e = getenv("CVX_PACKED_ORDER");
    return !(e && e[0] == 'b');
}

hipError_t launch_igemm_packed(const ConvGeom& g, const Plan& p, const float* x, const float* wp,
                               const float* scale, const float* bias, const float* res, float* y,
                               void* ws, hipStream_t s)
{
    const int kind = p.tile.kind;
    const int tc = p.tile.tc;
    const int splits = p.tile.splitk;
    if (!packed_tile_fits(g, kind, tc, nullptr)) return hipErrorInvalidValue;
    if (splits < 1 || (splits > 1 && ws == nullptr)) return hipErrorInvalidValue;
    const bool vec = g.w % 4 == 0 && al16(x);
    const Region r = packed_region(g, kind, tc, vec);
    // the persistent form needs 16-byte staging; otherwise one workgroup per tile
    const bool persist = p.tile.persist > 0 && splits == 1 && vec && packed_persist_fits(g, kind, tc, p.tile.persist);
    const size_t lds = persist ? packed_persist_lds(g, kind, r) : packed_lds(g, kind, r);
    PackedArgs a;
    a.x = x;
    a.wp = kPacked[kind].nt == 0 ? wp + packed_copy_floats(g) : wp;  // the 16-pixel tile's copy
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
    a.tc = tc;
    a.tiles_per_img = (int)packed_tiles_per_image(g, kind, tc);
    a.splits = splits;
    a.nchunks = (g.cin + kCh - 1) / kCh;
    a.chunks_per_split = (a.nchunks + splits - 1) / splits;
    a.tiles_w = tc > 0 ? (g.ow + tc - 1) / tc : 0;
    a.run_in_row = tc == 0 && g.ow % packed_tile_n(kind) == 0;
    fastdiv_params(tc > 0 ? tc : 1, &a.m_tc, &a.l_tc);
    fastdiv_params(a.tiles_w > 0 ? a.tiles_w : 1, &a.m_tw, &a.l_tw);
    fastdiv_params(g.ow, &a.m_ow, &a.l_ow);
    a.PR = r.pr;
    a.PCW = r.pcw;
    a.EPR = r.epr;
    a.RE = r.re;
    a.rounds = r.rounds;
    a.REP = r.rep;
    fastdiv_params(r.pr * r.epr, &a.m_rc, &a.l_rc);
    fastdiv_params(r.epr, &a.m_c, &a.l_c);
    {
        const int rc = r.pr * r.epr;
        a.step_ci = 256 / rc;
        a.step_r = (256 % rc) / r.epr;
        a.step_c = (256 % rc) % r.epr;
    }
    fastdiv_params(g.n * a.tiles_per_img, &a.m_nb, &a.l_nb);
    fastdiv_params(splits, &a.m_sp, &a.l_sp);
    a.xsplit = splits > 1 && packed_split_xcd(s) ? 1 : 0;
    {
        const int nmb = (g.cout + 31) / 32;
        a.nms = a.xsplit ? nmb : nmb * splits;
        fastdiv_params(a.nms, &a.m_ms, &a.l_ms);
        a.spatial = packed_spatial_order(g, nmb) ? 1 : 0;
    }
    fastdiv_params(a.tiles_per_img, &a.m_tpi, &a.l_tpi);
    a.tr = tc > 0 ? packed_tile_n(kind) / tc : 0;
    a.wp_bytes = (unsigned)(packed_copy_floats(g) * 4);
    a.act = g.act;
    a.res_mode = g.res_mode;
    if (splits > 1) {
        a.partial = static_cast<float*>(ws);
        a.ctr = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) +
                                                      packed_partial_bytes(g, kind, tc, splits));
        a.epoch = packed_next_epoch();
    } else {
        a.partial = nullptr;
        a.ctr = nullptr;
        a.epoch = 0;
    }
    // 16-byte epilogue accesses when a lane's quad of pixels is contiguous and aligned
    const bool quads = tc > 0 ? (tc % 4 == 0 && g.ow % 4 == 0) : (g.oh * g.ow) % 4 == 0;
    a.vout = quads && al16(y) && (res == nullptr || al16(res)) && (ws == nullptr || al16(ws)) ? 1 : 0;
    const long tiles = (long)g.n * a.tiles_per_img * ((g.cout + 31) / 32);
    a.nv = (int)tiles;
    // XCD-local slices: a multiple of 8 x splits workgroups (the rest exit at once)
    const long wgs = a.xsplit ? (tiles * splits + 8L * splits - 1) / (8L * splits) * (8L * splits) : tiles * splits;
    dim3 grid((unsigned)(persist ? (long)p.tile.persist : wgs));
    if (g.k == 1)
        launch_packed_k<1>(kind, vec, persist, grid, lds, s, a);
    else
        launch_packed_k<3>(kind, vec, persist, grid, lds, s, a);
    return hipGetLastError();
}

}  // namespace cvx
