// k_chain.hip -- a run of dense 1x1 / 3x3 convolution layers (packed weights,
// folded BatchNorm, activation, residual) as ONE launch.
//
// The pages replay a whole network per inference and count the launch overhead
// and the small kernels between layers against it ("YOLO26N Inference
// Optimisation", "nsys kernel-level breakdown" and "Improvements" #5); one of
// them lists running the whole network in a single launch as the next step
// ("Как я свертки ускорял", "Идеи и следующие шаги", item 3).  At batch 1 a
// detector layer has one round of tiles or less on the chip, so every layer
// launched on its own pays a ramp-up and a drain in which most compute units
// idle.  Here the layers' tiles are one queue of work items, in layer order,
// and a fixed set of persistent workgroups (as many as fit the chip at once)
// takes them in that order: a workgroup's first item is its workgroup index,
// later ones come from an atomic counter.  A tile of layer L+1 starts as soon
// as the rows of layer L it reads are complete, so one layer's tail overlaps
// the next layer's head.
//
// Readiness.  Each layer keeps one counter per output row (and image): a
// finished tile adds, once its stores have completed, its pixels in every row
// it covers, so a row is complete when its counter reaches OW x (row blocks).
// A tile counts its rows before its workgroup waits for anything else.  Before staging
// a tile, the producer waves poll the counters of the input rows its window
// reads (and of its residual rows) with device-coherent loads, a bounded
// number of times.  Items are handed out in layer order and a workgroup
// processes its items in the order it got them, so the unfinished item with
// the smallest index only ever waits for finished items: the wait always ends
// while the workgroups holding earlier items are running (each workgroup's
// first item is its index, so the grid is at most what the device holds at
// once).  If a wait exceeds
// its bound anyway, the workgroup sets an abort word, writes NaN for that
// tile, and every later wait returns at once, so the kernel still drains.
//
// Cross-workgroup data.  Layer outputs are written with device-coherent
// stores (write-through past the XCD's own L2) and inputs and residuals are
// read with device-coherent loads, so a row written on one XCD is read
// correctly on another; a tile's stores have completed (waited on) before its
// rows are counted.  Weights, scales and biases are read-only and cached.
//
// Counter life cycle.  A small kernel launched just before the chain (on the
// same stream, so a captured graph replays it too) zeroes the queue, the
// abort word, the row counters and the split arrival counters; nothing in the
// workspace needs to be valid on entry.  Each row counter has a 128-byte line
// of its own, every tile counts its rows once (the last of its four consumer
// waves to finish its stores does it), and only one producer wave per
// workgroup polls, backing off, while the other three wait on a word in LDS.
//
// Tiles.  Every layer uses 32 output channels x 32 output pixels (a flat run,
// or a 2-D block of tc columns) and the single-layer kernel's division of
// labour: four producer waves stage 16-channel chunks global -> LDS, four
// consumer waves run v_mfma_f32_32x32x2_f32 with weights loaded into
// registers two stages ahead.  Three stage buffers and one barrier per stage
// within a tile; the cross-wave exchange has a region of its own, so the
// producers stage the next tile while the consumers finish the current one.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCh = 16;          // input channels per chunk
constexpr int kSC1 = 16;         // cache policy: device-coherent (sc1)
constexpr int kThreads = 512;    // four consumer and four producer waves
constexpr int kNR = 8;           // most 16-byte staging rounds per chunk
constexpr int kBCF3 = 5120;      // packed weight floats per (block, chunk), 3x3
constexpr int kBCF1 = 512;       // the same, 1x1
constexpr int kPitch = 36;       // LDS row pitch of the partial-sum exchange
constexpr int kExchFloats = 4 * 32 * kPitch;
constexpr int kQueue = 0;        // control word: items handed out past the first gridDim.x
constexpr int kAbort = 1;        // control word: a wait gave up
constexpr int kHdr = 32;         // words before the first row counter
constexpr int kRowStride = 32;   // words between row counters (one 128-byte line each)

}  // namespace

struct ChainLayer {
    const float* x;
    const float* wp;
    const float* scale;
    const float* bias;
    const float* res;
    float* y;
    float* partial;                // [splits][n][cout][OH*OW] when splits > 1
    unsigned* tctr;                // split arrival counter per (row block, image, tile)
    int in_dep, res_dep;           // producer of x / res in the run, or -1 (complete at launch)
    int in_rows, res_rows;         // their first row counter (row index in the control block)
    int out_rows;                  // this layer's first row counter
    int item0;                     // first work item of this layer
    int n, k, cin, H, W, cout, stride, pad, OH, OW;
    int nmb, splits, chunks_per_split, nchunks, tiles_per_img;
    int part_stride;               // floats per split slice of the partials
    int tc, tiles_w, run_in_row, tr;
    unsigned m_tc, l_tc, m_tw, l_tw, m_ow, l_ow;
    int PR, PCW, EPR, RE, rounds, REP;
    unsigned m_rc, l_rc, m_c, l_c;
    int step_ci, step_r, step_c;
    unsigned m_sp, l_sp, m_nmb, l_nmb, m_tpi, l_tpi;
    unsigned wp_bytes;
    unsigned in_target, res_target;  // a producer row is complete at this count
    int act, res_mode;
};

struct ChainArgs {
    ChainLayer L[kChainMax];
    unsigned* ctl;                 // control block (zeroed by k_chain_zero before the launch)
    int nlayers, total_items;
    int buf_floats;                // floats per stage buffer
    unsigned spin_limit;           // polls before a wait gives up
    int stall_layer;               // tests: this layer's inputs never become ready
};

static_assert(sizeof(ChainArgs) <= 4096, "kernel arguments are limited to 4 KB");

namespace {

__device__ __forceinline__ int pdiv(int n, unsigned m, unsigned l)
{
    unsigned hi = __umulhi((unsigned)n, m);
    return (int)((hi + (unsigned)n) >> l);
}

__device__ __forceinline__ void lds_load16_sc1(rsrc_t r, __attribute__((address_space(3))) void* d, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, kSC1);
}

__device__ __forceinline__ unsigned ld_agent(unsigned* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide: lanes 0..31 watch row counters [o0, o0+n0) until each reaches
// t0, lanes 32..63 rows [o1, o1+n1) until t1; polls back off to about 0.5 us
// apart, and the abort word is read every eighth poll.  False when the wait
// gave up (or another one did): the abort word is then set.
__device__ bool wait_rows(const ChainArgs& A, int o0, int n0, unsigned t0, int o1, int n1, unsigned t1)
{
    const int lane = threadIdx.x & 63;
    unsigned* p = nullptr;
    unsigned t = 0;
    if (lane < 32) {
        if (lane < n0) {
            p = A.ctl + kHdr + (o0 + lane) * kRowStride;
            t = t0;
        }
    } else if (lane - 32 < n1) {
        p = A.ctl + kHdr + (o1 + lane - 32) * kRowStride;
        t = t1;
    }
    for (unsigned it = 0;; ++it) {
        const unsigned v = p ? ld_agent(p) : 0u;
        if (__builtin_amdgcn_ballot_w64(v < t) == 0) return true;
        if ((it & 7) == 7 && (ld_agent(A.ctl + kAbort) != 0 || it >= A.spin_limit)) {
            st_agent(A.ctl + kAbort, 1u);
            return false;
        }
        if (it < 16)
            __builtin_amdgcn_s_sleep(2);
        else
            __builtin_amdgcn_s_sleep(16);
    }
}

// Counts a finished tile's rows (wave-wide): lane i < nr adds the tile's
// pixels in row oh0 + i to that row's counter, so a row is complete at
// OW x (row blocks).
__device__ __forceinline__ void signal_rows(const ChainArgs& A, int rows, int nr, int oh0, int q0, int q_end,
                                            int cols, int OW)
{
    const int lane = threadIdx.x & 63;
    if (lane < nr) {
        const int r = oh0 + lane;
        const int pix = q_end >= 0 ? min(q_end, (r + 1) * OW) - max(q0, r * OW) : cols;
        __hip_atomic_fetch_add(A.ctl + kHdr + (rows + lane) * kRowStride, (unsigned)pix, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

struct ChainShared {
    int next[2];       // the item after the current one (by tile parity)
    int go[2];         // producer wave 0's poll result for the tile: tile number + 1 (+ 2^30 if it gave up)
    int fin[2];        // consumer waves whose stores of the tile have completed
    int last;          // split reduction: this workgroup finishes the tile
};

template <int K>
__device__ __forceinline__ void chain_tile(const ChainArgs& A, const ChainLayer& a, int li, int mb, int sp,
                                           int b, int tile, int par, int seq, float* smem, ChainShared& sh)
{
    constexpr int CPS = K == 3 ? 1 : 4;  // chunks per pipeline stage
    constexpr int KK = K * K;
    constexpr int WF = K == 3 ? kBCF3 : kBCF1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    const int co0 = mb * 32;
    const int OHW = a.OH * a.OW;
    const int HW = a.H * a.W;
    int q0, q_end = 0, oh_ref, ix0, oh_last;
    if (a.tc == 0) {
        q0 = tile * 32;
        q_end = min(q0 + 32, OHW);
        oh_ref = pdiv(q0, a.m_ow, a.l_ow);
        ix0 = (a.run_in_row ? (q0 - oh_ref * a.OW) * a.stride : 0) - a.pad;
        oh_last = pdiv(q_end - 1, a.m_ow, a.l_ow);
    } else {
        const int band = pdiv(tile, a.m_tw, a.l_tw);
        const int tw = tile - band * a.tiles_w;
        oh_ref = band * a.tr;
        ix0 = tw * a.tc * a.stride - a.pad;
        q0 = tw * a.tc;
        oh_last = min(oh_ref + a.tr - 1, a.OH - 1);
    }
    const int gx0 = ix0 & ~3;  // staged columns start on a 16-byte boundary
    const int CHF = a.REP;
    const int BUF = A.buf_floats;
    float* exch = smem + 3 * BUF;
    const int c_begin = sp * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    const int nstages = (c_end - c_begin + CPS - 1) / CPS;
    const bool single = a.splits == 1;

    if (wave >= 4) {
        // ---------------------------------------------------------- producers
        const int ptid = tid - 256;
        const int pw = wave - 4;
        const int iy0 = oh_ref * a.stride - a.pad;
        unsigned goff[kNR];
        {
            int ci = pdiv(ptid, a.m_rc, a.l_rc);
            const int rem = ptid - ci * (a.PR * a.EPR);
            int r = pdiv(rem, a.m_c, a.l_c);
            int c = rem - r * a.EPR;
#pragma unroll
            for (int i = 0; i < kNR; ++i) {
                goff[i] = kOOB;
                if (i < a.rounds) {
                    const int iy = iy0 + r, gx = gx0 + 4 * c;
                    const bool ok = (ptid + 256 * i < a.RE) & ((unsigned)iy < (unsigned)a.H) & (gx >= 0) &
                                    (gx + 4 <= a.W);
                    const unsigned lin = __umul24((unsigned)ci, (unsigned)HW) +
                                         __umul24((unsigned)iy, (unsigned)a.W) + (unsigned)gx;
                    goff[i] = ok ? 4u * lin : kOOB;
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
        // The rows this tile reads must be complete before its input is
        // staged: producer wave 0 polls their counters, the other producer
        // waves wait for its word in LDS (tile number + 1, plus 2^30 when the
        // wait gave up and the tile is poisoned).
        if (a.in_dep >= 0 || a.res_dep >= 0) {
            if (pw == 0) {
                int o0 = 0, n0 = 0, o1 = 0, n1 = 0;
                if (a.in_dep >= 0) {
                    const int lo = max(0, oh_ref * a.stride - a.pad);
                    const int hi_ = min(a.H - 1, oh_last * a.stride - a.pad + K - 1);
                    o0 = a.in_rows + b * a.H + lo;
                    n0 = hi_ - lo + 1;
                }
                if (a.res_dep >= 0) {
                    o1 = a.res_rows + b * a.OH + oh_ref;
                    n1 = oh_last - oh_ref + 1;
                }
                const bool stall = li == A.stall_layer;
                const bool ok = wait_rows(A, o0, n0, stall ? 0xffffffffu : a.in_target, o1, n1,
                                          stall ? 0xffffffffu : a.res_target);
                if (lane == 0)
                    __hip_atomic_store(&sh.go[par], seq + 1 + (ok ? 0 : (1 << 30)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                while ((__hip_atomic_load(&sh.go[par], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) &
                        ((1 << 30) - 1)) != seq + 1)
                    __builtin_amdgcn_s_sleep(1);
            }
        } else if (pw == 0 && lane == 0) {
            __hip_atomic_store(&sh.go[par], seq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }

        const float* xim = a.x + (long)b * a.cin * HW;
        auto issue_x = [&](int st, int sb) {
#pragma unroll
            for (int j = 0; j < CPS; ++j) {
                const int chunk = c_begin + st * CPS + j;
                int cbase = sb + j * CHF;
                asm volatile("" : "+s"(cbase));
                const int left = chunk < c_end ? min(kCh, a.cin - chunk * kCh) : 0;
                const rsrc_t rc = make_rsrc(xim + (long)chunk * kCh * HW, 4u * (unsigned)(left * HW));
#pragma unroll
                for (int i = 0; i < kNR; ++i) {
                    if (i >= a.rounds) break;
                    auto* d = (__attribute__((address_space(3))) void*)(smem + cbase + 1024 * i + pw * 256);
                    lds_load16_sc1(rc, d, goff[i]);
                }
            }
        };
        if (nstages > 0) issue_x(0, 0);
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
        // The next work item, taken once this tile's loads are all issued: a
        // workgroup holds an item only from about when it can start it, so a
        // ready item never waits behind a long tile of the same workgroup.
        // The fetch overlaps the consumers' last stage, exchange and epilogue.
        if (tid == 256) {
            const int nx = (int)gridDim.x +
                           (int)__hip_atomic_fetch_add(A.ctl + kQueue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh.next[par] = min(nx, A.total_items);
        }
        // the consumers' exchange barriers (and the split's two)
        const int tail = single ? 2 : 4;
        for (int i = 0; i < tail; ++i) __syncthreads();
        return;
    }

    // -------------------------------------------------------------- consumers
    const int erow = 8 * wave + (lane >> 3);
    const int eco = co0 + erow;
    const bool row_ok = eco < a.cout;
    float sc = 0.0f, bi = 0.0f;

    const int RS = a.PR * a.PCW;
    int loff;
    {
        int oh, ow;
        if (a.tc == 0) {
            const int qc = min(q0 + l32, q_end - 1);
            oh = pdiv(qc, a.m_ow, a.l_ow);
            ow = qc - oh * a.OW;
        } else {
            const int jr = pdiv(l32, a.m_tc, a.l_tc);
            oh = min(oh_ref + jr, a.OH - 1);
            ow = min(q0 + (l32 - jr * a.tc), a.OW - 1);
        }
        loff = (oh - oh_ref) * a.stride * a.PCW + ow * a.stride - a.pad - gx0;
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    struct AT {
        f32x4 q[K == 3 ? 4 : 1];
        f32x2 t;
        __device__ float operator[](int f) const { return K == 3 ? (f < 16 ? q[f / 4][f % 4] : t[f - 16]) : t[f]; }
    };
    const rsrc_t rw = make_rsrc(a.wp, a.wp_bytes);
    const unsigned wrow = 4u * (unsigned)(mb * a.nchunks * WF + wave * (WF / 4)) + (K == 3 ? 16u : 8u) * (unsigned)lane;
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
    auto read_b = [&](int sb, int q, float (&bv)[KK]) {
        const int j = q >> 1, pp = q & 1;
        int base = sb + j * CHF + (2 * (2 * wave + pp) + hi) * RS;
        asm volatile("" : "+v"(base));
        const float* xa = smem + base + loff;
#pragma unroll
        for (int tap = 0; tap < KK; ++tap) bv[tap] = xa[(tap / K) * a.PCW + (tap % K)];
    };
    constexpr int NQ = CPS * 2;
    float b0[KK], b1[KK];
    AT a0[CPS], a1[CPS];
    auto stage = [&](int st, AT (&ac)[CPS], int sb, int nsb, bool more) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float (&cur)[KK] = (q & 1) ? b1 : b0;
            float (&nxt)[KK] = (q & 1) ? b0 : b1;
            const int j = q >> 1, pp = q & 1;
            if (q + 1 < NQ)
                read_b(sb, q + 1, nxt);
            else if (more)
                read_b(nsb, 0, nxt);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tap = 0; tap < KK; ++tap) {
                const float wv = ac[j][K == 3 ? 9 * pp + tap : pp];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(cur[tap], wv, acc, 0, 0, 0);
            }
        }
        load_a(st + 2, ac);
    };

    const unsigned plane_b = 4u * (unsigned)OHW;
    // byte offset of pixel quad k's first pixel in this image's output, or kOOB
    const unsigned img_b = plane_b * (unsigned)a.cout;  // one image's output
    auto at = [&](int e) {
        const int p = 4 * (lane & 7) + e;
        bool ok;
        int q;
        if (a.tc == 0) {
            q = q0 + p;
            ok = q < q_end;
        } else {
            const int jr = pdiv(p, a.m_tc, a.l_tc);
            const int oh = oh_ref + jr, ow = q0 + (p - jr * a.tc);
            ok = oh < a.OH && ow < a.OW;
            q = oh * a.OW + ow;
        }
        return ok && row_ok ? (unsigned)eco * plane_b + 4u * (unsigned)q : kOOB;
    };
    // one image's tensors: output, residual, and the split partial slices
    const long img_off = (long)b * a.cout * OHW;

    load_a(0, a0);
    load_a(1, a1);
    lds_barrier();  // B0: the input (and residual) rows are complete, stage 0 and 1 landed
    const int poison = sh.go[par] >> 30;
    f32x4 rv = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    {
        const bool want_res = a.res_mode != CVX_RES_NONE;
        const rsrc_t rr = make_rsrc(want_res ? a.res + img_off : a.res, want_res ? img_b : 0u);
        rv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)at(0), 0, kSC1));
    }
    if (single) {
        const unsigned o = row_ok ? 4u * (unsigned)eco : kOOB;
        sc = bload(make_rsrc(a.scale, 4u * (unsigned)a.cout), o);
        bi = bload(make_rsrc(a.bias, 4u * (unsigned)a.cout), o);
    }
    if (nstages > 0) read_b(0, 0, b0);
    {
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

    // Partial-sum exchange in a region of its own: wave w writes its 32x32
    // tile as [channel][pixel], then sums channels 8w..8w+7 of the four.
    __syncthreads();
    {
        float* red = exch + wave * 32 * kPitch + l32 * kPitch + 4 * hi;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(red + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
    __syncthreads();
    f32x4 v;
    {
        const int off = erow * kPitch + 4 * (lane & 7);
        v = *reinterpret_cast<const f32x4*>(exch + off);
#pragma unroll
        for (int s = 1; s < 4; ++s) v += *reinterpret_cast<const f32x4*>(exch + s * 32 * kPitch + off);
    }

    if (!single) {
        // As in the single-layer kernel: publish this slice's sums, count the
        // arrivals at the tile's counter (zeroed before the launch), and let
        // the last arrival add the slices in split order.
        {
            const rsrc_t rps = make_rsrc(a.partial + (long)sp * a.part_stride + img_off, img_b);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rps, (int)at(0), 0, kSC1);
            const unsigned o = row_ok ? 4u * (unsigned)eco : kOOB;
            sc = bload(make_rsrc(a.scale, 4u * (unsigned)a.cout), o);
            bi = bload(make_rsrc(a.bias, 4u * (unsigned)a.cout), o);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            unsigned* c = a.tctr + ((mb * a.n + b) * a.tiles_per_img + tile);
            const unsigned before = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh.last = before + 1 == (unsigned)a.splits;
        }
        __syncthreads();
        if (!sh.last) return;
        f32x4 tot = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s2 = 0; s2 < a.splits; ++s2) {
            const rsrc_t rps = make_rsrc(a.partial + (long)s2 * a.part_stride + img_off, img_b);
            tot += s2 == sp ? v
                            : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rps, (int)at(0), 0, kSC1));
        }
        v = tot;
    }

    if (poison) v = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    const rsrc_t ry = make_rsrc(a.y + img_off, img_b);
    f32x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float t = fmaf(sc, v[e], bi);
        if (a.res_mode == CVX_RES_BEFORE_ACT) t += rv[e];
        t = apply_act_fast(t, a.act);
        if (a.res_mode == CVX_RES_AFTER_ACT) t += rv[e];
        z[e] = t;
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, z), ry, (int)at(0), 0, kSC1);
    // Once this wave's stores have completed it checks in; the last of the
    // four consumer waves to do so counts the tile's rows.
    __builtin_amdgcn_s_waitcnt(0);
    int before = 0;
    if (lane == 0) before = __hip_atomic_fetch_add(&sh.fin[par], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before == 3) {
        if (lane == 0) __hip_atomic_store(&sh.fin[par], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        signal_rows(A, a.out_rows + b * a.OH + oh_ref, oh_last - oh_ref + 1, oh_ref, a.tc == 0 ? q0 : 0,
                    a.tc == 0 ? q_end : -1, a.tc == 0 ? 0 : min(a.tc, a.OW - q0), a.OW);
    }
}

}  // namespace

__global__ void __launch_bounds__(kThreads) k_chain(ChainArgs A)
{
    extern __shared__ __attribute__((aligned(16))) float smem[];
    __shared__ ChainShared sh;
    const int tid = threadIdx.x;
    if (tid < 2) {
        sh.go[tid] = 0;
        sh.fin[tid] = 0;
    }
    __syncthreads();
    int item = blockIdx.x, par = 0, seq = 0;
    while (item < A.total_items) {
        int li = 0;
        while (li + 1 < A.nlayers && item >= A.L[li + 1].item0) ++li;
        li = __builtin_amdgcn_readfirstlane(li);
        const ChainLayer& a = A.L[li];
        const int local = item - a.item0;
        const int t1 = pdiv(local, a.m_sp, a.l_sp);
        const int sp = local - t1 * a.splits;
        const int t2 = pdiv(t1, a.m_nmb, a.l_nmb);
        const int mb = t1 - t2 * a.nmb;
        const int b = pdiv(t2, a.m_tpi, a.l_tpi);
        const int tile = t2 - b * a.tiles_per_img;
        if (a.k == 3)
            chain_tile<3>(A, a, li, mb, sp, b, tile, par, seq, smem, sh);
        else
            chain_tile<1>(A, a, li, mb, sp, b, tile, par, seq, smem, sh);
        item = __builtin_amdgcn_readfirstlane(sh.next[par]);
        par ^= 1;
        ++seq;
    }
}

// Zeroes the words a chain launch counts with: the queue and the abort word,
// one counter per (layer, image, output row), one arrival counter per split
// tile.  Launched before every chain launch on the same stream (a kernel, so
// a captured graph replays it too).
__global__ void __launch_bounds__(256) k_chain_zero(unsigned* ctl, int rows, unsigned* tctr, int tctr_words)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < 2) ctl[i] = 0u;
    if (i < rows) ctl[kHdr + i * kRowStride] = 0u;
    if (i < tctr_words) tctr[i] = 0u;
}

// ------------------------------------------------------------------ host side
namespace {

constexpr int kKind = 0;  // the packed kernel's 32 x 32 tile

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

int chain_cps(int k) { return packed_chunks_per_stage(kKind, k); }

// output rows a tile covers at most
int chain_rows_out(const ConvGeom& g, int tc)
{
    if (tc > 0) return 32 / tc;
    return std::min(g.oh, (31 + g.ow - 1) / g.ow + 1);
}

struct DevInfo {
    int cus = 0;
    int per_cu[2] = {0, 0};  // workgroups per compute unit at the two LDS sizes last asked
    size_t lds[2] = {0, 0};
};

}  // namespace

bool chain_layer_fits(const ConvGeom& g, int tc, int* buf_floats)
{
    if (g.groups != 1 || (g.k != 1 && g.k != 3) || g.w_layout != CVX_W_PACKED) return false;
    if (g.w % 4 != 0) return false;  // 16-byte staging
    if (chain_cps(g.k) != (g.k == 3 ? 1 : 4)) return false;
    if (!packed_tile_fits(g, kKind, tc, nullptr)) return false;
    const bool quads = tc > 0 ? (tc % 4 == 0 && g.ow % 4 == 0) : (g.oh * g.ow) % 4 == 0;
    if (!quads) return false;
    const int ro = chain_rows_out(g, tc);
    if ((ro - 1) * g.stride + g.k > 32 || ro > 32) return false;  // rows one wave polls
    PackedStage st;
    packed_stage_geometry(g, kKind, tc, true, &st);
    if (st.rounds > kNR) return false;
    if (buf_floats) *buf_floats = chain_cps(g.k) * st.rep;
    return true;
}

static int chain_tiles_per_image(const ConvGeom& g, int tc) { return (int)packed_tiles_per_image(g, kKind, tc); }

static int chain_rows(const ChainLayerSpec* L, int n)
{
    int r = 0;
    for (int i = 0; i < n; ++i) r += L[i].g.n * L[i].g.oh;
    return r;
}

static int chain_tctr_words(const ChainLayerSpec* L, int n)
{
    int w = 0;
    for (int i = 0; i < n; ++i)
        if (L[i].splits > 1) w += ((L[i].g.cout + 31) / 32) * L[i].g.n * chain_tiles_per_image(L[i].g, L[i].tc);
    return w;
}

// Control block (queue, abort, a 128-byte line per row counter), the split
// arrival counters, then each split layer's partial sums.
size_t chain_workspace_bytes(const ChainLayerSpec* L, int n)
{
    size_t b = round256(((size_t)kHdr + (size_t)chain_rows(L, n) * kRowStride) * sizeof(unsigned));
    b += round256((size_t)chain_tctr_words(L, n) * sizeof(unsigned));
    for (int i = 0; i < n; ++i) {
        const ConvGeom& g = L[i].g;
        if (L[i].splits > 1) b += round256((size_t)L[i].splits * g.n * g.cout * g.oh * g.ow * sizeof(float));
    }
    return b;
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups of k_chain that fit the device at once (persistent grid).
static int chain_capacity(size_t lds)
{
    static std::mutex mu;
    static DevInfo info[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    DevInfo& d = info[dev];
    if (d.cus == 0 && hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    for (int j = 0; j < 2; ++j)
        if (d.lds[j] == lds && d.per_cu[j] > 0) return d.cus * d.per_cu[j];
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_chain, kThreads, lds) != hipSuccess || nb < 1)
        return 0;
    const int j = d.lds[0] == 0 ? 0 : 1;
    d.lds[j] = lds;
    d.per_cu[j] = nb;
    return d.cus * nb;
}

static unsigned env_uint(const char* name, unsigned dflt)
{
    const char* e = getenv(name);
    if (!e || !*e) return dflt;
    return (unsigned)strtoul(e, nullptr, 10);
}

hipError_t launch_chain(const ChainLayerSpec* S, int n, void* ws, hipStream_t s)
{
    if (n < 1 || n > kChainMax || ws == nullptr || !al16(ws)) return hipErrorInvalidValue;
    ChainArgs A;
    memset(&A, 0, sizeof(A));
    char* base = static_cast<char*>(ws);
    A.ctl = reinterpret_cast<unsigned*>(base);
    const int nrows = chain_rows(S, n);
    const int ntctr = chain_tctr_words(S, n);
    size_t off = round256(((size_t)kHdr + (size_t)nrows * kRowStride) * sizeof(unsigned));
    unsigned* tctr = reinterpret_cast<unsigned*>(base + off);
    off += round256((size_t)ntctr * sizeof(unsigned));
    int rows = 0, items = 0, buf = 0, tctr_used = 0;
    int row_off[kChainMax];
    for (int i = 0; i < n; ++i) {
        const ChainLayerSpec& sp = S[i];
        const ConvGeom& g = sp.g;
        int bf = 0;
        if (!chain_layer_fits(g, sp.tc, &bf)) return hipErrorInvalidValue;
        if (!al16(sp.x) || !al16(sp.y) || (sp.res && !al16(sp.res))) return hipErrorInvalidValue;
        if (sp.in_dep >= i || sp.res_dep >= i) return hipErrorInvalidValue;
        buf = std::max(buf, bf);
        ChainLayer& a = A.L[i];
        a.x = sp.x;
        a.wp = sp.wp;
        a.scale = sp.scale;
        a.bias = sp.bias;
        a.res = g.res_mode != CVX_RES_NONE ? sp.res : nullptr;
        a.y = sp.y;
        a.n = g.n;
        a.k = g.k;
        a.cin = g.cin;
        a.H = g.h;
        a.W = g.w;
        a.cout = g.cout;
        a.stride = g.stride;
        a.pad = g.pad;
        a.OH = g.oh;
        a.OW = g.ow;
        a.nmb = (g.cout + 31) / 32;
        a.splits = std::max(1, sp.splits);
        a.nchunks = (g.cin + kCh - 1) / kCh;
        a.chunks_per_split = (a.nchunks + a.splits - 1) / a.splits;
        if ((long)(a.splits - 1) * a.chunks_per_split >= a.nchunks) return hipErrorInvalidValue;
        a.tc = sp.tc;
        a.tiles_per_img = chain_tiles_per_image(g, sp.tc);
        a.tiles_w = sp.tc > 0 ? (g.ow + sp.tc - 1) / sp.tc : 0;
        a.run_in_row = sp.tc == 0 && g.ow % 32 == 0;
        a.tr = sp.tc > 0 ? 32 / sp.tc : 0;
        fastdiv_params(sp.tc > 0 ? sp.tc : 1, &a.m_tc, &a.l_tc);
        fastdiv_params(a.tiles_w > 0 ? a.tiles_w : 1, &a.m_tw, &a.l_tw);
        fastdiv_params(g.ow, &a.m_ow, &a.l_ow);
        PackedStage st;
        packed_stage_geometry(g, kKind, sp.tc, true, &st);
        a.PR = st.pr;
        a.PCW = st.pcw;
        a.EPR = st.epr;
        a.RE = st.re;
        a.rounds = st.rounds;
        a.REP = st.rep;
        fastdiv_params(st.pr * st.epr, &a.m_rc, &a.l_rc);
        fastdiv_params(st.epr, &a.m_c, &a.l_c);
        {
            const int rc = st.pr * st.epr;
            a.step_ci = 256 / rc;
            a.step_r = (256 % rc) / st.epr;
            a.step_c = (256 % rc) % st.epr;
        }
        fastdiv_params(a.splits, &a.m_sp, &a.l_sp);
        fastdiv_params(a.nmb, &a.m_nmb, &a.l_nmb);
        fastdiv_params(a.tiles_per_img, &a.m_tpi, &a.l_tpi);
        a.wp_bytes = (unsigned)(packed_copy_floats(g) * 4);
        a.act = g.act;
        a.res_mode = g.res_mode;
        a.in_dep = sp.in_dep;
        a.res_dep = g.res_mode != CVX_RES_NONE ? sp.res_dep : -1;
        row_off[i] = rows;
        a.out_rows = rows;
        rows += g.n * g.oh;
        a.in_rows = a.in_dep >= 0 ? row_off[a.in_dep] : 0;
        a.res_rows = a.res_dep >= 0 ? row_off[a.res_dep] : 0;
        // a row is complete once every row block has counted its pixels
        a.in_target = a.in_dep >= 0 ? (unsigned)(S[a.in_dep].g.ow * ((S[a.in_dep].g.cout + 31) / 32)) : 0u;
        a.res_target = a.res_dep >= 0 ? (unsigned)(S[a.res_dep].g.ow * ((S[a.res_dep].g.cout + 31) / 32)) : 0u;
        if (a.in_dep >= 0 && (S[a.in_dep].g.oh != g.h || S[a.in_dep].g.ow != g.w || S[a.in_dep].g.n != g.n))
            return hipErrorInvalidValue;
        if (a.res_dep >= 0 && (S[a.res_dep].g.oh != g.oh || S[a.res_dep].g.n != g.n)) return hipErrorInvalidValue;
        a.item0 = items;
        items += g.n * a.tiles_per_img * a.nmb * a.splits;
        a.part_stride = g.n * g.cout * g.oh * g.ow;
        if (a.splits > 1) {
            a.partial = reinterpret_cast<float*>(base + off);
            off += round256((size_t)a.splits * a.part_stride * sizeof(float));
            a.tctr = tctr + tctr_used;
            tctr_used += a.nmb * g.n * a.tiles_per_img;
        }
    }
    A.nlayers = n;
    A.total_items = items;
    A.buf_floats = buf;
    A.spin_limit = env_uint("CVX_CHAIN_SPIN", 1u << 18);
    {
        const char* e = getenv("CVX_CHAIN_STALL");
        A.stall_layer = e && *e ? atoi(e) : -1;
    }
    const size_t lds = ((size_t)3 * buf + kExchFloats) * sizeof(float);
    if (lds + 256 > kMaxLdsBytes) return hipErrorInvalidValue;
    const int cap = chain_capacity(lds);
    if (cap < 1) return hipErrorInvalidValue;
    // CVX_CHAIN_WGS caps the persistent grid (tuning)
    const int grid = std::min(std::min(items, cap), (int)env_uint("CVX_CHAIN_WGS", (unsigned)cap));
    const int zn = std::max(std::max(nrows, ntctr), 2);
    hipLaunchKernelGGL(k_chain_zero, dim3((unsigned)((zn + 255) / 256)), dim3(256), 0, s, A.ctl, nrows, tctr, ntctr);
    hipLaunchKernelGGL(k_chain, dim3((unsigned)grid), dim3(kThreads), lds, s, A);
    return hipGetLastError();
}

}  // namespace cvx
