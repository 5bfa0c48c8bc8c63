// k_igemm_packed.hip -- the dense 1x1 / 3x3 implicit-GEMM kernel reading weights
// that were packed once, at model load, into the matrix cores' operand order.
//
// Same computation as k_igemm.hip (M = c_out, N = output pixels, K = c_in*kh*kw on
// fp32 MFMA 32x32x2, folded BN / residual / activation in the epilogue); what
// differs is how operands reach the matrix cores:
//   * weights: a one-time transform (cvx_pack_weights) lays them out as
//       [32-row block][16-channel chunk][channel pair][tap quad][lane][4]
//     where lane l holds output channel 32*block + l%32 and input channel
//     16*chunk + 2*pair + l/32 -- exactly the A-operand lane layout of
//     v_mfma_f32_32x32x2_f32.  Each wave loads its A operands straight into
//     registers with coalesced 16-byte loads (1 KB per wave instruction); no LDS
//     traffic and no address arithmetic per element.  ("YOLO26N Inference
//     Optimisation", "NHWC migration", "Weight layout": weights are reordered
//     once at load time for the layout the kernels read.)
//   * inputs: the staged region (as in k_igemm.hip) goes global -> LDS with
//     LDS-direct buffer loads (no register round trip, no LDS write
//     instructions); out-of-range offsets deliver zeros, so padding is free.
//   * two LDS buffers and two register sets: the loads for chunk i+1 are issued
//     before the MFMAs of chunk i, and one barrier per chunk orders the buffers.
#include <stdio.h>

#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int pdiv(int n, unsigned m, unsigned l)
{
    unsigned hi = __umulhi((unsigned)n, m);
    return (int)((hi + (unsigned)n) >> l);
}

struct PackedArgs {
    const float* x;
    const float* wp;      // packed weights
    const float* scale;
    const float* bias;
    const float* res;
    float* y;
    float* partial;
    int cin, H, W, cout, stride, pad, OH, OW;
    int tiles_per_img, chunks_per_split, nchunks;
    int tc, tiles_w;
    unsigned m_tc, l_tc;
    unsigned m_tpi, l_tpi;   // fast division by tiles_per_img
    unsigned m_tw, l_tw;     // fast division by tiles_w (2-D tiles)
    int step_ci, step_r, step_c;  // 256 in the mixed radix (channel, row, column)
    int PR, PC;
    unsigned m_rc, l_rc, m_c, l_c, m_ow, l_ow;
    unsigned wp_bytes;
    int act, res_mode;
};

// Floats of one (block, chunk, pair) group of packed weights.
template <int K>
constexpr int pair_floats()
{
    return K == 3 ? 3 * 64 * 4 : 64;
}

template <int BM, int BN, int WM, int WN, int WK, int K, int NPX, int CPS>
__global__ void __launch_bounds__(256) k_igemm_packed(PackedArgs a)
{
    static_assert(WM * WN * WK == 4, "four waves per workgroup");
    constexpr int TM = BM / WM, TN = BN / WN;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile is made of 32x32 blocks");
    constexpr int MT = TM / 32, NT = TN / 32;
    constexpr int KK = K * K;
    constexpr int CK = 16;
    constexpr int PAIRS = CK / 2;
    static_assert(PAIRS % WK == 0, "channel pairs split evenly over WK waves");
    constexpr int PPW = PAIRS / WK;           // pairs per wave per chunk
    constexpr int TQ = K == 3 ? 3 : 1;        // 16-byte groups per pair (K=3)
    constexpr int PF = pair_floats<K>();

    extern __shared__ float smem[];

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
    const int b = pdiv(blockIdx.x, a.m_tpi, a.l_tpi);
    const int tile = blockIdx.x - b * a.tiles_per_img;
    const int co0 = blockIdx.y * BM;

    int q0 = 0, q_end = 0, oh_ref, ix0;
    if (a.tc == 0) {
        q0 = tile * BN;
        q_end = min(q0 + BN, OHW);
        oh_ref = pdiv(q0, a.m_ow, a.l_ow);
        const int ow_a = q0 - oh_ref * a.OW;
        const int oh_b = pdiv(q_end - 1, a.m_ow, a.l_ow);
        ix0 = (oh_ref == oh_b ? ow_a * a.stride : 0) - a.pad;
    } else {
        const int band = pdiv(tile, a.m_tw, a.l_tw);
        const int tw = tile - band * a.tiles_w;
        oh_ref = band * (BN / a.tc);
        ix0 = tw * a.tc * a.stride - a.pad;
        q0 = tw * a.tc;  // first output column of the tile
    }
    const int iy0 = oh_ref * a.stride - a.pad;
    const int RC = a.PR * a.PC;
    const int RE = CK * RC;
    const int REP = (RE + 255) & ~255;  // LDS pitch of one staged chunk
    const int BUF = CPS * REP;          // floats of one stage buffer

    // Input slots: element e = tid + 256*i of the staged region, as a byte offset
    // from the chunk's first channel plane within this image; kOOB (reads as 0)
    // outside the image or past the region.  Channels past c_in fall outside the
    // image's descriptor and read as 0 too.  (channel, row, column) of e is found
    // once and then stepped by 256 in mixed radix; rounds wholly past the region
    // are skipped (uniform).
    unsigned goff[NPX];
    {
        int ci = pdiv(tid, a.m_rc, a.l_rc);
        const int rem = tid - ci * RC;
        int r = pdiv(rem, a.m_c, a.l_c);
        int c = rem - r * a.PC;
#pragma unroll
        for (int i = 0; i < NPX; ++i) {
            goff[i] = kOOB;
            if (256 * i < RE) {
                const int e = tid + 256 * i;
                const int iy = iy0 + r, ix = ix0 + c;
                if (e < RE && iy >= 0 && iy < a.H && ix >= 0 && ix < a.W)
                    goff[i] = 4u * (unsigned)(ci * HW + iy * a.W + ix);
                c += a.step_c;
                const bool cc = c >= a.PC;
                c -= cc ? a.PC : 0;
                r += a.step_r + (cc ? 1 : 0);
                const bool rc = r >= a.PR;
                r -= rc ? a.PR : 0;
                ci += a.step_ci + (rc ? 1 : 0);
            }
        }
    }
    const rsrc_t rx = make_rsrc(a.x + (long)b * a.cin * HW, 4u * (unsigned)(a.cin * HW));
    const rsrc_t rw = make_rsrc(a.wp, a.wp_bytes);
    // packed-weight byte offset of (row block mt, chunk 0, pair jp) for this lane
    unsigned aoff[MT][PPW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int jp = 0; jp < PPW; ++jp) {
            const int blk = (co0 + wm0) / 32 + mt;
            const int pair = wk + WK * jp;
            aoff[mt][jp] = 4u * (unsigned)(((blk * a.nchunks) * PAIRS + pair) * PF +
                                           (K == 3 ? lane * 4 : lane));
        }
    const unsigned chunk_stride_b = 4u * (unsigned)(PAIRS * PF);

    // A operands: two register sets of one stage (CPS chunks) each
    f32x4 A0[CPS][MT][PPW][TQ], A1[CPS][MT][PPW][TQ];
    float S0[CPS][MT][PPW], S1[CPS][MT][PPW];  // K == 1

    const int c_begin = blockIdx.z * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);
    const int nstages = (c_end - c_begin + CPS - 1) / CPS;

    // Load operations of one stage, addressed by a compile-time index `op`: the
    // A loads (NA_ST of them) first, then the input rounds (CPS * NPX, rounds
    // wholly past the region skipped by a uniform branch).  A chunk past the
    // split's end loads through out-of-range offsets: zero weights and zero
    // inputs, so the MFMAs need no branches.
    constexpr int NA_C = K == 3 ? MT * PPW * TQ : MT * PPW;  // A loads per chunk
    constexpr int NA_ST = CPS * NA_C;
    constexpr int NOPS = NA_ST + CPS * NPX;
    auto load_op = [&](int op, int stage, int buf, auto& A, auto& S) {
        if (op < NA_ST) {
            const int j = op / NA_C;
            const int r0 = op % NA_C;
            const int chunk = c_begin + stage * CPS + j;
            const unsigned cb = chunk < c_end ? (unsigned)chunk * chunk_stride_b : kOOB;
            if constexpr (K == 3) {
                const int tq = r0 % TQ, jp = (r0 / TQ) % PPW, mt = r0 / (TQ * PPW);
                A[j][mt][jp][tq] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rw, (int)(((aoff[mt][jp] + 4u * 256u * tq) | (cb & kOOB)) + (cb & ~kOOB)),
                               0, 0));
            } else {
                const int jp = r0 % PPW, mt = r0 / PPW;
                S[j][mt][jp] = bload(rw, (aoff[mt][jp] | (cb & kOOB)) + (cb & ~kOOB));
            }
        } else {
            const int j = (op - NA_ST) / NPX;
            const int i = (op - NA_ST) % NPX;
            if (256 * i < RE) {
                const int chunk = c_begin + stage * CPS + j;
                const unsigned xb = chunk < c_end ? 4u * (unsigned)(chunk * CK * HW) : kOOB;
                float* dst = smem + buf * BUF + j * REP + wave * 64 + 256 * i;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (__attribute__((address_space(3))) void*)dst, 4,
                    (goff[i] | (xb & kOOB)) + (xb & ~kOOB), 0, 0, 0);
            }
        }
    };
    auto issue = [&](int stage, int buf, auto& A, auto& S) {
#pragma unroll
        for (int op = 0; op < NOPS; ++op) load_op(op, stage, buf, A, S);
    };

    // the first stage's loads go out before the rest of the set-up
    if (nstages > 0) issue(0, 0, A0, S0);

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
            oh = pdiv(qc, a.m_ow, a.l_ow);
            ow = qc - oh * a.OW;
        } else {
            const int jr = pdiv(j, a.m_tc, a.l_tc);
            oh = oh_ref + jr;
            ow = q0 + (j - jr * a.tc);
            ok = oh < a.OH && ow < a.OW;
            oh = min(oh, a.OH - 1);
            ow = min(ow, a.OW - 1);
        }
        loff[nt] = (oh - oh_ref) * a.stride * a.PC + ow * a.stride - a.pad - ix0;
        qout[nt] = ok ? oh * a.OW + ow : -1;
    }

    f32x16 acc[2][MT][NT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[h][mt][nt][r] = 0.0f;

    // One stage's MFMAs.  The B operands of the next channel pair are read from
    // LDS before the current pair's MFMAs are issued (the scheduling barrier keeps
    // them there), so LDS latency hides behind matrix work; taps alternate between
    // two accumulator chains.
    constexpr int NPAIR = CPS * PPW;
    auto read_b = [&](int buf, int q, float (&bv)[KK][NT]) {
        const int j = q / PPW, jp = q % PPW;
        const int ci = 2 * (wk + WK * jp) + hi;
        const float* xa = smem + buf * BUF + j * REP + ci * RC;
#pragma unroll
        for (int tap = 0; tap < KK; ++tap) {
            const int toff = (tap / K) * a.PC + (tap % K);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bv[tap][nt] = xa[loff[nt] + toff];
        }
    };
    auto compute = [&](int buf, auto& A, auto& S) {
        float b0[KK][NT], b1[KK][NT];
        read_b(buf, 0, b0);
#pragma unroll
        for (int q = 0; q < NPAIR; ++q) {
            float (&cur)[KK][NT] = (q & 1) ? b1 : b0;
            float (&nxt)[KK][NT] = (q & 1) ? b0 : b1;
            if (q + 1 < NPAIR) read_b(buf, q + 1, nxt);
            __builtin_amdgcn_sched_barrier(0);
            const int j = q / PPW, jp = q % PPW;
#pragma unroll
            for (int tap = 0; tap < KK; ++tap)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    float av;
                    if constexpr (K == 3)
                        av = A[j][mt][jp][tap / 4][tap % 4];
                    else
                        av = S[j][mt][jp];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        f32x16& c = acc[(tap + q) & 1][mt][nt];
                        c = __builtin_amdgcn_mfma_f32_32x32x2f32(av, cur[tap][nt], c, 0, 0, 0);
                    }
                }
        }
    };

    // Epilogue operands are independent of the reduction: issue their loads with
    // the first stage so they share its memory round trip.
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
    float sc[MT][16], bi[MT][16], rv[MT][NT][16];
    const bool final_pass = a.partial == nullptr;
    if (final_pass) {
        const rsrc_t rsb = make_rsrc(a.scale, 4u * (unsigned)a.cout);
        const rsrc_t rbb = make_rsrc(a.bias, 4u * (unsigned)a.cout);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = co0 + wm0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                const unsigned o = co < a.cout ? 4u * (unsigned)co : kOOB;
                sc[mt][r] = bload(rsb, o);
                bi[mt][r] = bload(rbb, o);
            }
        if (a.res_mode != CVX_RES_NONE) {
            const rsrc_t rr = make_rsrc(a.res, out_bytes);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        rv[mt][nt][r] =
                            bload(rr, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB));
        }
    }

    // Stages alternate between (LDS buffer 0, register set 0) and (1, 1).  Each
    // step: wait for this stage's loads, barrier (its LDS data visible to all
    // waves; every wave done with the other buffer), issue the next stage's loads
    // into the other buffer/set, then run this stage's MFMAs.
    for (int st = 0; st < nstages; st += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (st + 1 < nstages) issue(st + 1, 1, A1, S1);
        compute(0, A0, S0);
        if (st + 1 >= nstages) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (st + 2 < nstages) issue(st + 2, 0, A0, S0);
        compute(1, A1, S1);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[0][mt][nt] += acc[1][mt][nt];

    if constexpr (WK > 1) {
        __syncthreads();
        float* red = smem;
        constexpr int SLAB = MT * NT * 16 * 64;
        if (wk > 0) {
            float* d = red + (wmn * (WK - 1) + wk - 1) * SLAB;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d[((mt * NT + nt) * 16 + r) * 64 + lane] = acc[0][mt][nt][r];
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
                        acc[0][mt][nt][r] += src[((mt * NT + nt) * 16 + r) * 64 + lane];
        }
    }

    // epilogue: rows past c_out and pixels outside the tile use kOOB offsets
    if (!final_pass) {
        const rsrc_t rp = make_rsrc(a.partial + (long)blockIdx.z * (out_bytes / 4), out_bytes);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    bstore(rp, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB), acc[0][mt][nt][r]);
        return;
    }
    const rsrc_t ry = make_rsrc(a.y, out_bytes);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float z = fmaf(sc[mt][r], acc[0][mt][nt][r], bi[mt][r]);
                if (a.res_mode == CVX_RES_BEFORE_ACT) z += rv[mt][nt][r];
                z = apply_act_fast(z, a.act);
                if (a.res_mode == CVX_RES_AFTER_ACT) z += rv[mt][nt][r];
                bstore(ry, (rowoff[mt][r] | (qb[nt] & kOOB)) + (qb[nt] & ~kOOB), z);
            }
}

// One-time weight transform: OIHW -> [32-row block][16-channel chunk][pair]
// [tap quad][lane][4] (3x3) or [block][chunk][pair][lane] (1x1); zero where the
// row, channel or tap does not exist.
__global__ void __launch_bounds__(256) k_pack_weights(const float* __restrict__ w, int cout, int cin,
                                                      int k, int nchunks, long total,
                                                      float* __restrict__ wp)
{
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int kk = k * k;
    int co, ci, tap;
    if (k == 3) {
        const int j = (int)(idx & 3);
        const int lane = (int)((idx >> 2) & 63);
        const long g = idx >> 8;  // (block, chunk, pair, tq)
        const int tq = (int)(g % 3);
        const long g2 = g / 3;
        const int pair = (int)(g2 % 8);
        const long g3 = g2 / 8;
        const int chunk = (int)(g3 % nchunks);
        const int blk = (int)(g3 / nchunks);
        co = blk * 32 + (lane & 31);
        ci = chunk * 16 + 2 * pair + (lane >> 5);
        tap = tq * 4 + j;
    } else {
        const int lane = (int)(idx & 63);
        const long g = idx >> 6;
        const int pair = (int)(g % 8);
        const long g3 = g / 8;
        const int chunk = (int)(g3 % nchunks);
        const int blk = (int)(g3 / nchunks);
        co = blk * 32 + (lane & 31);
        ci = chunk * 16 + 2 * pair + (lane >> 5);
        tap = 0;
    }
    float v = 0.0f;
    if (co < cout && ci < cin && tap < kk) v = w[((long)co * cin + ci) * kk + tap];
    wp[idx] = v;
}

// ------------------------------------------------------------------ host side
struct PackedKind {
    int bm, bn, wm, wn, wk, npx;
    int cps3, cps1;  // chunks per pipeline stage for 3x3 and 1x1
};
static constexpr PackedKind kPacked[] = {
    {32, 32, 1, 1, 4, 24, 2, 8},
    {32, 64, 1, 2, 2, 24, 2, 8},
    {64, 64, 2, 2, 1, 24, 1, 4},
    {64, 128, 2, 2, 1, 24, 0, 4},  // 1x1 only (a 3x3 stage would not fit the registers)
};

int packed_chunks_per_stage(int tile, int k) { return k == 3 ? kPacked[tile].cps3 : kPacked[tile].cps1; }
constexpr int kNumPacked = sizeof(kPacked) / sizeof(kPacked[0]);

void packed_kernel_name(const ConvGeom& g, int tile, char* buf, int len)
{
    const PackedKind& t = kPacked[tile];
    snprintf(buf, len, "cvx::k_igemm_packed<%d, %d, %d, %d, %d, %d, %d, %d>", t.bm, t.bn, t.wm, t.wn,
             t.wk, g.k, t.npx, packed_chunks_per_stage(tile, g.k));
}

long packed_weight_floats(const ConvGeom& g)
{
    const long blocks = (g.cout + 31) / 32;
    const long nchunks = (g.cin + 15) / 16;
    return blocks * nchunks * 8 * (g.k == 3 ? 3 * 64 * 4 : 64);
}

hipError_t launch_pack_weights(const ConvGeom& g, const float* w, float* wp, hipStream_t s)
{
    const long total = packed_weight_floats(g);
    dim3 grid((unsigned)((total + 255) / 256));
    hipLaunchKernelGGL(k_pack_weights, grid, dim3(256), 0, s, w, g.cout, g.cin, g.k,
                       (g.cin + 15) / 16, total, wp);
    return hipGetLastError();
}

// the region geometry and tile counts are shared with the OIHW kernel
void igemm_region(const ConvGeom& g, int bn, int tc, int* pr, int* pc);
void fastdiv_params(int d, unsigned* m, unsigned* l);

bool packed_tile_fits(const ConvGeom& g, int tile, int tc, size_t* lds_bytes)
{
    if (packed_chunks_per_stage(tile, g.k) == 0) return false;
    if (!igemm_tile_fits(g, tile, tc, nullptr)) return false;
    const PackedKind& t = kPacked[tile];
    int pr, pc;
    igemm_region(g, t.bn, tc, &pr, &pc);
    const long re = (long)16 * pr * pc;
    if (re > 256L * t.npx) return false;
    if (packed_weight_floats(g) * 4 >= 0x7fffffffL) return false;
    const long rep = (re + 255) / 256 * 256;
    const size_t stage = 2 * (size_t)packed_chunks_per_stage(tile, g.k) * rep * sizeof(float);
    const size_t red = t.wk > 1 ? (size_t)(4 / t.wk) * (t.wk - 1) * (t.bm / t.wm / 32) *
                                      (t.bn / t.wn / 32) * 16 * 64 * sizeof(float)
                                : 0;
    const size_t lds = stage > red ? stage : red;
    if (lds > kMaxLdsBytes) return false;
    if (lds_bytes) *lds_bytes = lds;
    return true;
}

template <int K, int TILE>
static void launch_packed_tile(dim3 grid, size_t lds, hipStream_t s, const PackedArgs& a)
{
    constexpr PackedKind t = kPacked[TILE];
    constexpr int cps = K == 3 ? t.cps3 : t.cps1;
    if constexpr (cps == 0) return;
    else
    hipLaunchKernelGGL((k_igemm_packed<t.bm, t.bn, t.wm, t.wn, t.wk, K, t.npx, cps>), grid,
                       dim3(256), lds, s, a);
}

template <int K>
static void launch_packed_k(int tile, dim3 grid, size_t lds, hipStream_t s, const PackedArgs& a)
{
    switch (tile) {
    case 0: launch_packed_tile<K, 0>(grid, lds, s, a); break;
    case 1: launch_packed_tile<K, 1>(grid, lds, s, a); break;
    case 2: launch_packed_tile<K, 2>(grid, lds, s, a); break;
    case 3: launch_packed_tile<K, 3>(grid, lds, s, a); break;
    }
}

hipError_t launch_igemm_packed(const ConvGeom& g, const Plan& p, const float* x, const float* wp,
                               const float* scale, const float* bias, const float* res, float* y,
                               void* ws, hipStream_t s)
{
    const int tile = p.tile.kind;
    if (tile < 0 || tile >= kNumPacked || (g.k != 1 && g.k != 3)) return hipErrorInvalidValue;
    size_t lds = 0;
    if (!packed_tile_fits(g, tile, p.tile.tc, &lds)) return hipErrorInvalidValue;
    const PackedKind& t = kPacked[tile];
    PackedArgs a;
    a.x = x;
    a.wp = wp;
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
    fastdiv_params(a.tiles_per_img, &a.m_tpi, &a.l_tpi);
    fastdiv_params(a.tiles_w > 0 ? a.tiles_w : 1, &a.m_tw, &a.l_tw);
    a.nchunks = (g.cin + 15) / 16;
    a.chunks_per_split = (a.nchunks + p.tile.splitk - 1) / p.tile.splitk;
    igemm_region(g, t.bn, a.tc, &a.PR, &a.PC);
    fastdiv_params(a.PR * a.PC, &a.m_rc, &a.l_rc);
    fastdiv_params(a.PC, &a.m_c, &a.l_c);
    fastdiv_params(g.ow, &a.m_ow, &a.l_ow);
    {
        const int rc = a.PR * a.PC;
        a.step_ci = 256 / rc;
        const int rem = 256 % rc;
        a.step_r = rem / a.PC;
        a.step_c = rem % a.PC;
    }
    a.wp_bytes = (unsigned)(packed_weight_floats(g) * 4);
    a.act = g.act;
    a.res_mode = g.res_mode;
    dim3 grid((unsigned)(g.n * a.tiles_per_img), (unsigned)((g.cout + t.bm - 1) / t.bm),
              (unsigned)p.tile.splitk);
    if (g.k == 1)
        launch_packed_k<1>(tile, grid, lds, s, a);
    else
        launch_packed_k<3>(tile, grid, lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.partial == nullptr) return e;
    return launch_splitk_finish(g, p.tile.splitk, a.partial, scale, bias, res, y, s);
}

}  // namespace cvx
