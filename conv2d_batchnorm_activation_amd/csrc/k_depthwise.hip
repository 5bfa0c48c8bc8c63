// k_depthwise.hip -- depthwise 3x3 convolution + folded BN + activation
// (+ residual), a memory-bound direct kernel with an LDS halo tile.
//
// The operation is the one of "Как я свертки ускорял", "А теперь — хардкор на
// Metal", steps 1-5: each output channel sees only its own input plane, the 3x3
// window starts at output position * stride - 1 (pad 1 there; any pad here),
// out-of-image taps are zero, BN and the activation are applied in registers and
// each output is stored once.  Its arithmetic intensity is 0.9-2.2 FLOP/byte
// ("Ускоряем скорость", problem 3), far below the MI355X fp32 ridge, so the
// kernel is built around moving bytes:
//   * NCHW planes of consecutive (n, c) pairs are contiguous, so a workgroup
//     stages `ppb` whole planes (or a band of `toh` output rows of one large
//     plane) into LDS with one linear, coalesced sweep over global memory and
//     reads every input element from HBM exactly once;
//   * the zero padding is written into the LDS tile, so the 9-tap loop has no
//     bounds checks;
//   * outputs are written as dense NCHW rows: no tile ever writes past a row
//     end, whatever OW is (the edge-tile overrun of "YOLO26N Inference
//     Optimisation", "Bug fixed: TMA overflow", cannot happen by construction).
#include "bufio.h"
#include "cvx_internal.h"
#include "epilogue.h"

namespace cvx {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int S>
__global__ void __launch_bounds__(256) k_depthwise3x3(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, const float* __restrict__ res, float* __restrict__ y,
    int planes, int C, int H, int W, int OH, int OW, int pad, int ppb, int toh, int bands,
    int act, int res_mode)
{
    extern __shared__ float tile[];
    const int task = blockIdx.x;
    const int band = task % bands;
    const int plane0 = (task / bands) * ppb;
    const int np = min(ppb, planes - plane0);
    const int oh0 = band * toh;
    const int nrows = min(toh, OH - oh0);
    const int PR = (toh - 1) * S + 3;        // input rows staged per plane
    const int PW = W + 2 * pad;              // staged row width incl. zero padding
    const int iy0 = oh0 * S - pad;
    const int tile_elems = np * PR * PW;

    // stage: element e = (pl, r, c) of the halo tile, zero outside the image
    for (int e = threadIdx.x; e < tile_elems; e += 256) {
        const int pl = e / (PR * PW);
        const int rem = e - pl * PR * PW;
        const int r = rem / PW;
        const int c = rem - r * PW;
        const int iy = iy0 + r;
        const int ix = c - pad;
        float v = 0.0f;
        if (iy >= 0 && iy < H && ix >= 0 && ix < W)
            v = x[((long)(plane0 + pl) * H + iy) * W + ix];
        tile[e] = v;
    }
    __syncthreads();

    const int outs = np * nrows * OW;
    for (int e = threadIdx.x; e < outs; e += 256) {
        const int pl = e / (nrows * OW);
        const int rem = e - pl * nrows * OW;
        const int r = rem / OW;
        const int c = rem - r * OW;
        const int plane = plane0 + pl;
        const int ch = plane % C;
        const float* wp = w + ch * 9;
        const float* t = tile + (pl * PR + r * S) * PW + c * S;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) acc = fmaf(t[i * PW + j], wp[i * 3 + j], acc);
        const long idx = ((long)plane * OH + oh0 + r) * OW + c;
        y[idx] = epilogue(acc, scale[ch], bias[ch], act, res_mode, res, idx);
    }
}

// Small planes (a whole plane fits LDS many times over: the MNIST net's 28^2,
// 14^2 and 7^2 maps, the detector's 13^2): a workgroup takes `ppb` consecutive
// (image, channel) planes, which are one contiguous run of memory, and stages
// the run in LDS with LDS-direct loads -- 16 bytes per lane when the input is
// 16-byte aligned and the run starts on a 16-byte boundary -- all in flight at
// once, between two zeroed margins of `margin` floats, so every tap address of
// every output is inside the allocation (taps outside the plane are masked in
// registers, not by address arithmetic).  A plane's nine weights, scale and bias
// are staged in LDS with it and read as broadcasts by the lanes that work on the
// plane (scalar loads there would put a memory round trip in front of every
// plane): planes go one per
// wave, or, when a workgroup holds fewer than four, each to the whole
// workgroup.  The folded-BN values go to an LDS output run; after a barrier the
// run (consecutive planes: contiguous in memory too) gets the residual and the
// activation and is stored 16 bytes per lane when aligned (VOUT), so a
// workgroup's global traffic is a few wide, coalesced accesses.
template <int S, int VEC, int VOUT, int KM>
__global__ void __launch_bounds__(256) k_dw_planes(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, const float* __restrict__ res, float* __restrict__ y,
    int planes, int C, int H, int W, int OH, int OW, int pad, int ppb, int margin, int obuf_off,
    unsigned m_ow, unsigned l_ow, int act, int res_mode)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int plane0 = blockIdx.x * ppb;
    const int np = min(ppb, planes - plane0);
    const int HW = H * W;
    const int n = np * HW;  // floats of the run
    const int rounds = VEC ? (((n + 3) >> 2) + 255) >> 8 : (n + 255) >> 8;
    float* const tile = lds + margin;
    {
        const rsrc_t rx = make_rsrc(x, 4u * (unsigned)(planes * HW));
        const unsigned base = 4u * (unsigned)(plane0 * HW);
        for (int i = 0; i < rounds; ++i) {
            if constexpr (VEC) {
                const int q = t + 256 * i;
                int d = margin + 1024 * i + 256 * wave;
                asm volatile("" : "+s"(d));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + d), 16,
                                                         4 * q < n ? base + 16u * (unsigned)q : kOOB, 0, 0, 0);
            } else {
                const int e = t + 256 * i;
                int d = margin + 256 * i + 64 * wave;
                asm volatile("" : "+s"(d));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                         e < n ? base + 4u * (unsigned)e : kOOB, 0, 0, 0);
            }
        }
        // the margins: before the run, and from the end of the staged rounds on
        const int staged = VEC ? 1024 * rounds : 256 * rounds;
        for (int e = t; e < margin; e += 256) {
            lds[e] = 0.0f;
            lds[margin + staged + e] = 0.0f;
        }
    }
    const int OHW = OH * OW;
    float* const obuf = lds + obuf_off;  // [pl][o]: the workgroup's output run
    // each plane's nine weights, scale and bias, [pl][12], after the output run
    float* const prm = obuf + ((ppb * OHW + 3) & ~3);
    for (int e = t; e < np * 12; e += 256) {
        const int pl = e / 12, k = e - 12 * pl;
        const int ch = (plane0 + pl) % C;
        prm[e] = k < 9 ? w[ch * 9 + k] : k == 9 ? scale[ch] : k == 10 ? bias[ch] : 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    auto one = [&](int pl, int o, const float (&wk)[9], float sc, float bi) {
        const int oy = (int)((__umulhi((unsigned)o, m_ow) + (unsigned)o) >> l_ow);
        const int ox = o - oy * OW;
        const int iy0 = oy * S - pad, ix0 = ox * S - pad;
        const float* tp = tile + pl * HW + iy0 * W + ix0;  // tap (0, 0); inside the margins
        float acc = 0.0f;
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            float racc = 0.0f;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const float v = tp[kh * W + kw];
                racc = fmaf(wk[kh * 3 + kw], (unsigned)(ix0 + kw) < (unsigned)W ? v : 0.0f, racc);
            }
            acc += (unsigned)(iy0 + kh) < (unsigned)H ? racc : 0.0f;
        }
        obuf[pl * OHW + o] = fmaf(sc, acc, bi);
    };
    auto params = [&](int pl, float (&wk)[9], float& sc, float& bi) {
        const f32x4* q = reinterpret_cast<const f32x4*>(prm + 12 * pl);  // same address in every lane
        const f32x4 a = q[0], b = q[1], c = q[2];
        wk[0] = a[0]; wk[1] = a[1]; wk[2] = a[2]; wk[3] = a[3];
        wk[4] = b[0]; wk[5] = b[1]; wk[6] = b[2]; wk[7] = b[3];
        wk[8] = c[0];
        sc = c[1];
        bi = c[2];
    };
    if (KM > 0 && np >= 4) {
        // At most KM outputs per lane and plane: every plane of the run has the
        // same geometry, so each lane's tap offsets and edge masks are found
        // once; per plane it only reads, multiplies and masks, KM outputs at a
        // time, with the next plane's weights loading meanwhile.
        int tb[KM > 0 ? KM : 1];
        unsigned msk[KM > 0 ? KM : 1];  // bit 3*kh + kw: tap inside the image
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            const int o = min(lane + 64 * k, OHW - 1);
            const int oy = (int)((__umulhi((unsigned)o, m_ow) + (unsigned)o) >> l_ow);
            const int ox = o - oy * OW;
            const int iy0 = oy * S - pad, ix0 = ox * S - pad;
            tb[k] = iy0 * W + ix0;
            unsigned m = 0;
#pragma unroll
            for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                for (int kw = 0; kw < 3; ++kw)
                    m |= ((unsigned)(iy0 + kh) < (unsigned)H && (unsigned)(ix0 + kw) < (unsigned)W ? 1u : 0u)
                         << (3 * kh + kw);
            msk[k] = m;
        }
        float wk[9], sc, bi;
        if (wave < np) params(wave, wk, sc, bi);
        for (int pl = wave; pl < np; pl += 4) {
            float wn[9], scn, bin;
            if (pl + 4 < np) params(pl + 4, wn, scn, bin);
            const float* tp = tile + pl * HW;
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                if (64 * k >= OHW) break;  // uniform: blocks of 64 outputs the plane has
                float acc = 0.0f;
#pragma unroll
                for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) {
                        const float v = tp[tb[k] + kh * W + kw];
                        acc = fmaf(wk[kh * 3 + kw], (msk[k] >> (3 * kh + kw)) & 1u ? v : 0.0f, acc);
                    }
                const int o = lane + 64 * k;
                if (o < OHW) obuf[pl * OHW + o] = fmaf(sc, acc, bi);
            }
            if (pl + 4 < np) {
#pragma unroll
                for (int i = 0; i < 9; ++i) wk[i] = wn[i];
                sc = scn;
                bi = bin;
            }
        }
    } else if (np >= 4) {
        for (int pl = wave; pl < np; pl += 4) {
            float wk[9], sc, bi;
            params(pl, wk, sc, bi);
            for (int o = lane; o < OHW; o += 64) one(pl, o, wk, sc, bi);
        }
    } else {
        for (int pl = 0; pl < np; ++pl) {
            float wk[9], sc, bi;
            params(pl, wk, sc, bi);
            for (int o = t; o < OHW; o += 256) one(pl, o, wk, sc, bi);
        }
    }
    __syncthreads();

    // The output run: residual, activation, store.
    const unsigned out_bytes = 4u * (unsigned)(planes * OHW);
    const rsrc_t ry = make_rsrc(y, out_bytes);
    const rsrc_t rr = make_rsrc(res, res_mode != CVX_RES_NONE ? out_bytes : 0u);
    const unsigned obase = 4u * (unsigned)(plane0 * OHW);
    const int m = np * OHW;
    auto fin = [&](float z, float r) {
        if (res_mode == CVX_RES_BEFORE_ACT) z += r;
        z = apply_act_fast(z, act);
        if (res_mode == CVX_RES_AFTER_ACT) z += r;
        return z;
    };
    if constexpr (VOUT) {
        for (int q = t; 4 * q < m; q += 256) {
            const unsigned off = obase + 16u * (unsigned)q;
            f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
            if (res_mode != CVX_RES_NONE)
                r = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)off, 0, 0));
            const f32x4 z = *reinterpret_cast<const f32x4*>(obuf + 4 * q);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fin(z[e], r[e]);
            if (4 * q + 4 <= m) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry, (int)off, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = v[e];
                    if (4 * q + e < m) bstore(ry, off + 4u * e, f);
                }
            }
        }
    } else {
        for (int j = t; j < m; j += 256) {
            const unsigned off = obase + 4u * (unsigned)j;
            const float r = res_mode != CVX_RES_NONE ? bload(rr, off) : 0.0f;
            bstore(ry, off, fin(obuf[j], r));
        }
    }
}

// Row strips for the small planes of known widths (7, 13, 14, 28; pad 1, stride
// 1 or 2): a lane takes one output row of one plane and, for each of its three
// input rows, reads the row once (VW floats per LDS read) and feeds all OW
// outputs of the row from registers -- about three LDS reads per output instead
// of nine.  64 / OH planes share a wave.  The workgroup's planes are a run of
// consecutive channels (`ppb` divides C), so their weights, scales and biases
// are runs too and come to LDS with LDS-direct loads together with the input:
// no register round trip before the arithmetic starts.  Rows outside the plane
// contribute nothing (a select on the row's partial sums; the columns' zero
// padding is known at compile time).  The output run and its store are those
// of the plane kernel.
template <int W, int S, int VW>
__global__ void __launch_bounds__(256) k_dw_rows(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ scale,
    const float* __restrict__ bias, const float* __restrict__ res, float* __restrict__ y,
    int planes, int C, int H, int OH, int ppb, int obuf_off, int prm_off, unsigned m_oh,
    unsigned l_oh, int vec, int vout, int act, int res_mode)
{
    constexpr int OW = (W - 1) / S + 1;  // pad 1
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int plane0 = blockIdx.x * ppb;
    const int np = min(ppb, planes - plane0);
    const int ch0 = plane0 - (plane0 / C) * C;  // the run's first channel; ppb divides C
    const int HW = H * W;
    const int n = np * HW;
    {
        // the planes' run
        const rsrc_t rx = make_rsrc(x, 4u * (unsigned)(planes * HW));
        const unsigned base = 4u * (unsigned)(plane0 * HW);
        if (vec) {
            const int rounds = (((n + 3) >> 2) + 255) >> 8;
            for (int i = 0; i < rounds; ++i) {
                const int q = t + 256 * i;
                int d = 1024 * i + 256 * wave;
                asm volatile("" : "+s"(d));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + d), 16,
                                                         4 * q < n ? base + 16u * (unsigned)q : kOOB, 0, 0, 0);
            }
        } else {
            const int rounds = (n + 255) >> 8;
            for (int i = 0; i < rounds; ++i) {
                const int e = t + 256 * i;
                int d = 256 * i + 64 * wave;
                asm volatile("" : "+s"(d));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                         e < n ? base + 4u * (unsigned)e : kOOB, 0, 0, 0);
            }
        }
        // weights [pl][9], scales [pl], biases [pl], each region whole rounds of
        // 256 floats (lanes past a run still write their slot, with zero)
        const int wr = (9 * ppb + 255) >> 8, sr = (ppb + 255) >> 8;
        const rsrc_t rw = make_rsrc(w + ch0 * 9, 36u * (unsigned)np);
        for (int i = 0; i < wr; ++i) {
            const int e = t + 256 * i;
            int d = prm_off + 256 * i + 64 * wave;
            asm volatile("" : "+s"(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                     e < 9 * np ? 4u * (unsigned)e : kOOB, 0, 0, 0);
        }
        const rsrc_t rs = make_rsrc(scale + ch0, 4u * (unsigned)np);
        const rsrc_t rb = make_rsrc(bias + ch0, 4u * (unsigned)np);
        for (int i = 0; i < sr; ++i) {
            const int e = t + 256 * i;
            int d = prm_off + 256 * (wr + i) + 64 * wave;
            asm volatile("" : "+s"(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + d), 4,
                                                     e < np ? 4u * (unsigned)e : kOOB, 0, 0, 0);
            int d2 = prm_off + 256 * (wr + sr + i) + 64 * wave;
            asm volatile("" : "+s"(d2));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(lds + d2), 4,
                                                     e < np ? 4u * (unsigned)e : kOOB, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int OHW = OH * OW;
    float* const obuf = lds + obuf_off;
    const float* const wts = lds + prm_off;
    const float* const scs = wts + 256 * ((9 * ppb + 255) >> 8);
    const float* const bis = scs + 256 * ((ppb + 255) >> 8);
    const int ppw = 64 / OH;  // planes per wave pass (the host keeps OH <= 64)
    const int lp = (int)((__umulhi((unsigned)lane, m_oh) + (unsigned)lane) >> l_oh);
    const int oy = lane - lp * OH;
    for (int pl0 = wave * ppw; pl0 < np; pl0 += 4 * ppw) {
        const int pl = min(pl0 + lp, np - 1);
        const bool live = lp < ppw && pl0 + lp < np;
        float wk[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) wk[k] = wts[pl * 9 + k];
        const float sc = scs[pl], bi = bis[pl];
        float acc[OW];
#pragma unroll
        for (int o = 0; o < OW; ++o) acc[o] = 0.0f;
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int ih = oy * S - 1 + kh;
            const bool rok = (unsigned)ih < (unsigned)H;
            const float* rp = lds + pl * HW + (rok ? ih : 0) * W;
            float r[W];
#pragma unroll
            for (int c = 0; c < W; c += VW) {
                if constexpr (VW == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(rp + c);
                    r[c] = v[0]; r[c + 1] = v[1]; r[c + 2] = v[2]; r[c + 3] = v[3];
                } else if constexpr (VW == 2) {
                    typedef float f32x2 __attribute__((ext_vector_type(2)));
                    const f32x2 v = *reinterpret_cast<const f32x2*>(rp + c);
                    r[c] = v[0]; r[c + 1] = v[1];
                } else {
                    r[c] = rp[c];
                }
            }
#pragma unroll
            for (int o = 0; o < OW; ++o) {
                float racc = 0.0f;
#pragma unroll
                for (int kw = 0; kw < 3; ++kw) {
                    const int c = o * S - 1 + kw;
                    if (c >= 0 && c < W) racc = fmaf(wk[kh * 3 + kw], r[c], racc);
                }
                acc[o] += rok ? racc : 0.0f;
            }
        }
        if (live) {
            float* op = obuf + pl * OHW + oy * OW;
#pragma unroll
            for (int o = 0; o < OW; ++o) op[o] = fmaf(sc, acc[o], bi);
        }
    }
    __syncthreads();

    // The output run: residual, activation, store (as the plane kernel).
    const unsigned out_bytes = 4u * (unsigned)(planes * OHW);
    const rsrc_t ry = make_rsrc(y, out_bytes);
    const rsrc_t rr = make_rsrc(res, res_mode != CVX_RES_NONE ? out_bytes : 0u);
    const unsigned obase = 4u * (unsigned)(plane0 * OHW);
    const int m = np * OHW;
    auto fin = [&](float z, float rv) {
        if (res_mode == CVX_RES_BEFORE_ACT) z += rv;
        z = apply_act_fast(z, act);
        if (res_mode == CVX_RES_AFTER_ACT) z += rv;
        return z;
    };
    if (vout) {
        for (int q = t; 4 * q < m; q += 256) {
            const unsigned off = obase + 16u * (unsigned)q;
            f32x4 rv = {0.0f, 0.0f, 0.0f, 0.0f};
            if (res_mode != CVX_RES_NONE)
                rv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)off, 0, 0));
            const f32x4 z = *reinterpret_cast<const f32x4*>(obuf + 4 * q);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fin(z[e], rv[e]);
            if (4 * q + 4 <= m) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry, (int)off, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f = v[e];
                    if (4 * q + e < m) bstore(ry, off + 4u * e, f);
                }
            }
        }
    } else {
        for (int j = t; j < m; j += 256) {
            const unsigned off = obase + 4u * (unsigned)j;
            const float rv = res_mode != CVX_RES_NONE ? bload(rr, off) : 0.0f;
            bstore(ry, off, fin(obuf[j], rv));
        }
    }
}

void fastdiv_params(int d, unsigned* m, unsigned* l);

// Zeroed floats before and after the plane kernel's staged run: taps reach
// pad rows and columns before a plane and (3 - pad) rows past it, plus the
// row's last taps; a multiple of 4 keeps the run 16-byte aligned.
static int dw_planes_margin(const ConvGeom& g)
{
    return ((3 * g.w + 3) + 3) & ~3;
}

// LDS floats of the plane kernel's input part: margins and the staged run
// (whole 1 KB loads for 16-byte staging, whole 256-float rounds for 4-byte
// staging); the output run follows it.
static size_t dw_planes_in_floats(const ConvGeom& g, int ppb, bool vec)
{
    const long n = (long)ppb * g.h * g.w;
    const long run = vec ? (n + 1023) / 1024 * 1024 : (n + 255) / 256 * 256;
    return (size_t)(run + 2 * dw_planes_margin(g));
}

size_t dw_planes_lds_bytes(const ConvGeom& g, int ppb)
{
    return (dw_planes_in_floats(g, ppb, true) + (((size_t)ppb * g.oh * g.ow + 3) & ~(size_t)3) +
            12 * (size_t)ppb) * sizeof(float);
}

static inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The row-strip kernel's shapes: pad 1, widths with a compiled instance, at most
// 64 output rows (a plane's rows fit one wave).
bool dw_rows_shape(const ConvGeom& g)
{
    if (g.pad != 1 || g.oh > 64) return false;
    if (g.stride == 1) return g.w == 7 || g.w == 13 || g.w == 14 || g.w == 28;
    if (g.stride == 2) return g.w == 14 || g.w == 28;
    return false;
}

// LDS floats of the row kernel: the staged run (whole 1 KB loads), the output
// run, then weights [ppb][9], scales and biases.
static size_t dw_rows_run_floats(const ConvGeom& g, int ppb)
{
    const long n = (long)ppb * g.h * g.w;
    return (size_t)((n + 1023) / 1024 * 1024);
}

size_t dw_rows_lds_bytes(const ConvGeom& g, int ppb)
{
    const size_t wr = (9 * (size_t)ppb + 255) / 256, sr = ((size_t)ppb + 255) / 256;
    return (dw_rows_run_floats(g, ppb) + (((size_t)ppb * g.oh * g.ow + 3) & ~(size_t)3) +
            256 * (wr + 2 * sr)) * sizeof(float);
}

hipError_t launch_depthwise(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                            const float* scale, const float* bias, const float* res, float* y,
                            hipStream_t s)
{
    const int planes = g.n * g.cout;
    if (p.dw_toh == -1) {  // row-strip kernel
        const int ppb = p.dw_ppb;
        const int vec = al16(x) && ((long)ppb * g.h * g.w) % 4 == 0;
        const int vout = al16(y) && (res == nullptr || al16(res)) && ((long)ppb * g.oh * g.ow) % 4 == 0;
        const int obuf_off = (int)dw_rows_run_floats(g, ppb);
        const int prm_off = obuf_off + (int)((((size_t)ppb * g.oh * g.ow + 3) & ~(size_t)3));
        const size_t lds = dw_rows_lds_bytes(g, ppb);
        unsigned m_oh, l_oh;
        fastdiv_params(g.oh, &m_oh, &l_oh);
        dim3 grid((unsigned)((planes + ppb - 1) / ppb));
        const int hw = g.h * g.w;
#define CVX_DWR(W_, S_, VW_)                                                                        \
    hipLaunchKernelGGL((k_dw_rows<W_, S_, VW_>), grid, dim3(256), lds, s, x, w, scale, bias, res, y,  \
                       planes, g.cout, g.h, g.oh, ppb, obuf_off, prm_off, m_oh, l_oh, vec, vout, g.act, \
                       g.res_mode)
        if (g.stride == 1 && g.w == 7) CVX_DWR(7, 1, 1);
        else if (g.stride == 1 && g.w == 13) CVX_DWR(13, 1, 1);
        else if (g.stride == 1 && g.w == 14) { if (hw % 2 == 0) CVX_DWR(14, 1, 2); else CVX_DWR(14, 1, 1); }
        else if (g.stride == 1 && g.w == 28) { if (hw % 4 == 0) CVX_DWR(28, 1, 4); else CVX_DWR(28, 1, 1); }
        else if (g.stride == 2 && g.w == 14) { if (hw % 2 == 0) CVX_DWR(14, 2, 2); else CVX_DWR(14, 2, 1); }
        else if (g.stride == 2 && g.w == 28) { if (hw % 4 == 0) CVX_DWR(28, 2, 4); else CVX_DWR(28, 2, 1); }
        else return hipErrorInvalidValue;
#undef CVX_DWR
        return hipGetLastError();
    }
    if (p.dw_toh == 0) {  // plane kernel
        // 16-byte staging needs every run to start on a 16-byte boundary
        const bool vec = al16(x) && ((long)p.dw_ppb * g.h * g.w) % 4 == 0;
        // 16-byte output run: every run starts on a 16-byte boundary
        const bool vout = al16(y) && (res == nullptr || al16(res)) && ((long)p.dw_ppb * g.oh * g.ow) % 4 == 0;
        const int obuf_off = (int)dw_planes_in_floats(g, p.dw_ppb, vec);
        const size_t lds = ((size_t)obuf_off + (((size_t)p.dw_ppb * g.oh * g.ow + 3) & ~(size_t)3) +
                            12 * (size_t)p.dw_ppb) * sizeof(float);
        const int margin = dw_planes_margin(g);
        const bool small = g.oh * g.ow <= 256;  // at most four outputs per lane and plane
        unsigned m_ow, l_ow;
        fastdiv_params(g.ow, &m_ow, &l_ow);
        dim3 grid((unsigned)((planes + p.dw_ppb - 1) / p.dw_ppb));
#define CVX_DWP(S_, V_, VO_, KM_)                                                                      \
    hipLaunchKernelGGL((k_dw_planes<S_, V_, VO_, KM_>), grid, dim3(256), lds, s, x, w, scale, bias, res,  \
                       y, planes, g.cout, g.h, g.w, g.oh, g.ow, g.pad, p.dw_ppb, margin, obuf_off,        \
                       m_ow, l_ow, g.act, g.res_mode)
#define CVX_DWP_K(S_, V_, VO_)                               \
    if (small) CVX_DWP(S_, V_, VO_, 4);                      \
    else CVX_DWP(S_, V_, VO_, 0);
#define CVX_DWP_S(S_)                          \
    if (vec && vout) { CVX_DWP_K(S_, 1, 1) }   \
    else if (vec) { CVX_DWP_K(S_, 1, 0) }      \
    else if (vout) { CVX_DWP_K(S_, 0, 1) }     \
    else { CVX_DWP_K(S_, 0, 0) }
        if (g.stride == 1) {
            CVX_DWP_S(1)
        } else if (g.stride == 2) {
            CVX_DWP_S(2)
        } else {
            return hipErrorInvalidValue;
        }
#undef CVX_DWP_S
#undef CVX_DWP_K
#undef CVX_DWP
        return hipGetLastError();
    }
    const int bands = (g.oh + p.dw_toh - 1) / p.dw_toh;
    const int groups_of_planes = (planes + p.dw_ppb - 1) / p.dw_ppb;
    const int PR = (p.dw_toh - 1) * g.stride + 3;
    const size_t lds = (size_t)p.dw_ppb * PR * (g.w + 2 * g.pad) * sizeof(float);
    dim3 grid((unsigned)(groups_of_planes * bands));
    if (g.stride == 1)
        hipLaunchKernelGGL(k_depthwise3x3<1>, grid, dim3(256), lds, s, x, w, scale, bias, res, y,
                           planes, g.cout, g.h, g.w, g.oh, g.ow, g.pad, p.dw_ppb, p.dw_toh, bands,
                           g.act, g.res_mode);
    else if (g.stride == 2)
        hipLaunchKernelGGL(k_depthwise3x3<2>, grid, dim3(256), lds, s, x, w, scale, bias, res, y,
                           planes, g.cout, g.h, g.w, g.oh, g.ow, g.pad, p.dw_ppb, p.dw_toh, bands,
                           g.act, g.res_mode);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace cvx
