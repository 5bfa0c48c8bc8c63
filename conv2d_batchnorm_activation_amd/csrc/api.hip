// api.hip -- the C ABI of libcvx: host-side validation, per-shape planning and
// the layer-list executor.  Every check runs on the host before anything is
// enqueued; the only device work is the kernels in the k_*.hip files.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <unordered_map>
#include <utility>
#include <vector>

#include "cvx_internal.h"
#include "dsblock.h"

using namespace cvx;

namespace {

constexpr long kMaxElems = 0x7fffffffL;  // kernels index tensors with 32-bit element counts

inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
inline Range span(const void* p, size_t bytes)
{
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}
inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int out_extent(int in, int k, int stride, int pad)
{
    const int span_ = in + 2 * pad - k;
    return span_ < 0 ? 0 : span_ / stride + 1;
}

cvx_status geom_from_desc(const cvx_conv_desc* d, ConvGeom* g)
{
    if (d == nullptr) return CVX_ERR_NULL;
    if (d->act < CVX_ACT_NONE || d->act > CVX_ACT_SILU) return CVX_ERR_ARG;
    if (d->res_mode < CVX_RES_NONE || d->res_mode > CVX_RES_AFTER_ACT) return CVX_ERR_ARG;
    if (d->w_layout != CVX_W_OIHW && d->w_layout != CVX_W_PACKED) return CVX_ERR_ARG;
    if (d->n < 1 || d->c_in < 1 || d->h < 1 || d->w < 1 || d->c_out < 1) return CVX_ERR_SHAPE;
    if (d->kh < 1 || d->kw < 1 || d->stride < 1 || d->pad < 0 || d->groups < 1)
        return CVX_ERR_SHAPE;
    if (d->n > 65535) return CVX_ERR_SHAPE;
    if (d->c_in % d->groups != 0 || d->c_out % d->groups != 0) return CVX_ERR_SHAPE;
    if (d->kh != d->kw) return CVX_ERR_UNSUPPORTED;       // square windows only
    if (d->kh > 7 || d->stride > 4) return CVX_ERR_UNSUPPORTED;
    if (d->pad >= d->kh) return CVX_ERR_UNSUPPORTED;      // every output sees the image
    const int oh = out_extent(d->h, d->kh, d->stride, d->pad);
    const int ow = out_extent(d->w, d->kw, d->stride, d->pad);
    if (oh < 1 || ow < 1) return CVX_ERR_SHAPE;
    if ((long)d->n * d->c_in * d->h * d->w > kMaxElems) return CVX_ERR_SHAPE;
    if ((long)d->n * d->c_out * oh * ow > kMaxElems) return CVX_ERR_SHAPE;
    if ((long)d->c_out * (d->c_in / d->groups) * d->kh * d->kw > kMaxElems) return CVX_ERR_SHAPE;
    *g = {d->n, d->c_in, d->h, d->w, d->c_out, d->kh, d->stride, d->pad, d->groups,
          d->act, d->res_mode, oh, ow, d->w_layout};
    return CVX_OK;
}

// ------------------------------------------------------------------ planning
// Kernel family and tile parameters per layer shape ("YOLO26N Inference
// Optimisation", "Key observations" #1-#2 and "Improvements" #1, #3: one fixed
// tile configuration cannot serve both the large-map stem and the
// many-channel late layers, so a single dispatcher picks per shape).
bool plan_depthwise(const ConvGeom& g, Plan* p)
{
    if (!(g.groups == g.cin && g.cin == g.cout && g.k == 3)) return false;
    if (g.stride != 1 && g.stride != 2) return false;
    const int pw = g.w + 2 * g.pad;
    const int ohw = g.oh * g.ow;
    const int planes = g.n * g.cout;
    // Small planes: the plane kernel, `ppb` whole planes per workgroup -- small
    // enough that about eight workgroups share a compute unit when there are
    // planes enough (the per-plane arithmetic needs waves to hide its LDS
    // latency behind), at most about 8K floats of staging -- for tensors within
    // a buffer's 2^31-byte range.
    if ((long)g.h * g.w <= 4096 && (long)planes * g.h * g.w * 4 < 0x7fffffffL &&
        (long)planes * ohw * 4 < 0x7fffffffL) {
        const int cap = std::max(4, std::min(64, (int)(8192 / ((long)g.h * g.w))) & ~3);
        const int want = ((planes + 2047) / 2048 + 3) & ~3;  // ~8 workgroups per compute unit
        // Widths with a row-strip instance: the same size class, rounded down to
        // a divisor of C so that a workgroup's channels (and their weights, scales
        // and biases) are one run.
        // (Few large planes go to the plane kernel below, which spreads one
        // plane over the whole workgroup.)
        if (dw_rows_shape(g) && !(g.oh * g.ow >= 192 && (long)planes < 4L * 256)) {
            int ppb = std::max(1, std::min(cap, want));
            while (g.cout % ppb != 0) --ppb;
            if (dw_rows_lds_bytes(g, ppb) <= kMaxLdsBytes) {
                p->dw_ppb = ppb;
                p->dw_toh = -1;
                p->fam = FAM_DEPTHWISE;
                p->ws_bytes = 0;
                return true;
            }
        }
        int ppb = std::max(4, std::min(cap, want));
        // large planes with few of them: a plane per workgroup (all waves on it)
        if (g.oh * g.ow >= 192 && (long)planes < 4L * 256) ppb = 1;
        if (dw_planes_lds_bytes(g, ppb) > kMaxLdsBytes) return false;
        p->dw_ppb = ppb;
        p->dw_toh = 0;
        p->fam = FAM_DEPTHWISE;
        p->ws_bytes = 0;
        return true;
    }
    const size_t budget = 32 * 1024 / sizeof(float);  // floats of halo tile per workgroup
    if (ohw <= 1024 && (size_t)((g.oh - 1) * g.stride + 3) * pw <= budget) {
        // whole planes; several per workgroup when they are small
        const int plane_tile = ((g.oh - 1) * g.stride + 3) * pw;
        int ppb = std::max(1, 1024 / ohw);
        ppb = std::min<int>(ppb, (int)(budget / plane_tile));
        ppb = std::max(1, std::min(ppb, planes));
        p->dw_ppb = ppb;
        p->dw_toh = g.oh;
    } else {
        // bands of output rows of one plane
        int toh = std::max(1, 1024 / g.ow);
        while (toh > 1 && (size_t)((toh - 1) * g.stride + 3) * pw > budget) --toh;
        if ((size_t)(2 * g.stride + 3) * pw > budget && toh == 1 && (size_t)3 * pw > budget)
            return false;  // a single row does not fit the LDS budget
        p->dw_ppb = 1;
        p->dw_toh = std::min(toh, g.oh);
    }
    p->fam = FAM_DEPTHWISE;
    p->ws_bytes = 0;
    return true;
}

// Tuning and test override: CVX_IGEMM_TILE="kind,tc,splitk[,persist]" forces a
// tile configuration when it is valid for this shape (sweeps and coverage
// tests); persist > 0 asks for the persistent form with that many workgroups
// (rounded down to a multiple of 8, at most the tile count).
bool forced_tile(int* kind, int* tc, int* sk, int* persist)
{
    const char* env = getenv("CVX_IGEMM_TILE");
    int k, t, s, pe = 0;
    if (env == nullptr) return false;
    const int got = sscanf(env, "%d,%d,%d,%d", &k, &t, &s, &pe);
    if (got < 3) return false;
    *kind = k;
    *tc = t;
    *sk = s;
    *persist = got == 4 ? pe : 0;
    return true;
}

bool slices_ok(int nchunks, int sk)
{
    return sk >= 1 && sk <= nchunks && (long)(sk - 1) * ((nchunks + sk - 1) / sk) < nchunks;
}

// Measured winners for the detector's shapes: a GPU sweep timed every packed
// configuration of each layer alone (the pages' static per-shape table, filled
// by offline sweeps: "YOLO26N Inference Optimisation", "Improvements" #1 and
// "Key observations"); an entry is kept where the best beat the planner's
// choice by 2% or more in one sweep (repeated sweeps of the same build differ by
// 2-7% on some layers, so near-ties may flip between sweeps).  Other shapes go
// to the cost model below.
struct TileEntry {
    int n, cin, h, w, cout, k, stride, pad;
    int kind, tc, splitk;
};
constexpr TileEntry kTileTable[] = {
    // batch 1
    {1, 16, 320, 320, 32, 3, 2, 1, 1, 16, 1},   // stem2  7.70 -> 7.33 us (when not paired with stem1)
    {1, 64, 80, 80, 128, 3, 2, 1, 0, 16, 1},    // b      6.21 -> 6.07
    {1, 128, 40, 40, 128, 3, 1, 1, 0, 8, 1},    // d      8.66 -> 8.35
    {1, 128, 40, 40, 256, 3, 2, 1, 3, 8, 1},    // e      7.88 -> 6.85 (16-pixel tile; 32x32 needed a split)
    {1, 256, 20, 20, 256, 1, 1, 0, 3, 0, 1},    // f      5.55 -> 5.05 (16-pixel tile: 200 workgroups, not 104)
    {1, 256, 20, 20, 256, 3, 1, 1, 3, 0, 1},    // g     10.23 -> 9.31 (16-pixel tile; 32x32 needed a split)
    // batch 8
    {8, 16, 320, 320, 32, 3, 2, 1, 0, 16, 1},   // stem2 40.38 -> 37.07 (when not paired with stem1)
    {8, 32, 160, 160, 64, 3, 2, 1, 0, 16, 1},   // bridge 30.87 -> 29.99
    {8, 64, 80, 80, 64, 3, 1, 1, 0, 16, 1},     // a     44.32 -> 43.48
    {8, 64, 80, 80, 128, 3, 2, 1, 0, 8, 1},     // b     27.98 -> 27.04
    {8, 128, 40, 40, 128, 1, 1, 0, 1, 16, 1},   // c     14.23 -> 12.23
    {8, 128, 40, 40, 128, 3, 1, 1, 0, 0, 1},    // d     45.76 -> 42.18
    {8, 128, 40, 40, 256, 3, 2, 1, 0, 8, 1},    // e     26.67 -> 25.84
};

const TileEntry* table_tile(const ConvGeom& g)
{
    for (const TileEntry& e : kTileTable)
        if (e.n == g.n && e.cin == g.cin && e.h == g.h && e.w == g.w && e.cout == g.cout && e.k == g.k &&
            e.stride == g.stride && e.pad == g.pad)
            return &e;
    return nullptr;
}

// Packed-weight implicit GEMM: tile, tc and split count by a cost model of one
// MI355X in clocks.  A workgroup pays a fixed start (kernel arguments, address
// set-up, the cross-wave exchange and the epilogue) plus its first stage's loads,
// which nothing overlaps; after that the producers load stage s+1 while the
// consumers compute stage s, so a stage costs the larger of its matrix time
// (taps x 64 clocks per SIMD and chunk for every 16 pixels of the tile) and
// its load time (~30 clocks per vector-memory instruction the unit issues),
// plus a barrier.  A split into s slices adds ~4000 + 800*s*(tile pixels / 32)
// clocks (the partial sums' round trip through memory and the arrival count).  Up to packed_occupancy(kind)
// workgroups share a compute unit, each slowing the others by ~30%.
// `max_split` bounds the split (1 when no workspace is at hand).
bool plan_packed(const ConvGeom& g, Plan* p, int max_split = 8, int only_kind = -1)
{
    if (g.groups != 1 || (g.k != 1 && g.k != 3)) return false;
    if (g.cin * g.k * g.k < 16 || g.cin < 4) return false;  // too short a reduction
    const double kCUs = 256.0, kFixedClk = 4000.0, kLoadClk = 30.0, kBarrierClk = 150.0,
                 kSplitClk = 4000.0, kSplitEachClk = 800.0, kShare = 0.3;
    const int nchunks = (g.cin + 15) / 16;
    const int kk = g.k * g.k;
    const long mblocks = (g.cout + 31) / 32;
    double best = 1e300;
    GemmTile bt{-1, 0, 0, 0, 1};
    for (int kind = 0; kind < packed_num_kinds(); ++kind) {
        if (only_kind >= 0 && kind != only_kind) continue;
        const int bn = packed_tile_n(kind);
        const double nt = bn / 32.0;
        const int cps = packed_chunks_per_stage(kind, g.k);
        for (int tc = bn; tc >= 0; tc = tc > 4 ? tc / 2 : tc - 4) {
            size_t lds = 0;
            if (!packed_tile_fits(g, kind, tc, &lds)) continue;
            const int occ = std::max(1, std::min<int>(packed_occupancy(kind, g.k),
                                                      (int)(kMaxLdsBytes / std::max<size_t>(lds, 1))));
            const double loads = cps * kLoadClk * packed_loads_per_chunk(g, kind, tc);
            const double stage = std::max(cps * kk * 64.0 * (bn / 16), loads) + kBarrierClk;
            const long tiles = (long)g.n * packed_tiles_per_image(g, kind, tc) * mblocks;
            for (int sk = 1; sk <= max_split; ++sk) {
                if (!slices_ok(nchunks, sk)) continue;
                if ((long)sk * g.n * g.cout * g.oh * g.ow * 4 >= 0x7fffffffL) continue;
                const int per = (nchunks + sk - 1) / sk;
                const int stages = (per + cps - 1) / cps;
                const double wg = kFixedClk + loads + stages * stage +
                                  (sk > 1 ? kSplitClk + kSplitEachClk * nt * sk : 0.0);
                const long wgs = tiles * sk;
                const double per_cu = std::ceil(wgs / kCUs);  // workgroups one unit runs
                const double together = std::min<double>(per_cu, occ);
                const double cost = std::ceil(per_cu / together) * wg * (1.0 + kShare * (together - 1.0)) +
                                    1e-3 * wgs;  // ties: fewer workgroups
                if (cost < best) {
                    best = cost;
                    bt = GemmTile{kind, 32, bn, tc, sk};
                }
            }
        }
    }
    if (const TileEntry* e = table_tile(g)) {
        if ((only_kind < 0 || e->kind == only_kind) && e->splitk <= max_split && slices_ok(nchunks, e->splitk) &&
            packed_tile_fits(g, e->kind, e->tc, nullptr))
            bt = GemmTile{e->kind, 32, packed_tile_n(e->kind), e->tc, e->splitk};
    }
    int kind, tc, sk, pe;
    if (forced_tile(&kind, &tc, &sk, &pe) && kind >= 0 && kind < packed_num_kinds() &&
        (only_kind < 0 || kind == only_kind) && sk <= max_split && slices_ok(nchunks, sk) &&
        packed_tile_fits(g, kind, tc, nullptr)) {
        bt = GemmTile{kind, 32, packed_tile_n(kind), tc, sk, 0};
        if (pe > 0 && sk == 1) {
            const long tiles = packed_num_tiles(g, kind, tc);
            const int wgs = (int)(std::min<long>(pe, tiles) / 8 * 8);
            if (packed_persist_fits(g, kind, tc, wgs)) bt.persist = wgs;
        }
    }
    if (bt.kind < 0) return false;
    p->fam = FAM_IGEMM_PACKED;
    p->tile = bt;
    p->ws_bytes = packed_workspace_bytes(g, bt.kind, bt.tc, bt.splitk);
    return true;
}

// OIHW implicit GEMM (k_igemm.hip): tile choice by a small cost model of one
// MI355X: 256 compute units, one workgroup per unit per round, each unit
// retiring 256 fp32 MFMA FLOP per clock; every chunk of input channels costs a
// fixed staging overhead, every workgroup a fixed start-up latency, and a split
// reduction costs a finishing pass over the partial sums.
bool plan_igemm(const ConvGeom& g, Plan* p)
{
    if (g.groups != 1 || (g.k != 1 && g.k != 3)) return false;
    if (g.cin * g.k * g.k < 16 || g.cin < 4) return false;  // too short a reduction
    const double kCUs = 256.0, kFlopPerClk = 256.0, kChunkClk = 400.0, kStartClk = 3000.0,
                 kLaunchClk = 4000.0, kBytesPerClk = 2000.0;
    const int ck = igemm_chunk_channels();
    const int nchunks = (g.cin + ck - 1) / ck;
    const int kk = g.k * g.k;
    double best = 1e300;
    GemmTile bt{-1, 0, 0, 0, 1};
    for (int tile = 0; tile < igemm_num_tiles(); ++tile) {
        int bm, bn;
        igemm_tile_shape(tile, &bm, &bn);
        for (int tc = bn; tc >= 0; tc = tc > 4 ? tc / 2 : tc - 4) {
            if (!igemm_tile_fits(g, tile, tc, nullptr)) continue;
            const double stage_clk = igemm_stage_floats(g, tile, tc) / 256.0 * 6.0;
            const long tiles = (long)g.n * igemm_tiles_per_image(g, tile, tc) *
                               ((g.cout + bm - 1) / bm);
            for (int sk = 1; sk <= 8; ++sk) {
                if (!slices_ok(nchunks, sk)) continue;
                if ((long)sk * g.n * g.cout * g.oh * g.ow * 4 >= 0x7fffffffL) continue;
                const int per = (nchunks + sk - 1) / sk;
                const long wgs = tiles * sk;
                const double rounds = std::ceil(wgs / kCUs);
                const double chunk_mfma = 2.0 * bm * bn * ck * kk / kFlopPerClk;
                const double wg_clk = per * (chunk_mfma + kChunkClk + stage_clk) + kStartClk;
                double cost = rounds * wg_clk + 1e-3 * wgs;  // ties: fewer workgroups
                if (sk > 1)
                    cost += kLaunchClk +
                            (double)g.n * g.cout * g.oh * g.ow * 4.0 * (sk + 2) / kBytesPerClk;
                if (cost < best) {
                    best = cost;
                    bt = GemmTile{tile, bm, bn, tc, sk};
                }
            }
        }
    }
    int kind, tc, sk, pe;
    if (forced_tile(&kind, &tc, &sk, &pe) && kind >= 0 && kind < igemm_num_tiles() &&
        slices_ok(nchunks, sk) && igemm_tile_fits(g, kind, tc, nullptr)) {
        int bm, bn;
        igemm_tile_shape(kind, &bm, &bn);
        bt = GemmTile{kind, bm, bn, tc, sk};
    }
    if (bt.kind < 0) return false;
    p->fam = FAM_IGEMM;
    p->tile = bt;
    p->ws_bytes = bt.splitk > 1 ? (size_t)bt.splitk * g.n * g.cout * g.oh * g.ow * sizeof(float) : 0;
    return true;
}

void plan_direct(const ConvGeom& g, Plan* p)
{
    const int cout_g = g.cout / g.groups;
    p->fam = FAM_DIRECT;
    p->direct_cob = cout_g >= 16 ? 16 : cout_g >= 8 ? 8 : cout_g >= 4 ? 4 : 1;
    p->direct_stem = stem_shape(g) ? 1 : 0;
    p->ws_bytes = 0;
}

// CVX_GEMM1X1=0 never takes the 1x1 GEMM kernel, =1 takes it for every layer
// it fits (tests and sweeps); unset, for layers with at least kGemm1x1Waves
// output blocks.
int gemm1x1_mode()
{
    const char* e = getenv("CVX_GEMM1X1");
    return e == nullptr ? -1 : (e[0] == '1' ? 1 : 0);
}
constexpr long kGemm1x1Waves = 768;  // the detector's c and f at b=8 (1600, 832), not at b=1 (200, 104)

bool gemm1x1_wanted(const ConvGeom& g)
{
    const int m = gemm1x1_mode();
    return m == 1 || (m < 0 && gemm1x1_waves(g) >= kGemm1x1Waves);
}

cvx_status plan_uncached(const ConvGeom& g, Plan* p)
{
    *p = Plan{};
    if (plan_depthwise(g, p)) return CVX_OK;
    // 1x1 layers over batches of small planes: whole images per workgroup (a
    // forced packed tile keeps the packed kernel, for sweeps and tests)
    int fk, ft, fs, fp;
    if (g.w_layout == CVX_W_PACKED && !forced_tile(&fk, &ft, &fs, &fp) && pointwise_fits(g)) {
        p->fam = FAM_POINTWISE;
        p->ws_bytes = 0;
        return CVX_OK;
    }
    // 1x1 stride-1 layers with enough 32 x 32 output blocks to give most SIMDs
    // one: a wave per block over the whole reduction (a forced packed tile
    // keeps the packed kernel)
    if (g.w_layout == CVX_W_PACKED && !forced_tile(&fk, &ft, &fs, &fp) && gemm1x1_fits(g) && gemm1x1_wanted(g)) {
        p->fam = FAM_GEMM1X1;
        p->ws_bytes = 0;
        return CVX_OK;
    }
    if (g.w_layout == CVX_W_PACKED ? plan_packed(g, p) : plan_igemm(g, p)) return CVX_OK;
    plan_direct(g, p);
    const int cout_g = g.cout / g.groups;
    if ((long)g.groups * ((cout_g + p->direct_cob - 1) / p->direct_cob) > 65535)
        return CVX_ERR_UNSUPPORTED;
    return CVX_OK;
}

// Plans are a pure function of the geometry (and of a forced tile, when one is
// set), so they are remembered: a forward then plans each layer shape once, not
// on every call.  Bounded, and safe to use from several host threads.
struct PlanKey {
    ConvGeom g;
    int forced[4];
    int g1x1;  // CVX_GEMM1X1
    bool operator==(const PlanKey& o) const { return memcmp(this, &o, sizeof(PlanKey)) == 0; }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey& k) const
    {
        const unsigned char* b = reinterpret_cast<const unsigned char*>(&k);
        size_t h = 1469598103934665603ull;  // FNV-1a
        for (size_t i = 0; i < sizeof(PlanKey); ++i) h = (h ^ b[i]) * 1099511628211ull;
        return h;
    }
};

cvx_status make_plan(const ConvGeom& g, Plan* p)
{
    static std::mutex mu;
    static std::unordered_map<PlanKey, std::pair<cvx_status, Plan>, PlanKeyHash> cache;
    PlanKey key;
    memset(&key, 0, sizeof(key));  // padding takes part in the hash and comparison
    key.g = g;
    key.forced[0] = key.forced[1] = key.forced[2] = key.forced[3] = -1;
    forced_tile(&key.forced[0], &key.forced[1], &key.forced[2], &key.forced[3]);
    key.g1x1 = gemm1x1_mode();
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            *p = it->second.second;
            return it->second.first;
        }
    }
    const cvx_status st = plan_uncached(g, p);
    std::lock_guard<std::mutex> lock(mu);
    if (cache.size() >= 4096) cache.clear();
    cache.emplace(key, std::make_pair(st, *p));
    return st;
}

cvx_status launch_conv(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                       const float* scale, const float* bias, const float* res, float* y, void* ws,
                       hipStream_t s)
{
    hipError_t e = hipSuccess;
    switch (p.fam) {
    case FAM_DEPTHWISE: e = launch_depthwise(g, p, x, w, scale, bias, res, y, s); break;
    case FAM_DIRECT: e = launch_direct(g, p, x, w, scale, bias, res, y, s); break;
    case FAM_IGEMM: e = launch_igemm(g, p, x, w, scale, bias, res, y, ws, s); break;
    case FAM_IGEMM_PACKED: e = launch_igemm_packed(g, p, x, w, scale, bias, res, y, ws, s); break;
    case FAM_GEMM1X1: e = launch_gemm1x1(g, x, w, scale, bias, res, y, s); break;
    case FAM_POINTWISE:
        if (pointwise_aligned(x, res, y)) {
            e = launch_pointwise(g, x, w, scale, bias, res, y, s);
        } else {
            // 16-byte staging and stores need aligned tensors; otherwise the
            // packed kernel (same weights), unsplit: the plan has no workspace
            Plan q = Plan{};
            if (!plan_packed(g, &q, 1)) return CVX_ERR_UNSUPPORTED;
            e = launch_igemm_packed(g, q, x, w, scale, bias, res, y, nullptr, s);
        }
        break;
    }
    return e == hipSuccess ? CVX_OK : CVX_ERR_HIP;
}

size_t elems_in(const ConvGeom& g) { return (size_t)g.n * g.cin * g.h * g.w; }
size_t elems_out(const ConvGeom& g) { return (size_t)g.n * g.cout * g.oh * g.ow; }
size_t elems_oihw(const ConvGeom& g) { return (size_t)g.cout * (g.cin / g.groups) * g.k * g.k; }

// floats of the packed form of a layer's weights (a copy of OIHW unless the plan
// for the packed layout is the packed implicit-GEMM kernel)
size_t elems_packed(const ConvGeom& g)
{
    ConvGeom gp = g;
    gp.w_layout = CVX_W_PACKED;
    Plan p;
    if (make_plan(gp, &p) == CVX_OK &&
        (p.fam == FAM_IGEMM_PACKED || p.fam == FAM_POINTWISE || p.fam == FAM_GEMM1X1))
        return (size_t)packed_weight_floats(gp);
    return elems_oihw(g);
}

size_t elems_w(const ConvGeom& g)
{
    return g.w_layout == CVX_W_PACKED ? elems_packed(g) : elems_oihw(g);
}

}  // namespace

// The text cvx_conv_plan returns for a planned layer.
static void describe_plan(const ConvGeom& g, const Plan& p, char* buf, int buf_len)
{
    char kn[96];
    switch (p.fam) {
    case FAM_IGEMM_PACKED:
        if (p.tile.persist > 0) {  // named as launched on 16-byte aligned tensors
            packed_persist_kernel_name(g, p.tile.kind, kn, sizeof(kn));
            snprintf(buf, buf_len, "igemm_packed k%d s%d tile=%d bm=%d bn=%d tc=%d splitk=%d persist=%d kernel=%s",
                     g.k, g.stride, p.tile.kind, p.tile.bm, p.tile.bn, p.tile.tc, p.tile.splitk, p.tile.persist, kn);
        } else {
            packed_kernel_name(g, p.tile.kind, kn, sizeof(kn));
            snprintf(buf, buf_len, "igemm_packed k%d s%d tile=%d bm=%d bn=%d tc=%d splitk=%d kernel=%s",
                     g.k, g.stride, p.tile.kind, p.tile.bm, p.tile.bn, p.tile.tc, p.tile.splitk, kn);
        }
        break;
    case FAM_POINTWISE: pointwise_describe(g, nullptr, buf, buf_len); break;
    case FAM_GEMM1X1: gemm1x1_describe(g, buf, buf_len); break;
    case FAM_DEPTHWISE:
        if (p.dw_toh == -1) {  // named as launched on 16-byte aligned tensors
            const int hw = g.h * g.w;
            const int vw = g.w % 4 == 0 && hw % 4 == 0 ? 4 : g.w % 2 == 0 && hw % 2 == 0 ? 2 : 1;
            snprintf(buf, buf_len, "depthwise3x3 s%d rows ppb=%d splitk=1 kernel=cvx::k_dw_rows<%d, %d, %d>",
                     g.stride, p.dw_ppb, g.w, g.stride, vw);
        } else if (p.dw_toh == 0)  // named as launched on a 16-byte aligned input
            snprintf(buf, buf_len, "depthwise3x3 s%d planes ppb=%d splitk=1 kernel=cvx::k_dw_planes<%d, 1, 1, %d>",
                     g.stride, p.dw_ppb, g.stride, g.oh * g.ow <= 256 ? 4 : 0);
        else
            snprintf(buf, buf_len, "depthwise3x3 s%d ppb=%d toh=%d splitk=1 kernel=cvx::k_depthwise3x3<%d>",
                     g.stride, p.dw_ppb, p.dw_toh, g.stride);
        break;
    case FAM_DIRECT:
        if (p.direct_stem)
            snprintf(buf, buf_len, "stem k3 s%d splitk=1 kernel=cvx::k_stem<%d, %d, %d>", g.stride,
                     g.cin, stem_cob(g), g.stride);
        else
            snprintf(buf, buf_len, "direct k%d s%d cob=%d splitk=1 kernel=cvx::k_direct<%d>", g.k,
                     g.stride, p.direct_cob, p.direct_cob);
        break;
    case FAM_IGEMM:
        igemm_kernel_name(g, p.tile.kind, kn, sizeof(kn));
        snprintf(buf, buf_len, "igemm_mfma k%d s%d tile=%d bm=%d bn=%d tc=%d splitk=%d kernel=%s",
                 g.k, g.stride, p.tile.kind, p.tile.bm, p.tile.bn, p.tile.tc, p.tile.splitk, kn);
        break;
    }
}

extern "C" {

const char* cvx_status_str(cvx_status s)
{
    switch (s) {
    case CVX_OK: return "ok";
    case CVX_ERR_NULL: return "a required pointer is NULL";
    case CVX_ERR_SHAPE: return "sizes are non-positive, inconsistent or too large";
    case CVX_ERR_UNSUPPORTED: return "convolution not implemented by this library";
    case CVX_ERR_ALIGN: return "a tensor pointer is not 4-byte aligned";
    case CVX_ERR_ALIAS: return "the output overlaps an input";
    case CVX_ERR_WORKSPACE: return "workspace missing or too small";
    case CVX_ERR_HIP: return "HIP runtime error on launch";
    case CVX_ERR_ARG: return "enum or index argument out of range";
    case CVX_ERR_SCRATCH: return "the list needs more workspace than the static scratch array holds";
    default: return "unknown status";
    }
}

const char* cvx_version(void) { return "cvx 0.1 gfx950"; }

cvx_status cvx_conv_out_shape(const cvx_conv_desc* d, int* oh, int* ow)
{
    if (oh == nullptr || ow == nullptr) return CVX_ERR_NULL;
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    Plan p;
    st = make_plan(g, &p);
    if (st != CVX_OK) return st;
    *oh = g.oh;
    *ow = g.ow;
    return CVX_OK;
}

cvx_status cvx_conv_plan(const cvx_conv_desc* d, char* buf, int buf_len)
{
    if (buf == nullptr || buf_len < 1) return CVX_ERR_NULL;
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    Plan p;
    st = make_plan(g, &p);
    if (st != CVX_OK) return st;
    describe_plan(g, p, buf, buf_len);
    return CVX_OK;
}

size_t cvx_conv_workspace_bytes(const cvx_conv_desc* d)
{
    ConvGeom g;
    if (geom_from_desc(d, &g) != CVX_OK) return 0;
    Plan p;
    if (make_plan(g, &p) != CVX_OK) return 0;
    return p.ws_bytes;
}

size_t cvx_packed_weights_bytes(const cvx_conv_desc* d)
{
    ConvGeom g;
    if (geom_from_desc(d, &g) != CVX_OK) return 0;
    Plan p;
    if (make_plan(g, &p) != CVX_OK) return 0;
    return elems_packed(g) * sizeof(float);
}

cvx_status cvx_pack_weights(const cvx_conv_desc* d, const float* w_oihw, float* w_packed,
                            void* stream)
{
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    if (!w_oihw || !w_packed) return CVX_ERR_NULL;
    if (!aligned4(w_oihw) || !aligned4(w_packed)) return CVX_ERR_ALIGN;
    Plan p;
    st = make_plan(g, &p);
    if (st != CVX_OK) return st;
    const size_t np = elems_packed(g), no = elems_oihw(g);
    if (overlap(span(w_packed, np * sizeof(float)), span(w_oihw, no * sizeof(float))))
        return CVX_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ConvGeom gp = g;
    gp.w_layout = CVX_W_PACKED;
    Plan pp;
    make_plan(gp, &pp);
    const bool packed = pp.fam == FAM_IGEMM_PACKED || pp.fam == FAM_POINTWISE || pp.fam == FAM_GEMM1X1;
    hipError_t e = packed ? launch_pack_weights(g, w_oihw, w_packed, s)
                                              : launch_copy(w_oihw, w_packed, (long)no, s);
    return e == hipSuccess ? CVX_OK : CVX_ERR_HIP;
}

cvx_status cvx_fold_bn(const float* gamma, const float* beta, const float* mean, const float* var,
                       float eps, int c, float* scale, float* bias, void* stream)
{
    if (!gamma || !beta || !mean || !var || !scale || !bias) return CVX_ERR_NULL;
    if (c < 1) return CVX_ERR_SHAPE;
    if (!(eps > 0.0f)) return CVX_ERR_ARG;
    for (const void* p : {(const void*)gamma, (const void*)beta, (const void*)mean,
                          (const void*)var, (const void*)scale, (const void*)bias})
        if (!aligned4(p)) return CVX_ERR_ALIGN;
    const size_t b = (size_t)c * sizeof(float);
    const Range outs[2] = {span(scale, b), span(bias, b)};
    if (overlap(outs[0], outs[1])) return CVX_ERR_ALIAS;
    for (const float* in : {gamma, beta, mean, var})
        for (const Range& o : outs)
            if (overlap(o, span(in, b))) return CVX_ERR_ALIAS;
    hipError_t e = launch_fold_bn(gamma, beta, mean, var, eps, c, scale, bias,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CVX_OK : CVX_ERR_HIP;
}

cvx_status cvx_conv_bn_act(const cvx_conv_desc* d, const float* x, const float* w,
                           const float* scale, const float* bias, const float* residual, float* y,
                           void* workspace, size_t ws_bytes, void* stream)
{
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    if (!x || !w || !scale || !bias || !y) return CVX_ERR_NULL;
    if (g.res_mode != CVX_RES_NONE && residual == nullptr) return CVX_ERR_NULL;
    const float* res = g.res_mode != CVX_RES_NONE ? residual : nullptr;
    for (const void* p : {(const void*)x, (const void*)w, (const void*)scale, (const void*)bias,
                          (const void*)y})
        if (!aligned4(p)) return CVX_ERR_ALIGN;
    if (res && !aligned4(res)) return CVX_ERR_ALIGN;
    Plan p;
    st = make_plan(g, &p);
    if (st != CVX_OK) return st;
    const Range yr = span(y, elems_out(g) * sizeof(float));
    if (overlap(yr, span(x, elems_in(g) * sizeof(float))) ||
        overlap(yr, span(w, elems_w(g) * sizeof(float))) ||
        overlap(yr, span(scale, g.cout * sizeof(float))) ||
        overlap(yr, span(bias, g.cout * sizeof(float))) ||
        (res && overlap(yr, span(res, elems_out(g) * sizeof(float)))))
        return CVX_ERR_ALIAS;
    if (p.ws_bytes > 0) {
        if (workspace == nullptr || ws_bytes < p.ws_bytes) return CVX_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return CVX_ERR_ALIGN;
        const Range wr = span(workspace, p.ws_bytes);
        if (overlap(wr, yr) || overlap(wr, span(x, elems_in(g) * sizeof(float))) ||
            overlap(wr, span(w, elems_w(g) * sizeof(float))) ||
            (res && overlap(wr, span(res, elems_out(g) * sizeof(float)))))
            return CVX_ERR_ALIAS;
    }
    return launch_conv(g, p, x, w, scale, bias, res, y, workspace,
                       static_cast<hipStream_t>(stream));
}

cvx_status cvx_preprocess_u8(const unsigned char* src, int n, int src_h, int src_w,
                             long src_row_bytes, float* dst, int dst_h, int dst_w,
                             const float* mean, const float* stdv, void* stream)
{
    if (!src || !dst || !mean || !stdv) return CVX_ERR_NULL;
    if (n < 1 || n > 65535 || src_h < 1 || src_w < 1 || dst_h < 1 || dst_w < 1)
        return CVX_ERR_SHAPE;
    if (src_row_bytes < 3L * src_w) return CVX_ERR_SHAPE;
    if ((long)n * 3 * dst_h * dst_w > kMaxElems) return CVX_ERR_SHAPE;
    if (!aligned4(dst)) return CVX_ERR_ALIGN;
    for (int c = 0; c < 3; ++c)
        if (!(stdv[c] != 0.0f)) return CVX_ERR_ARG;
    const size_t src_bytes = (size_t)n * src_h * src_row_bytes;
    if (overlap(span(dst, (size_t)n * 3 * dst_h * dst_w * sizeof(float)), span(src, src_bytes)))
        return CVX_ERR_ALIAS;
    hipError_t e = launch_preprocess(src, n, src_h, src_w, src_row_bytes, dst, dst_h, dst_w, mean,
                                     stdv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CVX_OK : CVX_ERR_HIP;
}

cvx_status cvx_workgroup_xcds(int* xcd, int n_workgroups, void* stream)
{
    if (!xcd) return CVX_ERR_NULL;
    if (n_workgroups < 1 || n_workgroups > (1 << 20)) return CVX_ERR_SHAPE;
    if (!aligned4(xcd)) return CVX_ERR_ALIGN;
    return launch_workgroup_xcds(xcd, n_workgroups, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CVX_OK
               : CVX_ERR_HIP;
}

cvx_status cvx_gap_fc(const float* x, int n, int c, int h, int w, const float* fc_w,
                      const float* fc_b, int out_f, float* out, void* stream)
{
    if (!x || !fc_w || !fc_b || !out) return CVX_ERR_NULL;
    if (n < 1 || n > 65535 || c < 1 || c > 4096 || h < 1 || w < 1 || out_f < 1)
        return CVX_ERR_SHAPE;
    if ((long)n * c * h * w > kMaxElems) return CVX_ERR_SHAPE;
    for (const void* p : {(const void*)x, (const void*)fc_w, (const void*)fc_b, (const void*)out})
        if (!aligned4(p)) return CVX_ERR_ALIGN;
    const Range o = span(out, (size_t)n * out_f * sizeof(float));
    if (overlap(o, span(x, (size_t)n * c * h * w * sizeof(float))) ||
        overlap(o, span(fc_w, (size_t)out_f * c * sizeof(float))) ||
        overlap(o, span(fc_b, (size_t)out_f * sizeof(float))))
        return CVX_ERR_ALIAS;
    hipError_t e = launch_gap_fc(x, n, c, h * w, fc_w, fc_b, out_f, out,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CVX_OK : CVX_ERR_HIP;
}

}  // extern "C"

// ============================================================ layer lists
namespace {

// The stem prologue of list layer `l` (a CVX_L_PREPROC over contiguous frames).
StemPrologue prologue_of(const cvx_layer& l, const void* frames)
{
    StemPrologue pre;
    pre.src = static_cast<const unsigned char*>(frames);
    pre.src_h = l.conv.h;
    pre.src_w = l.conv.w;
    pre.row_bytes = 3L * l.conv.w;
    for (int c = 0; c < 3; ++c) {
        pre.mean[c] = l.mean[c];
        pre.stdv[c] = l.std[c];
    }
    return pre;
}

struct Shape {
    int n, c, h, w;
    size_t elems() const { return (size_t)n * c * h * w; }
};

struct NodePlan {
    Shape in, out;
    ConvGeom g;
    Plan p;
    bool fuse_next;      // GAP whose only reader is the following FC: run as one kernel
    bool skipped;        // FC folded into the preceding GAP
    bool merged;         // 1x1 shortcut computed inside its reader's kernel: no output
    int pair;            // the merged shortcut this layer computes with its own product, or -1
    int dsb_dw;          // pointwise layer run as a block with this depthwise layer (k_dsblock), or -1
    int dsb_skip;        // ... and with this 1x1 shortcut layer, or -1
    bool stem_next;      // stem whose output only the next layer reads: both run as one kernel there
    bool stem_kept;      // ... whose output still gets a region (a list input may be misaligned at launch)
    bool pre_into_pair;  // prologue whose output only a paired stem reads: the pair resizes the frame itself
    int last_use;        // last layer index reading this output
    size_t offset;       // workspace offset of the output (non-final layers)
    int chain_first;     // first layer of the chain run this layer belongs to, or -1
    int chain_len;       // (first layer of a run) layers in the run
    int chain_tc, chain_splits;  // the layer's tile in the chain
};

struct ListPlan {
    std::vector<NodePlan> nodes;
    Shape input;
    bool input_u8;
    size_t act_bytes;    // activation region
    size_t layer_ws;     // largest per-layer workspace (after the activations)
    size_t total() const { return act_bytes + layer_ws; }
};

constexpr size_t kAlign = 256;
constexpr size_t kDistinctBytes = size_t(256) << 20;  // intermediates each in a region of their own
constexpr int kReuseGap = 2;                          // layers after its last read a buffer waits
inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The tile a chained layer uses: the packed planner's choice among 32 x 32
// tiles (its tc and split count), or the first 32 x 32 tile the chain takes.
bool chain_choose(const ConvGeom& g, int* tc, int* splits)
{
    Plan p;
    if (plan_packed(g, &p, 8, 0) && chain_layer_fits(g, p.tile.tc, nullptr)) {
        *tc = p.tile.tc;
        *splits = p.tile.splitk;
        return true;
    }
    for (int t : {0, 32, 16, 8, 4}) {
        if (chain_layer_fits(g, t, nullptr)) {
            *tc = t;
            *splits = 1;
            return true;
        }
    }
    return false;
}

cvx_status plan_list(const cvx_layer* L, int nl, ListPlan* lp)
{
    if (L == nullptr) return CVX_ERR_NULL;
    if (nl < 1 || nl > 4096) return CVX_ERR_SHAPE;
    lp->nodes.assign(nl, NodePlan{});
    lp->input_u8 = L[0].kind == CVX_L_PREPROC;
    bool have_input = false;
    auto input_shape = [&](const Shape& s) -> bool {
        if (!have_input) {
            lp->input = s;
            have_input = true;
            return true;
        }
        return lp->input.n == s.n && lp->input.c == s.c && lp->input.h == s.h &&
               lp->input.w == s.w;
    };
    for (int i = 0; i < nl; ++i) {
        const cvx_layer& l = L[i];
        NodePlan& np = lp->nodes[i];
        np.last_use = i;
        np.pair = -1;
        np.dsb_dw = -1;
        np.dsb_skip = -1;
        if (l.kind < CVX_L_CONV || l.kind > CVX_L_PREPROC) return CVX_ERR_ARG;
        if (l.in < CVX_INPUT || l.in >= i) return CVX_ERR_ARG;
        if (l.kind == CVX_L_PREPROC) {
            if (i != 0 || l.in != CVX_INPUT) return CVX_ERR_ARG;
            const cvx_conv_desc& d = l.conv;
            if (d.n < 1 || d.n > 65535 || d.h < 1 || d.w < 1 || l.dst_h < 1 || l.dst_w < 1)
                return CVX_ERR_SHAPE;
            if ((long)d.n * 3 * l.dst_h * l.dst_w > kMaxElems) return CVX_ERR_SHAPE;
            for (int c = 0; c < 3; ++c)
                if (!(l.std[c] != 0.0f)) return CVX_ERR_ARG;
            lp->input = {d.n, 3, d.h, d.w};  // u8 frames [n][h][w][3]
            have_input = true;
            np.in = lp->input;
            np.out = {d.n, 3, l.dst_h, l.dst_w};
            continue;
        }
        if (l.in == CVX_INPUT && lp->input_u8) return CVX_ERR_ARG;  // raw frames feed only layer 0
        Shape in = l.in == CVX_INPUT ? Shape{l.conv.n, l.conv.c_in, l.conv.h, l.conv.w}
                                     : lp->nodes[l.in].out;
        if (l.in == CVX_INPUT && !input_shape(in)) return CVX_ERR_SHAPE;
        if (l.in >= 0) lp->nodes[l.in].last_use = i;
        np.in = in;
        if (l.kind == CVX_L_CONV) {
            const cvx_conv_desc& d = l.conv;
            if (d.n != in.n || d.c_in != in.c || d.h != in.h || d.w != in.w) return CVX_ERR_SHAPE;
            cvx_status st = geom_from_desc(&d, &np.g);
            if (st != CVX_OK) return st;
            st = make_plan(np.g, &np.p);
            if (st != CVX_OK) return st;
            if (!l.w || !l.scale || !l.bias) return CVX_ERR_NULL;
            np.out = {d.n, d.c_out, np.g.oh, np.g.ow};
            if (d.res_mode != CVX_RES_NONE) {
                if (l.res < CVX_INPUT || l.res >= i) return CVX_ERR_ARG;
                Shape r = l.res == CVX_INPUT ? lp->input : lp->nodes[l.res].out;
                if (l.res == CVX_INPUT && (!have_input || lp->input_u8)) return CVX_ERR_ARG;
                if (r.n != np.out.n || r.c != np.out.c || r.h != np.out.h || r.w != np.out.w)
                    return CVX_ERR_SHAPE;
                if (l.res >= 0) lp->nodes[l.res].last_use = i;
            } else if (l.res != CVX_NO_RES) {
                return CVX_ERR_ARG;
            }
        } else if (l.kind == CVX_L_GAP) {
            if (l.conv.n != in.n || l.conv.c_in != in.c || l.conv.h != in.h || l.conv.w != in.w)
                return CVX_ERR_SHAPE;
            if (in.c > 4096) return CVX_ERR_SHAPE;
            np.out = {in.n, in.c, 1, 1};
        } else {  // FC
            if (in.h != 1 || in.w != 1 || l.conv.n != in.n || l.conv.c_in != in.c)
                return CVX_ERR_SHAPE;
            if (l.conv.c_out < 1 || in.c > 4096) return CVX_ERR_SHAPE;
            if (!l.w || !l.bias) return CVX_ERR_NULL;
            np.out = {in.n, l.conv.c_out, 1, 1};
        }
    }
    if (!have_input) return CVX_ERR_ARG;
    // GAP immediately followed by its only reader, an FC: one kernel
    for (int i = 0; i + 1 < nl; ++i) {
        if (L[i].kind == CVX_L_GAP && L[i + 1].kind == CVX_L_FC && L[i + 1].in == i &&
            lp->nodes[i].last_use == i + 1) {
            lp->nodes[i].fuse_next = true;
            lp->nodes[i + 1].skipped = true;
            // the fused kernel (run at i) writes the fc output (node i+1)
            // while it still reads the pool's input: keep that input live
            // through i+1 so placement never puts the fc output on it
            if (L[i].in >= 0)
                lp->nodes[L[i].in].last_use = std::max(lp->nodes[L[i].in].last_use, i + 1);
        }
    }
    // A 1x1 shortcut convolution (BN, no activation) whose one reader is a
    // later pointwise layer adding it before its activation: both are one
    // product over the two inputs' channels (k_pointwise with two sources), and
    // the shortcut's output is never written.  Both inputs are intermediate
    // outputs (256-byte aligned) and so is the result, as the kernel needs.
    std::vector<int> readers(nl, 0);
    for (int i = 0; i < nl; ++i) {
        if (L[i].kind == CVX_L_PREPROC) continue;
        if (L[i].in >= 0) ++readers[L[i].in];
        if (L[i].kind == CVX_L_CONV && L[i].conv.res_mode != CVX_RES_NONE && L[i].res >= 0) ++readers[L[i].res];
    }
    for (int i = 0; i + 1 < nl; ++i) {
        const cvx_layer& l = L[i];
        NodePlan& np = lp->nodes[i];
        if (l.kind != CVX_L_CONV || np.p.fam != FAM_POINTWISE || l.conv.res_mode != CVX_RES_BEFORE_ACT ||
            l.res < 0 || l.in < 0)
            continue;
        const int j = l.res;
        const cvx_layer& sl = L[j];
        NodePlan& sp = lp->nodes[j];
        if (sl.kind != CVX_L_CONV || sp.p.fam != FAM_POINTWISE || sl.conv.act != CVX_ACT_NONE ||
            sl.conv.res_mode != CVX_RES_NONE || sl.in < 0 || readers[j] != 1 || sp.merged || sp.pair >= 0)
            continue;
        if (!pointwise_pair_fits(np.g, sp.g)) continue;
        sp.merged = true;
        np.pair = j;
        lp->nodes[sl.in].last_use = std::max(lp->nodes[sl.in].last_use, i);
    }
    // A stem layer (k_stem: 3x3, one or three input channels) with 16 output
    // channels whose only reader is the next layer, a packed dense 3x3: the two
    // run as one kernel (k_stem_pair) and the stem's output is not written.
    // When the stem reads the list input, whose alignment is known only at
    // launch, its output keeps a region for the two-kernel fallback.
    // CVX_STEM_PAIR=0 runs them apart.
    const char* pair_env = getenv("CVX_STEM_PAIR");
    if (!(pair_env && pair_env[0] == '0')) {
        for (int i = 0; i + 1 < nl; ++i) {
            const cvx_layer& l = L[i];
            const cvx_layer& nx = L[i + 1];
            NodePlan& np = lp->nodes[i];
            const NodePlan& nn = lp->nodes[i + 1];
            if (l.kind != CVX_L_CONV || nx.kind != CVX_L_CONV || nx.in != i || readers[i] != 1) continue;
            if (np.p.fam != FAM_DIRECT || !np.p.direct_stem || np.merged || np.pair >= 0) continue;
            if (nn.p.fam != FAM_IGEMM_PACKED || !stem_pair_fits(np.g, nn.g, nullptr)) continue;
            np.stem_next = true;
            np.stem_kept = l.in == CVX_INPUT;
            if (l.in >= 0) lp->nodes[l.in].last_use = std::max(lp->nodes[l.in].last_use, i + 1);
            // the prologue before it, read by nothing else: the pair resizes and
            // normalises the frame itself (CVX_STEM_PAIR_U8=0 keeps it apart).
            // Its output keeps a region, for frames off a 16-byte boundary.
            const char* u8_env = getenv("CVX_STEM_PAIR_U8");
            if (i == 1 && l.in == 0 && L[0].kind == CVX_L_PREPROC && readers[0] == 1 && !(u8_env && u8_env[0] == '0')) {
                const StemPrologue pre = prologue_of(L[0], nullptr);
                if (stem_pair_fits(np.g, nn.g, &pre)) lp->nodes[0].pre_into_pair = true;
            }
        }
    }
    // A depthwise 3x3 layer whose one reader is a 1x1 layer, plus that layer's
    // shortcut (the block input, or a 1x1 strided convolution of it read only
    // there): at small batches the block runs as one kernel (k_dsblock) and
    // neither the depthwise output nor the shortcut's is written.  Measured
    // on the MNIST net it is slower than the separate kernels at every batch
    // (b=1: 75 against 46-58 us a forward): with 12-21 workgroups a block, each
    // recomputing the depthwise layer for its channel group, the workgroups'
    // serial work outweighs the two launches saved.  Opt-in: CVX_DSBLOCK=1.
    const char* dsb_env = getenv("CVX_DSBLOCK");
    if (dsb_env && dsb_env[0] == '1') {
        for (int i = 0; i < nl; ++i) {
            const cvx_layer& l = L[i];
            NodePlan& np = lp->nodes[i];
            if (l.kind != CVX_L_CONV || l.in < 0 || np.merged || np.pair >= 0 || np.stem_next) continue;
            const int d = l.in;
            if (L[d].kind != CVX_L_CONV || readers[d] != 1) continue;
            NodePlan& dp = lp->nodes[d];
            if (dp.p.fam != FAM_DEPTHWISE || dp.merged || dp.pair >= 0 || dp.stem_next) continue;
            if (d > 0 && lp->nodes[d - 1].stem_next) continue;
            // a shortcut that cannot run inside (an activation, other readers)
            // is added like any residual tensor
            int j = -1;
            if (l.conv.res_mode == CVX_RES_BEFORE_ACT && l.res >= 0 && l.res != L[d].in) {
                const cvx_layer& sl = L[l.res];
                const NodePlan& sp = lp->nodes[l.res];
                if (sl.kind == CVX_L_CONV && sl.in == L[d].in && readers[l.res] == 1 && !sp.merged &&
                    sp.pair < 0 && !sp.stem_next && dsblock_fits(dp.g, np.g, &sp.g))
                    j = l.res;
            }
            if (j < 0 && !dsblock_fits(dp.g, np.g, nullptr)) continue;
            dp.merged = true;
            np.dsb_dw = d;
            if (j >= 0) {
                lp->nodes[j].merged = true;
                np.dsb_skip = j;
            }
            if (L[d].in >= 0) lp->nodes[L[d].in].last_use = std::max(lp->nodes[L[d].in].last_use, i);
        }
    }
    // Placement of intermediate outputs.  A kernel that writes a buffer another
    // kernel has just read runs markedly slower than one writing memory that
    // was not read since (MNIST conv1's 38.5 MB output: 16.7 against 10.8 us),
    // so when all intermediates together fit kDistinctBytes each gets its own
    // region; past that, first fit over live ranges, where a buffer read by
    // one of the last kReuseGap layers still counts as busy.
    lp->act_bytes = 0;
    lp->layer_ws = 0;
    size_t total = 0;
    auto unwritten = [&](const NodePlan& n) {
        return n.fuse_next || n.merged || (n.stem_next && !n.stem_kept);
    };
    for (int i = 0; i < nl - 1; ++i)
        if (!unwritten(lp->nodes[i])) total += round_up(lp->nodes[i].out.elems() * sizeof(float));
    // CVX_FORWARD_REUSE=1 takes the reuse branch for any size (tests of the
    // placement at small batches)
    const char* reuse_env = getenv("CVX_FORWARD_REUSE");
    const bool distinct = total <= kDistinctBytes && !(reuse_env && reuse_env[0] == '1');
    std::vector<int> placed;
    for (int i = 0; i < nl - 1; ++i) {
        NodePlan& np = lp->nodes[i];
        if (unwritten(np)) {  // pooled vector / shortcut / paired stem never materialised
            np.offset = 0;
            continue;
        }
        const size_t sz = round_up(np.out.elems() * sizeof(float));
        size_t off = 0;
        if (distinct) {
            off = lp->act_bytes;
        } else {
            std::vector<std::pair<size_t, size_t>> busy;
            for (int j : placed) {
                const NodePlan& o = lp->nodes[j];
                if (o.last_use + kReuseGap >= i)  // live while layer i writes, or read just before
                    busy.push_back({o.offset, o.offset + round_up(o.out.elems() * sizeof(float))});
            }
            std::sort(busy.begin(), busy.end());
            for (auto& b : busy) {
                if (off + sz <= b.first) break;
                off = std::max(off, b.second);
            }
        }
        np.offset = off;
        lp->act_bytes = std::max(lp->act_bytes, off + sz);
        placed.push_back(i);
    }
    for (int i = 0; i < nl; ++i)
        if (L[i].kind == CVX_L_CONV) lp->layer_ws = std::max(lp->layer_ws, lp->nodes[i].p.ws_bytes);
    lp->act_bytes = round_up(lp->act_bytes);
    // With CVX_CHAIN=1, runs of consecutive dense packed layers become one
    // chain launch each (k_chain.hip).  Measured on the detector it is slower
    // than one launch per layer at batch 1 and 8 -- a layer there is one round
    // of tiles, so the chain's critical path through the layers' rows is the
    // sum of the tiles' durations plus the signalling -- so it is off by
    // default.  Only with every intermediate in a region of its own: a
    // chain's layers run at the same time, so no output may overwrite a buffer
    // another layer of the run still reads.
    for (int i = 0; i < nl; ++i) {
        lp->nodes[i].chain_first = -1;
        lp->nodes[i].chain_len = 0;
    }
    const char* chain_env = getenv("CVX_CHAIN");
    if (distinct && chain_env && chain_env[0] == '1') {
        std::vector<char> ok(nl, 0);
        for (int i = 0; i < nl; ++i) {
            NodePlan& np = lp->nodes[i];
            if (L[i].kind != CVX_L_CONV || np.merged || np.pair >= 0 || np.dsb_dw >= 0 || np.p.fam != FAM_IGEMM_PACKED)
                continue;
            if (i > 0 && lp->nodes[i - 1].stem_next) continue;  // runs with its stem
            ok[i] = chain_choose(np.g, &np.chain_tc, &np.chain_splits) ? 1 : 0;
        }
        std::vector<ChainLayerSpec> spec;
        for (int i = 0; i < nl;) {
            if (!ok[i]) {
                ++i;
                continue;
            }
            int j = i;
            while (j < nl && ok[j] && j - i < kChainMax) ++j;
            if (j - i >= 2) {
                spec.assign(j - i, ChainLayerSpec{});
                for (int k = i; k < j; ++k) {
                    ChainLayerSpec& c = spec[k - i];
                    c.g = lp->nodes[k].g;
                    c.tc = lp->nodes[k].chain_tc;
                    c.splits = lp->nodes[k].chain_splits;
                    lp->nodes[k].chain_first = i;
                }
                lp->nodes[i].chain_len = j - i;
                lp->layer_ws = std::max(lp->layer_ws, chain_workspace_bytes(spec.data(), j - i));
            }
            i = j;
        }
    }
    return CVX_OK;
}

}  // namespace

extern "C" {

cvx_status cvx_forward_out_shape(const cvx_layer* layers, int n_layers, int out_shape[4])
{
    if (out_shape == nullptr) return CVX_ERR_NULL;
    ListPlan lp;
    cvx_status st = plan_list(layers, n_layers, &lp);
    if (st != CVX_OK) return st;
    const Shape& o = lp.nodes.back().out;
    out_shape[0] = o.n;
    out_shape[1] = o.c;
    out_shape[2] = o.h;
    out_shape[3] = o.w;
    return CVX_OK;
}

size_t cvx_forward_workspace_bytes(const cvx_layer* layers, int n_layers, cvx_status* status)
{
    ListPlan lp;
    cvx_status st = plan_list(layers, n_layers, &lp);
    if (status) *status = st;
    return st == CVX_OK ? lp.total() : 0;
}

cvx_status cvx_forward_plan(const cvx_layer* layers, int n_layers, char* buf, int buf_len)
{
    if (buf == nullptr || buf_len < 1) return CVX_ERR_NULL;
    ListPlan lp;
    cvx_status st = plan_list(layers, n_layers, &lp);
    if (st != CVX_OK) return st;
    int pos = 0;
    buf[0] = '\0';
    for (int i = 0; i < n_layers && pos < buf_len - 1; ++i) {
        const cvx_layer& l = layers[i];
        const NodePlan& np = lp.nodes[i];
        char line[320];
        switch (l.kind) {
        case CVX_L_PREPROC:
            if (np.pre_into_pair)
                snprintf(line, sizeof(line), "merged into 2");
            else
                snprintf(line, sizeof(line), "preprocess");
            break;
        case CVX_L_CONV:
            if (np.chain_first >= 0) {
                const int f = np.chain_first;
                snprintf(line, sizeof(line), "chain %d-%d k%d s%d tile=0 bm=32 bn=32 tc=%d splitk=%d kernel=cvx::k_chain",
                         f, f + lp.nodes[f].chain_len - 1, np.g.k, np.g.stride, np.chain_tc, np.chain_splits);
            } else if (np.merged) {
                int into = -1;
                for (int j = i + 1; j < n_layers; ++j)
                    if (lp.nodes[j].pair == i || lp.nodes[j].dsb_dw == i || lp.nodes[j].dsb_skip == i) into = j;
                snprintf(line, sizeof(line), "merged into %d", into);
            } else if (np.dsb_dw >= 0) {
                char d[256];
                dsblock_describe(lp.nodes[np.dsb_dw].g, np.g, np.dsb_skip >= 0, d, sizeof(d));
                if (np.dsb_skip >= 0)
                    snprintf(line, sizeof(line), "%s dw=%d shortcut=%d", d, np.dsb_dw, np.dsb_skip);
                else
                    snprintf(line, sizeof(line), "%s dw=%d", d, np.dsb_dw);
            } else if (np.pair >= 0) {
                char d[256];
                pointwise_describe(np.g, &lp.nodes[np.pair].g, d, sizeof(d));
                snprintf(line, sizeof(line), "%s shortcut=%d", d, np.pair);
            } else if (np.stem_next) {
                snprintf(line, sizeof(line), "merged into %d", i + 1);
            } else if (i > 0 && lp.nodes[i - 1].stem_next) {
                char d[256];
                const bool u8 = i == 2 && lp.nodes[0].pre_into_pair;
                const StemPrologue pre = u8 ? prologue_of(layers[0], nullptr) : StemPrologue{};
                stem_pair_describe(lp.nodes[i - 1].g, np.g, u8 ? &pre : nullptr, d, sizeof(d));
                snprintf(line, sizeof(line), "%s stem=%d", d, i - 1);
            } else {
                describe_plan(np.g, np.p, line, sizeof(line));
            }
            break;
        case CVX_L_GAP:
            snprintf(line, sizeof(line), np.fuse_next ? "gap+fc kernel=cvx::k_gap_fc" : "gap kernel=cvx::k_gap_fc");
            break;
        default:
            if (np.skipped)
                snprintf(line, sizeof(line), "merged into %d", i - 1);
            else
                snprintf(line, sizeof(line), "fc kernel=cvx::k_gap_fc");
            break;
        }
        const int w = snprintf(buf + pos, buf_len - pos, "%s%d %s", i ? "\n" : "", i, line);
        pos = std::min(buf_len - 1, pos + std::max(w, 0));
    }
    return CVX_OK;
}

cvx_status cvx_forward(const cvx_layer* layers, int n_layers, const void* input, float* output,
                       void* workspace, size_t ws_bytes, void* stream)
{
    ListPlan lp;
    cvx_status st = plan_list(layers, n_layers, &lp);
    if (st != CVX_OK) return st;
    if (!input || !output) return CVX_ERR_NULL;
    if (!aligned4(output) || (!lp.input_u8 && !aligned4(input))) return CVX_ERR_ALIGN;
    const size_t need = lp.total();
    if (need > 0) {
        if (!workspace || ws_bytes < need) return CVX_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return CVX_ERR_ALIGN;
    }
    const size_t in_bytes = lp.input_u8 ? (size_t)lp.input.n * lp.input.h * lp.input.w * 3
                                        : lp.input.elems() * sizeof(float);
    const Range out_r = span(output, lp.nodes.back().out.elems() * sizeof(float));
    if (overlap(out_r, span(input, in_bytes))) return CVX_ERR_ALIAS;
    if (need > 0 && (overlap(out_r, span(workspace, need)) ||
                     overlap(span(input, in_bytes), span(workspace, need))))
        return CVX_ERR_ALIAS;
    for (int i = 0; i < n_layers; ++i) {
        const cvx_layer& l = layers[i];
        if (l.kind == CVX_L_CONV) {
            for (const void* p : {(const void*)l.w, (const void*)l.scale, (const void*)l.bias})
                if (!aligned4(p)) return CVX_ERR_ALIGN;
            const NodePlan& np = lp.nodes[i];
            // weights must not overlap anything the list writes
            const Range wr = span(l.w, elems_w(np.g) * sizeof(float));
            if (overlap(wr, out_r) || (need > 0 && overlap(wr, span(workspace, need))))
                return CVX_ERR_ALIAS;
        } else if (l.kind == CVX_L_FC) {
            if (!aligned4(l.w) || !aligned4(l.bias)) return CVX_ERR_ALIGN;
        }
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    auto out_ptr = [&](int i) -> float* {
        return i == n_layers - 1 ? output : reinterpret_cast<float*>(ws + lp.nodes[i].offset);
    };
    auto in_ptr = [&](int i) -> const float* {
        return i == CVX_INPUT ? static_cast<const float*>(input) : out_ptr(i);
    };
    void* layer_ws = ws ? ws + lp.act_bytes : nullptr;
    int chain_end = -1;  // layers before this index ran inside a chain launch
    // frames the stem pair can read itself: 16-byte aligned (rows are whole
    // 16-byte runs, checked when planning)
    const bool frames_fused = lp.nodes[0].pre_into_pair && (reinterpret_cast<uintptr_t>(input) & 15u) == 0;
    for (int i = 0; i < n_layers; ++i) {
        const cvx_layer& l = layers[i];
        const NodePlan& np = lp.nodes[i];
        if (np.skipped || np.merged || i < chain_end) continue;
        hipError_t e = hipSuccess;
        cvx_status cs = CVX_OK;
        if (np.stem_next) {
            // runs with the next layer, unless its input is off a 16-byte boundary
            const float* x = in_ptr(l.in);
            if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) continue;
            cs = launch_conv(np.g, np.p, x, l.w, l.scale, l.bias, nullptr, out_ptr(i), layer_ws, s);
            if (cs != CVX_OK) return cs;
            continue;
        }
        if (np.pre_into_pair && frames_fused) continue;  // the stem pair resizes the frame
        if (i > 0 && lp.nodes[i - 1].stem_next) {
            const cvx_layer& sl = layers[i - 1];
            const float* x = in_ptr(sl.in);
            if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) {
                const float* res = l.conv.res_mode != CVX_RES_NONE ? in_ptr(l.res) : nullptr;
                const bool u8 = i == 2 && lp.nodes[0].pre_into_pair && frames_fused;
                const StemPrologue pre = u8 ? prologue_of(layers[0], input) : StemPrologue{};
                e = launch_stem_pair(lp.nodes[i - 1].g, x, u8 ? &pre : nullptr, sl.w, sl.scale, sl.bias, np.g, l.w,
                                     l.scale, l.bias, res, out_ptr(i), s);
                if (e != hipSuccess) return CVX_ERR_HIP;
                continue;
            }
        }
        if (np.chain_first == i && np.chain_len >= 2) {
            ChainLayerSpec spec[kChainMax];
            const int n = np.chain_len;
            bool aligned = true;
            for (int k = 0; k < n; ++k) {
                const cvx_layer& lk = layers[i + k];
                const NodePlan& nk = lp.nodes[i + k];
                ChainLayerSpec& c = spec[k];
                c.g = nk.g;
                c.tc = nk.chain_tc;
                c.splits = nk.chain_splits;
                c.x = in_ptr(lk.in);
                c.wp = lk.w;
                c.scale = lk.scale;
                c.bias = lk.bias;
                c.res = lk.conv.res_mode != CVX_RES_NONE ? in_ptr(lk.res) : nullptr;
                c.y = out_ptr(i + k);
                c.in_dep = lk.in >= i && lk.in < i + n ? lk.in - i : -1;
                c.res_dep = lk.conv.res_mode != CVX_RES_NONE && lk.res >= i && lk.res < i + n ? lk.res - i : -1;
                for (const void* p : {(const void*)c.x, (const void*)c.y, (const void*)c.res})
                    if (p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0) aligned = false;
            }
            // a list input off a 16-byte boundary: one launch per layer instead
            if (aligned) {
                e = launch_chain(spec, n, layer_ws, s);
                if (e != hipSuccess) return CVX_ERR_HIP;
                chain_end = i + n;
                continue;
            }
        }
        switch (l.kind) {
        case CVX_L_PREPROC:
            e = launch_preprocess(static_cast<const unsigned char*>(input), np.in.n, np.in.h,
                                  np.in.w, 3L * np.in.w, out_ptr(i), l.dst_h, l.dst_w, l.mean,
                                  l.std, s);
            break;
        case CVX_L_CONV: {
            if (np.dsb_dw >= 0) {
                const cvx_layer& dl = layers[np.dsb_dw];
                const NodePlan& dn = lp.nodes[np.dsb_dw];
                auto packed_1x1 = [](const NodePlan& n) {
                    return n.g.w_layout == CVX_W_PACKED &&
                           (n.p.fam == FAM_IGEMM_PACKED || n.p.fam == FAM_POINTWISE || n.p.fam == FAM_GEMM1X1);
                };
                DsBlockArgs a{};
                a.x = in_ptr(dl.in);
                a.dw_w = dl.w;
                a.dw_scale = dl.scale;
                a.dw_bias = dl.bias;
                a.pw_w = l.w;
                a.pw_scale = l.scale;
                a.pw_bias = l.bias;
                if (np.dsb_skip >= 0) {
                    const cvx_layer& sl = layers[np.dsb_skip];
                    a.skip_w = sl.w;
                    a.skip_scale = sl.scale;
                    a.skip_bias = sl.bias;
                    a.skip_packed = packed_1x1(lp.nodes[np.dsb_skip]);
                } else if (l.conv.res_mode != CVX_RES_NONE) {
                    a.res = in_ptr(l.res);
                }
                a.y = out_ptr(i);
                a.n = dn.g.n;
                a.cin = dn.g.cin;
                a.h = dn.g.h;
                a.w = dn.g.w;
                a.cout = np.g.cout;
                a.oh = np.g.oh;
                a.ow = np.g.ow;
                a.stride = dn.g.stride;
                a.dw_act = dn.g.act;
                a.pw_act = np.g.act;
                a.res_mode = np.g.res_mode;
                a.pw_packed = packed_1x1(np);
                e = launch_dsblock(a, s);
                break;
            }
            if (np.pair >= 0) {
                const cvx_layer& sl = layers[np.pair];
                e = launch_pointwise_pair(np.g, in_ptr(l.in), l.w, l.scale, l.bias, lp.nodes[np.pair].g,
                                          in_ptr(sl.in), sl.w, sl.scale, sl.bias, out_ptr(i), s);
                break;
            }
            const float* res = l.conv.res_mode != CVX_RES_NONE ? in_ptr(l.res) : nullptr;
            cs = launch_conv(np.g, np.p, in_ptr(l.in), l.w, l.scale, l.bias, res, out_ptr(i),
                             layer_ws, s);
            break;
        }
        case CVX_L_GAP:
            if (np.fuse_next) {
                const cvx_layer& fc = layers[i + 1];
                e = launch_gap_fc(in_ptr(l.in), np.in.n, np.in.c, np.in.h * np.in.w, fc.w, fc.bias,
                                  fc.conv.c_out, out_ptr(i + 1), s);
            } else {
                e = launch_gap_fc(in_ptr(l.in), np.in.n, np.in.c, np.in.h * np.in.w, nullptr,
                                  nullptr, 0, out_ptr(i), s);
            }
            break;
        case CVX_L_FC:
            e = launch_gap_fc(in_ptr(l.in), np.in.n, np.in.c, 1, l.w, l.bias, l.conv.c_out,
                              out_ptr(i), s);
            break;
        }
        if (e != hipSuccess) return CVX_ERR_HIP;
        if (cs != CVX_OK) return cs;
    }
    return CVX_OK;
}

}  // extern "C"

// ============================================================ channels-last
static bool nhwc_dtype_known(int dt) { return dt == CVX_DT_F32 || dt == CVX_DT_F16 || dt == CVX_DT_BF16; }
static size_t nhwc_dtype_bytes(int dt) { return dt == CVX_DT_F32 ? 4 : 2; }

extern "C" {

size_t cvx_nhwc_packed_weights_bytes(const cvx_conv_desc* d, int dtype)
{
    ConvGeom g;
    if (geom_from_desc(d, &g) != CVX_OK || !nhwc_supported(g, dtype)) return 0;
    return (size_t)nhwc_packed_weight_elems(g, dtype) * nhwc_dtype_bytes(dtype);
}

cvx_status cvx_nhwc_plan(const cvx_conv_desc* d, int dtype, char* buf, int buf_len)
{
    if (buf == nullptr || buf_len < 1) return CVX_ERR_NULL;
    if (!nhwc_dtype_known(dtype)) return CVX_ERR_ARG;
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    if (!nhwc_supported(g, dtype)) return CVX_ERR_UNSUPPORTED;
    nhwc_describe(g, dtype, buf, buf_len);
    return CVX_OK;
}

cvx_status cvx_nhwc_pack_weights(const cvx_conv_desc* d, int dtype, const float* w_oihw, void* w_packed,
                                 void* stream)
{
    if (!nhwc_dtype_known(dtype)) return CVX_ERR_ARG;
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    if (!w_oihw || !w_packed) return CVX_ERR_NULL;
    if (!nhwc_supported(g, dtype)) return CVX_ERR_UNSUPPORTED;
    if (!aligned4(w_oihw) || (reinterpret_cast<uintptr_t>(w_packed) & 15u) != 0) return CVX_ERR_ALIGN;
    const size_t nb = (size_t)nhwc_packed_weight_elems(g, dtype) * nhwc_dtype_bytes(dtype);
    if (overlap(span(w_packed, nb), span(w_oihw, elems_oihw(g) * sizeof(float)))) return CVX_ERR_ALIAS;
    return launch_pack_nhwc(g, dtype, w_oihw, w_packed, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CVX_OK
               : CVX_ERR_HIP;
}

cvx_status cvx_conv_bn_act_nhwc(const cvx_conv_desc* d, int dtype, const void* x, const void* w_packed,
                                const float* scale, const float* bias, const void* residual, void* y, void* stream)
{
    if (!nhwc_dtype_known(dtype)) return CVX_ERR_ARG;
    ConvGeom g;
    cvx_status st = geom_from_desc(d, &g);
    if (st != CVX_OK) return st;
    if (!x || !w_packed || !scale || !bias || !y) return CVX_ERR_NULL;
    if (g.res_mode != CVX_RES_NONE && residual == nullptr) return CVX_ERR_NULL;
    if (!nhwc_supported(g, dtype)) return CVX_ERR_UNSUPPORTED;
    const void* res = g.res_mode != CVX_RES_NONE ? residual : nullptr;
    for (const void* p : {x, w_packed, (const void*)y})
        if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return CVX_ERR_ALIGN;
    if (res && (reinterpret_cast<uintptr_t>(res) & 15u) != 0) return CVX_ERR_ALIGN;
    if (!aligned4(scale) || !aligned4(bias)) return CVX_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(scale) & 15u) != 0 || (reinterpret_cast<uintptr_t>(bias) & 15u) != 0)
        return CVX_ERR_ALIGN;  // read four channels at a time
    const size_t sz = nhwc_dtype_bytes(dtype);
    const Range yr = span(y, elems_out(g) * sz);
    if (overlap(yr, span(x, elems_in(g) * sz)) ||
        overlap(yr, span(w_packed, (size_t)nhwc_packed_weight_elems(g, dtype) * sz)) ||
        overlap(yr, span(scale, g.cout * sizeof(float))) || overlap(yr, span(bias, g.cout * sizeof(float))) ||
        (res && overlap(yr, span(res, elems_out(g) * sz))))
        return CVX_ERR_ALIAS;
    return launch_conv_nhwc(g, dtype, x, w_packed, scale, bias, res, y, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? CVX_OK
               : CVX_ERR_HIP;
}

}  // extern "C"

// ====================================================== allocation-free forward
// For callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it): the intermediates and split
// partial sums live in one static device array per GPU.  Its device address is
// looked up once per device, with that device current, and kept; host code
// never passes the array's own name to a kernel (on the host that name is a
// stand-in, not a device address).
namespace {

constexpr size_t kScratchBytes = CVX_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

cvx_status scratch_for_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CVX_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return CVX_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return CVX_OK;
}

}  // namespace

extern "C" {

size_t cvx_static_scratch_bytes(void) { return kScratchBytes; }

cvx_status cvx_forward_noalloc(const cvx_layer* layers, int n_layers, const void* input,
                               float* output, void* stream)
{
    cvx_status st = CVX_OK;
    const size_t need = cvx_forward_workspace_bytes(layers, n_layers, &st);
    if (st != CVX_OK) return st;
    if (need > kScratchBytes) return CVX_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != CVX_OK) return st;
    return cvx_forward(layers, n_layers, input, output, ws, kScratchBytes, stream);
}

}  // extern "C"
