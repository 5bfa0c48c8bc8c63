// cvx_internal.h -- declarations shared by the host dispatcher and the kernel
// translation units of libcvx.  Not part of the public ABI (include/cvx.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cvx.h"

namespace cvx {

// Kernel families.  The dispatcher picks one per layer shape.
enum Family : int {
    FAM_DEPTHWISE = 0,  // depthwise 3x3 direct kernel, LDS halo tile per plane
    FAM_DIRECT = 1,     // direct VALU kernel (tiny c_in stems, grouped, large k)
    FAM_IGEMM = 2,      // implicit GEMM on fp32 MFMA (dense 1x1 and 3x3), OIHW weights
    FAM_IGEMM_PACKED = 3,  // the same, weights pre-packed in MFMA operand order
    FAM_POINTWISE = 4,  // 1x1 over batches of small planes, whole images per workgroup (packed weights)
    FAM_GEMM1X1 = 5,    // 1x1 stride 1 as a GEMM per image, a wave per 32x32 block over all of c_in (packed weights)
};

// Geometry of one convolution, derived from a validated cvx_conv_desc.
struct ConvGeom {
    int n, cin, h, w, cout, k, stride, pad, groups, act, res_mode;
    int oh, ow;
    int w_layout;  // CVX_W_OIHW or CVX_W_PACKED
};

// Tile configuration for the implicit-GEMM family.
struct GemmTile {
    int kind;         // index into the compiled tile table (k_igemm.hip)
    int bm, bn;       // output tile: bm output channels x bn output pixels
    int tc;           // 0: bn consecutive pixels; else 2-D tile of bn/tc rows x tc columns
    int splitk;       // number of K slices (1 = no split); >1 uses the workspace
    int persist;      // packed family: workgroups of the persistent form (0: one per tile)
};

struct Plan {
    Family fam;
    GemmTile tile;     // FAM_IGEMM only
    int dw_ppb;        // FAM_DEPTHWISE: planes per workgroup
    int dw_toh;        // FAM_DEPTHWISE: output rows per workgroup (0: plane kernel, -1: row-strip kernel)
    int direct_cob;    // FAM_DIRECT: output channels per thread
    int direct_stem;   // FAM_DIRECT: the stem kernel (k_stem) when tensors are 16-byte aligned
    size_t ws_bytes;   // workspace the plan needs
};

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// caller; the launchers assume shapes match the kernels' grid assumptions.
hipError_t launch_fold_bn(const float* gamma, const float* beta, const float* mean,
                          const float* var, float eps, int c, float* scale, float* bias,
                          hipStream_t s);

hipError_t launch_depthwise(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                            const float* scale, const float* bias, const float* res, float* y,
                            hipStream_t s);

hipError_t launch_direct(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                         const float* scale, const float* bias, const float* res, float* y,
                         hipStream_t s);

hipError_t launch_igemm(const ConvGeom& g, const Plan& p, const float* x, const float* w,
                        const float* scale, const float* bias, const float* res, float* y,
                        void* ws, hipStream_t s);

// 3x3 pad-1 stride-1/2 layers with 1 or 3 input channels and widths a multiple of
// 4 (the detector and MNIST stems) run on k_stem.
bool stem_shape(const ConvGeom& g);
// output channels per k_stem workgroup (8 or 16)
int stem_cob(const ConvGeom& g);
// LDS bytes of the depthwise plane kernel for `ppb` planes per workgroup.
size_t dw_planes_lds_bytes(const ConvGeom& g, int ppb);
// The depthwise row-strip kernel (known widths, pad 1) and its LDS bytes.
bool dw_rows_shape(const ConvGeom& g);
size_t dw_rows_lds_bytes(const ConvGeom& g, int ppb);

hipError_t launch_gap_fc(const float* x, int n, int c, int hw, const float* fc_w,
                         const float* fc_b, int out_f, float* out, hipStream_t s);

hipError_t launch_preprocess(const unsigned char* src, int n, int src_h, int src_w,
                             long src_row_bytes, float* dst, int dst_h, int dst_w,
                             const float mean[3], const float stdv[3], hipStream_t s);

// Exact symbol of the kernel a plan launches, as profilers print it
// ("cvx::k_igemm_packed<32, 32, 1, 1, 4, 3, 24, 2>").
void igemm_kernel_name(const ConvGeom& g, int tile, char* buf, int len);
void packed_kernel_name(const ConvGeom& g, int tile, char* buf, int len);
void packed_persist_kernel_name(const ConvGeom& g, int tile, char* buf, int len);

hipError_t launch_igemm_packed(const ConvGeom& g, const Plan& p, const float* x, const float* wp,
                               const float* scale, const float* bias, const float* res, float* y,
                               void* ws, hipStream_t s);

// Pointwise family (k_pointwise.hip): 1x1, no padding, packed weights, c_in a
// multiple of 16 and c_out of 32, planes small enough for a whole image per
// workgroup; x, y and the residual 16-byte aligned at launch.
bool pointwise_fits(const ConvGeom& g);
bool pointwise_aligned(const float* x, const float* res, const float* y);
void pointwise_describe(const ConvGeom& g, const ConvGeom* g2, char* buf, int len);
hipError_t launch_pointwise(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                            const float* bias, const float* res, float* y, hipStream_t s);
// A 1x1 layer g and a second 1x1 convolution g2 (same batch, c_out and output
// plane, its own input x2) in one kernel: y = act(BN(g's conv) + BN2(g2's conv)).
bool pointwise_pair_fits(const ConvGeom& g, const ConvGeom& g2);
hipError_t launch_pointwise_pair(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                                 const float* bias, const ConvGeom& g2, const float* x2, const float* wp2,
                                 const float* scale2, const float* bias2, float* y, hipStream_t s);

hipError_t launch_pack_weights(const ConvGeom& g, const float* w, float* wp, hipStream_t s);

// 1x1 GEMM family (k_gemm1x1.hip): stride 1, no padding, packed 1x1 weights,
// c_in >= 16.  gemm1x1_waves is the number of 32 x 32 output blocks (one wave each).
bool gemm1x1_fits(const ConvGeom& g);
long gemm1x1_waves(const ConvGeom& g);
void gemm1x1_describe(const ConvGeom& g, char* buf, int len);
hipError_t launch_gemm1x1(const ConvGeom& g, const float* x, const float* wp, const float* scale,
                          const float* bias, const float* res, float* y, hipStream_t s);

// Stem pair (k_stem_pair.hip): a k_stem-shaped layer g1 with 16 output channels
// and no residual, and the packed 3x3 layer g2 that alone reads its output, in
// one kernel.  Layer 1's input is x (16-byte aligned), or, with `pre`, a u8 HWC
// frame the kernel resizes and normalises into it as the stem prologue does
// (frame 16-byte aligned, rows a multiple of 16 bytes).
struct StemPrologue {
    const unsigned char* src;
    int src_h, src_w;
    long row_bytes;
    float mean[3], stdv[3];
};
bool stem_pair_fits(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre);
void stem_pair_describe(const ConvGeom& g1, const ConvGeom& g2, const StemPrologue* pre, char* buf, int len);
hipError_t launch_stem_pair(const ConvGeom& g1, const float* x, const StemPrologue* pre, const float* w1,
                            const float* scale1, const float* bias1, const ConvGeom& g2, const float* wp,
                            const float* scale2, const float* bias2, const float* res, float* y, hipStream_t s);

hipError_t launch_splitk_finish(const ConvGeom& g, int splitk, const float* partial,
                                const float* scale, const float* bias, const float* res, float* y,
                                hipStream_t s);

hipError_t launch_copy(const float* src, float* dst, long n, hipStream_t s);

// Packed-weight implicit-GEMM family (k_igemm_packed.hip).  A configuration is
// a kind (tile of 32 x packed_tile_n(kind) outputs), tc and a split count.
// floats of the packed weight buffer: two copies of the same weights, in the
// lane orders of the 32x32x2 (32 x 32*NT tiles, the pointwise, 1x1 GEMM, chain
// and stem-pair kernels) and 16x16x4 (the 16-pixel tile) matrix instructions;
// a kernel reads one copy and bounds its weight descriptor to it
long packed_weight_floats(const ConvGeom& g);
long packed_copy_floats(const ConvGeom& g);
int packed_num_kinds();
int packed_tile_n(int kind);
int packed_chunks_per_stage(int kind, int k);
long packed_tiles_per_image(const ConvGeom& g, int kind, int tc);
bool packed_tile_fits(const ConvGeom& g, int kind, int tc, size_t* lds_bytes);
size_t packed_workspace_bytes(const ConvGeom& g, int kind, int tc, int splits);
// vector-memory instructions a workgroup issues per 16-channel chunk
int packed_loads_per_chunk(const ConvGeom& g, int kind, int tc);
// workgroups of a configuration that fit one compute unit together
int packed_occupancy(int kind, int k);
// workgroup order of a layer: pixel tiles slowest (true) or row blocks slowest
bool packed_spatial_order(const ConvGeom& g, int nmb);
// Staged input region of one 16-channel chunk of a tile: rows, LDS floats per
// row, 16-byte (vec) or 4-byte elements per row and per chunk, 256-lane load
// rounds, LDS floats per chunk.
struct PackedStage {
    int pr, pcw, epr, re, rounds, rep;
};
void packed_stage_geometry(const ConvGeom& g, int kind, int tc, bool vec, PackedStage* st);
// Persistent form: `wgs` workgroups (a multiple of 8, at most the tile count)
// each running several tiles; no split, 16-byte staging, two or more stages.
bool packed_persist_fits(const ConvGeom& g, int kind, int tc, int wgs);
bool packed_split_xcd(hipStream_t s);
hipError_t launch_workgroup_xcds(int* xcd, int n, hipStream_t s);
// workgroups of the persistent form that fit the device at once
int packed_persist_capacity(const ConvGeom& g, int kind, int tc);
long packed_num_tiles(const ConvGeom& g, int kind, int tc);
// A fresh nonzero tag per launch for counters that outlive a launch.
unsigned long long packed_next_epoch();
void fastdiv_params(int d, unsigned* m, unsigned* l);

// ------------------------------------------------------ channels-last layers
// Dense 1x1/3x3 on NHWC tensors stored as fp32 or fp16 (k_nhwc.hip).
bool nhwc_supported(const ConvGeom& g, int dtype);
long nhwc_packed_weight_elems(const ConvGeom& g, int dtype);
hipError_t launch_pack_nhwc(const ConvGeom& g, int dtype, const float* w, void* wp, hipStream_t s);
hipError_t launch_conv_nhwc(const ConvGeom& g, int dtype, const void* x, const void* wp, const float* scale,
                            const float* bias, const void* res, void* y, hipStream_t s);
void nhwc_describe(const ConvGeom& g, int dtype, char* buf, int len);

// ---------------------------------------------------------------- layer chain
// A run of dense 1x1/3x3 layers with packed weights, run as one launch
// (k_chain.hip).  Each layer reads its input (and residual) either from a
// tensor complete before the launch or from an earlier layer of the run.
constexpr int kChainMax = 10;
struct ChainLayerSpec {
    ConvGeom g;
    int tc, splits;            // 32x32 tiles: tc = 0 flat runs, else 2-D tiles tc columns wide
    int in_dep, res_dep;       // index in the run of the layer producing x / res, or -1
    const float *x, *wp, *scale, *bias, *res;
    float* y;
};
// tile geometry the chain supports for this layer (32x32 tiles, 16-byte staging,
// whole-quad epilogue), its LDS floats per stage buffer when it does
bool chain_layer_fits(const ConvGeom& g, int tc, int* buf_floats);
size_t chain_workspace_bytes(const ChainLayerSpec* L, int n);
hipError_t launch_chain(const ChainLayerSpec* L, int n, void* ws, hipStream_t s);

// igemm helpers used by the planner (defined next to the kernel).
void igemm_region(const ConvGeom& g, int bn, int tc, int* pr, int* pc);
int igemm_num_tiles();
void igemm_tile_shape(int tile, int* bm, int* bn);
bool igemm_tile_fits(const ConvGeom& g, int tile, int tc, size_t* lds_bytes);
long igemm_tiles_per_image(const ConvGeom& g, int tile, int tc);
long igemm_stage_floats(const ConvGeom& g, int tile, int tc);  // per chunk
int igemm_chunk_channels();

// LDS one workgroup may use on gfx950 (160 KB per compute unit)
constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace cvx
