/*
 * cvx.h -- C ABI of libcvx: fused convolution + folded BatchNorm + activation
 * for AMD MI355X (gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are fp32, dense and contiguous.  Activations are NCHW: element
 *    (n, c, h, w) sits at n*C*H*W + c*H*W + h*W + w ("YOLO26N Inference
 *    Optimisation", section "NHWC migration", "What NHWC is and why it matters").
 *    Convolution weights are OIHW: [c_out][c_in/groups][kh][kw], the order the
 *    MNIST page's PyTorch weights use ("Как я свертки ускорял", "Ускоряем скорость").
 *  - Every tensor pointer is a DEVICE pointer (HBM), 4-byte aligned, unless the
 *    argument says "host".  The caller owns all memory; the library borrows the
 *    pointers until the work it enqueued has finished, keeps no reference and
 *    never allocates device memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued asynchronously; no call synchronises the device or the stream.
 *  - Errors are returned as cvx_status codes.  All argument validation happens on
 *    the host before anything is enqueued, so an error return means nothing was
 *    launched (except CVX_ERR_HIP, which reports a failed launch).
 *  - Calls are thread-safe: the library has no mutable global state.
 */
#ifndef CVX_H
#define CVX_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbol (the library is built with hidden default visibility). */
#define CVX_API __attribute__((visibility("default")))

typedef int cvx_status;

enum {
    CVX_OK = 0,
    CVX_ERR_NULL = -1,        /* a required pointer is NULL                        */
    CVX_ERR_SHAPE = -2,       /* sizes are non-positive, inconsistent or too large */
    CVX_ERR_UNSUPPORTED = -3, /* valid convolution this library does not implement */
    CVX_ERR_ALIGN = -4,       /* a tensor pointer is not 4-byte aligned            */
    CVX_ERR_ALIAS = -5,       /* the output overlaps an input                      */
    CVX_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required           */
    CVX_ERR_HIP = -7,         /* the HIP runtime reported an error on launch       */
    CVX_ERR_ARG = -8,         /* an enum or index argument is out of range         */
    CVX_ERR_SCRATCH = -9      /* cvx_forward_noalloc: the list needs more workspace
                                 than the static scratch array holds               */
};

/* Activation applied in the epilogue. ReLU = max(0, v) ("Как я свертки ускорял",
 * "А теперь — хардкор на Metal", step 4); SiLU = v / (1 + exp(-v)) (the
 * activation of the fused kernels in "YOLO26N Inference Optimisation",
 * "nsys kernel-level breakdown"). */
enum { CVX_ACT_NONE = 0, CVX_ACT_RELU = 1, CVX_ACT_SILU = 2 };

/* Where the optional residual r is added, with z = scale*conv + bias:
 *   CVX_RES_BEFORE_ACT: y = act(z + r)  -- the MNIST block adds its shortcut
 *                       before the final ReLU ("Как я свертки ускорял",
 *                       "Пациента на стол");
 *   CVX_RES_AFTER_ACT : y = act(z) + r  -- the residual add that followed the
 *                       fused conv+BN+SiLU kernel ("YOLO26N Inference
 *                       Optimisation", "Improvements", #7, now in the epilogue). */
enum { CVX_RES_NONE = 0, CVX_RES_BEFORE_ACT = 1, CVX_RES_AFTER_ACT = 2 };

/* Layout of the weight buffer a layer is given.  OIHW: [c_out][c_in/groups][kh][kw]
 * as is.  PACKED: the buffer cvx_pack_weights produced from the OIHW weights for the
 * same descriptor (a one-time transform at model load into the order the matrix
 * cores read; "YOLO26N Inference Optimisation", "NHWC migration", "Weight
 * layout").  Both give the same results; PACKED is the fast path. */
enum { CVX_W_OIHW = 0, CVX_W_PACKED = 1 };

/* One convolution layer.  Output extent: oh = (h + 2*pad - kh)/stride + 1 (floor),
 * likewise ow.  Supported: 1 <= kh, kw <= 7, 1 <= stride <= 4, 0 <= pad < k,
 * groups dividing c_in and c_out; dilation 1.  n*c*h*w of every tensor must stay
 * below 2^31 elements. */
typedef struct cvx_conv_desc {
    int n, c_in, h, w;   /* input  [n][c_in][h][w]                 */
    int c_out, kh, kw;   /* weight [c_out][c_in/groups][kh][kw]    */
    int stride, pad;     /* same in both spatial dimensions        */
    int groups;          /* 1 = dense; c_in = c_out = groups: depthwise */
    int act;             /* CVX_ACT_*                              */
    int res_mode;        /* CVX_RES_*                              */
    int w_layout;        /* CVX_W_OIHW or CVX_W_PACKED             */
} cvx_conv_desc;

/* Human-readable text for a status code (static storage, never NULL). */
CVX_API const char *cvx_status_str(cvx_status s);

/* Library version string, e.g. "cvx 0.1 gfx950" (static storage). */
CVX_API const char *cvx_version(void);

/* Host-only query: output extent of `d`.  Validates `d` exactly as
 * cvx_conv_bn_act does (without pointers).  Touches no GPU. */
CVX_API cvx_status cvx_conv_out_shape(const cvx_conv_desc *d, int *oh, int *ow);

/* Host-only query: which kernel family and tile configuration the dispatcher
 * selects for `d` ("YOLO26N Inference Optimisation", "Improvements", #1 and #3:
 * one code path whose tile parameters are chosen per layer shape).  Writes a
 * short NUL-terminated description into buf (at most buf_len bytes, truncated
 * to fit): family, tile, split-K factor ("splitk=S"; with OIHW weights S > 1
 * adds a second, finishing launch) and, after "kernel=", the main kernel's
 * symbol as profilers print it.  256 bytes always suffice. */
CVX_API cvx_status cvx_conv_plan(const cvx_conv_desc *d, char *buf, int buf_len);

/* Workspace bytes cvx_conv_bn_act needs for `d` (0 when the selected kernel
 * needs none).  Host-only. */
CVX_API size_t cvx_conv_workspace_bytes(const cvx_conv_desc *d);

/* Bytes of the weight buffer cvx_pack_weights writes for `d` (whatever
 * d->w_layout says).  Host only; 0 on an invalid descriptor. */
CVX_API size_t cvx_packed_weights_bytes(const cvx_conv_desc *d);

/*
 * cvx_pack_weights -- one-time weight transform for layers run with
 * w_layout = CVX_W_PACKED.  For the dense 1x1/3x3 kernels the OIHW weights are
 * reordered into the matrix cores' operand order (zero-padded to whole 32-row
 * and 16-channel groups, a 3x3 chunk's 18 taps per lane in five 16-byte slots);
 * the weights are stored twice, in the two lane orders of the 32x32x2 and the
 * 16x16x4 matrix instructions (the second copy serves the 16-pixel tile), so
 * every plan of the shape reads the same buffer;
 * for the other kernels the packed form is a copy
 * of the OIHW weights.  The packed form does not depend on anything but the
 * descriptor's shape fields.
 *   w_oihw : device [c_out][c_in/groups][kh][kw], read only.
 *   w_packed: device, cvx_packed_weights_bytes(d) bytes, written; must not overlap w_oihw.
 */
CVX_API cvx_status cvx_pack_weights(const cvx_conv_desc *d, const float *w_oihw, float *w_packed,
                                    void *stream);

/*
 * cvx_fold_bn -- fold inference BatchNorm into a per-channel affine map:
 *     scale[i] = gamma[i] / sqrt(var[i] + eps),  bias[i] = beta[i] - mean[i]*scale[i]
 * so that BN(v) = scale*v + bias.  The BatchNorm form is (v - mean)/sqrt(var + eps)
 * * gamma + beta ("Как я свертки ускорял", "А теперь — хардкор на Metal", step 4);
 * folding it before inference is the "weight folding" of "YOLO26N Inference
 * Optimisation", "Baseline benchmark".  Weights are left untouched: scale and bias
 * are applied in the convolution epilogue.
 *   gamma, beta, mean, var : device, [c] each, read only.
 *   scale, bias            : device, [c] each, written.  Must not overlap the inputs.
 *   eps > 0; c >= 1.
 */
CVX_API cvx_status cvx_fold_bn(const float *gamma, const float *beta, const float *mean,
                       const float *var, float eps, int c, float *scale, float *bias,
                       void *stream);

/*
 * cvx_conv_bn_act -- one fused layer:
 *     z[n][co][oh][ow] = scale[co] * sum_{ci,i,j} x[n][g*Cg+ci][oh*s-p+i][ow*s-p+j]
 *                                     * w[co][ci][i][j]  +  bias[co]
 *     y = act(z [+ r]) [+ r]        (placement of r by d->res_mode)
 * a zero-padded cross-correlation ("Как я свертки ускорял", "А теперь — хардкор на
 * Metal", steps 2-5: window origin = output position * stride - pad, out-of-image
 * taps read as zero, BN and the activation applied while the sum is still in
 * registers, one store per output), in one launch per layer.  When the selected
 * plan splits the reduction over several workgroups, the workspace holds their
 * partial sums and one arrival counter per output tile; with packed weights the
 * last workgroup of a tile adds the partial sums in split order (results do not
 * depend on timing), with OIHW weights a second launch does.
 *   d        : host, layer description.
 *   x        : device [n][c_in][h][w].
 *   w        : device; [c_out][c_in/groups][kh][kw] when d->w_layout is CVX_W_OIHW,
 *              the cvx_pack_weights output for d when it is CVX_W_PACKED.
 *   scale,bias: device [c_out] (from cvx_fold_bn).
 *   residual : device [n][c_out][oh][ow]; required iff d->res_mode != CVX_RES_NONE,
 *              may equal x (read only) but must not overlap y.
 *   y        : device [n][c_out][oh][ow]; must not overlap x, w, scale, bias, residual.
 *              Only the n*c_out*oh*ow elements are written (no row padding).
 *   workspace: device scratch of cvx_conv_workspace_bytes(d) bytes, 16-byte
 *              aligned (may be NULL when that is 0); contents on entry are ignored.
 *              Two calls in flight at once (e.g. on two streams) must not share a
 *              workspace.
 */
CVX_API cvx_status cvx_conv_bn_act(const cvx_conv_desc *d, const float *x, const float *w,
                           const float *scale, const float *bias, const float *residual,
                           float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * cvx_preprocess_u8 -- stem prologue in one pass: u8 HWC RGB frames ->
 * bilinear resize with half-pixel centres (source coordinate
 * s = (d + 0.5) * src/dst - 0.5, clamped below at 0; the upper neighbour clamped
 * to the last row/column) -> v/255 -> (v - mean[c]) / std[c] -> fp32 CHW.
 * The u8 frame is read once and the fp32 tensor written once; interpolated values
 * are not rounded back to u8 ("A fused Ampere preprocess kernel", "The theory"
 * and "My notes from Day 7": the resize is the half-pixel bilinear function).
 *   src          : device, n frames, frame b at src + b*src_h*src_row_bytes,
 *                  pixel (y, x) channel c at + y*src_row_bytes + 3*x + c.
 *   src_row_bytes: >= 3*src_w.
 *   dst          : device [n][3][dst_h][dst_w].
 *   mean, std    : HOST arrays of 3 floats; std[c] != 0.
 */
CVX_API cvx_status cvx_preprocess_u8(const unsigned char *src, int n, int src_h, int src_w,
                             long src_row_bytes, float *dst, int dst_h, int dst_w,
                             const float *mean, const float *std, void *stream);

/*
 * cvx_gap_fc -- classifier tail: v[b][c] = mean over the h*w plane of x[b][c];
 * out[b][o] = sum_c fc_w[o][c] * v[b][c] + fc_b[o] ("Как я свертки ускорял",
 * "Пациента на стол": average pool to 1x1, flatten, Linear).  One launch.
 *   x: device [n][c][h][w]; fc_w: device [out_f][c]; fc_b: device [out_f];
 *   out: device [n][out_f], must not overlap the inputs.
 */
CVX_API cvx_status cvx_gap_fc(const float *x, int n, int c, int h, int w, const float *fc_w,
                      const float *fc_b, int out_f, float *out, void *stream);

/* ---------------------------------------------------------------- layer lists */
enum {
    CVX_L_CONV = 0,    /* cvx_conv_bn_act                                    */
    CVX_L_GAP = 1,     /* global average pool: [n][c][h][w] -> [n][c][1][1]   */
    CVX_L_FC = 2,      /* fc on [n][c][1][1] -> [n][c_out][1][1] (w, bias)   */
    CVX_L_PREPROC = 3  /* cvx_preprocess_u8; only as layer 0 on the raw input */
};

#define CVX_INPUT (-1)  /* `in` / `res` index meaning the network input */
#define CVX_NO_RES (-2) /* `res` index meaning no residual               */

typedef struct cvx_layer {
    int kind;              /* CVX_L_*                                              */
    int in;                /* index of the layer whose output this reads; CVX_INPUT */
    int res;               /* residual source index, CVX_INPUT, or CVX_NO_RES       */
    cvx_conv_desc conv;    /* CONV: full description; GAP: n, c_in, h, w;
                              FC: n, c_in (in features), c_out; PREPROC: n, and
                              h, w = source frame height and width                */
    const float *w;        /* CONV: weights in conv.w_layout; FC: [c_out][c_in]    */
    const float *scale;    /* CONV: folded scale [c_out] (device)                  */
    const float *bias;     /* CONV: folded bias [c_out]; FC: bias [c_out] (device) */
    int dst_h, dst_w;      /* PREPROC: output extent                               */
    float mean[3], std[3]; /* PREPROC: per-channel normalisation (by value)        */
} cvx_layer;

/* Output shape [n][c][h][w] of the last layer of a list (host only; validates
 * the whole list: every `in`/`res` index must name an earlier layer or the
 * input, shapes must chain, residual shapes must equal output shapes). */
CVX_API cvx_status cvx_forward_out_shape(const cvx_layer *layers, int n_layers, int out_shape[4]);

/* Workspace bytes cvx_forward needs: intermediate activations (each 256-byte
 * aligned) plus the largest per-layer workspace.  Intermediates that total at
 * most 256 MiB each get a region of their own (a kernel writing memory another
 * kernel has just read runs slower); larger lists reuse a region once no later
 * layer reads it and two further layers have run.  Host only.  Returns 0 and
 * sets *status on an invalid list when status != NULL. */
CVX_API size_t cvx_forward_workspace_bytes(const cvx_layer *layers, int n_layers, cvx_status *status);

/* Host-only query: the launch plan of a layer list, one line per layer ("i
 * <text>", lines separated by '\n'): a convolution's cvx_conv_plan text; for a
 * pointwise layer that computes its block's 1x1 shortcut in the same kernel,
 * the pair's description and "shortcut=j"; "merged into i" for a layer run
 * inside layer i's kernel (that shortcut, or an FC after its GAP); "chain i-j
 * ..." for a layer of a chain launch (see cvx_forward); "gap", "gap+fc", "fc"
 * or "preprocess" otherwise.  Validates the list as
 * cvx_forward_out_shape does; writes at most buf_len bytes (truncated to fit,
 * always NUL-terminated).  320 bytes per layer always suffice. */
CVX_API cvx_status cvx_forward_plan(const cvx_layer *layers, int n_layers, char *buf, int buf_len);

/*
 * cvx_forward -- run an ordered layer list on one stream, with no host
 * synchronisation: layer i reads the output of layer `in` (and the residual from
 * layer `res`), so a list expresses chains and the MNIST block's shortcut.  The
 * last layer writes `output`; the others write into `workspace`.  This is the
 * whole-network launch sequence the pages replay per inference ("YOLO26N
 * Inference Optimisation", "Baseline benchmark" and "nsys kernel-level
 * breakdown": kernels, not copies, take the time).  A 1x1 shortcut (BN, no
 * activation, packed weights) whose only reader is a later packed 1x1 layer
 * adding it before its activation runs inside that layer's kernel, as one
 * product over both inputs' channels; its output is then never written.
 * With the environment variable CVX_CHAIN=1, a run of 2 to 10 consecutive
 * dense 1x1/3x3 layers with packed weights (rows a multiple of four floats)
 * runs as one persistent launch whose tiles start once the rows they read are
 * complete ("Как я свертки ускорял", "Идеи и следующие шаги", item 3: the
 * whole network in one launch): same results, a larger workspace (the run's
 * row counters).  It is off by default, as one launch per layer is faster on
 * the detector workloads.  A wait in it that exceeds its bound poisons the
 * affected outputs with NaN instead of hanging.
 * With CVX_DSBLOCK=1, a depthwise 3x3 layer (pad 1, no residual) whose only
 * reader is a 1x1 stride-1 layer runs with that layer, and with its 1x1
 * shortcut of the block input (BN, no activation, added before the
 * activation) when it has one, as one kernel at small batches ("Как я свертки
 * ускорял", "А теперь — хардкор на Metal": one launch for the block); the
 * depthwise and shortcut outputs are then never written.  Same results; off by
 * default, as the separate kernels are faster on the MNIST net.
 *   input : device; fp32 NCHW, or u8 NHWC frames when layer 0 is CVX_L_PREPROC.
 *   output: device, shape from cvx_forward_out_shape; must not overlap input/workspace.
 *   workspace: device, >= cvx_forward_workspace_bytes(...) bytes, 256-byte aligned.
 */
CVX_API cvx_status cvx_forward(const cvx_layer *layers, int n_layers, const void *input, float *output,
                       void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------ channels-last variant */
/* Element type of a channels-last layer's activations and weights.  Sums are
 * always accumulated in fp32 and the folded BatchNorm, residual and activation
 * are applied in fp32; CVX_DT_F16 rounds the stored output to IEEE half and
 * CVX_DT_BF16 to bfloat16 (8-bit exponent, 8-bit significand), both to
 * nearest even.  bf16 keeps fp32's range, so activations that would overflow
 * half stay finite, at a coarser step (2^-8 of the value). */
enum { CVX_DT_F32 = 0, CVX_DT_F16 = 1, CVX_DT_BF16 = 2 };

/* Bytes of the packed weights cvx_nhwc_pack_weights writes for `d` and
 * `dtype` (0 when the layer is not supported by the channels-last kernels).
 * Host only. */
CVX_API size_t cvx_nhwc_packed_weights_bytes(const cvx_conv_desc *d, int dtype);

/* Host-only query: the channels-last kernel and tile chosen for `d`, like
 * cvx_conv_plan. */
CVX_API cvx_status cvx_nhwc_plan(const cvx_conv_desc *d, int dtype, char *buf, int buf_len);

/*
 * cvx_nhwc_pack_weights -- one-time transform of OIHW fp32 weights into the
 * order the channels-last kernels read (the weights reordered once to match
 * the NHWC layout: "YOLO26N Inference Optimisation", "NHWC migration --
 * detailed scope", "Weight layout"), rounded to `dtype` (fp16 and bf16 round
 * to nearest even).  Padded with zeros to whole 32-row and 16/32-channel
 * groups.
 *   w_oihw  : device fp32 [c_out][c_in][kh][kw], read only.
 *   w_packed: device, cvx_nhwc_packed_weights_bytes(d, dtype) bytes, written.
 */
CVX_API cvx_status cvx_nhwc_pack_weights(const cvx_conv_desc *d, int dtype, const float *w_oihw,
                                         void *w_packed, void *stream);

/*
 * cvx_conv_bn_act_nhwc -- the fused layer of cvx_conv_bn_act on channels-last
 * tensors: x [n][h][w][c_in], y and residual [n][oh][ow][c_out], all of
 * element type `dtype`; the same arithmetic (cross-correlation, folded BN,
 * residual before or after the activation), fp32 accumulation
 * ("YOLO26N Inference Optimisation", "NHWC migration -- detailed scope";
 * "Как я свертки ускорял", "Идеи и следующие шаги", item 1: fp16).
 * Supported: groups 1, 1x1 or 3x3, stride 1 or 2, c_in a multiple of 4 (fp32)
 * or 8 (fp16, bf16), c_out a multiple of 4; else CVX_ERR_UNSUPPORTED.
 * An unknown dtype is CVX_ERR_ARG.
 * d->w_layout is ignored (the weights are cvx_nhwc_pack_weights' output).
 *   scale, bias: device fp32 [c_out] (cvx_fold_bn).
 *   x, y, residual: device, 16-byte aligned; y must not overlap the inputs;
 *   residual required iff d->res_mode != CVX_RES_NONE (may equal x).
 */
CVX_API cvx_status cvx_conv_bn_act_nhwc(const cvx_conv_desc *d, int dtype, const void *x,
                                        const void *w_packed, const float *scale, const float *bias,
                                        const void *residual, void *y, void *stream);

/* ------------------------------------------------------ placement report */
/*
 * cvx_workgroup_xcds -- where a launch's workgroups run.  Launches n_workgroups
 * workgroups of 64 threads on `stream`; workgroup i writes to xcd[i] the index
 * of the XCD (the die, with its own L2 cache) that ran it.  A diagnostic, not a
 * step of the operation: the split reduction of the implicit-GEMM kernel puts
 * the slices of a tile on workgroups whose indices agree modulo 8, and relies on
 * such workgroups sharing an XCD; this call lets a caller confirm that on its
 * device.  Asynchronous.
 *   xcd: device, n_workgroups ints, 4-byte aligned, written.
 *   n_workgroups: 1 .. 1048576.
 * Errors: CVX_ERR_NULL, CVX_ERR_SHAPE (count out of range), CVX_ERR_ALIGN,
 * CVX_ERR_HIP (launch failed).
 */
CVX_API cvx_status cvx_workgroup_xcds(int *xcd, int n_workgroups, void *stream);

/* ------------------------------------------------- allocation-free variant */
/* Size of the static device scratch array cvx_forward_noalloc uses (32 MiB),
 * held by each GPU the library runs on until the process ends. */
#define CVX_STATIC_SCRATCH_BYTES (32u << 20)

/* CVX_STATIC_SCRATCH_BYTES, for callers that load the library dynamically. */
CVX_API size_t cvx_static_scratch_bytes(void);

/*
 * cvx_forward_noalloc -- cvx_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same layers, kernels and results as cvx_forward, with
 * the workspace (intermediate activations, split partial sums and their
 * arrival counters) taken from a static device array of
 * CVX_STATIC_SCRATCH_BYTES per GPU instead of a caller buffer.  Calls no
 * hipMalloc, hipFree or other allocating routine.  The array's device address
 * is looked up once per device, on the first call with that device current.
 *   layers, n_layers, input, output, stream: as for cvx_forward.
 *   Returns CVX_ERR_SCRATCH (nothing launched) when
 *   cvx_forward_workspace_bytes(layers, n_layers) exceeds CVX_STATIC_SCRATCH_BYTES,
 *   and every error cvx_forward returns.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: intermediates are written
 * before they are read, and split arrival counters carry a per-launch tag).
 * Calls that overlap on one GPU (two streams, or two host threads) race on the
 * array: serialise them.
 */
CVX_API cvx_status cvx_forward_noalloc(const cvx_layer *layers, int n_layers, const void *input,
                                       float *output, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CVX_H */
