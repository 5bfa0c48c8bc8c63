/*
 * cvx_oracle.c -- plain, slow, obviously correct fp64 CPU oracle for the fused
 * convolution + BatchNorm + activation layer and its stem prologue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no source, header, table or helper with the HIP library.
 *
 * Every function computes its definition directly, in double precision, with no
 * blocking, fusion or reordering of the sums.  The only concession to speed is an
 * OpenMP loop over independent output planes, which does not change any sum.
 *
 * Sources (titles of the pages that define the operation):
 *   [P1] "YOLO26N Inference Optimisation" (vision-rs docs)
 *   [P2] "Как я свертки ускорял" ("How I sped up convolutions")
 *   [P3] "A fused Ampere preprocess kernel"
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1
#define ORC_ACT_SILU 2

#define ORC_RES_NONE 0
#define ORC_RES_BEFORE_ACT 1
#define ORC_RES_AFTER_ACT 2

/* Output extent of a padded, strided window: floor((in + 2*pad - k) / stride) + 1. */
int oracle_out_extent(int in, int k, int stride, int pad)
{
    int span = in + 2 * pad - k;
    if (span < 0 || stride < 1) return 0;
    return span / stride + 1;
}

/*
 * Grouped 2-D cross-correlation (no kernel flip), zero padding.
 * [P2] "А теперь — хардкор на Metal", steps 2-3: the window's top-left corner
 * is the output position times the stride minus the padding; taps that fall
 * outside the image contribute nothing (virtual zero).
 * [P1] "NHWC migration", "What NHWC is": NCHW offset n*C*H*W + c*H*W + h*W + w.
 * Weights are OIHW: [cout][cin/groups][kh][kw].
 *
 * out[b][co][oy][ox] = sum_{c < cin/groups} sum_{i < kh} sum_{j < kw}
 *       x[b][g*cin_g + c][oy*stride - pad + i][ox*stride - pad + j] * w[co][c][i][j]
 * with g = co / (cout/groups).
 */
void oracle_conv2d(const double *x, int n, int cin, int h, int w,
                   const double *wt, int cout, int kh, int kw,
                   int stride, int pad, int groups, double *out)
{
    const int oh = oracle_out_extent(h, kh, stride, pad);
    const int ow = oracle_out_extent(w, kw, stride, pad);
    const int cin_g = cin / groups;
    const int cout_g = cout / groups;
    const long planes = (long)n * cout;

#pragma omp parallel for schedule(dynamic, 1)
    for (long pc = 0; pc < planes; ++pc) {
        const long b = pc / cout;
        const int co = (int)(pc % cout);
        const int g = co / cout_g;
        for (int oy = 0; oy < oh; ++oy) {
            for (int ox = 0; ox < ow; ++ox) {
                double acc = 0.0;
                for (int c = 0; c < cin_g; ++c) {
                    const int ci = g * cin_g + c;
                    for (int i = 0; i < kh; ++i) {
                        const int iy = oy * stride - pad + i;
                        if (iy < 0 || iy >= h) continue;
                        for (int j = 0; j < kw; ++j) {
                            const int ix = ox * stride - pad + j;
                            if (ix < 0 || ix >= w) continue;
                            const double xv = x[((b * cin + ci) * (long)h + iy) * w + ix];
                            const double wv = wt[(((long)co * cin_g + c) * kh + i) * kw + j];
                            acc += xv * wv;
                        }
                    }
                }
                out[((b * cout + co) * (long)oh + oy) * ow + ox] = acc;
            }
        }
    }
}

/* Inference BatchNorm on one value, unfolded:
 * (v - mean) / sqrt(var + eps) * gamma + beta.
 * [P2] "А теперь — хардкор на Metal", step 4 (the full form; the copy in [P1]
 * "NHWC migration" drops the variance term, read as an extraction slip). */
static double bn_unfolded(double v, double gamma, double beta, double mean, double var, double eps)
{
    return (v - mean) / sqrt(var + eps) * gamma + beta;
}

/* ReLU = max(0, v) ([P2] step 4); SiLU = v * sigmoid(v) = v / (1 + exp(-v)),
 * the textbook definition of the activation the [P1] kernels are named after. */
static double activation(double v, int act)
{
    if (act == ORC_ACT_RELU) return v > 0.0 ? v : 0.0;
    if (act == ORC_ACT_SILU) return v / (1.0 + exp(-v));
    return v;
}

/* Apply act to an array in place (exposed for the activation pins). */
void oracle_activation(double *v, long count, int act)
{
    for (long i = 0; i < count; ++i) v[i] = activation(v[i], act);
}

/*
 * Fused layer, computed unfused: convolution, then unfolded BatchNorm per output
 * channel, then the residual and the activation.
 *   res_mode BEFORE_ACT: y = act(bn(conv) + r)   ([P2] "Пациента на стол": the
 *                        block adds its shortcut before the final ReLU)
 *   res_mode AFTER_ACT : y = act(bn(conv)) + r   ([P1] "Improvements" #7: the
 *                        residual add that followed the fused conv+BN+SiLU kernel)
 * residual has the output's shape and may be NULL when res_mode is NONE.
 */
void oracle_conv_bn_act(const double *x, int n, int cin, int h, int w,
                        const double *wt, int cout, int kh, int kw,
                        int stride, int pad, int groups,
                        const double *gamma, const double *beta,
                        const double *mean, const double *var, double eps,
                        int act, int res_mode, const double *residual, double *y)
{
    const int oh = oracle_out_extent(h, kh, stride, pad);
    const int ow = oracle_out_extent(w, kw, stride, pad);
    const long plane = (long)oh * ow;
    oracle_conv2d(x, n, cin, h, w, wt, cout, kh, kw, stride, pad, groups, y);
    const long planes = (long)n * cout;
#pragma omp parallel for schedule(static)
    for (long pc = 0; pc < planes; ++pc) {
        const int co = (int)(pc % cout);
        for (long q = 0; q < plane; ++q) {
            const long idx = pc * plane + q;
            double z = bn_unfolded(y[idx], gamma[co], beta[co], mean[co], var[co], eps);
            if (res_mode == ORC_RES_BEFORE_ACT) {
                z = activation(z + residual[idx], act);
            } else if (res_mode == ORC_RES_AFTER_ACT) {
                z = activation(z, act) + residual[idx];
            } else {
                z = activation(z, act);
            }
            y[idx] = z;
        }
    }
}

/* BatchNorm folded to a per-channel affine map, the reading of the "weight
 * folding" named in [P1] "Baseline benchmark":
 *   scale = gamma / sqrt(var + eps),  bias = beta - mean * scale,
 * so that bn(v) = scale * v + bias. */
void oracle_fold_bn(const double *gamma, const double *beta, const double *mean,
                    const double *var, double eps, int c, double *scale, double *bias)
{
    for (int i = 0; i < c; ++i) {
        scale[i] = gamma[i] / sqrt(var[i] + eps);
        bias[i] = beta[i] - mean[i] * scale[i];
    }
}

/* Global average pool: v[b][c] = (1 / (h*w)) * sum over the plane.
 * ([P2] "Пациента на стол": AdaptiveAvgPool2d(1) before the classifier.) */
void oracle_gap(const double *x, int n, int c, int h, int w, double *out)
{
    const long plane = (long)h * w;
    for (long pc = 0; pc < (long)n * c; ++pc) {
        double s = 0.0;
        for (long q = 0; q < plane; ++q) s += x[pc * plane + q];
        out[pc] = s / (double)plane;
    }
}

/* Fully connected layer: out[b][o] = sum_i W[o][i] * v[b][i] + bias[o].
 * ([P2] "Пациента на стол": Linear(192, num_classes) after the pool.) */
void oracle_fc(const double *v, int n, int in_f, const double *wt, const double *bias,
               int out_f, double *out)
{
    for (int b = 0; b < n; ++b) {
        for (int o = 0; o < out_f; ++o) {
            double s = 0.0;
            for (int i = 0; i < in_f; ++i) s += wt[(long)o * in_f + i] * v[(long)b * in_f + i];
            out[(long)b * out_f + o] = s + bias[o];
        }
    }
}

/*
 * Stem prologue: u8 HWC (RGB) -> bilinear resize with half-pixel centres ->
 * /255 -> per-channel (v - mean_c) / std_c -> f32 CHW, in one pass.
 * [P3] "The theory": read the u8 frame once, keep the middle values in
 * registers, write the f32 tensor once; "My notes from Day 7": the resize must
 * be the function OpenCV computes, i.e. bilinear with half-pixel centres.
 *
 * Source coordinate of destination column dx: sx = (dx + 0.5) * (Ws / Wd) - 0.5,
 * clamped below at 0; x0 = floor(sx), x1 = min(x0 + 1, Ws - 1), fx = sx - x0.
 * Same for rows.  The interpolation is done on the raw u8 values as reals, with
 * no rounding back to u8 (the fused path keeps the middle values in registers).
 * src rows are src_row_bytes apart; pixel (y, x) channel ch is at
 * src[img*src_h*src_row_bytes + y*src_row_bytes + 3*x + ch].
 */
void oracle_preprocess(const uint8_t *src, int n, int src_h, int src_w, long src_row_bytes,
                       int dst_h, int dst_w, const double *mean, const double *stdv, double *dst)
{
    const double ry = (double)src_h / (double)dst_h;
    const double rx = (double)src_w / (double)dst_w;
    for (int b = 0; b < n; ++b) {
        const uint8_t *img = src + (long)b * src_h * src_row_bytes;
        for (int dy = 0; dy < dst_h; ++dy) {
            double sy = ((double)dy + 0.5) * ry - 0.5;
            if (sy < 0.0) sy = 0.0;
            int y0 = (int)floor(sy);
            if (y0 > src_h - 1) y0 = src_h - 1;
            const int y1 = y0 + 1 < src_h ? y0 + 1 : src_h - 1;
            const double fy = sy - (double)y0;
            for (int dx = 0; dx < dst_w; ++dx) {
                double sx = ((double)dx + 0.5) * rx - 0.5;
                if (sx < 0.0) sx = 0.0;
                int x0 = (int)floor(sx);
                if (x0 > src_w - 1) x0 = src_w - 1;
                const int x1 = x0 + 1 < src_w ? x0 + 1 : src_w - 1;
                const double fx = sx - (double)x0;
                for (int ch = 0; ch < 3; ++ch) {
                    const double p00 = img[(long)y0 * src_row_bytes + 3 * x0 + ch];
                    const double p01 = img[(long)y0 * src_row_bytes + 3 * x1 + ch];
                    const double p10 = img[(long)y1 * src_row_bytes + 3 * x0 + ch];
                    const double p11 = img[(long)y1 * src_row_bytes + 3 * x1 + ch];
                    const double top = (1.0 - fx) * p00 + fx * p01;
                    const double bot = (1.0 - fx) * p10 + fx * p11;
                    const double v = (1.0 - fy) * top + fy * bot;
                    dst[(((long)b * 3 + ch) * dst_h + dy) * dst_w + dx] =
                        (v / 255.0 - mean[ch]) / stdv[ch];
                }
            }
        }
    }
}

/* Threads the OpenMP runtime will use (reported with the CPU baseline). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
