// epilogue.h -- the fused per-output epilogue every convolution kernel ends with.
//
// z = scale[c] * acc + bias[c]            folded BatchNorm (the affine form of
//                                         (v - mean)/sqrt(var + eps)*gamma + beta)
// RES_BEFORE_ACT: y = act(z + r)           the MNIST block's shortcut
// RES_AFTER_ACT : y = act(z) + r           the detector's residual add
// act: none, ReLU = max(0, v), SiLU = v / (1 + exp(-v)).
// Applied while the sum is still in registers, then one store per output
// ("Как я свертки ускорял", "А теперь — хардкор на Metal", steps 4-5;
// "YOLO26N Inference Optimisation", "Improvements", #7).
#pragma once

#include <hip/hip_runtime.h>

#include "cvx.h"

namespace cvx {

__device__ __forceinline__ float apply_act(float v, int act)
{
    if (act == CVX_ACT_RELU) return fmaxf(v, 0.0f);
    if (act == CVX_ACT_SILU) return v / (1.0f + expf(-v));
    return v;
}

// Same activation with the hardware exponential and reciprocal instructions
// (v_exp_f32, v_rcp_f32: about 1 ulp each, far inside the 1e-4 parity bound; a
// correctly rounded reciprocal would expand to a dozen instructions per
// output); exp(-v) overflowing to +inf gives a zero reciprocal and -0 for very
// negative v, as the exact form does.
__device__ __forceinline__ float apply_act_fast(float v, int act)
{
    if (act == CVX_ACT_RELU) return fmaxf(v, 0.0f);
    if (act == CVX_ACT_SILU) return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
    return v;
}

// `r` is read only when res_mode != CVX_RES_NONE.
__device__ __forceinline__ float epilogue(float acc, float sc, float bi, int act, int res_mode,
                                          const float* __restrict__ r, long idx)
{
    float z = fmaf(sc, acc, bi);
    if (res_mode == CVX_RES_BEFORE_ACT) return apply_act(z + r[idx], act);
    if (res_mode == CVX_RES_AFTER_ACT) return apply_act(z, act) + r[idx];
    return apply_act(z, act);
}

}  // namespace cvx
