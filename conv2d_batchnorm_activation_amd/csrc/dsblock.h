// dsblock.h -- the depthwise-separable block kernel (k_dsblock.hip): its
// arguments, the planner's test and the launcher.  Not part of the public ABI.
#pragma once

#include "cvx_internal.h"

namespace cvx {

// A depthwise-separable block in one launch (k_dsblock.hip): depthwise 3x3
// (+BN, act) -> pointwise 1x1 (+BN) + shortcut -> act, for small batches.
struct DsBlockArgs {
    const float* x;                 // block input [n][cin][h][w]
    const float* dw_w;              // [cin][9]
    const float* dw_scale;
    const float* dw_bias;
    const float* pw_w;              // 1x1 [cout][cin] (OIHW) or the packed 1x1 order
    const float* pw_scale;
    const float* pw_bias;
    const float* skip_w;            // projection shortcut weights, or null
    const float* skip_scale;
    const float* skip_bias;
    const float* res;               // identity shortcut [n][cout][oh][ow] (res_mode != NONE, no projection)
    float* y;                       // [n][cout][oh][ow]
    int n, cin, h, w, cout, oh, ow, stride;
    int dw_act, pw_act, res_mode;
    bool pw_packed, skip_packed;
    int runp;                       // set by launch_dsblock: staged floats per input plane
    long pw_elems, skip_elems;      // set by launch_dsblock: floats the weight reads may touch
};
constexpr long kDsBlockMaxGroups = 512;  // workgroups above which the block runs as separate layers
bool dsblock_fits(const ConvGeom& dw, const ConvGeom& pw, const ConvGeom* skip);
void dsblock_describe(const ConvGeom& dw, const ConvGeom& pw, bool proj, char* buf, int len);
hipError_t launch_dsblock(DsBlockArgs a, hipStream_t s);

}  // namespace cvx
