// bufio.h -- raw buffer loads and stores (vector memory, 32-bit byte offsets).
//
// A buffer descriptor carries its size; the hardware range-checks every access
// against it: an out-of-range load returns 0 and an out-of-range store is
// dropped.  Kernels use this for zero padding and edge masking without branches
// or per-element selects: an invalid element gets an offset >= 2^31, past any
// tensor this library accepts (the host limits every buffer to < 2^31 bytes).
#pragma once

#include <hip/hip_runtime.h>

namespace cvx {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Offset that is out of range for every descriptor (sizes are < 2^31 bytes).
constexpr unsigned kOOB = 0x80000000u;

// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family GPUs:
// 32-bit data format, default swizzle and cache policy.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRawBufferWord3);
}

// The b32 builtins move raw 32-bit words: reinterpret, never convert.
__device__ __forceinline__ float bload(rsrc_t r, unsigned off_bytes)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off_bytes, 0, 0));
}

__device__ __forceinline__ void bstore(rsrc_t r, unsigned off_bytes, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off_bytes, 0, 0);
}

}  // namespace cvx
