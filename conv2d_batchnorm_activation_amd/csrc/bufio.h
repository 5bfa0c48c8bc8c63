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

// Touches every 64-byte line of the kernel's argument block with scalar loads
// issued together and waits once.  Left alone, the compiler loads the fields
// in several batches, each waited on before the next is issued, so a large
// argument block costs several memory round trips per workgroup; afterwards
// every field is a scalar-cache hit.
template <int BYTES>
__device__ __forceinline__ void warm_kernargs()
{
    typedef const __attribute__((address_space(4))) unsigned* kptr;
    const kptr k = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
    unsigned v = k[(BYTES - 4) / 4];
#pragma unroll
    for (int o = 0; o < BYTES - 4; o += 64) v |= k[o / 4];
    asm volatile("" ::"s"(v));
}

// Waits until at most n of this wave's vector-memory operations are outstanding
// (loads complete in issue order), leaving the other counters alone.  The count
// is an immediate, so one instruction per value; above 35 it waits for all.
__device__ __forceinline__ void wait_vm_at_most(int n)
{
#define CVX_VM(k) \
    case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
    switch (n) {
        CVX_VM(0) CVX_VM(1) CVX_VM(2) CVX_VM(3) CVX_VM(4) CVX_VM(5) CVX_VM(6) CVX_VM(7) CVX_VM(8) CVX_VM(9)
        CVX_VM(10) CVX_VM(11) CVX_VM(12) CVX_VM(13) CVX_VM(14) CVX_VM(15) CVX_VM(16) CVX_VM(17) CVX_VM(18)
        CVX_VM(19) CVX_VM(20) CVX_VM(21) CVX_VM(22) CVX_VM(23) CVX_VM(24) CVX_VM(25) CVX_VM(26) CVX_VM(27)
        CVX_VM(28) CVX_VM(29) CVX_VM(30) CVX_VM(31) CVX_VM(32) CVX_VM(33) CVX_VM(34) CVX_VM(35)
        default: __builtin_amdgcn_s_waitcnt(0); break;
    }
#undef CVX_VM
}

// Workgroup barrier that orders LDS accesses only: global loads in flight stay
// in flight across it (a plain __syncthreads() also waits for those).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace cvx
