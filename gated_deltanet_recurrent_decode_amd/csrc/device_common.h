// device_common.h -- small device helpers shared by the gfx950 kernels of libgdn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 that already holds a bf16 value -> its bit pattern (exact truncation).
__device__ __forceinline__ uint16_t f32_to_bf16_exact(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }

// SiLU with IEEE division and the device library's expf.
__device__ __forceinline__ float silu(float y) { return y / (1.0f + expf(-y)); }

// Barrier for LDS hand-offs only: waits for this wave's LDS traffic and joins
// the workgroup, without waiting for outstanding global loads (which a full
// __syncthreads() fence would), so the state tile keeps streaming in across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Butterfly sum over the lanes whose index differs in bits [log2(from), 6):
// afterwards every participating lane holds the identical sum (IEEE addition
// is commutative, so both partners of each exchange compute the same value).
template <int FROM>
__device__ __forceinline__ float xor_sum(float v)
{
#pragma unroll
    for (int off = FROM; off < 64; off <<= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

} // namespace gdn
