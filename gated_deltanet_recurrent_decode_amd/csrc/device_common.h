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

// The value of lane (lane ^ D) for D = 1, 2, 4, 8 within a 16-lane row, by
// DPP moves (no LDS round trip): quad permutations for 1 and 2, a shift left
// or right by 4 picked by lane bit 2 for 4, a rotation by 8 for 8.
template <int D>
__device__ __forceinline__ float dpp_xor(float v)
{
    const int x = __float_as_int(v);
    if constexpr (D == 1)
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false)); // quad_perm [1,0,3,2]
    if constexpr (D == 2)
        return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false)); // quad_perm [2,3,0,1]
    if constexpr (D == 4) {
        const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);   // row_shl:4, lane + 4
        const int down = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false); // row_shr:4, lane - 4
        return __int_as_float((__lane_id() & 4) ? down : up);
    }
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false)); // row_ror:8
}

// Butterfly sum over the lanes whose index differs in bits [log2(from), 6):
// afterwards every participating lane holds the identical sum (IEEE addition
// is commutative, so both partners of each exchange compute the same value).
// Distances up to 8 move by DPP; 16 and 32 by gfx950's row swaps, whose two
// results are a lane's own value and its partner's, in one order or the other.
template <int FROM>
__device__ __forceinline__ float xor_sum(float v)
{
    if constexpr (FROM <= 1)
        v += dpp_xor<1>(v);
    if constexpr (FROM <= 2)
        v += dpp_xor<2>(v);
    if constexpr (FROM <= 4)
        v += dpp_xor<4>(v);
    if constexpr (FROM <= 8)
        v += dpp_xor<8>(v);
    if constexpr (FROM <= 16) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const float other = (__lane_id() & 16) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
        v += other;
    }
    if constexpr (FROM <= 32) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const float other = (__lane_id() & 32) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
        v += other;
    }
    return v;
}

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

} // namespace gdn
