// step_common.h -- pieces shared by the decode-step kernels of libgdn (gfx950):
// the thread layout of a head tile, buffer resources, the width-4 conv tap,
// and the cache policies of the state traffic.
#pragma once

#include "device_common.h"

namespace gdn {

// Thread layout of one head slice (d_k rows x DVS columns): eight row groups
// always, CG = DVS/4 float4 column groups, so NTH = 8 * CG threads.  Thread
// (rg, cg) holds rows rg, rg+8, ..., columns 4cg..4cg+3.  Fixing the row
// groups at eight makes the order of every sum over d_k the same for every
// column split and head grouping: in-thread over m, then the pairwise tree
// ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7)) over row groups -- so twin and
// in-place launches, and padded and unpadded buckets, give identical bits.
// Both step kernels keep the row groups in lane bits 3-5 (a wave holds 32
// columns of all eight row groups), so the tree ends inside the wave.
template <int DK, int DVS, int HPW>
struct StepCfg {
    static constexpr int RG = 8;                   // row groups
    static constexpr int CG = DVS / 4;             // float4 column groups in a head slice
    static constexpr int NTH = RG * CG;            // threads per head slice
    static constexpr int RPT = DK / RG;            // state rows held by each thread
    static constexpr int NT = NTH * HPW;           // threads per workgroup
    static constexpr int NCH = 2 * DK + HPW * DVS; // conv channels the workgroup needs
    static_assert(CG >= 8 && CG <= 64 && 64 % CG == 0, "a wave must hold whole row groups");
    static_assert(DK % RG == 0, "rows must tile the row groups");
    static_assert(NTH % 64 == 0, "a head slice is whole waves of eight column groups");
    static_assert(NT <= 1024, "workgroup too large");
};

// Raw buffer resource over one head's d_k x d_v fp32 tile: every state access
// is a 32-bit per-lane offset plus a uniform row offset, so the sixteen loads
// of a thread share one address register, and nothing outside the tile can
// be touched (out-of-range lanes read 0 and drop their stores).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(float *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// A byte offset past the end of every buffer resource used here: a load there
// returns 0 and a store there is dropped, with no memory access.
constexpr uint32_t kOOB = 0x80000000u;

// Raw buffer resources over bf16 and fp32 arrays of `bytes` bytes (under 2 GiB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bf16_rsrc(const uint16_t *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rsrc(const float *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint2 load_b64(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// One channel of the width-4 conv with SiLU, from bf16 values already moved
// into the high half of a 32-bit word (so they read as fp32): taps 0-1 in
// w01, taps 2-3 in w23 (tap 3 multiplies the current token), the three
// window values oldest first, the token, and the bias (added when present).
__device__ __forceinline__ float conv_tap4(uint32_t w01, uint32_t w23, uint32_t a0, uint32_t a1, uint32_t a2,
                                           uint32_t xv, uint32_t bias, bool has_bias)
{
    float acc = __uint_as_float(w01 << 16) * __uint_as_float(a0);
    acc = fmaf(__uint_as_float(w01 & 0xffff0000u), __uint_as_float(a1), acc);
    acc = fmaf(__uint_as_float(w23 << 16), __uint_as_float(a2), acc);
    acc = fmaf(__uint_as_float(w23 & 0xffff0000u), __uint_as_float(xv), acc);
    if (has_bias)
        acc += __uint_as_float(bias);
    return silu(acc);
}

// Cache-policy bits of the buffer accesses (gfx950): 1 = sc0, 2 = nt, 16 = sc1.
// A state tile is read once and written once per step and is not touched
// again until the next step of the layer, long after the caches have turned
// over.  Loads stream (nt): measured on MI355X, streaming reads run at ~7.1
// TB/s against ~6.3 for plain ones.  Stores stream too, twin or in place.
// Measured with at least 768 MiB of state written between two visits of a
// slot (so nothing is left of it in the 256 MB Infinity Cache, which takes in
// written lines but not streamed reads): 64 rows 28.3 us with streaming
// stores against 30.5 written through (sc0 sc1) and 30.7 plain; 128 rows 54.2
// against 58.3 and 59.2.  Written-through stores only look faster when the
// next read of the slot comes soon enough to hit the Infinity Cache.  On the
// current tile kernel at 64 rows: 27.7 us a step streaming, 29.5 written
// through, 30.2 plain.
constexpr int kLoadPolicy = 2;
constexpr int kStorePolicy = 2;
// Four waves per SIMD for the twin single-token kernel: a 64-row step (1024
// head tiles of 256 threads) is then resident on the 256 compute units all at
// once.  The in-place kernel carries all G value heads of a key head and T
// tokens and is left to the compiler (forcing four waves there spills).
constexpr int kWavesPerEU = 4;


} // namespace gdn
