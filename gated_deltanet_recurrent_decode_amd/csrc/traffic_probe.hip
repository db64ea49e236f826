// traffic_probe.hip -- the decode step's state traffic with no arithmetic (gfx950).
//
// Calibration in the manner of mstar PR #1139, "Numbers": a kernel with the
// GDN step's reads and writes and no math, plus its read-only and write-only
// halves, gives the practical bandwidth ceiling of this access pattern.  Modes
// 0-3 use the grid, thread layout, slot addressing and cache policies of the
// fused step with one head per workgroup and whole d_v rows.  Mode 4 moves the
// same bytes as mode 2 as one plain contiguous copy of B consecutive slots, the
// best case for HBM: the distance between the two is what slot addressing and
// per-tile dependencies cost.

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Cache-policy bits as the step uses them: streaming loads and stores.
constexpr int kProbeLoad = 2;
constexpr int kProbeStore = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(float *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

template <int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void traffic_probe_kernel(ProbeParams p)
{
    // the step's whole-tile layout: eight row groups, wave w holding columns
    // 32 w .. 32 w + 31, lane l column group 8 w + l % 8 and row group l / 8
    constexpr int RG = 8, RPT = DK / RG;
    static_assert(NTH == 2 * DV && DV % 32 == 0, "two threads a column, as in the step");
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int cg = (tid >> 6) * 8 + (lane & 7);
    const int h = blockIdx.x % p.H;
    const int r = blockIdx.x / p.H;
    const int rs = p.read_slot[r];
    const int ws = (p.mode == 0 || p.mode == 3) ? rs : p.write_slot[r];
    if (rs <= 0 || rs >= p.N || ws <= 0 || ws >= p.N)
        return;
    const __amdgpu_buffer_rsrc_t rd = probe_rsrc(p.state + ((size_t)rs * p.H + h) * TILE, TILE * 4u);
    const __amdgpu_buffer_rsrc_t wr = probe_rsrc(p.state + ((size_t)ws * p.H + h) * TILE, TILE * 4u);
    const uint32_t voff = (uint32_t)((rg * DV + 4 * cg) * 4);
    float4 s[RPT];
    if (p.mode != 1) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            s[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, voff, m * RG * DV * 4, kProbeLoad));
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            s[m] = make_float4(p.one, p.one, p.one, p.one);
    }
    if (p.mode == 0) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            acc += s[m].x + s[m].y + s[m].z + s[m].w;
        if (acc == -3.0e38f) // never true for finite state; keeps the loads alive
            p.sink[0] = acc;
        return;
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float4 v = make_float4(s[m].x * p.one, s[m].y * p.one, s[m].z * p.one, s[m].w * p.one);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), wr, voff, m * RG * DV * 4,
                                               kProbeStore);
    }
}

// Mode 4: the B slots from read_slot[0] on -> the B slots from write_slot[0]
// on, one contiguous copy: each thread moves four 16-byte elements per pass,
// all four loads in flight before the stores.  A range that does not lie in
// [1, N) makes the launch a no-op (the host has checked that B slots are
// under 2 GiB, so every byte offset fits 32 bits).
__global__ __launch_bounds__(256) void stream_copy_kernel(ProbeParams p, uint32_t slot_floats)
{
    const int rs = p.read_slot[0], ws = p.write_slot[0];
    if (rs < 1 || ws < 1 || (long long)rs + p.B > p.N || (long long)ws + p.B > p.N)
        return;
    const uint32_t n4 = slot_floats / 4u * (uint32_t)p.B;
    const __amdgpu_buffer_rsrc_t S = probe_rsrc(p.state + (size_t)rs * slot_floats, n4 * 16u);
    const __amdgpu_buffer_rsrc_t D = probe_rsrc(p.state + (size_t)ws * slot_floats, n4 * 16u);
    const uint32_t stride = gridDim.x * 256u * 4u;
    for (uint32_t i = blockIdx.x * 1024u + threadIdx.x; i < n4; i += stride) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) // past-the-end lanes read 0 from the buffer bounds
            v[u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(S, (i + 256u * u) * 16u, 0,
                                                                                   kProbeLoad));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 w = make_float4(v[u].x * p.one, v[u].y * p.one, v[u].z * p.one, v[u].w * p.one);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), D, (i + 256u * u) * 16u, 0,
                                                   kProbeStore);
        }
    }
}

template <int DK, int DV>
static hipError_t launch_probe(const ProbeParams &p, hipStream_t stream)
{
    constexpr int NTH = 2 * DV;
    const long long tiles = (long long)p.B * p.H;
    if (tiles <= 0)
        return hipSuccess;
    ProbeParams q = p;
    if (p.mode == 4) {
        uint32_t slot_floats = (uint32_t)p.H * DK * DV;
        const uint32_t n4 = slot_floats / 4u * (uint32_t)p.B;
        const uint32_t blocks = (n4 + 1023u) / 1024u;
        const unsigned grid = blocks < 4096u ? blocks : 4096u;
        void *args[] = {&q, &slot_floats};
        return hipLaunchKernel(reinterpret_cast<const void *>(&stream_copy_kernel), dim3(grid), dim3(256), args, 0,
                               stream);
    }
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&traffic_probe_kernel<DK, DV, NTH>), dim3((unsigned)tiles),
                           dim3(NTH), args, 0, stream);
}

hipError_t launch_traffic_probe(const ProbeParams &p, int d_k, int d_v, hipStream_t stream)
{
    if (d_k == 128 && d_v == 128) return launch_probe<128, 128>(p, stream);
    if (d_k == 64 && d_v == 64) return launch_probe<64, 64>(p, stream);
    if (d_k == 128 && d_v == 64) return launch_probe<128, 64>(p, stream);
    if (d_k == 64 && d_v == 128) return launch_probe<64, 128>(p, stream);
    return hipErrorInvalidValue;
}

} // namespace gdn
