// traffic_probe.hip -- calibration kernels: the decode step's state traffic
// with no arithmetic, in several workgroup designs (gfx950).
//
// The method of mstar PR #1139, "Numbers": a kernel with the GDN step's reads
// and writes and no math, plus its read-only and write-only halves, gives the
// practical bandwidth ceiling of the step's access pattern.  Here the same
// traffic can be taken by several designs, so that the ceiling is the best of
// them rather than one kernel:
//   - tile designs: the fused step's thread layout (a wave holds the eight row
//     groups of 32 columns, 256 threads a 128-wide tile), one, two or four
//     whole tiles a workgroup; with more than one, every wave waits for the
//     whole workgroup's loads before any store, as the step does;
//   - chunk designs: plain one-shot copies, each workgroup moving one
//     contiguous chunk of a tile (256 threads x 16, 8 or 1 16-byte loads a
//     lane, or 1024 threads x 1);
//   - either over the step's own slots (tile t of row r at slot read_slot[r])
//     or over contiguous slots (B consecutive slots from read_slot[0], written
//     to B consecutive slots from write_slot[0]);
//   - optionally holding every workgroup's stores until a set time after it
//     started, which puts the whole launch's reads ahead of its writes (HBM
//     serves a mix of reads and writes far worse than either alone); this
//     only measures what such phasing is worth;
//   - an empty kernel and a kernel that loads one slot index and then one
//     piece of that slot's tile: the launch floor of small batches.
// Every access is a buffer access through a resource sized to its tile or
// chunk, and every slot is range-checked, so nothing outside the pool can be
// touched whatever the slot arrays hold.

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Cache-policy bits as the step uses them: streaming loads and stores.
constexpr int kProbeLoad = 2;
constexpr int kProbeStore = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

// Byte offsets (from the pool's start) of the read and write copy of head
// tile t (row t / H, head t % H); false when a slot is unusable (the
// workgroup then moves nothing).
__device__ __forceinline__ bool probe_tile(const ProbeParams &p, int t, size_t tile_bytes, size_t &src, size_t &dst)
{
    const int r = t / p.H, h = t % p.H;
    int rs, ws;
    const bool own = p.traffic == 0 || p.traffic == 3; // read only, or written back in place
    if (p.layout == 1) {
        const int r0 = p.read_slot[0], w0 = own ? r0 : p.write_slot[0];
        if (r0 < 1 || (long long)r0 + p.B > p.N || w0 < 1 || (long long)w0 + p.B > p.N)
            return false;
        rs = r0 + r;
        ws = w0 + r;
    } else {
        rs = p.read_slot[r];
        ws = own ? rs : p.write_slot[r];
    }
    if (rs < 1 || rs >= p.N || ws < 1 || ws >= p.N)
        return false;
    src = ((size_t)rs * p.H + h) * tile_bytes;
    dst = ((size_t)ws * p.H + h) * tile_bytes;
    return true;
}

// The constant clock (100 MHz), read only when a hold is asked for, and only
// after the slot indices are in: the compiler treats the clock read as a
// memory side effect, and with one ahead of them it no longer loads the slot
// indices through the scalar cache (measured: every chunk design ~2 us slower).
__device__ __forceinline__ uint64_t probe_clock(uint32_t hold)
{
    return hold ? __builtin_amdgcn_s_memrealtime() : 0;
}

// Hold this wave until `hold` ticks of the 100 MHz constant clock after t0.
__device__ __forceinline__ void probe_hold(uint64_t t0, uint32_t hold)
{
    if (hold == 0)
        return;
    while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)hold)
        __builtin_amdgcn_s_sleep(4);
}

// Tile designs: TPW whole d_k x d_v tiles a workgroup, 2 d_v threads a tile,
// at the step's occupancy (its registers allow four waves a SIMD; the launch
// reserves LDS so that no more workgroups share a CU than the step's do).
template <int DK, int DV, int TPW>
__global__ __launch_bounds__(2 * DV * TPW) void probe_tile_kernel(ProbeParams p)
{
    constexpr int RG = 8, RPT = DK / RG, NTS = 2 * DV;
    static_assert(DV % 32 == 0, "a wave holds 32 columns");
    constexpr uint32_t TILE = (uint32_t)DK * DV * 4u;
    const int tid = threadIdx.x;
    const int sub = __builtin_amdgcn_readfirstlane(tid / NTS);
    const int ht = tid - sub * NTS;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int cg = (ht >> 6) * 8 + (lane & 7);
    const int t = blockIdx.x * TPW + sub;
    size_t so = 0, dof = 0;
    const bool ok = t < p.B * p.H && probe_tile(p, t, TILE, so, dof);
    char *pool = reinterpret_cast<char *>(p.state);
    const __amdgpu_buffer_rsrc_t rd = probe_rsrc(pool + so, ok ? TILE : 0u);
    const __amdgpu_buffer_rsrc_t wr = probe_rsrc(pool + dof, ok ? TILE : 0u);
    const uint32_t voff = (uint32_t)((rg * DV + 4 * cg) * 4);
    if (p.traffic == 1) { // write only: ones
        const uint64_t t0 = probe_clock(p.hold_ticks);
        probe_hold(t0, p.hold_ticks);
        const unsigned one = __float_as_uint(p.one);
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{one, one, one, one}, wr, voff, m * RG * DV * 4, kProbeStore);
        return;
    }
    u32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_amdgcn_raw_buffer_load_b128(rd, voff, m * RG * DV * 4, kProbeLoad);
    __builtin_amdgcn_sched_barrier(0); // every load goes out before the clock is read
    const uint64_t t0 = probe_clock(p.hold_ticks);
    if (p.traffic == 0) {
        unsigned acc = 0;
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            acc += s[m].x ^ s[m].y ^ s[m].z ^ s[m].w;
        if (acc == 0x9e3779b9u && p.one == 3.0f) // never true: p.one is 1; keeps the loads alive
            p.sink[0] = (float)acc;
        return;
    }
    if constexpr (TPW > 1) {
        // as the step: every wave of the workgroup has its data before any stores
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    }
    probe_hold(t0, p.hold_ticks);
    // stores straight from the registers the loads filled: staging the data
    // through other registers made the compiler write a staging register
    // right behind a 16-byte store that had not read it yet (seen on MI355X)
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(s[m], wr, voff, m * RG * DV * 4, kProbeStore);
}

// Chunk designs: workgroup c moves chunk c of NTH * L * 16 bytes, thread i
// the 16-byte elements i, i + NTH, ... of it (a wave instruction covers 1 KiB).
template <int NTH, int L>
__global__ __launch_bounds__(NTH) void probe_chunk_kernel(ProbeParams p, uint32_t tile_bytes)
{
    constexpr uint32_t CH = (uint32_t)NTH * L * 16u;
    const int per = (int)(tile_bytes / CH);
    const int c = blockIdx.x;
    size_t so = 0, dof = 0;
    const bool ok = c < p.B * p.H * per && probe_tile(p, c / per, tile_bytes, so, dof);
    const size_t part = (size_t)(c % per) * CH;
    char *pool = reinterpret_cast<char *>(p.state);
    const __amdgpu_buffer_rsrc_t rd = probe_rsrc(pool + so + part, ok ? CH : 0u);
    const __amdgpu_buffer_rsrc_t wr = probe_rsrc(pool + dof + part, ok ? CH : 0u);
    const uint32_t vo = threadIdx.x * 16u;
    if (p.traffic == 1) { // write only: ones
        const uint64_t t0 = probe_clock(p.hold_ticks);
        probe_hold(t0, p.hold_ticks);
        const unsigned one = __float_as_uint(p.one);
#pragma unroll
        for (int m = 0; m < L; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{one, one, one, one}, wr, vo, m * NTH * 16, kProbeStore);
        return;
    }
    u32x4 v[L];
#pragma unroll
    for (int m = 0; m < L; ++m)
        v[m] = __builtin_amdgcn_raw_buffer_load_b128(rd, vo, m * NTH * 16, kProbeLoad);
    __builtin_amdgcn_sched_barrier(0);
    const uint64_t t0 = probe_clock(p.hold_ticks);
    if (p.traffic == 0) {
        unsigned acc = 0;
#pragma unroll
        for (int m = 0; m < L; ++m)
            acc += v[m].x ^ v[m].y ^ v[m].z ^ v[m].w;
        if (acc == 0x9e3779b9u && p.one == 3.0f)
            p.sink[0] = (float)acc;
        return;
    }
    probe_hold(t0, p.hold_ticks);
#pragma unroll
    for (int m = 0; m < L; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(v[m], wr, vo, m * NTH * 16, kProbeStore);
}

// The launch floor: a kernel that does nothing.
__global__ __launch_bounds__(64) void probe_empty_kernel(ProbeParams p)
{
    if (p.one == 3.0f && threadIdx.x == 0) // never true
        p.sink[0] = 1.0f;
}

// The small-batch floor: load a slot index, then one 16-byte piece a lane of
// that slot's first tile (a dependent pair of loads, as every step starts).
__global__ __launch_bounds__(256) void probe_slot_load_kernel(ProbeParams p, uint32_t tile_bytes)
{
    const int rs = p.read_slot[0];
    const bool ok = rs >= 1 && rs < p.N;
    char *pool = reinterpret_cast<char *>(p.state);
    const __amdgpu_buffer_rsrc_t rd = probe_rsrc(pool + (ok ? (size_t)rs * p.H * tile_bytes : 0), ok ? 4096u : 0u);
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rd, threadIdx.x * 16u, 0, kProbeLoad);
    if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9e3779b9u && p.one == 3.0f)
        p.sink[0] = 1.0f;
}

template <int NTH, int L>
static hipError_t launch_chunk(ProbeParams q, uint32_t tile_bytes, hipStream_t stream)
{
    constexpr uint32_t CH = (uint32_t)NTH * L * 16u;
    if (tile_bytes % CH != 0)
        return hipErrorInvalidValue;
    const long long chunks = (long long)q.B * q.H * (tile_bytes / CH);
    void *args[] = {&q, &tile_bytes};
    return hipLaunchKernel(reinterpret_cast<const void *>(&probe_chunk_kernel<NTH, L>), dim3((unsigned)chunks),
                           dim3(NTH), args, 0, stream);
}

template <int DK, int DV, int TPW>
static hipError_t launch_tiles(ProbeParams q, hipStream_t stream)
{
    const long long tiles = (long long)q.B * q.H;
    void *args[] = {&q};
    // the step's 128 x 128 kernels fit four 256-thread tiles on a CU (registers):
    // reserve a quarter of the 160 KiB LDS per tile so the probe fits no more
    const size_t lds = DK == 128 && DV == 128 && TPW < 4 ? (size_t)TPW * 40 * 1024 : 0;
    return hipLaunchKernel(reinterpret_cast<const void *>(&probe_tile_kernel<DK, DV, TPW>),
                           dim3((unsigned)((tiles + TPW - 1) / TPW)), dim3(2 * DV * TPW), args, lds, stream);
}

template <int DK, int DV>
static hipError_t launch_probe(const ProbeParams &p, hipStream_t stream)
{
    const uint32_t tile_bytes = (uint32_t)DK * DV * 4u;
    ProbeParams q = p;
    switch (p.shape) {
    case 0: return launch_tiles<DK, DV, 1>(q, stream);
    case 1: return DK == 128 && DV == 128 ? launch_tiles<DK, DV, 2>(q, stream) : hipErrorInvalidValue;
    case 2: return DK == 128 && DV == 128 ? launch_tiles<DK, DV, 4>(q, stream) : hipErrorInvalidValue;
    case 3: return launch_chunk<256, 16>(q, tile_bytes, stream);
    case 4: return launch_chunk<256, 8>(q, tile_bytes, stream);
    case 5: return launch_chunk<256, 1>(q, tile_bytes, stream);
    case 6: return launch_chunk<1024, 1>(q, tile_bytes, stream);
    case 7: {
        void *args[] = {&q};
        return hipLaunchKernel(reinterpret_cast<const void *>(&probe_empty_kernel), dim3(1), dim3(64), args, 0,
                               stream);
    }
    case 8: {
        uint32_t tb = tile_bytes;
        void *args[] = {&q, &tb};
        return hipLaunchKernel(reinterpret_cast<const void *>(&probe_slot_load_kernel), dim3(1), dim3(256), args, 0,
                               stream);
    }
    }
    return hipErrorInvalidValue;
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
