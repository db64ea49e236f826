// gdn_step_tile.hip -- the single-token decode step, by head tiles, for
// gfx950: every twin-slot step, and in-place steps whose key heads each have
// one value head.
//
// The same computation as the key-head-group kernel in gdn_step.hip (conv
// decode + SiLU, L2 norms, gated delta rule, read-out), with the same thread
// layout and the same fixed summation order, so both give identical bits.  A
// twin step reads one slot of the request's pair and writes the other (mstar
// PR #1139, "What changed"); in place it writes back to the slot it read,
// which is only safe here when no other workgroup reads the tile's q/k conv
// windows, i.e. with one value head per key head.  A workgroup takes one head
// tile (row, value head, column slice), or two or three whole tiles when that
// keeps each compute unit's reads ahead of its writes (see dispatch_tile).
// The loads are straight-line: a
// padding row (read slot 0) or a row with an unusable slot gets buffer
// resources of size 0, so its loads return zeros without touching memory.
// Without a branch between the slot lookup and the loads, every load is issued
// after a short chain of scalar waits, and each later wait covers exactly the
// loads it needs (measured on MI355X: 0.5-1 us faster at 64 rows than the same
// arithmetic with an early exit and pointer-based loads).  Once every load is
// issued, such a row's workgroups write only its read-out (zeros, or NaN for
// an unusable slot) and leave: a 128-row bucket with 46 real rows then takes
// 22.3 us against 25.9 when they ran the arithmetic on zeros.
//
// Each wave holds all eight row groups of 32 columns, so the projections'
// sums over d_k end inside the wave (lane butterflies) with no LDS round trip
// and no barrier; one barrier publishes the conv outputs, and a multi-tile
// workgroup meets a second one between its last load and its first store.  At
// d_k = d_v = 128 the kernel takes 122 VGPRs (107 with several tiles a
// workgroup), four waves per SIMD, with no spill (measured on MI355X against
// the layout that summed the row groups across waves in LDS: 64 rows 28.4 ->
// 27.6 us a step).

#include "gdn_internal.h"
#include "step_common.h"

#include <atomic>

namespace gdn {

// Everything one head tile carries from its loads to its stores.
template <int DK, int DVS>
struct TileState {
    using Cfg = StepCfg<DK, DVS, 1>;
    static constexpr int NCL = Cfg::NCH / 4;                  // conv lanes (channel quads)
    static constexpr int NCQ = (NCL + Cfg::NT - 1) / Cfg::NT; // quads per thread
    int r, hv, hk, col0, rs, ws;
    bool valid, real, own_qk;
    uint16_t fill;
    float g, beta;
    int e4[NCQ], c[NCQ];
    bool lane_ok[NCQ], own[NCQ];
    uint4 wlo[NCQ], whi[NCQ];
    uint2 wn0[NCQ], wn1[NCQ], wn2[NCQ], xq[NCQ], bq[NCQ];
    float4 s[Cfg::RPT];
};

// What the first round of scalar loads needs, passed as separate leading
// kernel arguments, which the build has the hardware preload into scalar
// registers (gfx950 kernel argument preloading): the slots and gates are then
// requested at once, beside the rest of the arguments.
struct TileArgs {
    const int32_t *read_slot, *write_slot;
    const float *g, *beta;
    int B, H_v, G;
};

// Tile index -> (row, value head, column slice), its slots and gates.  Tiles
// are ordered row-major, then value head, then column slice.
template <int DK, int DV, int DVS, bool TWIN>
__device__ __forceinline__ void tile_locate(TileState<DK, DVS> &t, int tile, const TileArgs &a, const StepParams &p)
{
    constexpr int NS = DV / DVS;
    const int ntiles = a.B * a.H_v * NS;
    t.valid = tile < ntiles;
    const int tt = t.valid ? tile : 0;
    const int cs = tt % NS;
    const int rh = tt / NS;
    t.hv = rh % a.H_v;
    t.r = rh / a.H_v;
    t.hk = t.hv / a.G;
    t.col0 = cs * DVS;
    t.own_qk = (t.hv % a.G == 0) && cs == 0; // the tile that writes back the key head's q/k windows
    // the gates and both slots in one round of scalar loads
    t.g = a.g[(size_t)t.r * a.H_v + t.hv];
    t.beta = a.beta[(size_t)t.r * a.H_v + t.hv];
    constexpr bool twin = TWIN;
    const int32_t rs = a.read_slot[t.r];
    const int32_t ws = twin ? a.write_slot[t.r] : rs;
    t.rs = rs;
    t.ws = ws;
    // unusable: a slot out of range (a negative one too, as unsigned), or a
    // twin row writing over its own read slot or into the null slot (which
    // must stay zero: it never holds a row).  Bitwise, not short-circuit: the
    // branches of || would hold later loads back behind the slots' wait.
    const uint32_t n = (uint32_t)p.N;
    const bool bad = ((uint32_t)rs >= n) | ((uint32_t)ws >= n) | (twin & ((ws == rs) | (ws == 0)));
    t.real = t.valid & (rs != 0) & !bad;
    t.fill = rs == 0 ? (uint16_t)0 : (uint16_t)0x7fc0;
}

// The conv inputs of the tile's channels (q and k of its key head, v of its
// columns): each conv lane takes four consecutive channels -- 16-byte weight
// loads, 8-byte window, x and bias loads, raw bf16 bits.
template <int DK, int DV, int DVS>
__device__ __forceinline__ void tile_issue_small(TileState<DK, DVS> &t, const StepParams &p, int ht)
{
    using TT = TileState<DK, DVS>;
    constexpr int NT = TT::Cfg::NT;
    const int C = p.C;
    const uint32_t cbytes = (uint32_t)C * 2u;
    const __amdgpu_buffer_rsrc_t cw = bf16_rsrc(p.conv_w, cbytes * 4u);
    // unusable rows read through empty resources (multiplied by the flag,
    // not chosen: a choice here becomes a branch)
    const uint32_t real = (uint32_t)t.real;
    const __amdgpu_buffer_rsrc_t win =
        bf16_rsrc(p.conv_state + (size_t)(t.rs * (int)real) * 3 * C, 3u * cbytes * real);
    const __amdgpu_buffer_rsrc_t xr = bf16_rsrc(p.x + (size_t)t.r * p.x_row_stride, cbytes * real);
    const __amdgpu_buffer_rsrc_t br = bf16_rsrc(p.conv_b ? p.conv_b : p.conv_w, p.conv_b ? cbytes : 0u);
#pragma unroll
    for (int q = 0; q < TT::NCQ; ++q) {
        const int li = ht + q * NT;
        t.lane_ok[q] = li < TT::NCL;
        const int e = t.lane_ok[q] ? 4 * li : 0;
        t.e4[q] = e;
        const bool isq = e < DK;
        const bool isk = !isq && e < 2 * DK;
        t.c[q] = isq ? t.hk * DK + e
                 : isk ? p.H_k * DK + t.hk * DK + (e - DK)
                       : 2 * p.H_k * DK + t.hv * DV + t.col0 + (e - 2 * DK);
        t.own[q] = t.lane_ok[q] && ((isq || isk) ? t.own_qk : true);
        const uint32_t o2 = t.lane_ok[q] ? (uint32_t)t.c[q] * 2u : kOOB;
        const uint32_t o8 = t.lane_ok[q] ? (uint32_t)t.c[q] * 8u : kOOB;
        t.wlo[q] = load_b128(cw, o8);
        t.whi[q] = load_b128(cw, o8 + 16u);
        t.wn0[q] = load_b64(win, o2);
        t.wn1[q] = load_b64(win, o2 + cbytes);
        t.wn2[q] = load_b64(win, o2 + 2u * cbytes);
        t.xq[q] = load_b64(xr, o2);
        t.bq[q] = load_b64(br, o2);
    }
}

// The tile's fp32 state slice -> registers (16-byte streaming loads; each wave
// instruction covers whole 128-byte lines).
template <int DK, int DV, int DVS>
__device__ __forceinline__ void tile_issue_state(TileState<DK, DVS> &t, const StepParams &p, uint32_t voff)
{
    using Cfg = typename TileState<DK, DVS>::Cfg;
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    const __amdgpu_buffer_rsrc_t rd =
        tile_rsrc(p.state + ((size_t)(t.rs * (int)t.real) * p.H_v + t.hv) * TILE, TILE * 4u * (uint32_t)t.real);
    const uint32_t vo = voff + (uint32_t)(t.col0 * 4);
#pragma unroll
    for (int m = 0; m < Cfg::RPT; ++m)
        t.s[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd, vo, m * Cfg::RG * DV * 4,
                                                                                 kLoadPolicy));
}

// Conv + SiLU -> LDS, L2 norms, projections, the fixed-order reduction, the
// delta update, the read-out, and the stores of o, the advanced conv windows
// and the new state.
template <int DK, int DV, int DVS, bool INPLACE>
__device__ __forceinline__ void tile_process(TileState<DK, DVS> &t, const StepParams &p, int cg, int rg, int lane,
                                             int ht, uint32_t voff, float *y_lds)
{
    using TT = TileState<DK, DVS>;
    using Cfg = typename TT::Cfg;
    constexpr int RG = Cfg::RG, RPT = Cfg::RPT, NCH = Cfg::NCH;
    constexpr int NCW = (TT::NCL + 63) / 64; // waves' worth of conv lanes
    const bool has_bias = p.conv_b != nullptr;

    // ---- conv decode + SiLU -> LDS; the window advances in registers
#pragma unroll
    for (int q = 0; q < TT::NCQ; ++q) {
        if (!t.real || ((ht + q * Cfg::NT) >> 6) >= NCW) // wave-uniform; no memory access inside
            continue;
        const uint4 wl = t.wlo[q], wh = t.whi[q];
        const uint2 a0 = t.wn0[q], a1 = t.wn1[q], a2 = t.wn2[q], xx = t.xq[q], bb = t.bq[q];
        float4 y;
        y.x = conv_tap4(wl.x, wl.y, a0.x << 16, a1.x << 16, a2.x << 16, xx.x << 16, bb.x << 16, has_bias);
        y.y = conv_tap4(wl.z, wl.w, a0.x & 0xffff0000u, a1.x & 0xffff0000u, a2.x & 0xffff0000u,
                        xx.x & 0xffff0000u, bb.x & 0xffff0000u, has_bias);
        y.z = conv_tap4(wh.x, wh.y, a0.y << 16, a1.y << 16, a2.y << 16, xx.y << 16, bb.y << 16, has_bias);
        y.w = conv_tap4(wh.z, wh.w, a0.y & 0xffff0000u, a1.y & 0xffff0000u, a2.y & 0xffff0000u,
                        xx.y & 0xffff0000u, bb.y & 0xffff0000u, has_bias);
        *reinterpret_cast<float4 *>(&y_lds[t.lane_ok[q] ? t.e4[q] : NCH]) = y;
        t.wn0[q] = a1;
        t.wn1[q] = a2;
        t.wn2[q] = xx;
    }
    lds_barrier();

    // ---- L2 norms of q and k (every wave computes the same sums)
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    float4 a = f4_zero(), b = f4_zero();
    float rk = 0.f, kq = 0.f;
    const float alpha = expf(t.g);
    const float bt = t.beta;
    if (t.real) {
#pragma unroll
    for (int i = lane; i < DK; i += 64) {
        const float qv = y_lds[i], kv = y_lds[DK + i];
        sq = fmaf(qv, qv, sq);
        sk = fmaf(kv, kv, sk);
        sqk = fmaf(qv, kv, sqk);
    }
    sq = xor_sum<1>(sq);
    sk = xor_sum<1>(sk);
    sqk = xor_sum<1>(sqk);
    const float rq = 1.0f / sqrtf(sq + p.l2_eps);
    rk = 1.0f / sqrtf(sk + p.l2_eps);
    const float qs = rq * p.q_scale;
    kq = sqk * rk * qs; // k^ . q^

    // ---- projections of the state onto k^ and q^
    float4 pa = f4_zero(), pb = f4_zero();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const float kh = y_lds[DK + i] * rk;
        const float qh = y_lds[i] * qs;
        pa.x = fmaf(t.s[m].x, kh, pa.x);
        pa.y = fmaf(t.s[m].y, kh, pa.y);
        pa.z = fmaf(t.s[m].z, kh, pa.z);
        pa.w = fmaf(t.s[m].w, kh, pa.w);
        pb.x = fmaf(t.s[m].x, qh, pb.x);
        pb.y = fmaf(t.s[m].y, qh, pb.y);
        pb.z = fmaf(t.s[m].z, qh, pb.z);
        pb.w = fmaf(t.s[m].w, qh, pb.w);
    }
    // the eight row groups are lane bits 3-5 of one wave: butterflies over
    // bits 3, 4, 5 form the pairwise tree ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7))
    // in every lane, with no LDS round trip and no barrier
    pa.x = xor_sum<8>(pa.x);
    pa.y = xor_sum<8>(pa.y);
    pa.z = xor_sum<8>(pa.z);
    pa.w = xor_sum<8>(pa.w);
    pb.x = xor_sum<8>(pb.x);
    pb.y = xor_sum<8>(pb.y);
    pb.z = xor_sum<8>(pb.z);
    pb.w = xor_sum<8>(pb.w);
    a = pa;
    b = pb;
    }
    if (!t.real)
        return;

    // ---- delta update in registers, and the read-out
    const float *vv = &y_lds[2 * DK + 4 * cg];
    float4 u;
    u.x = bt * (vv[0] - alpha * a.x);
    u.y = bt * (vv[1] - alpha * a.y);
    u.z = bt * (vv[2] - alpha * a.z);
    u.w = bt * (vv[3] - alpha * a.w);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float kh = y_lds[DK + rg + RG * m] * rk;
        t.s[m].x = fmaf(kh, u.x, alpha * t.s[m].x);
        t.s[m].y = fmaf(kh, u.y, alpha * t.s[m].y);
        t.s[m].z = fmaf(kh, u.z, alpha * t.s[m].z);
        t.s[m].w = fmaf(kh, u.w, alpha * t.s[m].w);
    }
    const float o0 = fmaf(u.x, kq, alpha * b.x);
    const float o1 = fmaf(u.y, kq, alpha * b.y);
    const float o2 = fmaf(u.z, kq, alpha * b.z);
    const float o3 = fmaf(u.w, kq, alpha * b.w);
    const uint32_t f2 = (uint32_t)t.fill * 0x10001u;
    const u32x2 pk = {t.real ? ((uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16)) : f2,
                      t.real ? ((uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16)) : f2};
    // o: row group 0 of every column group (lanes 0-7 of each wave)
    const __amdgpu_buffer_rsrc_t orow =
        bf16_rsrc(p.out + ((size_t)t.r * p.H_v + t.hv) * DV, t.valid ? (uint32_t)DV * 2u : 0u);
    __builtin_amdgcn_raw_buffer_store_b64(pk, orow, rg == 0 ? (uint32_t)(t.col0 + 4 * cg) * 2u : kOOB, 0, 0);

    // ---- advanced conv windows of the channels this tile owns: a shift of
    // bf16 values, stored as the bits they were read as.  Streaming stores,
    // like the state's: a window is read again only at the layer's next step
    // (measured on MI355X at 64 rows: 27.45 against 27.6 us a step plain)
    const uint32_t cbytes = (uint32_t)p.C * 2u;
    const __amdgpu_buffer_rsrc_t wwin = bf16_rsrc(p.conv_state + (size_t)(t.real ? t.ws : 0) * 3 * p.C,
                                                  t.real ? 3u * cbytes : 0u);
#pragma unroll
    for (int q = 0; q < TT::NCQ; ++q) {
        if (((ht + q * Cfg::NT) >> 6) >= NCW) // waves with no conv lane own nothing
            continue;
        const uint32_t o2w = t.own[q] ? (uint32_t)t.c[q] * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{t.wn0[q].x, t.wn0[q].y}, wwin, o2w, 0, kStorePolicy);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{t.wn1[q].x, t.wn1[q].y}, wwin, o2w + cbytes, 0, kStorePolicy);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{t.wn2[q].x, t.wn2[q].y}, wwin, o2w + 2u * cbytes, 0, kStorePolicy);
    }

    // ---- new state -> write slot
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    const __amdgpu_buffer_rsrc_t wr =
        tile_rsrc(p.state + ((size_t)(t.real ? t.ws : 0) * p.H_v + t.hv) * TILE, t.real ? TILE * 4u : 0u);
    const uint32_t vo = voff + (uint32_t)(t.col0 * 4);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t.s[m]), wr, vo, m * RG * DV * 4,
                                               kStorePolicy);
}

template <int DK, int DV, int DVS, bool INPLACE, int TPW>
__global__ __launch_bounds__(2 * DVS * TPW) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void gdn_step_tile_kernel(const int32_t *read_slot, const int32_t *write_slot, const float *g, const float *beta, int B,
                          int H_v, int G, int xcd_groups, StepParams p)
{
    using TT = TileState<DK, DVS>;
    using Cfg = typename TT::Cfg;
    constexpr int CG = Cfg::CG, NCH = Cfg::NCH, NTS = Cfg::NT;
    static_assert(NTS == 2 * DVS, "launch bound must match the layout");
    static_assert(Cfg::RG == 8 && DVS % 32 == 0, "a wave holds the eight row groups of 32 columns");

    __shared__ float y_all[TPW][NCH + 4]; // + a padding slot for spare conv lanes

    // TPW head tiles a workgroup, 2 DVS threads each.  Thread layout inside a
    // tile: wave w holds columns 32 w .. 32 w + 31 of the slice, lane l column
    // group 8 w + l % 8 (four columns) and row group l / 8, i.e. rows l / 8,
    // l / 8 + 8, ..., so a row's projection is a sum inside one wave
    const int tid = threadIdx.x;
    const int sub = __builtin_amdgcn_readfirstlane(tid / NTS); // wave-uniform
    const int ht = tid - sub * NTS;
    const int lane = tid & 63;
    const int rg = lane >> 3;
    const int cg = (ht >> 6) * 8 + (lane & 7);
    const uint32_t voff = (uint32_t)((rg * DV + 4 * cg) * 4);
    float *y_lds = y_all[sub];

    // workgroup -> tile group; with xcd_groups (the grid size, 0: off),
    // workgroups (which the hardware deals to the eight XCDs in turn) are
    // renumbered so that each XCD gets a contiguous run of tile groups.  The
    // grid size comes with the arguments: read from the dispatch packet it
    // took a round of scalar loads of its own.
    const int n = xcd_groups, x = blockIdx.x % 8, q = n / 8, rr = n % 8;
    const int grp = n ? x * q + min(x, rr) + (int)blockIdx.x / 8 : (int)blockIdx.x;
    TT t;
    tile_locate<DK, DV, DVS, !INPLACE>(t, grp * TPW + sub, TileArgs{read_slot, write_slot, g, beta, B, H_v, G}, p);
    tile_issue_small<DK, DV, DVS>(t, p, ht);
    __builtin_amdgcn_sched_barrier(0); // the small loads stay ahead of the tile loads
    tile_issue_state<DK, DV, DVS>(t, p, voff);
    // every load is in flight; keep the scheduler from sinking any below the first wait
    __builtin_amdgcn_sched_barrier(0);
    if (!t.real) {
        // a padding row or an unusable slot: its loads above touched no memory;
        // write the read-out fill, fold in the commit, and skip the arithmetic
        const uint32_t f2 = (uint32_t)t.fill * 0x10001u;
        const __amdgpu_buffer_rsrc_t orow =
            bf16_rsrc(p.out + ((size_t)t.r * p.H_v + t.hv) * DV, t.valid ? (uint32_t)DV * 2u : 0u);
        if (ht < CG)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{f2, f2}, orow, (uint32_t)(t.col0 + 4 * ht) * 2u, 0, 0);
        if (p.next_read_slot && ht == 0 && t.valid && t.hv == 0 && t.col0 == 0) {
            p.next_read_slot[t.r] = t.ws;
            p.next_write_slot[t.r] = t.rs;
        }
        if constexpr (TPW == 1)
            return;
    }
    // the tiles of real rows do the work; the others only meet the workgroup
    // barrier after the conv
    tile_process<DK, DV, DVS, INPLACE>(t, p, cg, rg, lane, ht, voff, y_lds);

    // fused commit: the workgroup of a row's first tile writes the swapped
    // pair into the next step's slot arrays (distinct from the ones this step
    // reads, so there is no race)
    if (t.real && p.next_read_slot && ht == 0 && t.hv == 0 && t.col0 == 0) {
        p.next_read_slot[t.r] = t.ws;
        p.next_write_slot[t.r] = t.rs;
    }
}

template <int DK, int DV, int DVS, int TPW>
static hipError_t launch_tile(const StepParams &p, hipStream_t stream)
{
    StepParams q = p;
    q.n_slices = DV / DVS;
    const long long tiles = (long long)p.B * p.H_v * q.n_slices;
    if (tiles <= 0)
        return hipSuccess;
    const unsigned groups = (unsigned)((tiles + TPW - 1) / TPW);
    int xcd_groups = p.xcd_groups ? (int)groups : 0;
    const int32_t *rs = p.read_slot, *ws = p.write_slot;
    const float *g = p.g, *beta = p.beta;
    int B = p.B, H_v = p.H_v, G = p.G;
    void *args[] = {&rs, &ws, &g, &beta, &B, &H_v, &G, &xcd_groups, &q};
    const void *k = p.twin ? reinterpret_cast<const void *>(&gdn_step_tile_kernel<DK, DV, DVS, false, TPW>)
                           : reinterpret_cast<const void *>(&gdn_step_tile_kernel<DK, DV, DVS, true, TPW>);
    return hipLaunchKernel(k, dim3(groups), dim3(2 * DVS * TPW), args, 0, stream);
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Launch shape.  Up to 2047 head tiles a step is one round of workgroups on
// the 256 CUs, and its time follows the CUs that get the most tiles.
//
// Tiles a workgroup (twin writes of 128 x 128 tiles).  When a round puts
// three or four tiles on every CU, one workgroup of four tiles a CU (1024
// threads, a quarter of the workgroups to dispatch and to start) beats four
// workgroups of one.  Measured on MI355X, 16 heads, slots cold and scattered,
// us a step, one tile / two tiles with all of a workgroup's loads in before
// any store / four tiles, each wave storing as soon as its own tile is
// updated: 48 rows 22.0 / 21.6 / 20.3, 56 rows 25.8 / 23.5 / 22.5, 64 rows
// 27.7 / 26.3 / 25.65.  The wait for the workgroup's loads helped two tiles
// and costs four (26.4 at 64 rows), so it is gone; three tiles measured
// 29.4 at 64 rows.  One tile stays best at 128 rows (53.6 against 54.0) and
// in place at 64 and 128 rows (27.7 against 27.9 and 28.4).
//
// Column slices per head otherwise.  Halving the tiles evens out the CUs' share
// when heads mod 256 is between 1 and 128 (two half tiles where one CU had a
// whole one more than another); otherwise whole tiles win, as slicing adds the
// q/k conv a slice more.  Measured on MI355X with the state cold, 16 heads a
// row, us a step whole against sliced: 8 rows 6.66 / 5.78, 12 rows 7.20 / 7.26,
// 16 rows 8.13 / 8.46, 24 rows 12.61 / 11.06, 40 rows 19.18 / 18.41.  Under 128
// tiles two slices of 64 columns beat four of 32, whose 64-thread workgroups
// run the whole q/k conv on one wave (1 row 4.94 against 5.16 us, 2 rows 5.10
// against 5.30, 4 rows 5.32 against 5.48).  Never in place: every slice
// reads the head's q/k conv windows and one of them writes them back, so in
// place a slice that starts late could read an advanced window; with whole
// tiles and one value head per key head, no other workgroup reads them.
//
// In place, workgroups are handed to the XCDs in contiguous runs of tiles
// (64 rows 28.5 -> 28.1 us, 128 rows 53.7 -> 52.7); for twin writes that
// order measured equal or slower and is not used.
template <int DK, int DV>
static hipError_t dispatch_tile(const StepParams &p, hipStream_t stream)
{
    StepParams q = p;
    q.xcd_groups = p.twin ? 0 : 1; // launch_tile sets the grid size
    const long long heads = (long long)p.B * p.H_v;
    const long long rem = heads % 256;
    if constexpr (DK == 128 && DV == 128) {
        const long long cus = device_cus();
        if (p.twin && heads * 2 > 5 * cus && heads <= 4 * cus)
            return launch_tile<DK, DV, DV, 4>(q, stream);
    }
    if (!p.twin || heads >= 2048 || (heads >= 128 && (rem == 0 || rem > 128)))
        return launch_tile<DK, DV, DV, 1>(q, stream);
    return launch_tile<DK, DV, DV / 2, 1>(q, stream);
}

static hipError_t dispatch_dims(const StepParams &p, int d_k, int d_v, hipStream_t stream)
{
    if (d_k == 128 && d_v == 128) return dispatch_tile<128, 128>(p, stream);
    if (d_k == 64 && d_v == 64) return dispatch_tile<64, 64>(p, stream);
    if (d_k == 128 && d_v == 64) return dispatch_tile<128, 64>(p, stream);
    if (d_k == 64 && d_v == 128) return dispatch_tile<64, 128>(p, stream);
    return hipErrorInvalidValue;
}

// Twin steps of 128 x 128 heads that need more than one round of the
// four-tile workgroups (over 4 heads a CU) go as P launches over consecutive
// rows, P = ceil(heads / 4 CUs), when each part still puts more than 2.5
// heads on every CU: each launch is then one round of four-tile workgroups.
// Rows are independent (a key head's windows belong to one row), so the
// parts give the bits of one launch.  Measured on MI355X, same session, us a
// step: 128 rows of 16 heads 52.6 -> 49.9; the 9B-like layer (64 rows of 32
// value heads) 51.4 -> 48.6.
hipError_t launch_gdn_step_tile(const StepParams &p, int d_k, int d_v, hipStream_t stream)
{
    const long long heads = (long long)p.B * p.H_v, cus = device_cus();
    const long long parts = (heads + 4 * cus - 1) / (4 * cus);
    if (p.twin && d_k == 128 && d_v == 128 && parts > 1 && parts <= p.B && heads * 2 > 5 * cus * parts) {
        hipError_t e = hipSuccess;
        for (long long k = 0; k < parts && e == hipSuccess; ++k) {
            const int r0 = (int)(p.B * k / parts), r1 = (int)(p.B * (k + 1) / parts);
            StepParams q = p;
            q.B = r1 - r0;
            q.x = p.x + (size_t)r0 * p.x_row_stride;
            q.g = p.g + (size_t)r0 * p.T * p.H_v;
            q.beta = p.beta + (size_t)r0 * p.T * p.H_v;
            q.read_slot = p.read_slot + r0;
            q.write_slot = p.write_slot + r0;
            q.out = p.out + (size_t)r0 * p.T * p.H_v * d_v;
            if (p.next_read_slot) {
                q.next_read_slot = p.next_read_slot + r0;
                q.next_write_slot = p.next_write_slot + r0;
            }
            e = dispatch_dims(q, d_k, d_v, stream);
        }
        return e;
    }
    return dispatch_dims(p, d_k, d_v, stream);
}

} // namespace gdn
