// gdn_step.hip -- the fused Gated DeltaNet decode step for gfx950.
//
// One workgroup owns a tile (row r, key head hk, HPW value heads of that key
// head, DVS of the d_v state columns).  Per tile it:
//   1. issues the loads of its fp32 state slices (d_k x DVS per head, 16-byte
//      loads, each wave instruction covering whole 128-byte lines), so HBM
//      streams while the rest of the prologue runs;
//   2. runs the conv decode + SiLU of the channels it needs (q and k of hk, v
//      of its heads' columns) into LDS, and writes the advanced conv window of
//      the channels it owns to the write slot;
//   3. L2-normalises q and k (wave butterflies over LDS, done redundantly by
//      every wave so no extra barrier is needed);
//   4. per head: one pass over the register-resident state gives both
//      a = S^T k^ and b = S^T q^ (in-thread over its rows, butterfly across
//      the row groups of a wave, LDS across waves, all in a fixed order);
//      u = beta (v - alpha a); S' = alpha S + k^ u^T; o = alpha b + u (k^.q^),
//      which equals S'^T q^;
//   5. stores S' to the write slot (the read slot in place) and o as bf16.
// The delta rule is Gated DeltaNet's (decay, predict with the decayed state,
// correct, read out); the slot handling follows mstar PR #1139, "What
// changed" (twin slots, keep_in_place) and "Tests" (padding on slot 0).
//
// No MFMA: per state element the step does a handful of FMAs against 8 bytes
// of HBM traffic, far under the fp32 ridge point, so the kernel is written for
// bandwidth: wide coalesced loads, every tile loaded once, no re-reads.

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {

// Thread layout of one head slice (d_k rows x DVS columns): eight row groups
// always, CG = DVS/4 float4 column groups, so NTH = 8 * CG threads.  Thread
// (rg, cg) holds rows rg, rg+8, ..., columns 4cg..4cg+3.  Fixing the row
// groups at eight makes the order of every sum over d_k the same for every
// column split and head grouping: in-thread over m, then the pairwise tree
// ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7)) over row groups -- so twin and
// in-place launches, and padded and unpadded buckets, give identical bits.
template <int DK, int DVS, int HPW>
struct StepCfg {
    static constexpr int RG = 8;                   // row groups
    static constexpr int CG = DVS / 4;             // float4 column groups in a head slice
    static constexpr int NTH = RG * CG;            // threads per head slice
    static constexpr int RPT = DK / RG;            // state rows held by each thread
    static constexpr int NWH = NTH / 64;           // waves per head slice
    static constexpr int NT = NTH * HPW;           // threads per workgroup
    static constexpr int NCH = 2 * DK + HPW * DVS; // conv channels the workgroup needs
    static_assert(CG >= 8 && CG <= 64 && 64 % CG == 0, "a wave must hold whole row groups");
    static_assert(DK % RG == 0, "rows must tile the row groups");
    static_assert(NWH == 1 || NWH == 2 || NWH == 4, "pairwise tree over at most four waves");
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

// Cache-policy bits of the buffer accesses (gfx950): 2 = nt (streaming).  A
// state tile is read once and written once per step and is not touched again
// until the next step of the layer, long after the caches have turned over,
// so both directions stream past the caches.  On MI355X this is what lets the
// write stream overlap the read stream of other tiles: plain stores allocate
// in the caches and their evictions compete with the reads, and streaming
// reads leave the Infinity Cache to the small per-row inputs.
constexpr int kLoadPolicy = 2;
constexpr int kStorePolicy = 2;
// Four waves per SIMD for the whole-tile single-token kernel: a 64-row step
// (1024 head tiles of 256 threads) is then resident on the 256 compute units
// all at once.  The multi-token kernels carry more live state and are left
// to the compiler (forcing four waves there spills to scratch).
constexpr int kWavesPerEU = 4;

template <int DK, int DV, int DVS, int HPW, bool MT>
__global__ __launch_bounds__(2 * DVS * HPW) __attribute__((amdgpu_waves_per_eu((!MT && DVS == DV) ? kWavesPerEU : 1)))
void gdn_step_kernel(StepParams p)
{
    using Cfg = StepCfg<DK, DVS, HPW>;
    static_assert(Cfg::NT == 2 * DVS * HPW, "launch bound must match the layout");
    constexpr int NT = Cfg::NT, NTH = Cfg::NTH, CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT, NWH = Cfg::NWH;
    constexpr int NCH = Cfg::NCH;

    __shared__ float y_lds[NCH + 4]; // + a padding slot for spare conv lanes
    __shared__ float4 red_lds[HPW][NWH][2][CG];

    const int tid = threadIdx.x;
    // head of the group this thread updates; NTH is a multiple of the wave size,
    // so this is wave-uniform -- say so, or every buffer access that depends on
    // it would be compiled as a loop over lanes
    const int hloc = __builtin_amdgcn_readfirstlane(tid / NTH);
    const int ht = tid - hloc * NTH; // thread index inside its head slice
    const int cg = ht % CG;
    const int rg = ht / CG;
    const int wv = ht >> 6;
    const int lane = tid & 63;

    // tile -> (row, key head, head group, column slice)
    int tile = blockIdx.x;
    const int cs = tile % p.n_slices;
    tile /= p.n_slices;
    const int ngrp = p.G / HPW;
    const int grp = tile % ngrp;
    tile /= ngrp;
    const int hk = tile % p.H_k;
    const int r = tile / p.H_k;
    const int hv0 = hk * p.G + grp * HPW;
    const int col0 = cs * DVS;
    const int T = MT ? p.T : 1;

    const int rs = p.read_slot[r];
    const int ws = p.twin ? p.write_slot[r] : rs;
    const bool bad = rs < 0 || rs >= p.N || ws < 0 || ws >= p.N || (p.twin && ws == rs);
    // fused commit: one workgroup per row writes the swapped pair into the
    // next step's slot arrays (distinct from the ones every workgroup of this
    // step reads, so there is no race)
    if (p.next_read_slot && hk == 0 && grp == 0 && cs == 0 && tid == 0) {
        p.next_read_slot[r] = ws;
        p.next_write_slot[r] = rs;
    }
    if (rs == 0 || bad) {
        // padding row (or a row with an unusable slot): touch no slot; out gets
        // +0.0 for padding and NaN for the unusable slot.
        const uint16_t fill = rs == 0 ? (uint16_t)0 : (uint16_t)0x7fc0;
        for (int e = tid; e < T * HPW * DVS; e += NT) {
            const int t = e / (HPW * DVS);
            const int h = (e / DVS) % HPW;
            const int j = e % DVS;
            p.out[(((size_t)r * T + t) * p.H_v + hv0 + h) * DV + col0 + j] = fill;
        }
        return;
    }

    // ---- conv inputs of token 0 first: they are few and on the critical path,
    // and loads complete in order, so issuing them before the state tile lets
    // the conv run while the tile is still streaming in.  Each conv lane takes
    // four consecutive channels: 8-byte loads of its window rows, x and bias,
    // 16-byte loads of its weights, all raw bf16 bits.  NCL lanes do the conv,
    // whole waves except the last, whose spare lanes read lane 0's channels and
    // write their result to a padding slot of y_lds.
    constexpr int NCL = NCH / 4;               // conv lanes (channel quads)
    constexpr int NCW = (NCL + 63) / 64;       // waves' worth of conv lanes
    constexpr int NCQ = (NCL + NT - 1) / NT;   // quads per thread
    const bool own_qk = (grp == 0 && cs == 0);
    const int C = p.C;
    const int hv = hv0 + hloc;
    // gates of token 0, also ahead of the state tile
    float g_t = p.g[(size_t)r * T * p.H_v + hv];
    float b_t = p.beta[(size_t)r * T * p.H_v + hv];
    const uint16_t *xrow = p.x + (size_t)r * p.x_row_stride;
    const uint16_t *cs_rd = p.conv_state + (size_t)rs * 3 * C;
    uint16_t *cs_wr = p.conv_state + (size_t)ws * 3 * C;
    const uint16_t *bias_src = p.conv_b ? p.conv_b : p.conv_w; // conv_w: in-bounds stand-in, unused
    bool conv_wave[NCQ], conv_lane[NCQ], own[NCQ];
    int c[NCQ], e4[NCQ];
    uint4 wlo[NCQ], whi[NCQ];
    uint2 wn0[NCQ], wn1[NCQ], wn2[NCQ], xq[NCQ], bq[NCQ];
#pragma unroll
    for (int k = 0; k < NCQ; ++k) {
        const int li = tid + k * NT;
        conv_wave[k] = (li >> 6) < NCW; // wave-uniform (NT is a multiple of 64)
        conv_lane[k] = li < NCL;
        e4[k] = conv_lane[k] ? 4 * li : 0; // first channel of the quad
        const int e = e4[k];
        const bool isq = e < DK;
        const bool isk = !isq && e < 2 * DK;
        const int ve = e >= 2 * DK ? e - 2 * DK : 0;
        const int h = ve / DVS;
        c[k] = isq ? hk * DK + e
               : isk ? p.H_k * DK + hk * DK + (e - DK)
                     : 2 * p.H_k * DK + (hv0 + h) * DV + col0 + (ve - h * DVS);
        own[k] = conv_lane[k] && ((isq || isk) ? own_qk : true);
        wlo[k] = whi[k] = make_uint4(0, 0, 0, 0);
        wn0[k] = wn1[k] = wn2[k] = xq[k] = bq[k] = make_uint2(0, 0);
        if (conv_wave[k]) {
            const int ck = c[k];
            wlo[k] = *reinterpret_cast<const uint4 *>(p.conv_w + (size_t)ck * 4);
            whi[k] = *reinterpret_cast<const uint4 *>(p.conv_w + (size_t)ck * 4 + 8);
            wn0[k] = *reinterpret_cast<const uint2 *>(cs_rd + ck);
            wn1[k] = *reinterpret_cast<const uint2 *>(cs_rd + C + ck);
            wn2[k] = *reinterpret_cast<const uint2 *>(cs_rd + 2 * C + ck);
            xq[k] = *reinterpret_cast<const uint2 *>(xrow + ck);
            bq[k] = *reinterpret_cast<const uint2 *>(bias_src + ck);
        }
    }
    // conv inputs stay ahead of the tile loads
    __builtin_amdgcn_sched_barrier(0);

    // ---- state slice -> registers
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    const __amdgpu_buffer_rsrc_t rd_tile = tile_rsrc(p.state + ((size_t)rs * p.H_v + hv) * TILE, TILE * 4u);
    const uint32_t voff = (uint32_t)((rg * DV + col0 + 4 * cg) * 4);
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd_tile, voff, m * RG * DV * 4, kLoadPolicy));
    // Every load of the step is now in flight.  Keep the scheduler from sinking
    // any of them below the first wait: under a saturated memory system a load
    // issued after the flood of tile loads queues behind all of them.
    __builtin_amdgcn_sched_barrier(0);

    const bool has_bias = p.conv_b != nullptr;
    for (int t = 0; t < T; ++t) {
        if (MT && t > 0) {
            lds_barrier(); // the previous token's readers of y_lds / red_lds are done
#pragma unroll
            for (int k = 0; k < NCQ; ++k)
                if (conv_wave[k])
                    xq[k] = *reinterpret_cast<const uint2 *>(xrow + (size_t)t * C + c[k]);
            g_t = p.g[((size_t)r * T + t) * p.H_v + hv];
            b_t = p.beta[((size_t)r * T + t) * p.H_v + hv];
        }

        // ---- conv decode + SiLU of this workgroup's channels -> LDS; the
        // window (raw bf16 bits) advances in registers
#pragma unroll
        for (int k = 0; k < NCQ; ++k) {
            if (!conv_wave[k])
                continue;
            const uint4 wl = wlo[k], wh = whi[k];
            const uint2 a0 = wn0[k], a1 = wn1[k], a2 = wn2[k], xx = xq[k], bb = bq[k];
            float4 y;
            y.x = conv_tap4(wl.x, wl.y, a0.x << 16, a1.x << 16, a2.x << 16, xx.x << 16, bb.x << 16, has_bias);
            y.y = conv_tap4(wl.z, wl.w, a0.x & 0xffff0000u, a1.x & 0xffff0000u, a2.x & 0xffff0000u,
                            xx.x & 0xffff0000u, bb.x & 0xffff0000u, has_bias);
            y.z = conv_tap4(wh.x, wh.y, a0.y << 16, a1.y << 16, a2.y << 16, xx.y << 16, bb.y << 16, has_bias);
            y.w = conv_tap4(wh.z, wh.w, a0.y & 0xffff0000u, a1.y & 0xffff0000u, a2.y & 0xffff0000u,
                            xx.y & 0xffff0000u, bb.y & 0xffff0000u, has_bias);
            *reinterpret_cast<float4 *>(&y_lds[conv_lane[k] ? e4[k] : NCH]) = y;
            wn0[k] = a1;
            wn1[k] = a2;
            wn2[k] = xx;
        }
        lds_barrier();

        // ---- L2 norms of q and k (every wave computes the same sums)
        float sq = 0.f, sk = 0.f, sqk = 0.f;
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
        const float rk = 1.0f / sqrtf(sk + p.l2_eps);
        const float qs = rq * p.q_scale;
        const float kq = sqk * rk * qs; // k^ . q^

        // ---- projections of the state onto k^ and q^
        const size_t gi = ((size_t)r * T + t) * p.H_v + hv;
        const float alpha = expf(g_t);
        const float bt = b_t;
        float4 pa = f4_zero(), pb = f4_zero();
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float kh = y_lds[DK + i] * rk;
            const float qh = y_lds[i] * qs;
            pa.x = fmaf(s[m].x, kh, pa.x);
            pa.y = fmaf(s[m].y, kh, pa.y);
            pa.z = fmaf(s[m].z, kh, pa.z);
            pa.w = fmaf(s[m].w, kh, pa.w);
            pb.x = fmaf(s[m].x, qh, pb.x);
            pb.y = fmaf(s[m].y, qh, pb.y);
            pb.z = fmaf(s[m].z, qh, pb.z);
            pb.w = fmaf(s[m].w, qh, pb.w);
        }
        pa.x = xor_sum<CG>(pa.x);
        pa.y = xor_sum<CG>(pa.y);
        pa.z = xor_sum<CG>(pa.z);
        pa.w = xor_sum<CG>(pa.w);
        pb.x = xor_sum<CG>(pb.x);
        pb.y = xor_sum<CG>(pb.y);
        pb.z = xor_sum<CG>(pb.z);
        pb.w = xor_sum<CG>(pb.w);
        if (lane < CG) {
            red_lds[hloc][wv][0][cg] = pa;
            red_lds[hloc][wv][1][cg] = pb;
        }
        lds_barrier();
        // the higher row-group bits live in the wave index: finish the same
        // pairwise tree across the waves of this head slice
        float4 av[NWH], bv[NWH];
#pragma unroll
        for (int w = 0; w < NWH; ++w) {
            av[w] = red_lds[hloc][w][0][cg];
            bv[w] = red_lds[hloc][w][1][cg];
        }
#pragma unroll
        for (int st = 1; st < NWH; st *= 2) {
#pragma unroll
            for (int w = 0; w + st < NWH; w += 2 * st) {
                av[w].x += av[w + st].x; av[w].y += av[w + st].y; av[w].z += av[w + st].z; av[w].w += av[w + st].w;
                bv[w].x += bv[w + st].x; bv[w].y += bv[w + st].y; bv[w].z += bv[w + st].z; bv[w].w += bv[w + st].w;
            }
        }
        const float4 a = av[0], b = bv[0];

        // ---- delta update in registers, and the read-out
        const float *vv = &y_lds[2 * DK + hloc * DVS + 4 * cg];
        float4 u;
        u.x = bt * (vv[0] - alpha * a.x);
        u.y = bt * (vv[1] - alpha * a.y);
        u.z = bt * (vv[2] - alpha * a.z);
        u.w = bt * (vv[3] - alpha * a.w);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float kh = y_lds[DK + rg + RG * m] * rk;
            s[m].x = fmaf(kh, u.x, alpha * s[m].x);
            s[m].y = fmaf(kh, u.y, alpha * s[m].y);
            s[m].z = fmaf(kh, u.z, alpha * s[m].z);
            s[m].w = fmaf(kh, u.w, alpha * s[m].w);
        }
        if (rg == 0) {
            const float o0 = fmaf(u.x, kq, alpha * b.x);
            const float o1 = fmaf(u.y, kq, alpha * b.y);
            const float o2 = fmaf(u.z, kq, alpha * b.z);
            const float o3 = fmaf(u.w, kq, alpha * b.w);
            const u32x2 pk = {(uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16),
                              (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16)};
            __builtin_nontemporal_store(pk, reinterpret_cast<u32x2 *>(p.out + (gi * DV + col0 + 4 * cg)));
        }
    }

    // ---- advanced conv windows of the channels this workgroup owns: a shift
    // of bf16 values, stored as the bits they were read as
#pragma unroll
    for (int k = 0; k < NCQ; ++k) {
        if (own[k]) {
            uint16_t *dst = cs_wr + c[k];
            __builtin_nontemporal_store(u32x2{wn0[k].x, wn0[k].y}, reinterpret_cast<u32x2 *>(dst));
            __builtin_nontemporal_store(u32x2{wn1[k].x, wn1[k].y}, reinterpret_cast<u32x2 *>(dst + C));
            __builtin_nontemporal_store(u32x2{wn2[k].x, wn2[k].y}, reinterpret_cast<u32x2 *>(dst + 2 * C));
        }
    }

    // ---- new state -> write slot (the read slot in place)
    const __amdgpu_buffer_rsrc_t wr_tile = tile_rsrc(p.state + ((size_t)ws * p.H_v + hv) * TILE, TILE * 4u);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), wr_tile, voff, m * RG * DV * 4,
                                               kStorePolicy);
}

template <int DK, int DV, int DVS, int HPW, bool MT>
static hipError_t launch_step(const StepParams &p, hipStream_t stream)
{
    const long long tiles = (long long)p.B * p.H_k * (p.G / HPW) * (DV / DVS);
    if (tiles <= 0)
        return hipSuccess;
    StepParams q = p;
    q.n_slices = DV / DVS;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_step_kernel<DK, DV, DVS, HPW, MT>),
                           dim3((unsigned)tiles), dim3(StepCfg<DK, DVS, HPW>::NT), args, 0, stream);
}

// Column slices per head for a twin step: split d_v only when the rows give
// very few workgroups (with the state cold in HBM, whole tiles win from 16
// rows of 16 heads up; slices stay >= 32 columns).
static int pick_slices(const StepParams &p, int dv)
{
    const long long heads = (long long)p.B * p.H_v;
    if (heads >= 128)
        return 1;
    if (heads >= 32 || dv < 128)
        return 2;
    return 4;
}

template <int DK, int DV>
static hipError_t dispatch_dims(const StepParams &p, hipStream_t stream)
{
    if (!p.twin) {
        // in place: one workgroup owns every channel of its key head (all G
        // value heads, all columns), so no other workgroup reads a conv window
        // it overwrites
        switch (p.G) {
        case 1: return launch_step<DK, DV, DV, 1, true>(p, stream);
        case 2: return launch_step<DK, DV, DV, 2, true>(p, stream);
        case 4: return launch_step<DK, DV, DV, 4, true>(p, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (pick_slices(p, DV)) {
    case 1: return launch_step<DK, DV, DV, 1, false>(p, stream);
    case 2: return launch_step<DK, DV, DV / 2, 1, false>(p, stream);
    default: return launch_step<DK, DV, (DV / 4 >= 32 ? DV / 4 : 32), 1, false>(p, stream);
    }
}

hipError_t launch_gdn_step(const StepParams &p, int d_k, int d_v, hipStream_t stream)
{
    if (d_k == 128 && d_v == 128) return dispatch_dims<128, 128>(p, stream);
    if (d_k == 64 && d_v == 64) return dispatch_dims<64, 64>(p, stream);
    if (d_k == 128 && d_v == 64) return dispatch_dims<128, 64>(p, stream);
    if (d_k == 64 && d_v == 128) return dispatch_dims<64, 128>(p, stream);
    return hipErrorInvalidValue;
}

} // namespace gdn
