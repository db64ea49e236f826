// gdn_step.hip -- the fused Gated DeltaNet decode step for gfx950, in place
// (keep_in_place), T tokens a row.
//
// One workgroup owns one key head of a row (or several: four of one value
// head each, or two of two, for single-token steps where that is faster) with
// all of their value heads, so no other workgroup reads a conv window it
// overwrites.  The tokens go in blocks of up to eight.  Per block the
// workgroup:
//   1. issues the loads of the block's conv inputs (weights, bias, the window
//      before the block, x of its tokens) and gates; before the first block
//      it then issues the loads of its value heads' fp32 state tiles (d_k x
//      d_v each, 16-byte loads, each wave instruction covering whole 128-byte
//      lines), so the conv runs while HBM streams the tiles;
//   2. runs the conv decode + SiLU of its channels (q and k of the key head, v
//      of its value heads) for every token of the block into LDS, and the
//      gates exp(g), beta;
//   3. L2-normalises each token's q and k (one wave a token and key head, the
//      sums in the same lane order as the single-token kernel) and leaves q^
//      (times q_scale) and k^ in LDS;
//   4. per token and head: one pass over the register-resident state gives
//      both a = S^T k^ and b = S^T q^ (in-thread over its rows, then
//      butterflies across the eight row groups, which sit in lane bits 3-5 of
//      one wave, so the sum ends inside the wave in a fixed order);
//      u = beta (v - alpha a); S' = alpha S + k^ u^T; o = alpha b + u (k^.q^),
//      which equals S'^T q^;
//   5. after the last token, stores the state and the advanced window back to
//      the read slot; o goes out as bf16 every token.
// Steps 2-3 leave every register they used free again before the state
// update, so the kernel fits four waves a SIMD with no spills at any head
// grouping.  The delta rule is Gated DeltaNet's (decay, predict with the
// decayed state, correct, read out); the slot handling follows mstar PR #1139,
// "What changed" (keep_in_place for prefill, split walks and the mixed step's
// decode half) and "Tests" (padding on slot 0).  Single-token steps that
// allow one head tile per workgroup (every twin step, and in place with one
// value head per key head) run in gdn_step_tile.hip instead, with the same
// thread layout and the same arithmetic in the same order, so both give the
// same bits; this kernel takes token walks, per-token states, in-place GQA,
// and the single-token in-place sizes that run faster grouped (see
// walk_key_heads).
//
// No MFMA: per state element the step does a handful of FMAs against 8 bytes
// of HBM traffic, far under the fp32 ridge point, so the kernel is written for
// bandwidth: wide coalesced loads, every tile loaded once, no re-reads.

#include "gdn_internal.h"
#include "step_common.h"

namespace gdn {

// Tokens whose conv outputs are computed together before their state updates.
constexpr int kWalkBlock = 8;

// Everything a conv lane loads for one block of tokens.
template <int NCQ, int TB>
struct ConvIn {
    uint4 wlo[NCQ], whi[NCQ]; // taps 0-3 of its four channels
    uint2 a0[NCQ], a1[NCQ], a2[NCQ]; // the window before the block, oldest first
    uint2 bq[NCQ];
    uint2 xs[NCQ][TB];        // x of the block's tokens (0 past the last token)
    float g, beta;            // gate of (token tid / HPW, value head tid % HPW)
};

// G value heads a key head, KPW key heads a workgroup (HPW = G KPW head
// slices); TOKENS: per-token states (p.token_slots set), a separate
// instantiation, so the plain walk carries none of its registers.
template <int DK, int DV, int G, int KPW, bool TOKENS>
__global__ __launch_bounds__(2 * DV * G * KPW) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void gdn_step_kernel(const int32_t *read_slot, int H_k, int N, StepParams p)
{
    constexpr int HPW = G * KPW;
    using Cfg = StepCfg<DK, DV, HPW>;
    constexpr int NT = Cfg::NT, NTH = Cfg::NTH, RG = Cfg::RG, RPT = Cfg::RPT;
    constexpr int NCHK = 2 * DK + G * DV; // conv channels of one key head: q, k, its value heads' v
    constexpr int NCH = KPW * NCHK;
    constexpr int TB = kWalkBlock;
    constexpr int NW = NT / 64;                // waves
    constexpr int NCL = NCH / 4;               // conv lanes (channel quads)
    constexpr int NCW = (NCL + 63) / 64;       // waves' worth of conv lanes
    constexpr int NCQ = (NCL + NT - 1) / NT;   // quads per thread
    static_assert(TB * HPW <= NT, "one gate load a thread");
    static_assert(TB >= 3, "the window before a later block is the previous block's last three tokens");

    // the block's conv outputs (+ a padding slot for spare conv lanes); after
    // the norm phase q and k hold q^ q_scale and k^
    __shared__ float y_blk[TB][NCH + 4];
    __shared__ float kq_blk[TB][KPW];     // k^ . q^ of each token and key head
    __shared__ float2 gate_blk[TB][HPW];  // exp(g), beta of each token and value head
    // each conv lane's own inputs, parked here as soon as they arrive so no
    // register holds them through the conv: rows 0-2 the window before the
    // block (oldest first), rows 3.. the block's x, then the bias and the
    // four 8-byte pieces of the weights.  One array indexed [row][lane], so
    // every access is one per-lane address plus a constant.
    constexpr int RB = 3 + TB, RW = RB + 1, NROW = RW + 4;
    __shared__ uint2 conv_st[NROW][NCL];

    const int tid = threadIdx.x;
    // head of the group this thread updates; NTH is a multiple of the wave size,
    // so this is wave-uniform -- say so, or every buffer access that depends on
    // it would be compiled as a loop over lanes
    const int hloc = __builtin_amdgcn_readfirstlane(tid / NTH);
    const int ht = tid - hloc * NTH; // thread index inside its head slice
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // each wave holds 32 columns (eight column groups in lane bits 0-2) of
    // all eight row groups (lane bits 3-5)
    const int cg = (ht >> 6) * 8 + (lane & 7);
    const int rg = lane >> 3;

    // workgroup -> (row, group of KPW key heads); the value heads of key head
    // hk are hk*G .. hk*G + G-1, so the workgroup's are hv0 .. hv0 + HPW-1.
    // The read slot's pointer, H_k and N come as leading arguments that the
    // build has the hardware preload into scalar registers (gfx950 kernel
    // argument preloading), so the slot load leaves beside the load of the
    // other arguments.
    const int ngrp = H_k / KPW;
    const int hk0 = (int)(blockIdx.x % ngrp) * KPW;
    const int r = blockIdx.x / ngrp;
    const int hv0 = hk0 * G;
    const int T = p.T;

    const int rs_in = read_slot[r];
    bool bad = (uint32_t)rs_in >= (uint32_t)N; // a negative slot too
    if (TOKENS && rs_in != 0) {
        // per-token states: every kept slot must be a usable slot other than the read slot
        for (int t = 0; t < T; ++t) {
            const int ts = p.token_slots[(size_t)r * T + t];
            bad = bad || ts < 0 || ts >= N || ts == rs_in;
        }
    }
    // a padding row (read slot 0) or a row with an unusable slot touches no
    // slot: its loads below go through empty resources (sizes multiplied by
    // the flag; a choice would become a branch that holds the loads back
    // behind the slot's wait), then it writes the read-out fill and leaves
    const bool real = rs_in != 0 && !bad;
    const uint32_t realu = (uint32_t)real;
    const int rs = rs_in * (int)real;

    // ---- conv lanes: each takes four consecutive channels, whole waves except
    // the last, whose spare lanes read nothing and write their result to the
    // padding slot of y_blk
    const int C = p.C;
    const uint32_t cbytes = (uint32_t)C * 2u;
    // channel of x / conv_w / the window for the first channel e of a quad:
    // per key head of the workgroup, its q and k, then v of its value heads
    auto channel = [&](int e) {
        const int kl = e / NCHK;
        const int e2 = e - kl * NCHK;
        const int hk = hk0 + kl;
        const bool isq = e2 < DK;
        const bool isk = !isq && e2 < 2 * DK;
        const int ve = e2 >= 2 * DK ? e2 - 2 * DK : 0;
        const int h = ve / DV;
        return isq ? hk * DK + e2
               : isk ? H_k * DK + hk * DK + (e2 - DK)
                     : 2 * H_k * DK + (hk * G + h) * DV + (ve - h * DV);
    };
    bool conv_wave[NCQ], conv_lane[NCQ];
    int c[NCQ], e4[NCQ];
#pragma unroll
    for (int k = 0; k < NCQ; ++k) {
        const int li = tid + k * NT;
        conv_wave[k] = (li >> 6) < NCW; // wave-uniform (NT is a multiple of 64)
        conv_lane[k] = li < NCL;
        e4[k] = conv_lane[k] ? 4 * li : 0; // first channel of the quad
        c[k] = channel(e4[k]);
    }
    const __amdgpu_buffer_rsrc_t xr = bf16_rsrc(p.x + (size_t)r * p.x_row_stride, (uint32_t)T * cbytes * realu);
    const __amdgpu_buffer_rsrc_t cw = bf16_rsrc(p.conv_w, cbytes * 4u);
    const __amdgpu_buffer_rsrc_t br = bf16_rsrc(p.conv_b ? p.conv_b : p.conv_w, p.conv_b ? cbytes : 0u);
    const __amdgpu_buffer_rsrc_t win = bf16_rsrc(p.conv_state + (size_t)rs * 3 * C, 3u * cbytes * realu);
    const uint32_t gbytes = (uint32_t)T * (uint32_t)p.H_v * 4u * realu;
    const __amdgpu_buffer_rsrc_t gr = f32_rsrc(p.g + (size_t)r * T * p.H_v, gbytes);
    const __amdgpu_buffer_rsrc_t bt_r = f32_rsrc(p.beta + (size_t)r * T * p.H_v, gbytes);
    const bool has_bias = p.conv_b != nullptr;
    // o of this row: T tokens x H_v heads x d_v
    const __amdgpu_buffer_rsrc_t orow =
        bf16_rsrc(p.out + (size_t)r * T * p.H_v * DV, (uint32_t)T * (uint32_t)p.H_v * DV * 2u);

    // The loads of a block's conv inputs and gates; all offsets of lanes with
    // nothing to read, and of tokens past the last, fall outside their
    // resources and read 0, so the block needs no branch around a load.
    // Both take their lane offsets from a copy of the thread index the
    // compiler cannot see through, so nothing they compute is kept in a
    // register across the token blocks.
    auto issue = [&](ConvIn<NCQ, TB> &in, int t0) {
        int tt = tid;
        asm volatile("" : "+v"(tt));
#pragma unroll
        for (int k = 0; k < NCQ; ++k) {
            const int li = tt + k * NT;
            const bool lane_ok = li < NCL;
            in.wlo[k] = in.whi[k] = make_uint4(0, 0, 0, 0);
            in.a0[k] = in.a1[k] = in.a2[k] = in.bq[k] = make_uint2(0, 0);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                in.xs[k][tb] = make_uint2(0, 0);
            if (!conv_wave[k])
                continue;
            // kOOB plus any row offset below 2 GiB stays past the end of every
            // resource, and so does the offset of a token past the last: no
            // select per load
            const int ch = channel(lane_ok ? 4 * li : 0);
            const uint32_t o2 = lane_ok ? (uint32_t)ch * 2u : kOOB;
            const uint32_t o8 = lane_ok ? (uint32_t)ch * 8u : kOOB;
            in.wlo[k] = load_b128(cw, o8);
            in.whi[k] = load_b128(cw, o8 + 16u);
            in.bq[k] = load_b64(br, o2);
            // the window before token t0: the slot's own window for the first
            // block, the previous block's last three tokens after that
            const __amdgpu_buffer_rsrc_t wsrc = t0 == 0 ? win : xr;
            const uint32_t wbase = t0 == 0 ? 0u : (uint32_t)(t0 - 3) * cbytes;
            in.a0[k] = load_b64(wsrc, o2 + wbase);
            in.a1[k] = load_b64(wsrc, o2 + wbase + cbytes);
            in.a2[k] = load_b64(wsrc, o2 + wbase + 2u * cbytes);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                in.xs[k][tb] = load_b64(xr, o2 + (uint32_t)(t0 + tb) * cbytes);
        }
        const int gt = tt / HPW, gh = tt % HPW;
        const uint32_t go = tt < TB * HPW && t0 + gt < T
                                ? (uint32_t)(((t0 + gt) * p.H_v + hv0 + gh) * 4)
                                : kOOB;
        in.g = load_f32(gr, go);
        in.beta = load_f32(bt_r, go);
    };

    // Park a block's conv inputs in LDS, each conv lane its own, and its gates
    // as exp(g), beta.  This waits for the block's conv loads only: they were
    // issued before anything still in flight.
    auto stash = [&](const ConvIn<NCQ, TB> &in) {
        int tt = tid;
        asm volatile("" : "+v"(tt));
#pragma unroll
        for (int k = 0; k < NCQ; ++k) {
            const int li = tt + k * NT;
            if (li >= NCL)
                continue;
            conv_st[RW][li] = make_uint2(in.wlo[k].x, in.wlo[k].y);
            conv_st[RW + 1][li] = make_uint2(in.wlo[k].z, in.wlo[k].w);
            conv_st[RW + 2][li] = make_uint2(in.whi[k].x, in.whi[k].y);
            conv_st[RW + 3][li] = make_uint2(in.whi[k].z, in.whi[k].w);
            conv_st[RB][li] = in.bq[k];
            conv_st[0][li] = in.a0[k];
            conv_st[1][li] = in.a1[k];
            conv_st[2][li] = in.a2[k];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                conv_st[3 + tb][li] = in.xs[k][tb];
        }
        if (tt < TB * HPW)
            gate_blk[tt / HPW][tt % HPW] = make_float2(expf(in.g), in.beta);
    };

    ConvIn<NCQ, TB> in;
    issue(in, 0);
    // conv inputs stay ahead of the tile loads: they are few and on the
    // critical path, and loads complete in order
    __builtin_amdgcn_sched_barrier(0);

    // ---- state slice -> registers
    const int hv = hv0 + hloc;
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    const __amdgpu_buffer_rsrc_t rd_tile = tile_rsrc(p.state + ((size_t)rs * p.H_v + hv) * TILE, TILE * 4u * realu);
    const uint32_t voff = (uint32_t)((rg * DV + 4 * cg) * 4);
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rd_tile, voff, m * RG * DV * 4, kLoadPolicy));
    // Every load of the first block is now in flight.  Keep the scheduler from
    // sinking any of them below the first wait: under a saturated memory
    // system a load issued after the flood of tile loads queues behind all of
    // them.
    __builtin_amdgcn_sched_barrier(0);
    if (!real) {
        // out gets +0.0 for padding and NaN for an unusable slot
        const uint16_t fill = rs_in == 0 ? (uint16_t)0 : (uint16_t)0x7fc0;
        for (int e = tid; e < T * HPW * DV; e += NT) {
            const int t = e / (HPW * DV);
            const int h = (e / DV) % HPW;
            const int j = e % DV;
            p.out[(((size_t)r * T + t) * p.H_v + hv0 + h) * DV + j] = fill;
        }
        return;
    }
    stash(in);

    for (int t0 = 0;;) {
        const int nb = T - t0 < TB ? T - t0 : TB;

        // ---- conv decode + SiLU of the block's tokens -> y_blk.  Token tb
        // reads rows tb..tb+3 of its lane's parked sequence: the window
        // before it and its x.  (The compiler barrier keeps the stash from
        // being forwarded in registers.)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < NCQ; ++k) {
            const int li = tid + k * NT;
            if (!conv_wave[k])
                continue;
            const int lr = conv_lane[k] ? li : 0; // spare lanes compute lane 0's channels into the padding slot
            const uint2 w0 = conv_st[RW][lr], w1 = conv_st[RW + 1][lr], w2 = conv_st[RW + 2][lr],
                        w3 = conv_st[RW + 3][lr];
            const uint4 wl = make_uint4(w0.x, w0.y, w1.x, w1.y), wh = make_uint4(w2.x, w2.y, w3.x, w3.y);
            const uint2 bb = conv_st[RB][lr];
            const int yo = conv_lane[k] ? e4[k] : NCH;
            for (int tb = 0; tb < nb; ++tb) {
                const uint2 a0 = conv_st[tb][lr], a1 = conv_st[tb + 1][lr], a2 = conv_st[tb + 2][lr];
                const uint2 xx = conv_st[tb + 3][lr];
                float4 y;
                y.x = conv_tap4(wl.x, wl.y, a0.x << 16, a1.x << 16, a2.x << 16, xx.x << 16, bb.x << 16, has_bias);
                y.y = conv_tap4(wl.z, wl.w, a0.x & 0xffff0000u, a1.x & 0xffff0000u, a2.x & 0xffff0000u,
                                xx.x & 0xffff0000u, bb.x & 0xffff0000u, has_bias);
                y.z = conv_tap4(wh.x, wh.y, a0.y << 16, a1.y << 16, a2.y << 16, xx.y << 16, bb.y << 16, has_bias);
                y.w = conv_tap4(wh.z, wh.w, a0.y & 0xffff0000u, a1.y & 0xffff0000u, a2.y & 0xffff0000u,
                                xx.y & 0xffff0000u, bb.y & 0xffff0000u, has_bias);
                *reinterpret_cast<float4 *>(&y_blk[tb][yo]) = y;
                if (TOKENS) {
                    // speculative verify: the window after this token goes to
                    // the token's own slot (0: not kept)
                    const int ts = p.token_slots[(size_t)r * T + t0 + tb];
                    if (ts != 0) {
                        const __amdgpu_buffer_rsrc_t tw = bf16_rsrc(p.conv_state + (size_t)ts * 3 * C, 3u * cbytes);
                        const uint32_t o2 = conv_lane[k] ? (uint32_t)c[k] * 2u : kOOB;
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{a1.x, a1.y}, tw, o2, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{a2.x, a2.y}, tw, o2 + cbytes, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{xx.x, xx.y}, tw, o2 + 2u * cbytes, 0, 0);
                    }
                }
            }
            if (!TOKENS && t0 + nb == T) {
                // the advanced window of a channel this workgroup owns, back to
                // the read slot: a shift of bf16 values, stored as the bits
                // they were read as (no other workgroup reads it)
                const uint2 n0 = conv_st[nb][lr], n1 = conv_st[nb + 1][lr], n2 = conv_st[nb + 2][lr];
                const uint32_t o2 = conv_lane[k] ? (uint32_t)c[k] * 2u : kOOB;
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{n0.x, n0.y}, win, o2, 0, kStorePolicy);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{n1.x, n1.y}, win, o2 + cbytes, 0, kStorePolicy);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{n2.x, n2.y}, win, o2 + 2u * cbytes, 0, kStorePolicy);
            }
        }
        lds_barrier();

        // ---- L2 norms of q and k, one wave a token and key head (lane l sums
        // elements l, l + 64, ...; then a butterfly over the wave), and q, k
        // rescaled in place
        for (int pr = wave; pr < nb * KPW; pr += NW) {
            const int tb = pr / KPW, kl = pr - tb * KPW;
            float *y = &y_blk[tb][kl * NCHK];
            float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
            for (int i = lane; i < DK; i += 64) {
                const float qv = y[i], kv = y[DK + i];
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
#pragma unroll
            for (int i = lane; i < DK; i += 64) {
                const float qv = y[i], kv = y[DK + i];
                y[i] = qv * qs;
                y[DK + i] = kv * rk;
            }
            if (lane == 0)
                kq_blk[tb][kl] = sqk * rk * qs; // k^ . q^
        }
        lds_barrier();

        // ---- per token: projections of the state onto k^ and q^, the delta
        // update in registers, and the read-out
        const int kl = hloc / G; // the thread's key head in the workgroup (uniform)
        for (int tb = 0; tb < nb; ++tb) {
            const float *y = &y_blk[tb][kl * NCHK];
            float4 pa = f4_zero(), pb = f4_zero();
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int i = rg + RG * m;
                const float kh = y[DK + i];
                const float qh = y[i];
                pa.x = fmaf(s[m].x, kh, pa.x);
                pa.y = fmaf(s[m].y, kh, pa.y);
                pa.z = fmaf(s[m].z, kh, pa.z);
                pa.w = fmaf(s[m].w, kh, pa.w);
                pb.x = fmaf(s[m].x, qh, pb.x);
                pb.y = fmaf(s[m].y, qh, pb.y);
                pb.z = fmaf(s[m].z, qh, pb.z);
                pb.w = fmaf(s[m].w, qh, pb.w);
            }
            // k^ is read again for the update below rather than held in
            // sixteen registers through the butterflies
            asm volatile("" ::: "memory");
            // butterflies over lane bits 3, 4, 5 form the pairwise tree
            // ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7)) over the row groups in every lane
            pa.x = xor_sum<8>(pa.x);
            pa.y = xor_sum<8>(pa.y);
            pa.z = xor_sum<8>(pa.z);
            pa.w = xor_sum<8>(pa.w);
            pb.x = xor_sum<8>(pb.x);
            pb.y = xor_sum<8>(pb.y);
            pb.z = xor_sum<8>(pb.z);
            pb.w = xor_sum<8>(pb.w);

            const float2 gb = gate_blk[tb][hloc];
            const float alpha = gb.x, bt = gb.y;
            const float kq = kq_blk[tb][kl];
            const float *vv = &y[2 * DK + (hloc - kl * G) * DV + 4 * cg];
            float4 u;
            u.x = bt * (vv[0] - alpha * pa.x);
            u.y = bt * (vv[1] - alpha * pa.y);
            u.z = bt * (vv[2] - alpha * pa.z);
            u.w = bt * (vv[3] - alpha * pa.w);
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const float kh = y[DK + rg + RG * m];
                s[m].x = fmaf(kh, u.x, alpha * s[m].x);
                s[m].y = fmaf(kh, u.y, alpha * s[m].y);
                s[m].z = fmaf(kh, u.z, alpha * s[m].z);
                s[m].w = fmaf(kh, u.w, alpha * s[m].w);
            }
            {
                // o: row group 0 of every column group (lanes 0-7 of each wave)
                const float o0 = fmaf(u.x, kq, alpha * pb.x);
                const float o1 = fmaf(u.y, kq, alpha * pb.y);
                const float o2 = fmaf(u.z, kq, alpha * pb.z);
                const float o3 = fmaf(u.w, kq, alpha * pb.w);
                const u32x2 pk = {(uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16),
                                  (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16)};
                const uint32_t oo = (uint32_t)(((t0 + tb) * p.H_v + hv) * DV + 4 * cg) * 2u;
                __builtin_amdgcn_raw_buffer_store_b64(pk, orow, rg == 0 ? oo : kOOB, 0, kStorePolicy);
            }
            if (TOKENS) {
                // speculative verify: the state after this token goes to the
                // token's own slot (0: not kept); the read slot stays as it was
                const int ts = p.token_slots[(size_t)r * T + t0 + tb];
                if (ts != 0) {
                    const __amdgpu_buffer_rsrc_t tok_tile =
                        tile_rsrc(p.state + ((size_t)ts * p.H_v + hv) * TILE, TILE * 4u);
#pragma unroll
                    for (int m = 0; m < RPT; ++m)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), tok_tile, voff,
                                                               m * RG * DV * 4, kStorePolicy);
                }
            }
        }

        t0 += TB;
        if (t0 >= T)
            break;
        // every wave is done with this block's LDS before the next one writes it
        lds_barrier();
        issue(in, t0);
        stash(in);
    }
    if (TOKENS)
        return;

    // ---- new state -> the read slot
    const __amdgpu_buffer_rsrc_t wr_tile = tile_rsrc(p.state + ((size_t)rs * p.H_v + hv) * TILE, TILE * 4u);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), wr_tile, voff, m * RG * DV * 4,
                                               kStorePolicy);
}

template <int DK, int DV, int G, int KPW>
static hipError_t launch_step(const StepParams &p, hipStream_t stream)
{
    if (p.H_k % KPW != 0)
        return hipErrorInvalidValue;
    const long long groups = (long long)p.B * (p.H_k / KPW);
    if (groups <= 0)
        return hipSuccess;
    StepParams q = p;
    q.n_slices = 1;
    const int32_t *rs = p.read_slot;
    int H_k = p.H_k, N = p.N;
    void *args[] = {&rs, &H_k, &N, &q};
    const void *k = reinterpret_cast<const void *>(&gdn_step_kernel<DK, DV, G, KPW, false>);
    if constexpr (KPW == 1) {
        if (p.token_slots)
            k = reinterpret_cast<const void *>(&gdn_step_kernel<DK, DV, G, KPW, true>);
    } else if (p.token_slots) {
        return hipErrorInvalidValue; // per-token states keep one key head a workgroup
    }
    return hipLaunchKernel(k, dim3((unsigned)groups), dim3(2 * DV * G * KPW), args, 0, stream);
}

// Key heads a workgroup.  Single-token in-place steps of 128 x 128 tiles
// whose value heads put 2.5 to 4 tiles on every CU (40-64 rows of 16 heads)
// take four value heads a workgroup -- four key heads of one value head each,
// or two of two -- in 1024 threads, one workgroup a CU.  Measured on MI355X
// at 64 rows, cold scattered slots, us a step: one value head a key head 27.6
// (the one-tile kernel) -> 26.65, two 26.9 -> 26.4.  Token walks keep one key
// head a workgroup (four tokens at 64 rows: 29.7 against 32.2 grouped), as do
// 16 and 128 rows (8.2 against 11.8, 52.0 against 54.5), where the grouped
// workgroups leave CUs idle or hold two to a CU.
int walk_key_heads(const StepParams &p, int d_k, int d_v)
{
    if (p.T != 1 || p.token_slots || p.twin || d_k != 128 || d_v != 128 || (p.G != 1 && p.G != 2))
        return 1;
    const long long heads = (long long)p.B * p.H_v, cus = device_cus();
    const int kpw = 4 / p.G;
    return heads * 2 > 5 * cus && heads <= 4 * cus && p.H_k % kpw == 0 ? kpw : 1;
}

template <int DK, int DV>
static hipError_t dispatch_dims(const StepParams &p, hipStream_t stream)
{
    if constexpr (DK == 128 && DV == 128) {
        const int kpw = walk_key_heads(p, DK, DV);
        if (kpw == 4)
            return launch_step<DK, DV, 1, 4>(p, stream);
        if (kpw == 2)
            return launch_step<DK, DV, 2, 2>(p, stream);
    }
    switch (p.G) {
    case 1: return launch_step<DK, DV, 1, 1>(p, stream);
    case 2: return launch_step<DK, DV, 2, 1>(p, stream);
    case 4: return launch_step<DK, DV, 4, 1>(p, stream);
    default: return hipErrorInvalidValue;
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
