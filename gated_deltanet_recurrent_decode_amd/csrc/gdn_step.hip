// gdn_step.hip -- the fused Gated DeltaNet decode step for gfx950, in place
// (keep_in_place), T tokens a row.
//
// One workgroup owns a key head of a row with all G of its value heads, so no
// other workgroup reads a conv window it overwrites.  Per workgroup it:
//   1. issues the loads of its G fp32 state tiles (d_k x d_v each, 16-byte
//      loads, each wave instruction covering whole 128-byte lines), so HBM
//      streams while the rest of the prologue runs;
//   2. per token: runs the conv decode + SiLU of its channels (q and k of the
//      key head, v of its value heads) into LDS, the window advancing in
//      registers;
//   3. L2-normalises q and k (wave butterflies over LDS, done redundantly by
//      every wave so no extra barrier is needed);
//   4. per head: one pass over the register-resident state gives both
//      a = S^T k^ and b = S^T q^ (in-thread over its rows, then butterflies
//      across the eight row groups, which sit in lane bits 3-5 of one wave, so
//      the sum ends inside the wave in a fixed order);
//      u = beta (v - alpha a); S' = alpha S + k^ u^T; o = alpha b + u (k^.q^),
//      which equals S'^T q^;
//   5. after the last token, stores the state and the advanced window back to
//      the read slot; o goes out as bf16 every token.
// The delta rule is Gated DeltaNet's (decay, predict with the decayed state,
// correct, read out); the slot handling follows mstar PR #1139, "What
// changed" (keep_in_place for prefill, split walks and the mixed step's decode
// half) and "Tests" (padding on slot 0).  Single-token steps that allow one
// head tile per workgroup (every twin step, and in place with one value head
// per key head) run in gdn_step_tile.hip instead, with the same thread layout
// and summation order; this kernel takes token walks, per-token states and
// in-place GQA.
//
// No MFMA: per state element the step does a handful of FMAs against 8 bytes
// of HBM traffic, far under the fp32 ridge point, so the kernel is written for
// bandwidth: wide coalesced loads, every tile loaded once, no re-reads.

#include "gdn_internal.h"
#include "step_common.h"

namespace gdn {

template <int DK, int DV, int HPW>
__global__ __launch_bounds__(2 * DV * HPW) void gdn_step_kernel(StepParams p)
{
    constexpr int DVS = DV; // whole tiles
    using Cfg = StepCfg<DK, DVS, HPW>;
    static_assert(Cfg::NT == 2 * DVS * HPW, "launch bound must match the layout");
    constexpr int NT = Cfg::NT, NTH = Cfg::NTH, RG = Cfg::RG, RPT = Cfg::RPT;
    constexpr int NCH = Cfg::NCH;

    // conv outputs (+ a padding slot for spare conv lanes), one set for even
    // and one for odd tokens: token t writes the set that token t - 2 read,
    // and a wave gets there only after every wave has passed token t - 1's
    // barrier, which waits for its LDS reads of token t - 2 to complete
    __shared__ float y_buf[2][NCH + 4];

    const int tid = threadIdx.x;
    // head of the group this thread updates; NTH is a multiple of the wave size,
    // so this is wave-uniform -- say so, or every buffer access that depends on
    // it would be compiled as a loop over lanes
    const int hloc = __builtin_amdgcn_readfirstlane(tid / NTH);
    const int ht = tid - hloc * NTH; // thread index inside its head slice
    const int lane = tid & 63;
    // each wave holds 32 columns (eight column groups in lane bits 0-2) of
    // all eight row groups (lane bits 3-5)
    const int cg = (ht >> 6) * 8 + (lane & 7);
    const int rg = lane >> 3;

    // workgroup -> (row, key head); its value heads are hk*G .. hk*G + G-1
    const int hk = blockIdx.x % p.H_k;
    const int r = blockIdx.x / p.H_k;
    const int hv0 = hk * p.G;
    constexpr int col0 = 0;
    const int T = p.T;

    const int rs = p.read_slot[r];
    bool bad = rs < 0 || rs >= p.N;
    if (p.token_slots && rs != 0) {
        // per-token states: every kept slot must be a usable slot other than the read slot
        for (int t = 0; t < T; ++t) {
            const int ts = p.token_slots[(size_t)r * T + t];
            bad = bad || ts < 0 || ts >= p.N || ts == rs;
        }
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
    const int C = p.C;
    const int hv = hv0 + hloc;
    // gates of token 0, also ahead of the state tile
    float g_t = p.g[(size_t)r * T * p.H_v + hv];
    float b_t = p.beta[(size_t)r * T * p.H_v + hv];
    const uint16_t *xrow = p.x + (size_t)r * p.x_row_stride;
    const uint16_t *cs_rd = p.conv_state + (size_t)rs * 3 * C;
    uint16_t *cs_wr = p.conv_state + (size_t)rs * 3 * C;
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
        own[k] = conv_lane[k]; // the workgroup owns every channel it reads
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
    uint2 xn[NCQ];     // the next token's x, loaded one token ahead
    float g_n = 0.f, b_n = 0.f;
    for (int t = 0; t < T; ++t) {
        float *y_lds = y_buf[t & 1];
        if (t > 0) {
#pragma unroll
            for (int k = 0; k < NCQ; ++k)
                xq[k] = xn[k];
            g_t = g_n;
            b_t = b_n;
        }
        if (t + 1 < T) {
            // loads of token t+1's inputs go out now and land while token t computes
#pragma unroll
            for (int k = 0; k < NCQ; ++k)
                xn[k] = conv_wave[k] ? *reinterpret_cast<const uint2 *>(xrow + (size_t)(t + 1) * C + c[k])
                                     : make_uint2(0, 0);
            g_n = p.g[((size_t)r * T + t + 1) * p.H_v + hv];
            b_n = p.beta[((size_t)r * T + t + 1) * p.H_v + hv];
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
        const float4 a = pa, b = pb;

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
        if (p.token_slots) {
            // speculative verify: the state and window after this token go to
            // the token's own slot (0: not kept); the read slot stays as it was
            const int ts = p.token_slots[(size_t)r * T + t];
            if (ts != 0) {
                uint16_t *cs_tok = p.conv_state + (size_t)ts * 3 * C;
#pragma unroll
                for (int k = 0; k < NCQ; ++k) {
                    if (own[k]) {
                        uint16_t *dst = cs_tok + c[k];
                        *reinterpret_cast<u32x2 *>(dst) = u32x2{wn0[k].x, wn0[k].y};
                        *reinterpret_cast<u32x2 *>(dst + C) = u32x2{wn1[k].x, wn1[k].y};
                        *reinterpret_cast<u32x2 *>(dst + 2 * C) = u32x2{wn2[k].x, wn2[k].y};
                    }
                }
                const __amdgpu_buffer_rsrc_t tok_tile =
                    tile_rsrc(p.state + ((size_t)ts * p.H_v + hv) * TILE, TILE * 4u);
#pragma unroll
                for (int m = 0; m < RPT; ++m)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), tok_tile, voff,
                                                           m * RG * DV * 4, kStorePolicy);
            }
        }
    }
    if (p.token_slots)
        return;

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

    // ---- new state -> the read slot
    const __amdgpu_buffer_rsrc_t wr_tile = tile_rsrc(p.state + ((size_t)rs * p.H_v + hv) * TILE, TILE * 4u);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[m]), wr_tile, voff, m * RG * DV * 4,
                                               kStorePolicy);
}

template <int DK, int DV, int HPW>
static hipError_t launch_step(const StepParams &p, hipStream_t stream)
{
    const long long tiles = (long long)p.B * p.H_k;
    if (tiles <= 0)
        return hipSuccess;
    StepParams q = p;
    q.n_slices = 1;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_step_kernel<DK, DV, HPW>), dim3((unsigned)tiles),
                           dim3(StepCfg<DK, DV, HPW>::NT), args, 0, stream);
}

template <int DK, int DV>
static hipError_t dispatch_dims(const StepParams &p, hipStream_t stream)
{
    switch (p.G) {
    case 1: return launch_step<DK, DV, 1>(p, stream);
    case 2: return launch_step<DK, DV, 2>(p, stream);
    case 4: return launch_step<DK, DV, 4>(p, stream);
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
