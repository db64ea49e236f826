// gdn_prefill.hip -- chunked Gated DeltaNet prefill, in place (gfx950).
//
// A prompt of L tokens updates its request's slot in place (mstar PR #1139,
// "What changed": prefill and split walks keep_in_place; PR #965 names the
// chunked GDN path).  What it computes is exactly the in-place decode step run
// over the L tokens in order -- conv decode + SiLU, L2 norms, and per token
// S <- alpha S; S <- S + beta k (v - S^T k)^T; o = S^T q -- but in the chunked
// form, so that the contractions are dense and run on the matrix cores.
//
// Chunked form (32 tokens a chunk, S0 the state entering the chunk, rows t of
// the chunk, gamma_t the running sum of the log decays inside the chunk):
//   U = (I + A)^-1 diag(beta) (V - diag(e^gamma) K S0),
//       A[t][s] = beta_t e^(gamma_t - gamma_s) (k_t . k_s) for s < t, else 0
//   O = diag(e^gamma) Q S0 + P U,  P[t][s] = e^(gamma_t - gamma_s) (q_t . k_s) for s <= t
//   S_next = e^gamma_last S0 + K^T diag(e^(gamma_last - gamma)) U
// which is the token-by-token recurrence unrolled over the chunk (u_t is the
// update vector beta_t (v_t - alpha_t S_{t-1}^T k_t), and unrolling S_{t-1}
// inside the chunk gives the triangular system).  (I + A)^-1 is unit lower
// triangular: its two 16x16 diagonal blocks come from forward substitution,
// the off-diagonal block is -T22 A21 T11, and U is then one more matrix-core
// product.  A chunk shorter than 32 is
// padded with zero tokens (k = q = v = 0, g = 0, beta = 0), which changes
// nothing.
//
// One workgroup (4 waves) per (sequence, key head), taking the key head's G
// value heads one after the other, so no other workgroup reads a conv window
// it writes back (the q and k windows go back after the last value head); the
// chunks of a sequence run in order.  The state lives in LDS as fp32; K S0, Q S0, K K^T,
// Q K^T, (I + A)^-1 (beta R), P U and K^T U are fp32 MFMA products
// (v_mfma_f32_16x16x4f32).  Everything is fp32, as in the decode kernels; the
// conv's SiLU uses the hardware exp and reciprocal (about an ulp each).

#include "gdn_internal.h"
#include "prefill_internal.h"
#include "step_common.h"

namespace gdn {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32; // tokens per chunk (two 16-row MFMA blocks)

// D += A * B for one 16x16 tile and a k-slice of 4: lane l supplies A[l%16][l/16]
// and B[l/16][l%16]; the tile's D[i][j] sits at lane j + 16 (i / 4), element i % 4.
__device__ __forceinline__ v4f mma16x16x4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DK, int DV>
struct PrefillCfg {
    static constexpr int NT = 256;                 // threads: four waves
    static constexpr int NCH = 2 * DK + DV;        // conv channels of a (key head, value head) pair
    static constexpr int NPAIR = NCH / 2;          // conv lanes, two channels each
    // LDS row pitches (floats), chosen so that every MFMA operand read hits each
    // of the 32 banks exactly twice: operands read along a row (A-style: lane
    // -> row, 4 consecutive k) need a pitch of 4 mod 32, operands read along a
    // column (B-style: lane -> column, 4 consecutive rows) 16 mod 32
    static constexpr int SP = DV + 16;             // S
    static constexpr int KP = DK + 4;              // Q and K
    static constexpr int VP = DV + 16;             // V / R / U
    static constexpr int AP = kChunk + 1;          // LDS row pitch of A and P
    static constexpr int CBW = DV / 16 / 4;        // 16-column blocks of O per wave
    static constexpr int RBW = DK / 16 / 4;        // 16-row blocks of S per wave
    static_assert(NPAIR <= NT, "one conv lane per channel pair");
    static_assert(CBW >= 1 && RBW >= 1, "head dims of 64 or 128");
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_prefill_kernel(PrefillParams p)
{
    using Cfg = PrefillCfg<DK, DV>;
    constexpr int NT = Cfg::NT, NPAIR = Cfg::NPAIR;
    constexpr int SP = Cfg::SP, KP = Cfg::KP, VP = Cfg::VP, AP = Cfg::AP;
    constexpr int CBW = Cfg::CBW, RBW = Cfg::RBW;
    constexpr int BT = kChunk;

    __shared__ float S[DK * SP];  // the state, S[i][j], i over keys
    __shared__ __align__(16) float Qs[BT * KP]; // q^ of the chunk's tokens (scaled by q_scale)
    __shared__ __align__(16) float Ks[BT * KP]; // k^
    __shared__ __align__(16) float Vs[BT * VP]; // v, then R = V - e^gamma K S0, then U
    __shared__ float Am[BT * AP]; // the strictly lower A
    __shared__ float Pm[BT * AP]; // P
    __shared__ float Tm[BT * AP]; // (I + A)^-1
    __shared__ float Mm[16 * 17]; // A21 T11
    __shared__ float gam[BT];     // running log decay inside the chunk
    __shared__ float bet[BT];     // beta (0 on padding tokens)
    __shared__ float eg[BT];      // e^gamma_t
    __shared__ float egl[BT];     // e^(gamma_last - gamma_t)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int li = lane & 15; // row (A) or column (B, D) inside a 16-block
    const int lk = lane >> 4; // k inside a 4-slice (A, B); row group of 4 (D)

    const int b = blockIdx.x / p.H_k;
    const int hk = blockIdx.x % p.H_k;
    const int t_begin = p.cu_seqlens[b];
    const int t_end = p.cu_seqlens[b + 1];
    const int s = p.slot[b];
    // a sequence whose range or slot is unusable touches nothing
    if (t_begin < 0 || t_end < t_begin || t_end > p.total || s < 0 || s >= p.N)
        return;
    if (s == 0) {
        // padding sequence on the null slot: its read-out is +0.0
        for (int e = tid; e < (t_end - t_begin) * p.G * DV; e += NT)
            p.out[((size_t)(t_begin + e / (p.G * DV)) * p.H_v + hk * p.G) * DV + e % (p.G * DV)] = 0;
        return;
    }
    if (t_end == t_begin)
        return;

    const int C = p.C;
    for (int hl = 0; hl < p.G; ++hl) {
    const int hv = hk * p.G + hl;
    if (hl > 0)
        __syncthreads(); // the previous value head's last reads of LDS are done
    constexpr uint32_t TILE = (uint32_t)DK * DV;
    float *tile = p.state + ((size_t)s * p.H_v + hv) * TILE;

    // ---- the state -> LDS (16-byte streaming loads)
    for (int e = tid; e < DK * DV / 4; e += NT) {
        const int i = e / (DV / 4), j4 = e % (DV / 4);
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(tile) + e);
        *reinterpret_cast<v4f *>(&S[i * SP + 4 * j4]) = v;
    }

    // ---- conv lanes: channel pair (e, e+1) of the workgroup's q | k | v channels
    const bool conv_lane = tid < NPAIR;
    const int e = conv_lane ? 2 * tid : 0;
    const bool isq = e < DK, isk = !isq && e < 2 * DK;
    const int c = isq ? hk * DK + e : isk ? p.H_k * DK + hk * DK + (e - DK) : 2 * p.H_k * DK + hv * DV + (e - 2 * DK);
    // q and k windows go back once, after the key head's last value head
    const bool own = conv_lane && ((isq || isk) ? (hl == p.G - 1) : true);
    // weights (taps 0..3, tap 3 on the current token), bias, window (oldest first), as fp32
    float w0[2], w1[2], w2[2], w3[2], bias[2], a0[2], a1[2], a2[2];
    const uint16_t *cs_rd = p.conv_state + (size_t)s * 3 * C;
    for (int h = 0; h < 2; ++h) {
        const uint16_t *wc = p.conv_w + (size_t)(c + h) * 4;
        w0[h] = bf16_to_f32(wc[0]);
        w1[h] = bf16_to_f32(wc[1]);
        w2[h] = bf16_to_f32(wc[2]);
        w3[h] = bf16_to_f32(wc[3]);
        bias[h] = p.conv_b ? bf16_to_f32(p.conv_b[c + h]) : 0.f;
        a0[h] = bf16_to_f32(cs_rd[c + h]);
        a1[h] = bf16_to_f32(cs_rd[C + c + h]);
        a2[h] = bf16_to_f32(cs_rd[2 * C + c + h]);
    }
    float *ydst = isq ? &Qs[e] : isk ? &Ks[e - DK] : &Vs[e - 2 * DK];
    const int ypitch = (isq || isk) ? KP : VP;
    const bool has_bias = p.conv_b != nullptr;

    // the first chunk's x (conv lanes) and gates (lanes < 32) go out now; each
    // chunk then loads the next one's while it computes
    uint32_t xb[BT];
    float g_in = 0.f, b_in = 0.f;
    auto load_chunk = [&](int t0n) {
        const int nn = t_end - t0n < BT ? t_end - t0n : BT;
#pragma unroll
        for (int tt = 0; tt < BT; ++tt)
            xb[tt] = (conv_lane && tt < nn)
                         ? *reinterpret_cast<const uint32_t *>(p.x + (size_t)(t0n + tt) * p.x_row_stride + c)
                         : 0u;
        const bool realg = tid < nn;
        g_in = realg ? p.g[(size_t)(t0n + tid) * p.H_v + hv] : 0.f;
        b_in = realg ? p.beta[(size_t)(t0n + tid) * p.H_v + hv] : 0.f;
    };
    load_chunk(t_begin);

    __syncthreads(); // the state is in LDS

    for (int t0 = t_begin; t0 < t_end; t0 += BT) {
        const int n = t_end - t0 < BT ? t_end - t0 : BT;

        // ---- conv decode + SiLU of the chunk's tokens (x already in registers);
        // zero rows past the end
        if (conv_lane) {
            // the pair's two outputs of a token are adjacent: one 8-byte store
#pragma unroll
            for (int tt = 0; tt < BT; ++tt) {
                float y0 = 0.f, y1 = 0.f;
                if (tt < n) {
                    const float x0 = __uint_as_float(xb[tt] << 16), x1 = __uint_as_float(xb[tt] & 0xffff0000u);
                    float acc0 = w0[0] * a0[0];
                    acc0 = fmaf(w1[0], a1[0], acc0);
                    acc0 = fmaf(w2[0], a2[0], acc0);
                    acc0 = fmaf(w3[0], x0, acc0);
                    float acc1 = w0[1] * a0[1];
                    acc1 = fmaf(w1[1], a1[1], acc1);
                    acc1 = fmaf(w2[1], a2[1], acc1);
                    acc1 = fmaf(w3[1], x1, acc1);
                    if (has_bias) {
                        acc0 += bias[0];
                        acc1 += bias[1];
                    }
                    y0 = acc0 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc0));
                    y1 = acc1 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc1));
                    a0[0] = a1[0]; a1[0] = a2[0]; a2[0] = x0;
                    a0[1] = a1[1]; a1[1] = a2[1]; a2[1] = x1;
                }
                *reinterpret_cast<float2 *>(&ydst[tt * ypitch]) = make_float2(y0, y1);
            }
        }
        if (tid < BT) {
            // the running log decay: an inclusive scan over the chunk's tokens
            // (five shuffle steps inside the first 32 lanes), and the decay
            // factors every later phase uses
            float gsum = g_in;
#pragma unroll
            for (int o = 1; o < BT; o <<= 1) {
                const float up = __shfl_up(gsum, o, 64);
                if (tid >= o)
                    gsum += up;
            }
            const float glast = __shfl(gsum, BT - 1, 64);
            gam[tid] = gsum;
            bet[tid] = b_in;
            eg[tid] = expf(gsum);
            egl[tid] = expf(glast - gsum);
        }
        // the next chunk's inputs load while this one computes
        if (t0 + BT < t_end)
            load_chunk(t0 + BT);
        __syncthreads();

        // ---- L2 norms of q and k: eight lanes a token, each summing DK/8
        // elements in runs of four (16-byte accesses, held in registers until
        // scaled), then three butterfly steps inside the eight; rows past the
        // end stay zero.
        {
            const int tt = tid >> 3, sub = tid & 7;
            constexpr int NR = DK / 32; // runs of four a lane
            v4f qr[NR], kr[NR];
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                qr[j] = *reinterpret_cast<const v4f *>(&Qs[tt * KP + 4 * sub + 32 * j]);
                kr[j] = *reinterpret_cast<const v4f *>(&Ks[tt * KP + 4 * sub + 32 * j]);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    sq = fmaf(qr[j][e4], qr[j][e4], sq);
                    sk = fmaf(kr[j][e4], kr[j][e4], sk);
                }
            }
            // the sums over each token's eight lanes: DPP butterflies (same pairs as an
            // xor shuffle, no LDS round trip)
            sq += dpp_xor<1>(sq);
            sk += dpp_xor<1>(sk);
            sq += dpp_xor<2>(sq);
            sk += dpp_xor<2>(sk);
            sq += dpp_xor<4>(sq);
            sk += dpp_xor<4>(sk);
            if (tt < n) {
                const float qs = (1.0f / sqrtf(sq + p.l2_eps)) * p.q_scale;
                const float rk = 1.0f / sqrtf(sk + p.l2_eps);
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    *reinterpret_cast<v4f *>(&Qs[tt * KP + 4 * sub + 32 * j]) =
                        v4f{qr[j][0] * qs, qr[j][1] * qs, qr[j][2] * qs, qr[j][3] * qs};
                    *reinterpret_cast<v4f *>(&Ks[tt * KP + 4 * sub + 32 * j]) =
                        v4f{kr[j][0] * rk, kr[j][1] * rk, kr[j][2] * rk, kr[j][3] * rk};
                }
            }
        }
        __syncthreads();

        // ---- K S0 and Q S0 (rows of the chunk x all of d_v): this wave's
        // column blocks, both row blocks; R = V - e^gamma K S0 goes over V
        v4f qs_acc[2][CBW], ks_acc[2][CBW];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < CBW; ++q)
                qs_acc[rb][q] = ks_acc[rb][q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const float aq0 = Qs[li * KP + k0 + lk], aq1 = Qs[(16 + li) * KP + k0 + lk];
            const float ak0 = Ks[li * KP + k0 + lk], ak1 = Ks[(16 + li) * KP + k0 + lk];
#pragma unroll
            for (int q = 0; q < CBW; ++q) {
                const float bs = S[(k0 + lk) * SP + (wv * CBW + q) * 16 + li];
                qs_acc[0][q] = mma16x16x4(aq0, bs, qs_acc[0][q]);
                qs_acc[1][q] = mma16x16x4(aq1, bs, qs_acc[1][q]);
                ks_acc[0][q] = mma16x16x4(ak0, bs, ks_acc[0][q]);
                ks_acc[1][q] = mma16x16x4(ak1, bs, ks_acc[1][q]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < CBW; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = rb * 16 + 4 * lk + r, j = (wv * CBW + q) * 16 + li;
                    Vs[tt * VP + j] -= eg[tt] * ks_acc[rb][q][r];
                }

        // ---- K K^T (waves 0, 1) and Q K^T (waves 2, 3): 32x32, two tiles a
        // wave; then the masked, decay-weighted A and P
        {
            const float *Asrc = wv < 2 ? Ks : Qs;
            const int rb = wv & 1;
            v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
            for (int k0 = 0; k0 < DK; k0 += 4) {
                const float a = Asrc[(rb * 16 + li) * KP + k0 + lk];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    acc[cb] = mma16x16x4(a, Ks[(cb * 16 + li) * KP + k0 + lk], acc[cb]);
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = rb * 16 + 4 * lk + r, ss = cb * 16 + li;
                    const float d = expf(gam[tt] - gam[ss]);
                    if (wv < 2)
                        Am[tt * AP + ss] = ss < tt ? bet[tt] * d * acc[cb][r] : 0.f;
                    else
                        Pm[tt * AP + ss] = ss <= tt ? d * acc[cb][r] : 0.f;
                }
        }
        __syncthreads();

        // ---- T = (I + A)^-1.  Diagonal blocks: column j of the inverse of a
        // unit lower 16x16 block by forward substitution (thread j of a block)
        if (tid < BT) {
            const int b0 = tid & 16, j = tid & 15;
            float xcol[16];
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                float acc = tt == j ? 1.f : 0.f;
#pragma unroll
                for (int ss = 0; ss < tt; ++ss)
                    acc = fmaf(-Am[(b0 + tt) * AP + b0 + ss], xcol[ss], acc);
                xcol[tt] = tt < j ? 0.f : acc;
                Tm[(b0 + tt) * AP + b0 + j] = xcol[tt];
                Tm[(b0 + tt) * AP + (b0 ^ 16) + j] = 0.f; // the upper block is 0; the lower one is set below
            }
        }
        __syncthreads();
        // off-diagonal block T21 = -T22 (A21 T11), one element a thread per product
        {
            const int r = tid >> 4, cc = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                acc = fmaf(Am[(16 + r) * AP + u], Tm[u * AP + cc], acc);
            Mm[r * 17 + cc] = acc;
            __syncthreads();
            float t21 = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                t21 = fmaf(Tm[(16 + r) * AP + 16 + u], Mm[u * 17 + cc], t21);
            Tm[(16 + r) * AP + cc] = -t21;
        }
        __syncthreads();

        // ---- U = T diag(beta) R: this wave's column blocks; U goes over R
        // (a wave reads and writes only its own columns)
        {
            v4f uacc[2][CBW];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int q = 0; q < CBW; ++q)
                    uacc[rb][q] = v4f{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int k0 = 0; k0 < BT; k0 += 4) {
                const float at0 = Tm[li * AP + k0 + lk], at1 = Tm[(16 + li) * AP + k0 + lk];
                const float bs = bet[k0 + lk];
#pragma unroll
                for (int q = 0; q < CBW; ++q) {
                    const float br = bs * Vs[(k0 + lk) * VP + (wv * CBW + q) * 16 + li];
                    uacc[0][q] = mma16x16x4(at0, br, uacc[0][q]);
                    uacc[1][q] = mma16x16x4(at1, br, uacc[1][q]);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int q = 0; q < CBW; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Vs[(rb * 16 + 4 * lk + r) * VP + (wv * CBW + q) * 16 + li] = uacc[rb][q][r];
        }
        __syncthreads();

        // ---- O = e^gamma Q S0 + P U -> out (bf16, rows of real tokens)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < CBW; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    qs_acc[rb][q][r] *= eg[rb * 16 + 4 * lk + r];
        #pragma unroll
            for (int k0 = 0; k0 < BT; k0 += 4) {
            const float ap0 = Pm[li * AP + k0 + lk], ap1 = Pm[(16 + li) * AP + k0 + lk];
#pragma unroll
            for (int q = 0; q < CBW; ++q) {
                const float bu = Vs[(k0 + lk) * VP + (wv * CBW + q) * 16 + li];
                qs_acc[0][q] = mma16x16x4(ap0, bu, qs_acc[0][q]);
                qs_acc[1][q] = mma16x16x4(ap1, bu, qs_acc[1][q]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < CBW; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = rb * 16 + 4 * lk + r;
                    if (tt < n)
                        p.out[((size_t)(t0 + tt) * p.H_v + hv) * DV + (wv * CBW + q) * 16 + li] =
                            f32_to_bf16_rne(qs_acc[rb][q][r]);
                }

        // ---- S_next = e^gamma_last S0 + K^T diag(e^(gamma_last - gamma)) U:
        // this wave's row blocks of S, every column block
        {
            // padding tokens carry g = 0, so the chunk's last gamma is its last real token's
            const float el = eg[BT - 1];
            v4f sacc[RBW][DV / 16];
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < DV / 16; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sacc[q][jb][r] = el * S[((wv * RBW + q) * 16 + 4 * lk + r) * SP + jb * 16 + li];
            #pragma unroll
            for (int k0 = 0; k0 < BT; k0 += 4) {
                const float sc = egl[k0 + lk];
#pragma unroll
                for (int q = 0; q < RBW; ++q) {
                    const float a = Ks[(k0 + lk) * KP + (wv * RBW + q) * 16 + li] * sc;
#pragma unroll
                    for (int jb = 0; jb < DV / 16; ++jb)
                        sacc[q][jb] = mma16x16x4(a, Vs[(k0 + lk) * VP + jb * 16 + li], sacc[q][jb]);
                }
            }
            // every wave's reads of S for this chunk are behind the barriers above,
            // except this wave's own rows, read just now
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < DV / 16; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[((wv * RBW + q) * 16 + 4 * lk + r) * SP + jb * 16 + li] = sacc[q][jb][r];
        }
        __syncthreads(); // S, Q, K, V are free for the next chunk
    }

    // ---- the state and the advanced window back to the slot
    for (int e2 = tid; e2 < DK * DV / 4; e2 += NT) {
        const int i = e2 / (DV / 4), j4 = e2 % (DV / 4);
        const v4f v = *reinterpret_cast<const v4f *>(&S[i * SP + 4 * j4]);
        __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(tile) + e2);
    }
    if (own) {
        uint16_t *cs_wr = p.conv_state + (size_t)s * 3 * C + c;
        // the window values are bf16 inputs carried exactly in fp32
        *reinterpret_cast<uint32_t *>(cs_wr) =
            (uint32_t)f32_to_bf16_exact(a0[0]) | ((uint32_t)f32_to_bf16_exact(a0[1]) << 16);
        *reinterpret_cast<uint32_t *>(cs_wr + C) =
            (uint32_t)f32_to_bf16_exact(a1[0]) | ((uint32_t)f32_to_bf16_exact(a1[1]) << 16);
        *reinterpret_cast<uint32_t *>(cs_wr + 2 * C) =
            (uint32_t)f32_to_bf16_exact(a2[0]) | ((uint32_t)f32_to_bf16_exact(a2[1]) << 16);
    }
    } // value heads
}

template <int DK, int DV>
static hipError_t launch_prefill_dims(const PrefillParams &p, hipStream_t stream)
{
    const long long wgs = (long long)p.B * p.H_k;
    if (wgs <= 0)
        return hipSuccess;
    PrefillParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_prefill_kernel<DK, DV>), dim3((unsigned)wgs),
                           dim3(PrefillCfg<DK, DV>::NT), args, 0, stream);
}

hipError_t launch_gdn_prefill(const PrefillParams &p, int d_k, int d_v, hipStream_t stream)
{
    if (d_k == 128 && d_v == 128) return launch_prefill_dims<128, 128>(p, stream);
    if (d_k == 64 && d_v == 64) return launch_prefill_dims<64, 64>(p, stream);
    if (d_k == 128 && d_v == 64) return launch_prefill_dims<128, 64>(p, stream);
    if (d_k == 64 && d_v == 128) return launch_prefill_dims<64, 128>(p, stream);
    return hipErrorInvalidValue;
}

} // namespace gdn
