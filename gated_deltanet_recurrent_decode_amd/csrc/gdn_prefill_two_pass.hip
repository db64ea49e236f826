// gdn_prefill_two_pass.hip -- chunked Gated DeltaNet prefill in two passes
// (gfx950), for calls with few prompts.
//
// The one-kernel prefill (gdn_prefill.hip) walks a prompt's chunks inside one
// workgroup per (sequence, key head), so a single prompt keeps only H_k
// compute units busy however long it is.  Here the work that does not depend
// on the state entering a chunk runs first, in parallel over every chunk of
// every prompt, and only dense products stay in the sequential walk:
//
//   with (I + A)^-1, A and P as in the chunked form (mstar PR #1139 prefill in
//   place; the chunked delta rule), R = V - e^gamma K S0 and U = (I+A)^-1 diag(beta) R,
//     U  = U~ - W S0,         U~ = (I+A)^-1 diag(beta) V,   W = (I+A)^-1 diag(beta e^gamma) K
//     O  = Q~ S0 + P U,       Q~ = diag(e^gamma) Q
//     S1 = e^gamma_last S0 + K~^T U,   K~ = diag(e^(gamma_last - gamma)) K
//
// Pass 1 (one workgroup per chunk and value head): conv + SiLU (the three
// inputs before the chunk come from the slot's window for a prompt's first
// chunk, else from x), L2 norms, the running log decay, K K^T and Q K^T -> A
// and P, (I + A)^-1 by blocked forward substitution, then W and U~ on the
// matrix cores; Q~, K~, W, U~, P and e^gamma_last go to the workspace.
// Pass 2 (one workgroup per sequence, value head and slice of d_v columns):
// the slice of the state in LDS, the chunks in order, each three matrix-core
// products and the read-out; then the state and the advanced conv window go
// back to the slot.  Pass 1 reads the old windows and pass 2 writes the new
// ones, so no workgroup can read a window another has already advanced.
// A map kernel first turns each sequence's length into its run of chunk
// indices (an exclusive scan), which pass 1 searches.

#include "gdn_internal.h"
#include "prefill_internal.h"
#include "step_common.h"

namespace gdn {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BT = 32;  // tokens per chunk
constexpr int NT = 256; // threads per workgroup: four waves

__device__ __forceinline__ v4f mma16(float a, float b, v4f c)
{
    // D += A B on one 16x16 tile and a k-slice of 4: lane l supplies A[l%16][l/16]
    // and B[l/16][l%16]; D[i][j] sits at lane j + 16 (i / 4), element i % 4
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A byte offset past the end of every buffer resource used here: a load there
// returns 0 and a store there is dropped, with no memory access.
constexpr uint32_t kOOB = 0x80000000u;

// Base and size are the same for the whole workgroup: they are moved to scalar
// registers here, or a value the compiler happened to compute on the vector
// unit (a clamp, a 64-bit multiply-add) makes it wrap every access in a loop
// over the lanes' distinct resources.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes)
{
    // readfirstlane works on int: each half goes back through uint32_t so that
    // the low word is not sign-extended into the high one
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(hi << 32 | lo), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ v4f buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ bool sequence_usable(const PrefillParams &p, int b, int &t_begin, int &t_end, int &s)
{
    t_begin = p.cu_seqlens[b];
    t_end = p.cu_seqlens[b + 1];
    s = p.slot[b];
    return t_begin >= 0 && t_end >= t_begin && t_end <= p.total && s >= 0 && s < p.N;
}

// ---------------------------------------------------------------- chunk map

__global__ __launch_bounds__(NT) void tp_chunk_map_kernel(TwoPassParams tp)
{
    const PrefillParams &p = tp.p;
    __shared__ int scan[NT];
    const int tid = threadIdx.x;
    int carry = 0;
    for (int base = 0; base <= p.B; base += NT) {
        const int b = base + tid;
        int cnt = 0;
        if (b < p.B) {
            int t_begin, t_end, s;
            if (sequence_usable(p, b, t_begin, t_end, s) && s > 0)
                cnt = (t_end - t_begin + BT - 1) / BT;
        }
        scan[tid] = cnt;
        __syncthreads();
        for (int o = 1; o < NT; o <<= 1) {
            const int v = tid >= o ? scan[tid - o] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        if (b <= p.B)
            tp.ws.chunk_start[b] = carry + scan[tid] - cnt;
        carry += scan[NT - 1];
        __syncthreads(); // scan[] is rewritten by the next tile
    }
}

// ---------------------------------------------------------------- pass 1

template <int DK, int DV>
__global__ __launch_bounds__(NT) void tp_intra_kernel(TwoPassParams tp)
{
    const PrefillParams &p = tp.p;
    constexpr int NPAIR = (2 * DK + DV) / 2; // conv lanes, two channels each
    // LDS pitches as in the one-kernel prefill: A-style operand reads along a
    // row want 4 mod 32, B-style reads down a column 16 mod 32
    constexpr int KP = DK + 4, VP = DV + 16, AP = BT + 1;
    static_assert(NPAIR <= NT, "one conv lane per channel pair");

    __shared__ __align__(16) float Qs[BT * KP];
    __shared__ __align__(16) float Ks[BT * KP];
    __shared__ __align__(16) float Vs[BT * VP];
    __shared__ float Am[BT * AP];
    __shared__ float Pm[BT * AP];
    __shared__ float Tm[BT * AP];
    __shared__ float Mm[16 * 17];
    __shared__ float gam[BT], bet[BT], eg[BT], egl[BT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lk = lane >> 4;
    const int gidx = blockIdx.x;
    const int hv = blockIdx.y;
    const int hk = hv / p.G;
    const int32_t *cs = tp.ws.chunk_start;
    if (gidx >= cs[p.B])
        return;
    // the sequence owning chunk gidx: the last b with chunk_start[b] <= gidx
    // (sequences with no chunks share their start with the next one)
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cs[mid] <= gidx)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int b = lo;
    const int c = gidx - cs[b];
    const int t_begin = p.cu_seqlens[b];
    const int L = p.cu_seqlens[b + 1] - t_begin;
    const int s = p.slot[b];
    const int t0 = t_begin + c * BT;
    const int n = L - c * BT < BT ? L - c * BT : BT;
    const int C = p.C;
    const size_t T = (size_t)p.total;

    // ---- conv lanes: channel pair (e, e+1) of the q | k | v channels of (hk, hv)
    const bool conv_lane = tid < NPAIR;
    const int e = conv_lane ? 2 * tid : 0;
    const bool isq = e < DK, isk = !isq && e < 2 * DK;
    const int ch = isq ? hk * DK + e : isk ? p.H_k * DK + hk * DK + (e - DK) : 2 * p.H_k * DK + hv * DV + (e - 2 * DK);
    float w0[2], w1[2], w2[2], w3[2], bias[2], h0[2], h1[2], h2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint16_t *wc = p.conv_w + (size_t)(ch + h) * 4;
        w0[h] = bf16_to_f32(wc[0]);
        w1[h] = bf16_to_f32(wc[1]);
        w2[h] = bf16_to_f32(wc[2]);
        w3[h] = bf16_to_f32(wc[3]);
        bias[h] = p.conv_b ? bf16_to_f32(p.conv_b[ch + h]) : 0.f;
    }
    // the three inputs before the chunk (oldest first)
    uint32_t hist[3];
    if (c == 0) {
        const uint16_t *win = p.conv_state + (size_t)s * 3 * C + ch;
#pragma unroll
        for (int k = 0; k < 3; ++k)
            hist[k] = *reinterpret_cast<const uint32_t *>(win + (size_t)k * C);
    } else {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            hist[k] = *reinterpret_cast<const uint32_t *>(p.x + (size_t)(t0 - 3 + k) * p.x_row_stride + ch);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        h0[h] = __uint_as_float(h ? hist[0] & 0xffff0000u : hist[0] << 16);
        h1[h] = __uint_as_float(h ? hist[1] & 0xffff0000u : hist[1] << 16);
        h2[h] = __uint_as_float(h ? hist[2] & 0xffff0000u : hist[2] << 16);
    }
    uint32_t xb[BT];
#pragma unroll
    for (int tt = 0; tt < BT; ++tt)
        xb[tt] = (conv_lane && tt < n) ? *reinterpret_cast<const uint32_t *>(p.x + (size_t)(t0 + tt) * p.x_row_stride + ch)
                                       : 0u;
    const float g_in = tid < n ? p.g[(size_t)(t0 + tid) * p.H_v + hv] : 0.f;
    const float b_in = tid < n ? p.beta[(size_t)(t0 + tid) * p.H_v + hv] : 0.f;

    // ---- conv + SiLU; rows past the chunk's last token stay zero
    if (conv_lane) {
        float *ydst = isq ? &Qs[e] : isk ? &Ks[e - DK] : &Vs[e - 2 * DK];
        const int ypitch = (isq || isk) ? KP : VP;
        const bool has_bias = p.conv_b != nullptr;
#pragma unroll
        for (int tt = 0; tt < BT; ++tt) {
            float y0 = 0.f, y1 = 0.f;
            if (tt < n) {
                const float x0 = __uint_as_float(xb[tt] << 16), x1 = __uint_as_float(xb[tt] & 0xffff0000u);
                float acc0 = w0[0] * h0[0];
                acc0 = fmaf(w1[0], h1[0], acc0);
                acc0 = fmaf(w2[0], h2[0], acc0);
                acc0 = fmaf(w3[0], x0, acc0);
                float acc1 = w0[1] * h0[1];
                acc1 = fmaf(w1[1], h1[1], acc1);
                acc1 = fmaf(w2[1], h2[1], acc1);
                acc1 = fmaf(w3[1], x1, acc1);
                if (has_bias) {
                    acc0 += bias[0];
                    acc1 += bias[1];
                }
                y0 = acc0 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc0));
                y1 = acc1 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc1));
                h0[0] = h1[0]; h1[0] = h2[0]; h2[0] = x0;
                h0[1] = h1[1]; h1[1] = h2[1]; h2[1] = x1;
            }
            ydst[tt * ypitch] = y0;
            ydst[tt * ypitch + 1] = y1;
        }
    }
    if (tid < BT) {
        // the running log decay inside the chunk and the factors derived from it
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
    __syncthreads();

    // ---- L2 norms of q and k: eight lanes a token
    {
        const int tt = tid >> 3, sub = tid & 7;
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = sub; i < DK; i += 8) {
            const float qv = Qs[tt * KP + i], kv = Ks[tt * KP + i];
            sq = fmaf(qv, qv, sq);
            sk = fmaf(kv, kv, sk);
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            sq += __shfl_xor(sq, o, 64);
            sk += __shfl_xor(sk, o, 64);
        }
        if (tt < n) {
            const float qs = (1.0f / sqrtf(sq + p.l2_eps)) * p.q_scale;
            const float rk = 1.0f / sqrtf(sk + p.l2_eps);
#pragma unroll
            for (int i = sub; i < DK; i += 8) {
                Qs[tt * KP + i] *= qs;
                Ks[tt * KP + i] *= rk;
            }
        }
    }
    __syncthreads();

    // ---- K K^T (waves 0, 1) and Q K^T (waves 2, 3) -> the masked, decay-weighted A and P
    {
        const float *Asrc = wv < 2 ? Ks : Qs;
        const int rb = wv & 1;
        v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const float a = Asrc[(rb * 16 + li) * KP + k0 + lk];
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                acc[cb] = mma16(a, Ks[(cb * 16 + li) * KP + k0 + lk], acc[cb]);
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

    // ---- (I + A)^-1: the two 16x16 diagonal blocks by forward substitution
    // (thread j of a block solves column j), then T21 = -T22 (A21 T11)
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
            Tm[(b0 + tt) * AP + (b0 ^ 16) + j] = 0.f;
        }
    }
    __syncthreads();
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

    // ---- W = T diag(beta e^gamma) K and U~ = T diag(beta) V on the matrix
    // cores: this wave's column blocks of each, both row blocks; rows of real
    // tokens go to the workspace (the others are zero by construction)
    {
        constexpr int WCB = DK / 64, UCB = DV / 64;
        v4f wacc[2][WCB], uacc[2][UCB];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int q = 0; q < WCB; ++q)
                wacc[rb][q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < UCB; ++q)
                uacc[rb][q] = v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k0 = 0; k0 < BT; k0 += 4) {
            const float at0 = Tm[li * AP + k0 + lk], at1 = Tm[(16 + li) * AP + k0 + lk];
            const float bs = bet[k0 + lk];
            const float bse = bs * eg[k0 + lk];
#pragma unroll
            for (int q = 0; q < WCB; ++q) {
                const float bk = bse * Ks[(k0 + lk) * KP + (wv * WCB + q) * 16 + li];
                wacc[0][q] = mma16(at0, bk, wacc[0][q]);
                wacc[1][q] = mma16(at1, bk, wacc[1][q]);
            }
#pragma unroll
            for (int q = 0; q < UCB; ++q) {
                const float bv = bs * Vs[(k0 + lk) * VP + (wv * UCB + q) * 16 + li];
                uacc[0][q] = mma16(at0, bv, uacc[0][q]);
                uacc[1][q] = mma16(at1, bv, uacc[1][q]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = rb * 16 + 4 * lk + r;
                if (tt < n) {
                    const size_t row = (size_t)hv * T + t0 + tt;
#pragma unroll
                    for (int q = 0; q < WCB; ++q)
                        tp.ws.ww[row * DK + (wv * WCB + q) * 16 + li] = wacc[rb][q][r];
#pragma unroll
                    for (int q = 0; q < UCB; ++q)
                        tp.ws.ut[row * DV + (wv * UCB + q) * 16 + li] = uacc[rb][q][r];
                }
            }
    }

    // ---- Q~, K~, the rows of P and e^gamma_last
    for (int e2 = tid; e2 < n * (DK / 4); e2 += NT) {
        const int tt = e2 / (DK / 4), i4 = e2 % (DK / 4);
        const size_t row = (size_t)hv * T + t0 + tt;
        const v4f qv = *reinterpret_cast<const v4f *>(&Qs[tt * KP + 4 * i4]);
        const v4f kv = *reinterpret_cast<const v4f *>(&Ks[tt * KP + 4 * i4]);
        *reinterpret_cast<v4f *>(tp.ws.qt + row * DK + 4 * i4) = qv * eg[tt];
        *reinterpret_cast<v4f *>(tp.ws.kt + row * DK + 4 * i4) = kv * egl[tt];
    }
    for (int e2 = tid; e2 < n * BT; e2 += NT) {
        const int tt = e2 / BT, ss = e2 % BT;
        tp.ws.pp[((size_t)hv * T + t0 + tt) * BT + ss] = Pm[tt * AP + ss];
    }
    if (tid == 0)
        tp.ws.el[(size_t)hv * T + t0] = eg[BT - 1]; // padding tokens carry g = 0
}

// ---------------------------------------------------------------- pass 2

template <int DK, int DV, int DVS>
__global__ __launch_bounds__(NT) void tp_inter_kernel(TwoPassParams tp)
{
    const PrefillParams &p = tp.p;
    constexpr int NSL = DV / DVS;
    constexpr int KP = DK + 4;                                  // W, Q~: A operands read along a row
    constexpr int K2P = DK + 16;                                // K~: the S update's A operand, read down a column
    constexpr int SP = DVS + ((DVS + 16) % 32 == 16 ? 16 : 32); // S and U: B operands, read down a column
    constexpr int PPI = BT + 4;                                 // P: A operand read along a row
    constexpr int CBS = DVS / 16;                               // column blocks of the slice
    // output tiles (row block, column block) of W S0, Q~ S0 and O a wave takes;
    // a 16-column slice has two, so waves 0-1 take W S0 and waves 2-3 Q~ S0 and O
    constexpr bool SPLIT = CBS == 1;
    constexpr int TPW = SPLIT ? 1 : 2 * CBS / 4;
    constexpr int RBW = DK / 16 / 4;                            // row blocks of S a wave updates
    constexpr int NW4 = BT * DK / 4 / NT;                       // float4 a thread stages of W, Q~, K~
    constexpr int NU4E = BT * DVS / 4;                          // float4 of U~ a chunk
    constexpr int NU4 = (NU4E + NT - 1) / NT;                   // ... a thread
    constexpr int NP4 = BT * BT / 4 / NT;                       // ... of P
    static_assert(NW4 >= 1 && NP4 == 1 && DVS >= 16, "slices of 16 columns or more");

    __shared__ __align__(16) float S[DK * SP];
    __shared__ __align__(16) float Wm[BT * KP];
    __shared__ __align__(16) float Qm[BT * KP];
    __shared__ __align__(16) float Km[BT * K2P];
    __shared__ __align__(16) float Um[BT * SP];
    __shared__ __align__(16) float Pm[BT * PPI];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lk = lane >> 4;
    const int sl = blockIdx.x % NSL;
    const int bh = blockIdx.x / NSL;
    const int hv = bh % p.H_v;
    const int b = bh / p.H_v;
    const int col0 = sl * DVS;
    int t_begin, t_end, s;
    if (!sequence_usable(p, b, t_begin, t_end, s))
        return; // an unusable range or slot touches nothing
    // one value for the whole workgroup: the buffer resources built from these
    // must sit in scalar registers
    t_begin = __builtin_amdgcn_readfirstlane(t_begin);
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    s = __builtin_amdgcn_readfirstlane(s);
    if (s == 0) {
        // padding sequence on the null slot: its read-out is +0.0
        for (int e = tid; e < (t_end - t_begin) * DVS; e += NT)
            p.out[((size_t)(t_begin + e / DVS) * p.H_v + hv) * DV + col0 + e % DVS] = 0;
        return;
    }
    if (t_end == t_begin)
        return;
    const size_t T = (size_t)p.total;
    float *tile = p.state + ((size_t)s * p.H_v + hv) * (size_t)(DK * DV);

    // ---- the state's column slice -> LDS (16-byte streaming loads)
    for (int e = tid; e < DK * DVS / 4; e += NT) {
        const int i = e / (DVS / 4), j4 = e % (DVS / 4);
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(tile + (size_t)i * DV + col0) + j4);
        *reinterpret_cast<v4f *>(&S[i * SP + 4 * j4]) = v;
    }

    // ---- a chunk's pass-1 results, staged in registers one chunk ahead.  The
    // loads are buffer loads over the chunk's real rows only (rows past the
    // prompt's end, or a chunk past it, read zeros without touching memory),
    // so the walk has no branch around a memory access and every wait in it
    // covers exactly the loads it needs, not the read-out stores in flight.
    v4f rw[NW4], rq[NW4], rk[NW4], ru[NU4], rp[NP4];
    float rel = 0.f;
    auto prefetch = [&](int c0) {
        c0 = __builtin_amdgcn_readfirstlane(c0);
        int nn = t_end - c0;
        nn = nn < 0 ? 0 : (nn > BT ? BT : nn);
        const size_t row0 = (size_t)hv * T + (size_t)c0;
        const __amdgpu_buffer_rsrc_t rW = buf_rsrc(tp.ws.ww + row0 * DK, (uint32_t)(nn * DK * 4));
        const __amdgpu_buffer_rsrc_t rQ = buf_rsrc(tp.ws.qt + row0 * DK, (uint32_t)(nn * DK * 4));
        const __amdgpu_buffer_rsrc_t rK = buf_rsrc(tp.ws.kt + row0 * DK, (uint32_t)(nn * DK * 4));
        const __amdgpu_buffer_rsrc_t rU =
            buf_rsrc(tp.ws.ut + row0 * DV + col0, nn > 0 ? (uint32_t)(((nn - 1) * DV + DVS) * 4) : 0u);
        const __amdgpu_buffer_rsrc_t rP = buf_rsrc(tp.ws.pp + row0 * BT, (uint32_t)(nn * BT * 4));
#pragma unroll
        for (int m = 0; m < NW4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (DK / 4), i4 = e4 % (DK / 4);
            const uint32_t off = (uint32_t)(tt * DK + 4 * i4) * 4u;
            rw[m] = buf_load4(rW, off);
            rq[m] = buf_load4(rQ, off);
            rk[m] = buf_load4(rK, off);
        }
#pragma unroll
        for (int m = 0; m < NU4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (DVS / 4), j4 = e4 % (DVS / 4);
            ru[m] = buf_load4(rU, e4 < NU4E ? (uint32_t)(tt * DV + 4 * j4) * 4u : kOOB);
        }
#pragma unroll
        for (int m = 0; m < NP4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (BT / 4), s4 = e4 % (BT / 4);
            rp[m] = buf_load4(rP, (uint32_t)(tt * BT + 4 * s4) * 4u);
        }
        rel = tp.ws.el[(size_t)hv * T + (size_t)__builtin_amdgcn_readfirstlane(c0 < t_end ? c0 : t_end - 1)];
    };
    prefetch(t_begin);

    for (int t0 = t_begin; t0 < t_end; t0 += BT) {
        const int n = t_end - t0 < BT ? t_end - t0 : BT;
        const float el = rel;
#pragma unroll
        for (int m = 0; m < NW4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (DK / 4), i4 = e4 % (DK / 4);
            *reinterpret_cast<v4f *>(&Wm[tt * KP + 4 * i4]) = rw[m];
            *reinterpret_cast<v4f *>(&Qm[tt * KP + 4 * i4]) = rq[m];
            *reinterpret_cast<v4f *>(&Km[tt * K2P + 4 * i4]) = rk[m];
        }
#pragma unroll
        for (int m = 0; m < NU4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (DVS / 4), j4 = e4 % (DVS / 4);
            if (e4 < NU4E)
                *reinterpret_cast<v4f *>(&Um[tt * SP + 4 * j4]) = ru[m];
        }
#pragma unroll
        for (int m = 0; m < NP4; ++m) {
            const int e4 = tid + NT * m, tt = e4 / (BT / 4), s4 = e4 % (BT / 4);
            *reinterpret_cast<v4f *>(&Pm[tt * PPI + 4 * s4]) = rp[m];
        }
        __syncthreads(); // the chunk is staged (and the previous chunk's S update is in)
        prefetch(t0 + BT);
        // the read-out rows of the chunk's real tokens; later rows fall outside
        const int t0u = __builtin_amdgcn_readfirstlane(t0), nu = __builtin_amdgcn_readfirstlane(n);
        const __amdgpu_buffer_rsrc_t rO = buf_rsrc(p.out + ((size_t)t0u * p.H_v + hv) * DV + col0,
                                                   (uint32_t)(((nu - 1) * p.H_v * DV + DVS) * 2));

        if constexpr (SPLIT) {
            // ---- waves 0-1: W S0 and U = U~ - W S0 on row block wv; waves 2-3:
            // Q~ S0 on row block wv - 2, then O = Q~ S0 + P U -> out
            const int rb = wv & 1;
            const bool is_w = wv < 2;
            const float *Asrc = is_w ? Wm : Qm;
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k0 = 0; k0 < DK; k0 += 4)
                acc = mma16(Asrc[(rb * 16 + li) * KP + k0 + lk], S[(k0 + lk) * SP + li], acc);
            if (is_w) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Um[(rb * 16 + 4 * lk + r) * SP + li] -= acc[r];
            }
            __syncthreads(); // U complete; every read of S0 for this chunk is done
            if (!is_w) {
#pragma unroll
                for (int k0 = 0; k0 < BT; k0 += 4)
                    acc = mma16(Pm[(rb * 16 + li) * PPI + k0 + lk], Um[(k0 + lk) * SP + li], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = rb * 16 + 4 * lk + r;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(acc[r]), rO,
                                                          (uint32_t)(tt * p.H_v * DV + li) * 2u, 0, 0);
                }
            }
        } else {
            // ---- W S0 and Q~ S0 on this wave's output tiles
            v4f aw[TPW], aq[TPW];
#pragma unroll
            for (int k = 0; k < TPW; ++k)
                aw[k] = aq[k] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 4) {
#pragma unroll
                for (int k = 0; k < TPW; ++k) {
                    const int ti = wv * TPW + k, rb = ti & 1, cb = ti >> 1;
                    const float bs = S[(k0 + lk) * SP + cb * 16 + li];
                    aw[k] = mma16(Wm[(rb * 16 + li) * KP + k0 + lk], bs, aw[k]);
                    aq[k] = mma16(Qm[(rb * 16 + li) * KP + k0 + lk], bs, aq[k]);
                }
            }
            // U = U~ - W S0 over the same tiles (a wave reads and writes only its own)
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int ti = wv * TPW + k, rb = ti & 1, cb = ti >> 1;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Um[(rb * 16 + 4 * lk + r) * SP + cb * 16 + li] -= aw[k][r];
            }
            __syncthreads(); // U complete; every read of S0 for this chunk is done

            // ---- O = Q~ S0 + P U -> out (rows of real tokens)
#pragma unroll
            for (int k0 = 0; k0 < BT; k0 += 4) {
#pragma unroll
                for (int k = 0; k < TPW; ++k) {
                    const int ti = wv * TPW + k, rb = ti & 1, cb = ti >> 1;
                    aq[k] = mma16(Pm[(rb * 16 + li) * PPI + k0 + lk], Um[(k0 + lk) * SP + cb * 16 + li], aq[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int ti = wv * TPW + k, rb = ti & 1, cb = ti >> 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = rb * 16 + 4 * lk + r;
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(aq[k][r]), rO,
                                                          (uint32_t)(tt * p.H_v * DV + cb * 16 + li) * 2u, 0, 0);
                }
            }
        }

        // ---- S1 = e^gamma_last S0 + K~^T U: this wave's row blocks, the slice's column blocks
        {
            v4f sacc[RBW][CBS];
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBS; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sacc[q][jb][r] = el * S[((wv * RBW + q) * 16 + 4 * lk + r) * SP + jb * 16 + li];
#pragma unroll
            for (int k0 = 0; k0 < BT; k0 += 4) {
#pragma unroll
                for (int q = 0; q < RBW; ++q) {
                    const float a = Km[(k0 + lk) * K2P + (wv * RBW + q) * 16 + li];
#pragma unroll
                    for (int jb = 0; jb < CBS; ++jb)
                        sacc[q][jb] = mma16(a, Um[(k0 + lk) * SP + jb * 16 + li], sacc[q][jb]);
                }
            }
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBS; ++jb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[((wv * RBW + q) * 16 + 4 * lk + r) * SP + jb * 16 + li] = sacc[q][jb][r];
        }
        __syncthreads(); // S, U and the staging buffers are free for the next chunk
    }

    // ---- the state's slice back to the slot
    for (int e = tid; e < DK * DVS / 4; e += NT) {
        const int i = e / (DVS / 4), j4 = e % (DVS / 4);
        const v4f v = *reinterpret_cast<const v4f *>(&S[i * SP + 4 * j4]);
        __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(tile + (size_t)i * DV + col0) + j4);
    }

    // ---- the advanced conv windows: the last three inputs of [window, prompt]
    // for this slice's v channels, and for the key head's q and k channels from
    // its first value head's first slice.  Nothing else reads or writes these
    // channels of this slot now: pass 1 is over.
    const int L = t_end - t_begin;
    const int C = p.C;
    const int hk = hv / p.G;
    const bool qk_owner = (hv % p.G == 0) && sl == 0;
    const int npair = DVS / 2 + (qk_owner ? DK : 0);
    uint16_t *win = p.conv_state + (size_t)s * 3 * C;
    for (int e = tid; e < npair; e += NT) {
        const int ch = e < DVS / 2 ? 2 * p.H_k * DK + hv * DV + col0 + 2 * e
                       : e < DVS / 2 + DK / 2 ? hk * DK + 2 * (e - DVS / 2)
                                             : p.H_k * DK + hk * DK + 2 * (e - DVS / 2 - DK / 2);
        uint32_t old[3], nw[3];
#pragma unroll
        for (int k = 0; k < 3; ++k)
            old[k] = *reinterpret_cast<const uint32_t *>(win + (size_t)k * C + ch);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int pos = L - 3 + k; // position in the prompt of the new tap k
            nw[k] = pos >= 0   ? *reinterpret_cast<const uint32_t *>(p.x + (size_t)(t_begin + pos) * p.x_row_stride + ch)
                    : pos == -1 ? old[2]
                    : pos == -2 ? old[1]
                                : old[0];
        }
#pragma unroll
        for (int k = 0; k < 3; ++k)
            *reinterpret_cast<uint32_t *>(win + (size_t)k * C + ch) = nw[k];
    }
}

template <int DK, int DV, int DVS>
hipError_t launch_inter(const TwoPassParams &tp, long long heads, hipStream_t stream)
{
    TwoPassParams q = tp;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&tp_inter_kernel<DK, DV, DVS>),
                           dim3((unsigned)(heads * (DV / DVS))), dim3(NT), args, 0, stream);
}

template <int DK, int DV>
hipError_t launch_dims(const TwoPassParams &tp, hipStream_t stream)
{
    const PrefillParams &p = tp.p;
    TwoPassParams q = tp;
    void *args[] = {&q};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_chunk_map_kernel), dim3(1), dim3(NT), args, 0,
                                   stream);
    if (e != hipSuccess)
        return e;
    // an upper bound on the chunk count: each sequence adds at most one partial chunk
    const long long gx = ((long long)p.total + BT - 1) / BT + p.B;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_intra_kernel<DK, DV>), dim3((unsigned)gx, (unsigned)p.H_v),
                        dim3(NT), args, 0, stream);
    if (e != hipSuccess)
        return e;
    // column slices: double them until the walk has 256 workgroups or the
    // slices are 16 columns wide
    const long long heads = (long long)p.B * p.H_v;
    int nsl = 1;
    while (nsl < DV / 16 && heads * nsl < 256)
        nsl *= 2;
    switch (nsl) {
    case 1: return launch_inter<DK, DV, DV>(tp, heads, stream);
    case 2: return launch_inter<DK, DV, DV / 2>(tp, heads, stream);
    case 4: return launch_inter<DK, DV, DV / 4>(tp, heads, stream);
    default: return launch_inter<DK, DV, (DV / 8 >= 16 ? DV / 8 : 16)>(tp, heads, stream);
    }
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

} // namespace

size_t two_pass_layout(int B, int total, int H_v, int d_k, int d_v, void *base, TwoPassWorkspace *ws)
{
    const size_t rows = (size_t)H_v * (size_t)total;
    size_t off = 0;
    const size_t o_cs = off;
    off = round_up(off + (size_t)(B + 1) * sizeof(int32_t));
    const size_t o_qt = off;
    off = round_up(off + rows * d_k * sizeof(float));
    const size_t o_kt = off;
    off = round_up(off + rows * d_k * sizeof(float));
    const size_t o_ww = off;
    off = round_up(off + rows * d_k * sizeof(float));
    const size_t o_ut = off;
    off = round_up(off + rows * d_v * sizeof(float));
    const size_t o_pp = off;
    off = round_up(off + rows * BT * sizeof(float));
    const size_t o_el = off;
    off = round_up(off + rows * sizeof(float));
    if (base && ws) {
        char *c = static_cast<char *>(base);
        ws->chunk_start = reinterpret_cast<int32_t *>(c + o_cs);
        ws->qt = reinterpret_cast<float *>(c + o_qt);
        ws->kt = reinterpret_cast<float *>(c + o_kt);
        ws->ww = reinterpret_cast<float *>(c + o_ww);
        ws->ut = reinterpret_cast<float *>(c + o_ut);
        ws->pp = reinterpret_cast<float *>(c + o_pp);
        ws->el = reinterpret_cast<float *>(c + o_el);
    }
    return off;
}

hipError_t launch_gdn_prefill_two_pass(const TwoPassParams &p, int d_k, int d_v, hipStream_t stream)
{
    if (p.p.B <= 0 || p.p.total <= 0)
        return hipSuccess;
    if (d_k == 128 && d_v == 128) return launch_dims<128, 128>(p, stream);
    if (d_k == 64 && d_v == 64) return launch_dims<64, 64>(p, stream);
    if (d_k == 128 && d_v == 64) return launch_dims<128, 64>(p, stream);
    if (d_k == 64 && d_v == 128) return launch_dims<64, 128>(p, stream);
    return hipErrorInvalidValue;
}

} // namespace gdn
