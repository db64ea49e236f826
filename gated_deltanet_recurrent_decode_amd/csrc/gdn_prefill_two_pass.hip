// gdn_prefill_two_pass.hip -- chunked Gated DeltaNet prefill in two passes
// (gfx950).
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
// Two workspace layouts (two_pass_slim picks one from the call's shape):
//
// Full (fewer prompt-head pairs than the compute units take, or a ragged last
// round).  Pass 1 (workgroups per value head, each walking every gx-th chunk
// of the call): conv + SiLU (the three inputs before the chunk come from the
// slot's window for a prompt's first chunk, else from x), L2 norms, the
// running log decay, K K^T and Q K^T -> A and P, (I + A)^-1 by blocked forward
// substitution, then W and U~ on the matrix cores; Q~, K~, W, U~, P and
// e^gamma_last go to the workspace.  Pass 2 (one workgroup per sequence,
// value head and slice of d_v columns): the chunks in order, each three
// matrix-core products and the read-out, with a 16-column slice of the state
// in registers and a wider one in LDS.
//
// Slim (256 or more pairs in nearly whole rounds of 256).  Pass 1 keeps only
// what needs the chunk's triangular solve, T' = (I + A)^-1 diag(beta), P and
// per-token row factors (an eighth of the full layout), and copies each
// prompt's old window; pass 2, a workgroup per sequence and value head, runs
// the conv again from x and forms U = T' (V - e^gamma K^ S0) on the matrix
// cores.
//
// In both, pass 2 then writes the state and the advanced conv window back to
// the slot.  Pass 1 reads the old windows and pass 2 writes the new ones, so
// no workgroup can read a window another has already advanced.
// A map kernel first turns each sequence's length into its run of chunk
// indices (an exclusive scan) and writes each chunk's record (first token,
// tokens, slot, and the sequence's index + 1 at its first chunk), which pass
// 1 reads with one load instead of searching the scan.

#include "gdn_internal.h"
#include "prefill_internal.h"
#include "step_common.h"

#include <climits>
#include <type_traits>

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

// fp32 -> bf16 bits, round to nearest even, a NaN kept quiet: the same bits as
// f32_to_bf16_rne, as selects instead of a branch around each store
__device__ __forceinline__ uint16_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x0040u;
    return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
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
    // every chunk's record: a thread a chunk finds its sequence in the scan just
    // written (the barrier above made this workgroup's stores visible to it)
    const int32_t *cs = tp.ws.chunk_start;
    const int nch = carry < tp.ws.nchunk ? carry : tp.ws.nchunk;
    for (int g = tid; g < nch; g += NT) {
        // the last b with chunk_start[b] <= g (sequences with no chunks share
        // their start with the next one)
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cs[mid] <= g)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int c = g - cs[lo];
        const int t_begin = p.cu_seqlens[lo];
        const int L = p.cu_seqlens[lo + 1] - t_begin;
        *reinterpret_cast<int4 *>(tp.ws.chunk_rec + 4 * (size_t)g) =
            make_int4(t_begin + c * BT, L - c * BT < BT ? L - c * BT : BT, p.slot[lo], c == 0 ? lo + 1 : 0);
    }
}

// ---------------------------------------------------------------- pass 1

// full layout: two workgroups a CU (LDS allows two), at most 256 registers a
// lane, which the compiler meets by recomputing LDS addresses inside the chunk
// loop; slim: three (at most 168 registers).
// SLIM: the slim layout (T', P and the row factors; no V, W or U~), the q | k
// conv spread over every lane in runs of tokens, and each prompt's old window
// copied to hw at its first chunk.
// The body of a pass-1 workgroup: (bx, hv) of a gx-wide grid takes the
// chunks lo + bx, lo + bx + gx, ... below hi (and below the call's count).
// With at most NT prompts the workgroup builds the chunk map itself (the
// chunk map kernel's scan, in LDS: kMapInLds) and, with write_map, also
// stores each prompt's first chunk for the walks.
template <int DK, int DV, bool SLIM>
__device__ __forceinline__ void intra_body(const TwoPassParams &tp, int bx, int gx, int hv, int lo, int hi,
                                           bool write_map)
{
    const PrefillParams &p = tp.p;
    constexpr int NPAIR = SLIM ? NT : (2 * DK + DV) / 2; // conv lanes, two channels each
    constexpr int NRUN = SLIM ? NT / DK : 1;             // runs of tokens (slim: DK pairs a run)
    constexpr int TPT = BT / NRUN;                       // tokens a run
    static_assert(!SLIM || (NT % DK == 0 && BT % NRUN == 0), "whole runs");
    // LDS pitches as in the one-kernel prefill: A-style operand reads along a
    // row want 4 mod 32, B-style reads down a column 16 mod 32
    constexpr int KP = DK + 4, VP = DV + 16, AP = BT + 1;
    static_assert(NPAIR <= NT, "one conv lane per channel pair");
    static_assert((2 * (DK / 16) * 64) % NT == 0, "whole store rounds");

    __shared__ __align__(16) float Qs[BT * KP];
    __shared__ __align__(16) float Ks[BT * KP];
    __shared__ __align__(16) float Vs[SLIM ? 4 : BT * (VP > KP ? VP : KP)]; // V, then W
    __shared__ float Am[BT * AP];
    __shared__ float Pm[BT * AP];
    __shared__ float Tm[BT * AP];
    __shared__ float Mm[16 * 17];
    __shared__ float gam[BT], bet[BT], eg[BT], egl[BT];
    // the chunk map of calls of at most NT prompts: each prompt's first chunk
    // (cstart[B] = the call's chunk count), its first token, length and slot
    __shared__ int cstart[NT + 1], ctb[NT], clen[NT], cslot[NT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lk = lane >> 4;
    const int hk = hv / p.G;
    const int C = p.C;
    const bool local_map = p.B <= NT;
    if (local_map) {
        // the chunk map kernel's scan: chunks of each usable prompt on a slot
        // other than the null slot, exclusive prefix sums in prompt order
        int cnt = 0, t_begin = 0, t_end = 0, s = 0;
        if (tid < p.B && sequence_usable(p, tid, t_begin, t_end, s) && s > 0)
            cnt = (t_end - t_begin + BT - 1) / BT;
        if (tid < p.B) {
            ctb[tid] = t_begin;
            clen[tid] = t_end - t_begin;
            cslot[tid] = s;
        }
        int *scan = reinterpret_cast<int *>(Am); // free until the chunk loop
        scan[tid] = cnt;
        __syncthreads();
        // inclusive sums: after the rounds with o < B every entry below B sums
        // all entries from 0 (the rounds beyond would only add zeros to them)
        for (int o = 1; o < p.B; o <<= 1) {
            const int v = tid >= o ? scan[tid - o] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        if (tid < p.B) {
            const int start = tid == 0 ? 0 : scan[tid - 1];
            cstart[tid] = start;
            if (write_map)
                tp.ws.chunk_start[tid] = start;
        }
        // the call's chunk count, the inclusive sum at B - 1: written apart
        // from the starts above, which cover tid < B only (with B = NT no
        // thread has tid = B)
        if (tid == 0) {
            const int total = p.B > 0 ? scan[p.B - 1] : 0;
            cstart[p.B] = total;
            if (write_map)
                tp.ws.chunk_start[p.B] = total;
        }
        __syncthreads();
    }
    const int32_t *cs = tp.ws.chunk_start;
    // chunks past the workspace's capacity exist only when ranges overlap,
    // which the contract excludes; they are skipped rather than written out of bounds
    const int ctotal = local_map ? cstart[p.B] : cs[p.B];
    const int nall = __builtin_amdgcn_readfirstlane(ctotal < tp.ws.nchunk ? ctotal : tp.ws.nchunk);
    const int nch = nall < hi ? nall : hi; // this body's chunks end here
    if (nch <= 0 || lo + bx >= nch)
        return;

    // ---- conv lanes: channel pair (e, e+1) of the q | k | v channels of (hk, hv)
    // (slim: the q | k channels, run `run` of the chunk's tokens)
    const bool conv_lane = tid < NPAIR;
    const int run = SLIM ? __builtin_amdgcn_readfirstlane(tid / DK) : 0; // the same across a wave
    const int e = SLIM ? 2 * (tid % DK) : conv_lane ? 2 * tid : 0;
    const bool isq = e < DK, isk = !isq && e < 2 * DK;
    const int ch = isq ? hk * DK + e : isk ? p.H_k * DK + hk * DK + (e - DK) : 2 * p.H_k * DK + hv * DV + (e - 2 * DK);
    float w0[2], w1[2], w2[2], w3[2], bias[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint16_t *wc = p.conv_w + (size_t)(ch + h) * 4;
        w0[h] = bf16_to_f32(wc[0]);
        w1[h] = bf16_to_f32(wc[1]);
        w2[h] = bf16_to_f32(wc[2]);
        w3[h] = bf16_to_f32(wc[3]);
        bias[h] = p.conv_b ? bf16_to_f32(p.conv_b[ch + h]) : 0.f;
    }

    // ---- a chunk's inputs: its record, the three inputs before it (from the
    // slot's window for a prompt's first chunk, else from x), its x rows and
    // gates.  The workgroup walks chunks lo + bx, + gx, ... and
    // loads the next one's inputs while it computes the current one; x and the
    // gates come through buffer resources over the chunk's real rows (later
    // rows read zeros), so no branch surrounds those loads.
    struct ChunkIn {
        uint32_t xb[TPT];
        uint32_t hist[3]; // the three inputs before the run: window or x
        float g_in, b_in;
        int t0, n, sl;
        int b1; // the sequence's index + 1 at its first chunk, else 0
    };
    // chunk g's record: (first token, tokens, slot, prompt + 1 at its first chunk, else 0)
    auto record = [&](int gq) -> int4 {
        if (!local_map)
            return *reinterpret_cast<const int4 *>(tp.ws.chunk_rec + 4 * (size_t)gq);
        // the last prompt whose first chunk is at or before g (prompts with no
        // chunks share their start with the next one)
        int a = 0, z = p.B - 1;
        while (a < z) {
            const int mid = (a + z + 1) >> 1;
            if (cstart[mid] <= gq)
                a = mid;
            else
                z = mid - 1;
        }
        const int c = gq - cstart[a];
        const int L = clen[a];
        return make_int4(ctb[a] + c * BT, L - c * BT < BT ? L - c * BT : BT, cslot[a], c == 0 ? a + 1 : 0);
    };
    auto load = [&](int gi, ChunkIn &in) {
        const int gq = __builtin_amdgcn_readfirstlane(gi < nch ? gi : nch - 1); // past the end: a real chunk, unused
        const int4 rec = record(gq);
        const int t0 = __builtin_amdgcn_readfirstlane(rec.x);
        const int n = __builtin_amdgcn_readfirstlane(rec.y);
        const int sl = __builtin_amdgcn_readfirstlane(rec.z);
        const int b1 = __builtin_amdgcn_readfirstlane(rec.w);
        const bool first = b1 != 0;
        const __amdgpu_buffer_rsrc_t rx =
            buf_rsrc(p.x + (size_t)t0 * p.x_row_stride, (uint32_t)(((n - 1) * p.x_row_stride + C) * 2));
        // the three inputs before the first run: the slot's window for a
        // prompt's first chunk, else x; before a later run (slim): x rows of
        // the chunk itself (a resource chosen per wave)
        const uint16_t *hb = first ? p.conv_state + (size_t)sl * 3 * C : p.x + (size_t)(t0 - 3) * p.x_row_stride;
        const int hs = first ? C : (int)p.x_row_stride;
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hb, (uint32_t)((2 * (int64_t)hs + C) * 2));
#pragma unroll
        for (int k = 0; k < 3; ++k)
            in.hist[k] = __builtin_amdgcn_raw_buffer_load_b32(
                run == 0 ? rh : rx,
                run == 0 ? (uint32_t)(k * hs + ch) * 2u : (uint32_t)((run * TPT - 3 + k) * p.x_row_stride + ch) * 2u, 0, 0);
        // (lanes without a channel pair load nothing: past the resource)
#pragma unroll
        for (int tt = 0; tt < TPT; ++tt)
            in.xb[tt] = __builtin_amdgcn_raw_buffer_load_b32(
                rx, conv_lane ? (uint32_t)((run * TPT + tt) * p.x_row_stride + ch) * 2u : kOOB, 0, 0);
        const __amdgpu_buffer_rsrc_t rg = buf_rsrc(p.g + (size_t)t0 * p.H_v, (uint32_t)(n * p.H_v * 4));
        const __amdgpu_buffer_rsrc_t rb_ = buf_rsrc(p.beta + (size_t)t0 * p.H_v, (uint32_t)(n * p.H_v * 4));
        const uint32_t goff = (uint32_t)((tid & (BT - 1)) * p.H_v + hv) * 4u; // lanes past BT: unused copies
        in.g_in = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
        in.b_in = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb_, goff, 0, 0));
        in.t0 = t0;
        in.n = n;
        in.sl = sl;
        in.b1 = b1;
    };

    ChunkIn cur, nxt;
    load(lo + bx, cur);
    for (int g = lo + bx; g < nch; g += gx) {
        const int n = cur.n;
        const uint32_t *hx = cur.hist;
        float h0[2], h1[2], h2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            h0[h] = __uint_as_float(h ? hx[0] & 0xffff0000u : hx[0] << 16);
            h1[h] = __uint_as_float(h ? hx[1] & 0xffff0000u : hx[1] << 16);
            h2[h] = __uint_as_float(h ? hx[2] & 0xffff0000u : hx[2] << 16);
        }

        // slim: a prompt's first chunk keeps its old window for the second pass
        // (q | k from the first run's lanes, the v channels copied here)
        if (SLIM && cur.b1 != 0) {
            if (run == 0) {
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    *reinterpret_cast<uint32_t *>(tp.ws.hw + ((size_t)(cur.b1 - 1) * 3 + k) * C + ch) = cur.hist[k];
            }
            for (int q = tid; q < DV / 2; q += NT) {
                const int cv = 2 * p.H_k * DK + hv * DV + 2 * q;
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    *reinterpret_cast<uint32_t *>(tp.ws.hw + ((size_t)(cur.b1 - 1) * 3 + k) * C + cv) =
                        *reinterpret_cast<const uint32_t *>(p.conv_state + ((size_t)cur.sl * 3 + k) * C + cv);
            }
        }

        // ---- conv + SiLU; rows past the chunk's last token stay zero
        if (conv_lane) {
            float *ydst = isq ? &Qs[e] : (SLIM || isk) ? &Ks[e - DK] : &Vs[e - 2 * DK];
            const int ypitch = (isq || isk) ? KP : VP;
            const bool has_bias = p.conv_b != nullptr;
            // the pair's two outputs of a token are adjacent: one 8-byte store.
            // Tokens past the chunk's end are computed on the zeros their loads
            // returned and stored as zero, with no branch per token.
#pragma unroll
            for (int tt = 0; tt < TPT; ++tt) {
                const float x0 = __uint_as_float(cur.xb[tt] << 16), x1 = __uint_as_float(cur.xb[tt] & 0xffff0000u);
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
                const bool live = run * TPT + tt < n;
                const float y0 = live ? acc0 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc0)) : 0.f;
                const float y1 = live ? acc1 * __builtin_amdgcn_rcpf(1.0f + __expf(-acc1)) : 0.f;
                h0[0] = h1[0]; h1[0] = h2[0]; h2[0] = x0;
                h0[1] = h1[1]; h1[1] = h2[1]; h2[1] = x1;
                *reinterpret_cast<float2 *>(&ydst[(run * TPT + tt) * ypitch]) = make_float2(y0, y1);
            }
        }
        // the next chunk's inputs load while this one computes; issued after
        // the conv, so only one chunk's x rows are live in registers at a time
        load(g + gx, nxt);
        if (tid < BT) {
            // the running log decay inside the chunk and the factors derived from it
            float gsum = cur.g_in;
#pragma unroll
            for (int o = 1; o < BT; o <<= 1) {
                const float up = __shfl_up(gsum, o, 64);
                if (tid >= o)
                    gsum += up;
            }
            const float glast = __shfl(gsum, BT - 1, 64);
            gam[tid] = gsum;
            bet[tid] = cur.b_in;
            eg[tid] = expf(gsum);
            egl[tid] = expf(glast - gsum);
        }
        __syncthreads();

        // ---- L2 norms of q and k: eight lanes a token, each lane four runs of
        // four values (16-byte accesses), held in registers until scaled
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
            const float qs = (1.0f / sqrtf(sq + p.l2_eps)) * p.q_scale;
            const float rk = 1.0f / sqrtf(sk + p.l2_eps);
            if constexpr (SLIM) {
                // the second pass's row factors (zero for a padding token)
                if (sub < 3) {
                    const size_t blk = (size_t)hv * tp.ws.nchunk + g;
                    const float f = sub == 0 ? rk * eg[tt] : sub == 1 ? qs * eg[tt] : rk * egl[tt];
                    tp.ws.fac[blk * 128 + sub * BT + tt] = tt < n ? f : 0.f;
                }
            }
            if (tt < n) {
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

        // ---- K K^T (waves 0, 1) and Q K^T (waves 2, 3) -> the masked, decay-weighted A and P
        {
            const float *Asrc = wv < 2 ? Ks : Qs;
            const int rb = __builtin_amdgcn_readfirstlane(wv & 1);
            v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
            // a dot product over k, so its k-steps may run in any order: step
            // (m, r) takes k = 16 m + 4 lk + r, and a lane's four values of a k
            // block are one 16-byte read.  Row block 0 against column block 1
            // lies above the diagonal, where both masks below give zero: not
            // computed.
            auto products = [&](auto ncb) {
                constexpr int NCB = decltype(ncb)::value;
#pragma unroll 4
                for (int m = 0; m < DK / 16; ++m) {
                    const v4f a4 = *reinterpret_cast<const v4f *>(&Asrc[(rb * 16 + li) * KP + 16 * m + 4 * lk]);
                    v4f b4[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        b4[cb] = *reinterpret_cast<const v4f *>(&Ks[(cb * 16 + li) * KP + 16 * m + 4 * lk]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            acc[cb] = mma16(a4[r], b4[cb][r], acc[cb]);
                }
            };
            if (rb == 0)
                products(std::integral_constant<int, 1>{});
            else
                products(std::integral_constant<int, 2>{});
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

        const size_t blk = (size_t)hv * tp.ws.nchunk + g;
        if constexpr (SLIM) {
            // ---- T' = T diag(beta) as the second pass's A operand (the layout of P below)
            const int idx = tid, l = idx & 63, m4 = (idx >> 6) & 1, rb = idx >> 7;
            v4f tv;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int ss = 16 * m4 + 4 * (l >> 4) + e4;
                tv[e4] = Tm[(rb * 16 + (l & 15)) * AP + ss] * bet[ss];
            }
            // block 1 (row block 0, tokens 16 ..: wave 1's) lies above the diagonal,
            // zero in T' and in P, and the second pass reads neither: not stored
            if (wv != 1)
                *reinterpret_cast<v4f *>(tp.ws.ta + blk * (BT * BT) + (size_t)idx * 4) = tv;
        } else {
        // ---- W = T diag(beta e^gamma) K and U~ = T diag(beta) V on the matrix
        // cores: this wave's column blocks of each, both row blocks.  Rows of
        // padding tokens come out zero (their rows of A, and beta, are zero).
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
                // T is lower triangular: row block 0 has no terms past k = 15 (zero
                // products, which would leave its sums as they are)
#pragma unroll
                for (int q = 0; q < WCB; ++q) {
                    const float bk = bse * Ks[(k0 + lk) * KP + (wv * WCB + q) * 16 + li];
                    if (k0 < 16)
                        wacc[0][q] = mma16(at0, bk, wacc[0][q]);
                    wacc[1][q] = mma16(at1, bk, wacc[1][q]);
                }
#pragma unroll
                for (int q = 0; q < UCB; ++q) {
                    const float bv = bs * Vs[(k0 + lk) * VP + (wv * UCB + q) * 16 + li];
                    if (k0 < 16)
                        uacc[0][q] = mma16(at0, bv, uacc[0][q]);
                    uacc[1][q] = mma16(at1, bv, uacc[1][q]);
                }
            }
            // U~ leaves in the accumulator layout it was computed in
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int q = 0; q < UCB; ++q)
                    *reinterpret_cast<v4f *>(tp.ws.ud + ((blk * 2 + rb) * (DV / 16) + wv * UCB + q) * 256 + lane * 4) =
                        uacc[rb][q];
            __syncthreads(); // every read of V is done: W goes over it
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int q = 0; q < WCB; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Vs[(rb * 16 + 4 * lk + r) * KP + (wv * WCB + q) * 16 + li] = wacc[rb][q][r];
        }
        __syncthreads();

        // ---- Q~, W, K~ and P in the order the second pass feeds them to the
        // matrix cores: 1 KiB blocks of one float4 a lane, lane j + 16 g of
        // block (row block rb, k block m4) holding X[16 rb + j][16 m4 + 4 g + r]
        // for r = 0..3 -- the k-steps of a 16-wide k block taken in the order
        // the accumulator layout holds rows (4 g + r), so that a state slice
        // kept in that layout is a B operand as it stands
        const float *Ws = Vs;
#pragma unroll
        for (int it = 0; it < 2 * (DK / 16) * 64 / NT; ++it) {
            const int idx = tid + it * NT;
            const int l = idx & 63, m4 = (idx >> 6) % (DK / 16), rb = idx / (64 * (DK / 16));
            const int row = rb * 16 + (l & 15);
            const int col = 16 * m4 + 4 * (l >> 4);
            const float er = eg[row];
            const v4f q4 = *reinterpret_cast<const v4f *>(&Qs[row * KP + col]);
            const v4f qv = {q4[0] * er, q4[1] * er, q4[2] * er, q4[3] * er};
            const v4f wv4 = *reinterpret_cast<const v4f *>(&Ws[row * KP + col]);
            *reinterpret_cast<v4f *>(tp.ws.qa + blk * (BT * DK) + (size_t)idx * 4) = qv;
            *reinterpret_cast<v4f *>(tp.ws.wa + blk * (BT * DK) + (size_t)idx * 4) = wv4;
        }
#pragma unroll
        for (int it = 0; it < (DK / 16) * 2 * 64 / NT; ++it) {
            const int idx = tid + it * NT;
            const int l = idx & 63, m4 = (idx >> 6) & 1, ib = idx >> 7;
            v4f kv;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int tt = 16 * m4 + 4 * (l >> 4) + e4;
                kv[e4] = Ks[tt * KP + ib * 16 + (l & 15)] * egl[tt];
            }
            *reinterpret_cast<v4f *>(tp.ws.ka + blk * (BT * DK) + (size_t)idx * 4) = kv;
        }
        } // full layout
        {
            const int idx = tid, l = idx & 63, m4 = (idx >> 6) & 1, rb = idx >> 7; // 256 float4: one a thread
            v4f pv;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                pv[e4] = Pm[(rb * 16 + (l & 15)) * AP + 16 * m4 + 4 * (l >> 4) + e4];
            if (!SLIM || wv != 1)
                *reinterpret_cast<v4f *>(tp.ws.pa + blk * (BT * BT) + (size_t)idx * 4) = pv;
        }
        // e^gamma_last (padding tokens carry g = 0): every lane stores the same
        // value to the same place, which needs no branch
        if constexpr (SLIM)
            tp.ws.fac[blk * 128 + 96] = eg[BT - 1];
        else
            tp.ws.el[blk] = eg[BT - 1];

        cur = nxt;
        __syncthreads(); // LDS is read to the end of the chunk; the next one rewrites it
    }
}

// pass 1 over the call's chunks lo .. hi - 1
template <int DK, int DV, bool SLIM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(SLIM ? 3 : 2, SLIM ? 3 : 2))) void tp_intra_kernel(TwoPassParams tp, int lo, int hi)
{
    intra_body<DK, DV, SLIM>(tp, blockIdx.x, gridDim.x, blockIdx.y, lo, hi, blockIdx.x == 0 && blockIdx.y == 0);
}

// ---------------------------------------------------------------- pass 2

// The advanced conv windows of a prompt: the last three inputs of [window,
// prompt] for the slice's v channels, and for the key head's q and k channels
// from its first value head's first slice.  Nothing else reads or writes these
// channels of this slot now: pass 1 is over.
template <int DK, int DV, int DVS, int NTH = NT>
__device__ __forceinline__ void advance_windows(const PrefillParams &p, int hv, int sl, int t_begin, int t_end, int s)
{
    const int tid = threadIdx.x;
    const int L = t_end - t_begin;
    const int C = p.C;
    const int hk = hv / p.G;
    const int col0 = sl * DVS;
    const bool qk_owner = (hv % p.G == 0) && sl == 0;
    const int npair = DVS / 2 + (qk_owner ? DK : 0);
    uint16_t *win = p.conv_state + (size_t)s * 3 * C;
    for (int e = tid; e < npair; e += NTH) {
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

// The (prompt, value head) pair and the column slice of pass-2 workgroup j, of
// nsl slices a head.  Workgroups go to the eight XCDs in turn, so the slices
// of a head are placed eight workgroups apart: they share one XCD, whose L2
// then fetches the head's operands once for all of them.  Pairs past the last
// whole group of eight are placed in order.
__device__ __forceinline__ void walk_place(int j, int heads, int nsl, int &bh, int &sl)
{
    const int h8 = heads & ~7;
    if (j < h8 * nsl) {
        const int k = j >> 3;
        bh = (k / nsl) * 8 + (j & 7);
        sl = k % nsl;
    } else {
        const int r = j - h8 * nsl;
        bh = h8 + r / nsl;
        sl = r % nsl;
    }
}

// Where a pass-2 workgroup's prompt stands: false when it has nothing to do
// (an unusable range or slot touches nothing; a padding prompt on the null
// slot gets its read-out of +0.0 here; an empty prompt does nothing).
template <int DV, int DVS, int NTH = NT>
__device__ __forceinline__ bool walk_setup(const TwoPassParams &tp, int b, int hv, int col0, int &t_begin, int &t_end,
                                           int &s, int &nchunks, size_t &blk0)
{
    const PrefillParams &p = tp.p;
    if (!sequence_usable(p, b, t_begin, t_end, s))
        return false;
    // one value for the whole workgroup: the buffer resources built from these
    // must sit in scalar registers
    t_begin = __builtin_amdgcn_readfirstlane(t_begin);
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    s = __builtin_amdgcn_readfirstlane(s);
    if (s == 0) {
        for (int e = threadIdx.x; e < (t_end - t_begin) * DVS; e += NTH)
            p.out[((size_t)(t_begin + e / DVS) * p.H_v + hv) * DV + col0 + e % DVS] = 0;
        return false;
    }
    if (t_end == t_begin)
        return false;
    nchunks = (t_end - t_begin + BT - 1) / BT;
    const int cs_b = __builtin_amdgcn_readfirstlane(tp.ws.chunk_start[b]);
    if (cs_b < 0 || (long long)cs_b + nchunks > tp.ws.nchunk)
        return false; // only with overlapping ranges (excluded by the contract): touch nothing
    blk0 = (size_t)hv * tp.ws.nchunk + (size_t)cs_b;
    return true;
}

// Slices of 32 or 64 columns: the slice of the state and U in LDS.  Wave w
// takes row block w & 1 of W S0, Q~ S0 and O and half the slice's column
// blocks, and row blocks w * DK / 64 .. of the state update.  The k-steps of
// every product run in pass 1's operand order (k = 16 m4 + 4 g + e4 at lane
// group g), and LDS holds S and U transposed (column-major), so a lane's four
// k-steps of a k block are four consecutive words: one 16-byte read, and the
// accumulator layout's four rows one 16-byte write.
// at most 256 registers a lane: two workgroups a CU (LDS allows two at 64 columns)
template <int DK, int DV, int DVS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void tp_inter_kernel(TwoPassParams tp)
{
    const PrefillParams &p = tp.p;
    constexpr int NSL = DV / DVS;
    // St[col][k] and Ut[col][token]: pitches of 4 mod 32 words put the 16
    // columns a lane group reads 4 banks apart (16-byte accesses, conflict-free)
    constexpr int SPT = DK + 4, UPT = BT + 4;
    constexpr int CBS = DVS / 16; // column blocks of the slice
    static_assert(CBS == 2 || CBS == 4, "16-column slices take tp_inter16_kernel");
    constexpr int CBW = CBS / 2;  // column blocks of W S0, Q~ S0 and O a wave takes
    constexpr int NA4 = DK / 16;  // float4 a lane holds of one A-operand tile over k = d_k
    constexpr int RBW = DK / 64;  // row blocks of S a wave updates
    constexpr int CHUNK_QK = BT * DK, CHUNK_P = BT * BT, CHUNK_U = BT * DV;

    __shared__ __align__(16) float St[DVS * SPT];
    __shared__ __align__(16) float Ut[DVS * UPT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lk = lane >> 4;
    int bh, sl;
    walk_place(blockIdx.x, p.B * p.H_v, NSL, bh, sl);
    const int hv = bh % p.H_v;
    const int b = bh / p.H_v;
    const int col0 = sl * DVS;
    int t_begin, t_end, s, nchunks;
    size_t blk0;
    if (!walk_setup<DV, DVS>(tp, b, hv, col0, t_begin, t_end, s, nchunks, blk0))
        return;
    float *tile = p.state + ((size_t)s * p.H_v + hv) * (size_t)(DK * DV);

    const int rb = wv & 1;
    const int cb0 = (wv >> 1) * CBW;

    // ---- the state's column slice -> LDS, transposed: a lane takes four rows
    // of one column (streaming loads, consecutive lanes on consecutive columns,
    // so each wave load covers whole rows) and writes them as one 16-byte run
    for (int e = tid; e < DK * DVS / 4; e += NT) {
        const int j = e % DVS, i4 = e / DVS;
        v4f v;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = __builtin_nontemporal_load(tile + (size_t)(4 * i4 + r) * DV + col0 + j);
        *reinterpret_cast<v4f *>(&St[j * SPT + 4 * i4]) = v;
    }

    // ---- this wave's operands of a chunk, loaded one chunk ahead straight
    // into registers.  Buffer loads over resources zero-sized past the last
    // chunk, so the walk has no branch around a memory access.  Every load,
    // even an empty one, takes the compute unit's address path (about 16
    // cycles for a 1 KiB wave load, shared by the four waves), so they are
    // interleaved with the matrix-core products below.
    constexpr int NLOAD = 2 * NA4 + 2 * RBW + 2 + CBW; // loads a wave issues a chunk
    v4f xw[NA4], xq[NA4], xk[RBW][2], xp[2], xu[CBW];
    float xel = 0.f;
    auto prefetch = [&](int c) {
        const bool real = c < nchunks;
        const size_t blk = blk0 + (size_t)(real ? c : 0);
        const __amdgpu_buffer_rsrc_t rK = buf_rsrc(tp.ws.ka + blk * CHUNK_QK + wv * RBW * 512, real ? RBW * 2048u : 0u);
        const __amdgpu_buffer_rsrc_t rW = buf_rsrc(tp.ws.wa + blk * CHUNK_QK + rb * NA4 * 256, real ? NA4 * 1024u : 0u);
        const __amdgpu_buffer_rsrc_t rQ = buf_rsrc(tp.ws.qa + blk * CHUNK_QK + rb * NA4 * 256, real ? NA4 * 1024u : 0u);
        const __amdgpu_buffer_rsrc_t rP = buf_rsrc(tp.ws.pa + blk * CHUNK_P + rb * 512, real ? 2048u : 0u);
        const __amdgpu_buffer_rsrc_t rU =
            buf_rsrc(tp.ws.ud + blk * CHUNK_U + (rb * (DV / 16) + col0 / 16 + cb0) * 256, real ? CBW * 1024u : 0u);
#pragma unroll
        for (int m4 = 0; m4 < NA4; ++m4) {
            xw[m4] = buf_load4(rW, (uint32_t)(m4 * 64 + lane) * 16u);
            xq[m4] = buf_load4(rQ, (uint32_t)(m4 * 64 + lane) * 16u);
        }
#pragma unroll
        for (int m4 = 0; m4 < 2; ++m4)
            xp[m4] = buf_load4(rP, (uint32_t)(m4 * 64 + lane) * 16u);
#pragma unroll
        for (int q = 0; q < CBW; ++q)
            xu[q] = buf_load4(rU, (uint32_t)(q * 64 + lane) * 16u);
#pragma unroll
        for (int q = 0; q < RBW; ++q)
#pragma unroll
            for (int m4 = 0; m4 < 2; ++m4)
                xk[q][m4] = buf_load4(rK, (uint32_t)((q * 2 + m4) * 64 + lane) * 16u);
        xel = tp.ws.el[blk];
    };
    prefetch(0);
    __syncthreads(); // the state is in LDS

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = t_begin + c * BT;
        const int n = t_end - t0 < BT ? t_end - t0 : BT;
        v4f aw_op[NA4], aq_op[NA4], ak_op[RBW][2], ap_op[2], au[CBW];
#pragma unroll
        for (int m4 = 0; m4 < NA4; ++m4) {
            aw_op[m4] = xw[m4];
            aq_op[m4] = xq[m4];
        }
#pragma unroll
        for (int q = 0; q < RBW; ++q) {
            ak_op[q][0] = xk[q][0];
            ak_op[q][1] = xk[q][1];
        }
        ap_op[0] = xp[0];
        ap_op[1] = xp[1];
#pragma unroll
        for (int q = 0; q < CBW; ++q)
            au[q] = xu[q];
        const float el = xel;
        prefetch(c + 1);
        // the read-out rows of the chunk's real tokens; later rows fall outside
        const int t0u = __builtin_amdgcn_readfirstlane(t0), nu = __builtin_amdgcn_readfirstlane(n);
        const __amdgpu_buffer_rsrc_t rO = buf_rsrc(p.out + ((size_t)t0u * p.H_v + hv) * DV + col0,
                                                   (uint32_t)(((nu - 1) * p.H_v * DV + DVS) * 2));

        // ---- W S0 and Q~ S0 on this wave's tiles (row block rb)
        v4f aw[CBW], aq[CBW];
#pragma unroll
        for (int q = 0; q < CBW; ++q)
            aw[q] = aq[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m4 = 0; m4 < NA4; ++m4) {
            v4f bs[CBW];
#pragma unroll
            for (int q = 0; q < CBW; ++q)
                bs[q] = *reinterpret_cast<const v4f *>(&St[((cb0 + q) * 16 + li) * SPT + 16 * m4 + 4 * lk]);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                for (int q = 0; q < CBW; ++q) {
                    aw[q] = mma16(aw_op[m4][e4], bs[q][e4], aw[q]);
                    aq[q] = mma16(aq_op[m4][e4], bs[q][e4], aq[q]);
                }
        }
        // interleave the next chunk's loads with these products, so their
        // address processing runs under the matrix cores instead of in front:
        // one load every four products (measured on MI355X against one every
        // two: 16 x 512 250 -> 245 us, 8 x 1024 259 -> 249)
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // one vector-memory read
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0); // four MFMA
        }
        // U = U~ - W S0 on the same tiles -> LDS
#pragma unroll
        for (int q = 0; q < CBW; ++q)
            *reinterpret_cast<v4f *>(&Ut[((cb0 + q) * 16 + li) * UPT + rb * 16 + 4 * lk]) =
                v4f{au[q][0] - aw[q][0], au[q][1] - aw[q][1], au[q][2] - aw[q][2], au[q][3] - aw[q][3]};
        __syncthreads(); // U complete; every read of S0 for this chunk is done

        // ---- O = Q~ S0 + P U -> out
#pragma unroll
        for (int m4 = 0; m4 < 2; ++m4) {
            v4f ub[CBW];
#pragma unroll
            for (int q = 0; q < CBW; ++q)
                ub[q] = *reinterpret_cast<const v4f *>(&Ut[((cb0 + q) * 16 + li) * UPT + 16 * m4 + 4 * lk]);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                for (int q = 0; q < CBW; ++q)
                    aq[q] = mma16(ap_op[m4][e4], ub[q][e4], aq[q]);
        }
#pragma unroll
        for (int q = 0; q < CBW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_buffer_store_b16(
                    f32_to_bf16_rne(aq[q][r]), rO,
                    (uint32_t)((rb * 16 + 4 * lk + r) * p.H_v * DV + (cb0 + q) * 16 + li) * 2u, 0, 0);

        // ---- S1 = e^gamma_last S0 + K~^T U: this wave's row blocks, the slice's column blocks
        {
            v4f sacc[RBW][CBS];
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBS; ++jb) {
                    const v4f s4 = *reinterpret_cast<const v4f *>(&St[(jb * 16 + li) * SPT + (wv * RBW + q) * 16 + 4 * lk]);
                    sacc[q][jb] = v4f{el * s4[0], el * s4[1], el * s4[2], el * s4[3]};
                }
#pragma unroll
            for (int m4 = 0; m4 < 2; ++m4)
#pragma unroll
                for (int jb = 0; jb < CBS; ++jb) {
                    const v4f ub = *reinterpret_cast<const v4f *>(&Ut[(jb * 16 + li) * UPT + 16 * m4 + 4 * lk]);
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                        for (int q = 0; q < RBW; ++q)
                            sacc[q][jb] = mma16(ak_op[q][m4][e4], ub[e4], sacc[q][jb]);
                }
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBS; ++jb)
                    *reinterpret_cast<v4f *>(&St[(jb * 16 + li) * SPT + (wv * RBW + q) * 16 + 4 * lk]) = sacc[q][jb];
        }
        __syncthreads(); // S and U are free for the next chunk
    }

    // ---- the state's slice back to the slot (the same mapping)
    for (int e = tid; e < DK * DVS / 4; e += NT) {
        const int j = e % DVS, i4 = e / DVS;
        const v4f v = *reinterpret_cast<const v4f *>(&St[j * SPT + 4 * i4]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_nontemporal_store(v[r], tile + (size_t)(4 * i4 + r) * DV + col0 + j);
    }
    advance_windows<DK, DV, DVS>(p, hv, sl, t_begin, t_end, s);
}

// 16-column slices: the slice of the state stays in registers.  Wave w holds
// row blocks w * RBW .. of the slice in the accumulator layout (lane j + 16 g,
// element r: row 4 g + r of the block, column j), which with pass 1's operand
// order is the B operand of a product over the state's rows as it stands:
// step (row block R, r) takes row 16 R + 4 g + r at lane group g.  Each wave
// forms W S0 and Q~ S0 over its own rows; one barrier a chunk sums the four
// partial products (in LDS, double-buffered by chunk parity, so the next
// chunk's writes cannot meet this chunk's reads) in a fixed order into
// U = U~ - W S0, which every wave then holds in the accumulator layout: the B
// operand, again as it stands, of its own rows' K~^T U and of a quarter of
// P U.  The read-out is spread over the four waves a chunk late: wave w takes
// P U for read-out row block w & 1 over tokens 16 (w >> 1) ..; waves 2-3 add
// the summed Q~ S0 partials and leave that in LDS, and waves 0-1 add it to
// theirs after the next chunk's barrier (one more barrier after the last
// chunk) and store the rows.
//
// The body of walk workgroup j over the call's chunks lo .. hi - 1 (global
// chunk indices): a prompt's chunks outside the range are left alone, and the
// state slice goes from the slot to registers and back around the range, so a
// prompt can be walked in consecutive ranges by consecutive launches.
template <int DK, int DV>
__device__ __forceinline__ void inter16_body(const TwoPassParams &tp, int j, int lo, int hi)
{
    const PrefillParams &p = tp.p;
    constexpr int NSL = DV / 16;
    constexpr int NRB = DK / 16; // row blocks of the state
    constexpr int RBW = NRB / 4; // row blocks a wave holds
    static_assert(NRB % 4 == 0, "whole row blocks a wave");
    constexpr int CHUNK_QK = BT * DK, CHUNK_P = BT * BT, CHUNK_U = BT * DV;

    // partial products: [chunk parity][wave][W S0, Q~ S0][row block][lane]
    __shared__ v4f part[2][4][2][2][64];
    // Q~ S0 + P U over tokens 16 .. 31 from waves 2-3: [chunk parity][row block][lane]
    __shared__ v4f osum[2][2][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, li = lane & 15, lk = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bh, sl;
    walk_place(j, p.B * p.H_v, NSL, bh, sl);
    const int hv = bh % p.H_v;
    const int b = bh / p.H_v;
    const int col0 = sl * 16;
    int t_begin, t_end, s, nchunks;
    size_t blk0;
    if (!walk_setup<DV, 16>(tp, b, hv, col0, t_begin, t_end, s, nchunks, blk0))
        return;
    // this prompt's chunks in the range
    const int cs_b = (int)(blk0 - (size_t)hv * tp.ws.nchunk);
    const int c_lo = lo > cs_b ? lo - cs_b : 0;
    const int c_hi = hi - cs_b < nchunks ? hi - cs_b : nchunks;
    if (c_lo >= c_hi)
        return;
    float *tile = p.state + ((size_t)s * p.H_v + hv) * (size_t)(DK * DV) + col0 + li;

    // ---- this wave's rows of the slice -> registers (a lane group's 16 lanes
    // read 64 contiguous bytes of a row)
    v4f st[RBW];
#pragma unroll
    for (int q = 0; q < RBW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            st[q][r] = __builtin_nontemporal_load(tile + (size_t)((wv * RBW + q) * 16 + 4 * lk + r) * DV);

    // ---- this wave's operands of a chunk: W and Q~ over its own rows (k
    // blocks wv * RBW ..), K~^T for its own rows, U~ of the slice, and its
    // quarter of P (row block wv & 1, k block wv >> 1), loaded one chunk ahead
    // (two chunks ahead, in two sets, measured no faster).
    constexpr int NLOAD = 6 * RBW + 3; // loads a wave issues a chunk
    struct Ops {
        v4f w[2][RBW], q[2][RBW], k[RBW][2], p, u[2];
        float el;
    };
    auto prefetch = [&](int c, Ops &x) {
        const bool real = c < c_hi;
        const size_t blk = blk0 + (size_t)(real ? c : 0);
        const __amdgpu_buffer_rsrc_t rW = buf_rsrc(tp.ws.wa + blk * CHUNK_QK, real ? CHUNK_QK * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rQ = buf_rsrc(tp.ws.qa + blk * CHUNK_QK, real ? CHUNK_QK * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rK = buf_rsrc(tp.ws.ka + blk * CHUNK_QK + wv * RBW * 512, real ? RBW * 2048u : 0u);
        const __amdgpu_buffer_rsrc_t rP = buf_rsrc(tp.ws.pa + blk * CHUNK_P, real ? CHUNK_P * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rU = buf_rsrc(tp.ws.ud + blk * CHUNK_U, real ? CHUNK_U * 4u : 0u);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int q = 0; q < RBW; ++q) {
                const uint32_t o = (uint32_t)((mb * NRB + wv * RBW + q) * 64 + lane) * 16u;
                x.w[mb][q] = buf_load4(rW, o);
                x.q[mb][q] = buf_load4(rQ, o);
            }
#pragma unroll
        for (int q = 0; q < RBW; ++q)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                x.k[q][tb] = buf_load4(rK, (uint32_t)((q * 2 + tb) * 64 + lane) * 16u);
        x.p = buf_load4(rP, (uint32_t)((((wv & 1) * 2 + (wv >> 1)) * 64 + lane) * 16u));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            x.u[tb] = buf_load4(rU, (uint32_t)((tb * NSL + sl) * 64 + lane) * 16u);
        x.el = tp.ws.el[blk];
    };
    // read-out row block wv (waves 0-1) of the chunk starting at token t0s,
    // ns real tokens; later rows fall outside the resource.  (Only waves 0-1
    // issue these: dropped stores on waves 2-3, which would make every
    // wave's count of memory operations the same, measured slower.)
    auto store_o = [&](const v4f o, int t0s, int ns) {
        const int t0u = __builtin_amdgcn_readfirstlane(t0s), nu = __builtin_amdgcn_readfirstlane(ns);
        const __amdgpu_buffer_rsrc_t rO =
            buf_rsrc(p.out + ((size_t)t0u * p.H_v + hv) * DV + col0, (uint32_t)(((nu - 1) * p.H_v * DV + 16) * 2));
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(o[r]), rO,
                                                  (uint32_t)((wv * 16 + 4 * lk + r) * p.H_v * DV + li) * 2u, 0, 0);
    };

    v4f o_lo = {0.f, 0.f, 0.f, 0.f}; // waves 0-1: the last chunk's P U over tokens 0 .. 15
    // chunk c's first products, from its operands in cur and the state entering
    // it, into LDS; chunk c + 1's loads go to nx, issued among the products
    auto first_products = [&](int c, const Ops &cur, Ops &nx) {
        prefetch(c + 1, nx);

        // ---- partial W S0 and Q~ S0 over this wave's rows
        v4f pw[2], pq[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            pw[mb] = pq[mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RBW; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    pw[mb] = mma16(cur.w[mb][q][r], st[q][r], pw[mb]);
                    pq[mb] = mma16(cur.q[mb][q][r], st[q][r], pq[mb]);
                }
        // the loads interleaved with these products, so their address
        // processing runs under the matrix cores
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // one vector-memory read
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // two MFMA
        }
        v4f(*pc)[2][2][64] = part[c & 1];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            pc[wv][0][mb][lane] = pw[mb];
            pc[wv][1][mb][lane] = pq[mb];
        }
    };
    // the rest of chunk c, after the barrier that follows its first products
    auto after_barrier = [&](int c, const Ops &cur) {
        const int t0 = t_begin + c * BT;
        v4f(*pc)[2][2][64] = part[c & 1];

        // ---- U = U~ - (W S0), the partials summed in wave order (the same
        // operands in the same order on every wave, so all four hold the same U)
        v4f u[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            v4f ws = pc[0][0][tb][lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const v4f x = pc[w][0][tb][lane];
                ws = v4f{ws[0] + x[0], ws[1] + x[1], ws[2] + x[2], ws[3] + x[3]};
            }
            u[tb] = v4f{cur.u[tb][0] - ws[0], cur.u[tb][1] - ws[1], cur.u[tb][2] - ws[2], cur.u[tb][3] - ws[3]};
        }

        // ---- the previous chunk's read-out rows (a whole chunk: only the last
        // can be partial), ahead of the state update, which then covers the
        // stores' latency
        if (wv < 2 && c > c_lo) {
            const v4f x = osum[(c - 1) & 1][wv][lane];
            store_o(v4f{x[0] + o_lo[0], x[1] + o_lo[1], x[2] + o_lo[2], x[3] + o_lo[3]}, t0 - BT, BT);
        }
        // ---- this wave's quarter of P U: read-out row block wv & 1, tokens 16 (wv >> 1) ..
        {
            const v4f ut = wv >= 2 ? u[1] : u[0];
            v4f op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                op = mma16(cur.p[r], ut[r], op);
            if (wv >= 2) {
                // + Q~ S0, its partials summed in wave order
                v4f o = pc[0][1][wv & 1][lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    const v4f x = pc[w][1][wv & 1][lane];
                    o = v4f{o[0] + x[0], o[1] + x[1], o[2] + x[2], o[3] + x[3]};
                }
                osum[c & 1][wv & 1][lane] = v4f{o[0] + op[0], o[1] + op[1], o[2] + op[2], o[3] + op[3]};
            } else {
                o_lo = op;
            }
        }

        // ---- S1 = e^gamma_last S0 + K~^T U on this wave's rows: each row
        // block's product over the two token blocks in separate accumulators,
        // interleaved, so no product waits on the one before it
        {
            v4f a0[RBW], a1[RBW];
#pragma unroll
            for (int q = 0; q < RBW; ++q) {
                a0[q] = v4f{cur.el * st[q][0], cur.el * st[q][1], cur.el * st[q][2], cur.el * st[q][3]};
                a1[q] = v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < RBW; ++q) {
                    a0[q] = mma16(cur.k[q][0][r], u[0][r], a0[q]);
                    a1[q] = mma16(cur.k[q][1][r], u[1][r], a1[q]);
                }
#pragma unroll
            for (int q = 0; q < RBW; ++q)
                st[q] = v4f{a0[q][0] + a1[q][0], a0[q][1] + a1[q][1], a0[q][2] + a1[q][2], a0[q][3] + a1[q][3]};
        }
    };

    // The walk turned so that one pass of the loop holds chunk c's state update
    // and chunk c + 1's first products: the products that need the new state
    // then follow its computation with no loop edge between (after the last
    // chunk they run on zero operands and their results are not read).
    // Two operand sets used in turn (chunk c in one, c + 1 in the other), so
    // no set is copied: a copy would wait for loads just issued.
    // The loop takes whole pairs and an odd last chunk follows it, so the loop
    // body has no branch: a path that skipped its second half would make every
    // wait at the top of the loop take all memory operations in flight.
    Ops opa, opb;
    prefetch(c_lo, opa);
    first_products(c_lo, opa, opb);
    int c = c_lo;
    for (; c + 1 < c_hi; c += 2) {
        __syncthreads();
        after_barrier(c, opa);
        first_products(c + 1, opb, opa);
        __syncthreads();
        after_barrier(c + 1, opb);
        first_products(c + 2, opa, opb);
    }
    if (c < c_hi) {
        __syncthreads();
        after_barrier(c, opa);
        first_products(c + 1, opb, opa);
    }
    // ---- the range's last chunk's read-out rows
    __syncthreads();
    if (wv < 2) {
        const int c = c_hi - 1, t0 = t_begin + c * BT;
        const v4f x = osum[c & 1][wv][lane];
        store_o(v4f{x[0] + o_lo[0], x[1] + o_lo[1], x[2] + o_lo[2], x[3] + o_lo[3]}, t0,
                t_end - t0 < BT ? t_end - t0 : BT);
    }

    // ---- the slice back to the slot
#pragma unroll
    for (int q = 0; q < RBW; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_nontemporal_store(st[q][r], tile + (size_t)((wv * RBW + q) * 16 + 4 * lk + r) * DV);
    if (c_hi == nchunks)
        advance_windows<DK, DV, 16>(p, hv, sl, t_begin, t_end, s);
}

// the 16-column walk over the call's chunks lo .. hi - 1
template <int DK, int DV>
__global__ __launch_bounds__(NT) void tp_inter16_kernel(TwoPassParams tp, int lo, int hi)
{
    inter16_body<DK, DV>(tp, blockIdx.x, lo, hi);
}

// One launch of the pipelined schedule (the full layout, when the 16-column
// walk leaves compute units idle): workgroups 0 .. n_walk - 1 walk chunks
// wlo .. whi - 1 while the rest run pass 1 over chunks plo .. phi - 1 (gx
// workgroups a value head) on the compute units the walk leaves free.  The
// two bodies' LDS together allow one workgroup a CU, so neither role shares a
// compute unit with the other; the kernel boundary orders a range's pass 1
// before its walk, and one range's walk before the next.
template <int DK, int DV>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void tp_pipe_kernel(TwoPassParams tp,
                                                                                                 int n_walk, int wlo,
                                                                                                 int whi, int gx,
                                                                                                 int plo, int phi)
{
    const int j = blockIdx.x;
    if (j < n_walk) {
        inter16_body<DK, DV>(tp, j, wlo, whi);
        return;
    }
    const int v = j - n_walk;
    intra_body<DK, DV, false>(tp, v % gx, gx, v / gx, plo, phi, false);
}

// The slim walk: one workgroup a (prompt, value head) over the slim layout,
// with the chunk's conv run here from x (once for the head), and a wave per
// 16-column block of the state.  Every wave meets the same barriers, so the
// head's waves move together (two workgroups sharing a compute unit had run
// apart: the older one takes the issue slots, the younger finishes alone).
// With K and Q the chunk's conv + SiLU outputs before normalisation (in LDS)
// and the state in LDS transposed, per chunk:
//   Y = K S0 and Z = Q S0, both row blocks of the wave's column block;
//   R = V - f_a Y, V the lane's own conv outputs at its accumulator-layout
//   places, f_a = k-norm e^gamma per row;  U = T' R, with R the B operand as
//   it stands;
//   O = f_b Z + P U -> out, f_b = q-norm q_scale e^gamma;
//   U'' = f_c U -> LDS, f_c = k-norm e^(gamma_last - gamma);
// and after the chunk's second barrier each wave updates its share of the
// state's 16 x 16 tiles (whole row blocks), S1 = e^gamma_last S0 + K^T U''.  U = T diag(beta) (V - e^gamma K^ S0) is the
// full layout's U~ - W S0, and K^T U'' its K~^T U.
// Two barriers a chunk: after the conv (K, Q and the previous update are in
// LDS) and after U'' (every read of the state, K and Q for the chunk is done,
// so the update and the next chunk's conv may write them).
// at most 256 registers a lane: two waves a SIMD (at d_v = 128 one
// workgroup of eight waves a CU, which its 120 KB of LDS allow)
template <int DK, int DV>
__global__ __launch_bounds__(DV * 4) __attribute__((amdgpu_waves_per_eu(2, 2))) void tp_slim_kernel(TwoPassParams tp)
{
    const PrefillParams &p = tp.p;
    constexpr int DVS = DV;
    constexpr int NW = DV / 16, NTS = 64 * NW;           // a wave per column block
    constexpr int KP = DK + 4, SPT = DK + 4, UPT = BT + 4; // 4 mod 32 words: 16-byte reads conflict-free
    constexpr int NA4 = DK / 16, NRB = DK / 16, NCB = DV / 16;
    // the state update's tiles: RBW row blocks x CBU column blocks a wave
    constexpr int RBW = NW <= NRB ? NRB / NW : 1;
    constexpr int CBU = NW <= NRB ? NCB : NCB / (NW / NRB);
    constexpr int NPQK = DK;                              // q | k channel pairs
    constexpr int NSPLIT = NTS / NPQK, TPT = BT / NSPLIT; // runs of tokens of the q | k conv
    static_assert(NTS % NPQK == 0 && BT % NSPLIT == 0 && TPT >= 1, "whole runs of tokens");
    static_assert(NRB % RBW == 0 && RBW * CBU * NW == NRB * NCB, "the state's tiles split evenly over the waves");
    constexpr int CHUNK_P = BT * BT;

    __shared__ __align__(16) float St[DVS * SPT];
    __shared__ __align__(16) float Ut[DVS * UPT];
    __shared__ __align__(16) float Qs[BT * KP];
    __shared__ __align__(16) float Ks[BT * KP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, li = lane & 15, lk = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hv = blockIdx.x % p.H_v;
    const int b = blockIdx.x / p.H_v;
    const int col0 = 0;
    // this wave's tiles of the state update: row blocks rb0 .., column blocks cbu0 ..
    const int rb0 = (wv % (NRB / RBW)) * RBW, cbu0 = (wv / (NRB / RBW)) * CBU;
    int t_begin, t_end, s, nchunks;
    size_t blk0;
    if (!walk_setup<DV, DVS, NTS>(tp, b, hv, col0, t_begin, t_end, s, nchunks, blk0))
        return;
    float *tile = p.state + ((size_t)s * p.H_v + hv) * (size_t)(DK * DV);
    const int C = p.C;
    const int hk = hv / p.G;

    // ---- conv roles.  q | k: thread tid takes channel pair pp over tokens
    // sp TPT ..; v: lane (li, lk) of wave w takes column 16 w + li of the
    // slice at tokens 16 rb + 4 lk + r, its places in the accumulator layout
    const int pp = tid % NPQK, sp = tid / NPQK; // sp is the same across a wave
    const int e = 2 * pp;
    const bool isq = e < DK;
    const int chqk = isq ? hk * DK + e : p.H_k * DK + hk * DK + (e - DK);
    float *ydst = isq ? &Qs[e] : &Ks[e - DK];
    const int chv = 2 * p.H_k * DK + hv * DV + col0 + 16 * wv + li;
    const bool has_bias = p.conv_b != nullptr;
    float wq[4][2], bq[2], wvc[4], bvc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wq[k][h] = bf16_to_f32(p.conv_w[(size_t)(chqk + h) * 4 + k]);
        bq[h] = has_bias ? bf16_to_f32(p.conv_b[chqk + h]) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        wvc[k] = bf16_to_f32(p.conv_w[(size_t)chv * 4 + k]);
    bvc = has_bias ? bf16_to_f32(p.conv_b[chv]) : 0.f;

    // ---- a chunk's x inputs, loaded one chunk ahead: the q | k pairs of the
    // thread's run with the three inputs before it, and the lane's v inputs
    // (tokens 16 rb + 4 lk - 3 ..).  Inputs before a prompt's first token come
    // from the window copy in hw (a separate register: an OR here would wait
    // for the loads).  Buffer resources over the chunk's rows, zero-sized past
    // the last chunk, so nothing branches around a load.
    struct XIn {
        uint32_t qk[TPT + 3], qkh[3]; // bf16 pairs
        uint32_t v[2][7], vh[3];      // bf16 in the low half
    };
    auto load_x = [&](int c, XIn &in) {
        const bool real = c < nchunks;
        const int cc = real ? c : 0;
        const int t0 = t_begin + cc * BT;
        const int n = t_end - t0 < BT ? t_end - t0 : BT;
        const int sh = cc == 0 ? 0 : 3; // rows of x before the chunk in the resource
        // (sizes times 0 or 1, not a choice: a choice here becomes a branch,
        // which would keep these loads out of the products they are issued among)
        const __amdgpu_buffer_rsrc_t rx =
            buf_rsrc(p.x + (size_t)(t0 - sh) * p.x_row_stride,
                     (uint32_t)(((size_t)(n - 1 + sh) * p.x_row_stride + C) * 2) * (uint32_t)real);
        const __amdgpu_buffer_rsrc_t rh =
            buf_rsrc(tp.ws.hw + (size_t)b * 3 * C, (uint32_t)(3 * C * 2) * (uint32_t)(real && cc == 0));
#pragma unroll
        for (int i = 0; i < TPT + 3; ++i) {
            const int t = sp * TPT - 3 + i;
            in.qk[i] = __builtin_amdgcn_raw_buffer_load_b32(
                rx, t + sh >= 0 ? (uint32_t)((t + sh) * p.x_row_stride + chqk) * 2u : kOOB, 0, 0);
            if (i < 3)
                in.qkh[i] = __builtin_amdgcn_raw_buffer_load_b32(rh, t < 0 ? (uint32_t)((t + 3) * C + chqk) * 2u : kOOB,
                                                                 0, 0);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 7; ++i) {
                const int t = 16 * rb + 4 * lk - 3 + i;
                in.v[rb][i] = __builtin_amdgcn_raw_buffer_load_b16(
                    rx, t + sh >= 0 ? (uint32_t)((t + sh) * p.x_row_stride + chv) * 2u : kOOB, 0, 0);
                if (rb == 0 && i < 3)
                    in.vh[i] = __builtin_amdgcn_raw_buffer_load_b16(
                        rh, t < 0 ? (uint32_t)((t + 3) * C + chv) * 2u : kOOB, 0, 0);
            }
    };
    // ---- a chunk's operands from the workspace: the nonzero blocks (row
    // block, token block) (0,0), (1,0), (1,1) of T' and P and the row factors
    // at the lane's rows (all read before the chunk's second barrier, so the
    // next chunk's load there reuses their registers), and e^gamma_last (read
    // at the chunk's end, and loaded there for the next: a value loaded while
    // the one before is still needed would be copied at the loop's edge,
    // which waits for every load in flight)
    struct Ops {
        v4f t[3], pm[3];
        v4f fa[2], fb[2], fc[2];
    };
    auto fac_rsrc = [&](int c) {
        const bool real = c < nchunks;
        return buf_rsrc(tp.ws.fac + (blk0 + (size_t)(real ? c : 0)) * 128, real ? 512u : 0u);
    };
    auto load_ops = [&](int c, Ops &o) {
        const bool real = c < nchunks;
        const size_t blk = blk0 + (size_t)(real ? c : 0);
        const __amdgpu_buffer_rsrc_t rT = buf_rsrc(tp.ws.ta + blk * CHUNK_P, real ? CHUNK_P * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rP = buf_rsrc(tp.ws.pa + blk * CHUNK_P, real ? CHUNK_P * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rF = fac_rsrc(c);
        constexpr int kBlk[3] = {0, 2, 3}; // [row block][token block] of the nonzero blocks
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            o.t[k] = buf_load4(rT, (uint32_t)(kBlk[k] * 64 + lane) * 16u);
            o.pm[k] = buf_load4(rP, (uint32_t)(kBlk[k] * 64 + lane) * 16u);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            o.fa[rb] = buf_load4(rF, (uint32_t)(0 * BT + 16 * rb + 4 * lk) * 4u);
            o.fb[rb] = buf_load4(rF, (uint32_t)(1 * BT + 16 * rb + 4 * lk) * 4u);
            o.fc[rb] = buf_load4(rF, (uint32_t)(2 * BT + 16 * rb + 4 * lk) * 4u);
        }
    };
    auto load_el = [&](int c) { return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(fac_rsrc(c), 96u * 4u, 0, 0)); };

    // ---- the state -> LDS, transposed (as the wide walk)
    for (int e2 = tid; e2 < DK * DVS / 4; e2 += NTS) {
        const int j = e2 % DVS, i4 = e2 / DVS;
        v4f v;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = __builtin_nontemporal_load(tile + (size_t)(4 * i4 + r) * DV + col0 + j);
        *reinterpret_cast<v4f *>(&St[j * SPT + 4 * i4]) = v;
    }
    XIn xin;
    Ops ops;
    load_x(0, xin);
    // x first, as in the loop: the conv at the loop's top then waits for x alone
    __builtin_amdgcn_sched_barrier(0);
    load_ops(0, ops);
    float el = load_el(0);

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = __builtin_amdgcn_readfirstlane(t_begin + c * BT);
        const int n = __builtin_amdgcn_readfirstlane(t_end - t0 < BT ? t_end - t0 : BT);

        // ---- conv + SiLU of the q | k run -> Qs, Ks (padding tokens: zero),
        // the same arithmetic as the first pass's
        {
            float h0[2], h1[2], h2[2];
            const uint32_t x0 = xin.qk[0] | xin.qkh[0], x1 = xin.qk[1] | xin.qkh[1], x2 = xin.qk[2] | xin.qkh[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                h0[h] = __uint_as_float(h ? x0 & 0xffff0000u : x0 << 16);
                h1[h] = __uint_as_float(h ? x1 & 0xffff0000u : x1 << 16);
                h2[h] = __uint_as_float(h ? x2 & 0xffff0000u : x2 << 16);
            }
#pragma unroll
            for (int tt = 0; tt < TPT; ++tt) {
                const uint32_t xb = xin.qk[3 + tt];
                const float xv[2] = {__uint_as_float(xb << 16), __uint_as_float(xb & 0xffff0000u)};
                float y[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float acc = wq[0][h] * h0[h];
                    acc = fmaf(wq[1][h], h1[h], acc);
                    acc = fmaf(wq[2][h], h2[h], acc);
                    acc = fmaf(wq[3][h], xv[h], acc);
                    if (has_bias)
                        acc += bq[h];
                    y[h] = sp * TPT + tt < n ? acc * __builtin_amdgcn_rcpf(1.0f + __expf(-acc)) : 0.f;
                    h0[h] = h1[h];
                    h1[h] = h2[h];
                    h2[h] = xv[h];
                }
                *reinterpret_cast<float2 *>(&ydst[(sp * TPT + tt) * KP]) = make_float2(y[0], y[1]);
            }
        }
        // ---- conv + SiLU of v at the lane's places (padding tokens: zero)
        v4f vv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float xs[7];
#pragma unroll
            for (int i = 0; i < 7; ++i)
                xs[i] = __uint_as_float((uint32_t)(xin.v[rb][i] | (rb == 0 && i < 3 ? xin.vh[i] : 0u)) << 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float acc = wvc[0] * xs[r];
                acc = fmaf(wvc[1], xs[r + 1], acc);
                acc = fmaf(wvc[2], xs[r + 2], acc);
                acc = fmaf(wvc[3], xs[r + 3], acc);
                if (has_bias)
                    acc += bvc;
                vv[rb][r] = 16 * rb + 4 * lk + r < n ? acc * __builtin_amdgcn_rcpf(1.0f + __expf(-acc)) : 0.f;
            }
        }
        __syncthreads(); // Q and K of this chunk; the state after the previous one

        // ---- K^T operands of this wave's state rows (token k-steps in the
        // accumulator layout's row order), taken now: after the next barrier
        // the next chunk's conv may rewrite K
        float kt[RBW][2][4];
#pragma unroll
        for (int q = 0; q < RBW; ++q)
#pragma unroll
            for (int m4 = 0; m4 < 2; ++m4)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    kt[q][m4][e4] = Ks[(16 * m4 + 4 * lk + e4) * KP + (rb0 + q) * 16 + li];

        // ---- Y = K S0 and Z = Q S0 on column block wv
        v4f y[2], z[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            y[rb] = z[rb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m4 = 0; m4 < NA4; ++m4) {
            const v4f bs = *reinterpret_cast<const v4f *>(&St[(wv * 16 + li) * SPT + 16 * m4 + 4 * lk]);
            v4f ka[2], qa[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                ka[rb] = *reinterpret_cast<const v4f *>(&Ks[(16 * rb + li) * KP + 16 * m4 + 4 * lk]);
                qa[rb] = *reinterpret_cast<const v4f *>(&Qs[(16 * rb + li) * KP + 16 * m4 + 4 * lk]);
            }
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    y[rb] = mma16(ka[rb][e4], bs[e4], y[rb]);
                    z[rb] = mma16(qa[rb][e4], bs[e4], z[rb]);
                }
        }
        // the next chunk's x loads go out among these products, so their
        // address processing runs under the matrix cores
        load_x(c + 1, xin);
#pragma unroll
        for (int i = 0; i < (TPT + 3) + 3 + 2 * 7 + 3; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // one vector-memory read
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0); // three MFMA
        }

        // ---- R = V - f_a Y, U = T' R (three independent chains of four)
        v4f rr[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rr[rb][r] = fmaf(-ops.fa[rb][r], y[rb][r], vv[rb][r]);
        v4f u0 = {0.f, 0.f, 0.f, 0.f}, u1a = u0, u1b = u0;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            u0 = mma16(ops.t[0][e4], rr[0][e4], u0);
            u1a = mma16(ops.t[1][e4], rr[0][e4], u1a);
            u1b = mma16(ops.t[2][e4], rr[1][e4], u1b);
        }
        const v4f u1 = {u1a[0] + u1b[0], u1a[1] + u1b[1], u1a[2] + u1b[2], u1a[3] + u1b[3]};

        // ---- O = f_b Z + P U -> out (rows of real tokens; later rows fall outside)
        {
            v4f o0 = {ops.fb[0][0] * z[0][0], ops.fb[0][1] * z[0][1], ops.fb[0][2] * z[0][2], ops.fb[0][3] * z[0][3]};
            v4f o1a = {ops.fb[1][0] * z[1][0], ops.fb[1][1] * z[1][1], ops.fb[1][2] * z[1][2], ops.fb[1][3] * z[1][3]};
            v4f o1b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                o0 = mma16(ops.pm[0][e4], u0[e4], o0);
                o1a = mma16(ops.pm[1][e4], u0[e4], o1a);
                o1b = mma16(ops.pm[2][e4], u1[e4], o1b);
            }
            const v4f o1 = {o1a[0] + o1b[0], o1a[1] + o1b[1], o1a[2] + o1b[2], o1a[3] + o1b[3]};
            const __amdgpu_buffer_rsrc_t rO =
                buf_rsrc(p.out + ((size_t)t0 * p.H_v + hv) * DV + col0, (uint32_t)(((n - 1) * p.H_v * DV + DVS) * 2));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                __builtin_amdgcn_raw_buffer_store_b16(bf16_bits(o0[r]), rO,
                                                      (uint32_t)((4 * lk + r) * p.H_v * DV + 16 * wv + li) * 2u, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16(
                    bf16_bits(o1[r]), rO, (uint32_t)((16 + 4 * lk + r) * p.H_v * DV + 16 * wv + li) * 2u, 0, 0);
            }
        }
        // ---- U'' = f_c U -> LDS (transposed, as the wide walk's U)
        *reinterpret_cast<v4f *>(&Ut[(16 * wv + li) * UPT + 4 * lk]) =
            v4f{ops.fc[0][0] * u0[0], ops.fc[0][1] * u0[1], ops.fc[0][2] * u0[2], ops.fc[0][3] * u0[3]};
        *reinterpret_cast<v4f *>(&Ut[(16 * wv + li) * UPT + 16 + 4 * lk]) =
            v4f{ops.fc[1][0] * u1[0], ops.fc[1][1] * u1[1], ops.fc[1][2] * u1[2], ops.fc[1][3] * u1[3]};
        load_ops(c + 1, ops);
        __syncthreads(); // U'' complete; this chunk's reads of the state, K and Q are done

        // ---- S1 = e^gamma_last S0 + K^T U'' on this wave's tiles
        {
            v4f sacc[RBW][CBU];
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBU; ++jb) {
                    const v4f s4 =
                        *reinterpret_cast<const v4f *>(&St[((cbu0 + jb) * 16 + li) * SPT + (rb0 + q) * 16 + 4 * lk]);
                    sacc[q][jb] = v4f{el * s4[0], el * s4[1], el * s4[2], el * s4[3]};
                }
#pragma unroll
            for (int m4 = 0; m4 < 2; ++m4)
#pragma unroll
                for (int jb = 0; jb < CBU; ++jb) {
                    const v4f ub = *reinterpret_cast<const v4f *>(&Ut[((cbu0 + jb) * 16 + li) * UPT + 16 * m4 + 4 * lk]);
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                        for (int q = 0; q < RBW; ++q)
                            sacc[q][jb] = mma16(kt[q][m4][e4], ub[e4], sacc[q][jb]);
                }
#pragma unroll
            for (int q = 0; q < RBW; ++q)
#pragma unroll
                for (int jb = 0; jb < CBU; ++jb)
                    *reinterpret_cast<v4f *>(&St[((cbu0 + jb) * 16 + li) * SPT + (rb0 + q) * 16 + 4 * lk]) = sacc[q][jb];
        }
        el = load_el(c + 1);
    }
    __syncthreads(); // the last update is in LDS

    // ---- the state's slice back to the slot (the same mapping)
    for (int e2 = tid; e2 < DK * DVS / 4; e2 += NTS) {
        const int j = e2 % DVS, i4 = e2 / DVS;
        const v4f v = *reinterpret_cast<const v4f *>(&St[j * SPT + 4 * i4]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_nontemporal_store(v[r], tile + (size_t)(4 * i4 + r) * DV + col0 + j);
    }
    advance_windows<DK, DV, DVS, NTS>(p, hv, 0, t_begin, t_end, s);
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
    int all_lo = 0, all_hi = INT_MAX;
    void *args[] = {&q, &all_lo, &all_hi};
    hipError_t e = hipSuccess;
    // up to NT prompts, pass 1 builds the chunk map in LDS (its first
    // workgroup stores the prompts' first chunks for the walks): no map launch
    if (p.B > NT)
        e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_chunk_map_kernel), dim3(1), dim3(NT), args, 0, stream);
    if (e != hipSuccess)
        return e;
    // pass 1 walks the chunks with about two resident workgroups a compute
    // unit (three in the slim layout), each taking every gx-th chunk of a head
    const long long nchunk_max = ((long long)p.total + BT - 1) / BT + p.B;
    long long gx = (tp.ws.slim ? 768 : 512) / p.H_v;
    gx = gx < 1 ? 1 : (gx > nchunk_max ? nchunk_max : gx);
    const long long heads = (long long)p.B * p.H_v;
    if (tp.ws.slim) {
        e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_intra_kernel<DK, DV, true>),
                            dim3((unsigned)gx, (unsigned)p.H_v), dim3(NT), args, 0, stream);
        if (e != hipSuccess)
            return e;
        return hipLaunchKernel(reinterpret_cast<const void *>(&tp_slim_kernel<DK, DV>), dim3((unsigned)heads),
                               dim3(4 * DV), args, 0, stream);
    }
    // column slices 64, 32 or 16 wide (two workgroups a CU fit; with whole
    // 128-column slices, one a CU, 16 x 512 took 10 us and 128 x 64 71 us
    // longer).  The walk's time follows the CUs that get the most workgroups,
    // each worth 1 / nsl of a head's work: take the nsl that makes
    // ceil(heads nsl / 256) / nsl least, the fewer slices on a tie (measured
    // on MI355X against doubling until 256 workgroups: 6 x 1024 221 -> 215 us,
    // 12 x 768 306 -> 296; the power-of-two batches keep their choice)
    int nsl = DV / 64 > 1 ? DV / 64 : 1;
    long long best = (heads * nsl + 255) / 256; // per-CU share, in units of 1 / nsl
    for (int n = 2 * nsl; n <= DV / 16; n *= 2) {
        const long long share = (heads * n + 255) / 256;
        if (share * nsl < best * n) { // share / n < best / nsl
            nsl = n;
            best = share;
        }
    }
    // The pipelined schedule: when the 16-column walk takes at most half the
    // compute units, the chunks go in consecutive ranges of 32; pass 1 of
    // range 0 runs alone, a workgroup a chunk, then launch k walks range k on
    // its workgroups while pass 1 of range k + 1 runs on the compute units
    // left free, a workgroup each.  At 16 value heads those 128 workgroups take
    // four chunks each, about as long as the walk takes over 32 chunks.
    const long long cus = device_cus();
    const long long n_walk = heads * nsl;
    // chunks of the call: at most one partial chunk a sequence
    const long long nchunk_hi = ((long long)p.total + BT - 1) / BT + p.B - 1;
    constexpr int S = 32;
    if (DV / nsl == 16 && n_walk * 2 <= cus && nchunk_hi >= 2 * S) {
        const long long K = (nchunk_hi + S - 1) / S;
        int lo0 = 0, hi0 = S;
        void *a0[] = {&q, &lo0, &hi0};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_intra_kernel<DK, DV, false>),
                            dim3((unsigned)S, (unsigned)p.H_v), dim3(NT), a0, 0, stream);
        const long long free_cus = cus - n_walk;
        int nw = (int)n_walk, gxp = (int)(free_cus / p.H_v > 0 ? free_cus / p.H_v : 1);
        for (long long k = 0; k + 1 < K && e == hipSuccess; ++k) {
            int wlo = (int)(k * S), whi = (int)((k + 1) * S);
            int plo = whi, phi = k + 2 < K ? (int)((k + 2) * S) : INT_MAX;
            void *ak[] = {&q, &nw, &wlo, &whi, &gxp, &plo, &phi};
            e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_pipe_kernel<DK, DV>),
                                dim3((unsigned)(n_walk + (long long)gxp * p.H_v)), dim3(NT), ak, 0, stream);
        }
        // the last range has no pass 1 beside it: the walk kernel alone
        int wl = (int)((K - 1) * S), wh = INT_MAX;
        void *al[] = {&q, &wl, &wh};
        if (e == hipSuccess)
            e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_inter16_kernel<DK, DV>), dim3((unsigned)n_walk),
                                dim3(NT), al, 0, stream);
        return e;
    }
    e = hipLaunchKernel(reinterpret_cast<const void *>(&tp_intra_kernel<DK, DV, false>),
                        dim3((unsigned)gx, (unsigned)p.H_v), dim3(NT), args, 0, stream);
    if (e != hipSuccess)
        return e;
    switch (DV / nsl) {
    case 16:
        return hipLaunchKernel(reinterpret_cast<const void *>(&tp_inter16_kernel<DK, DV>),
                               dim3((unsigned)(heads * (DV / 16))), dim3(NT), args, 0, stream);
    case 32: return launch_inter<DK, DV, 32>(tp, heads, stream);
    default: return launch_inter<DK, DV, 64>(tp, heads, stream);
    }
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

} // namespace

bool two_pass_slim(int B, int H_v, int d_k, int d_v)
{
    // the slim walk's workgroups (one a prompt and value head, one a compute
    // unit) fill the 256 compute units at least once, and their last round at
    // least three quarters: below that the full layout's column slices even
    // the rounds out (measured on MI355X: 320 pairs 399 us slim against 372
    // full, 384 pairs 417 against 417, 640 pairs 344 against 357)
    const long long heads = (long long)B * H_v, rounds = (heads + 255) / 256;
    return d_k % 64 == 0 && d_v % 64 == 0 && heads >= 256 && heads * 4 >= rounds * 256 * 3;
}

size_t two_pass_layout(int B, int total, int H_k, int H_v, int d_k, int d_v, void *base, TwoPassWorkspace *ws)
{
    // chunk blocks per head: an upper bound on the call's chunk count (each
    // sequence adds at most one partial chunk)
    const size_t nchunk = ((size_t)total + BT - 1) / BT + (size_t)B;
    const size_t blocks = (size_t)H_v * nchunk;
    const bool slim = two_pass_slim(B, H_v, d_k, d_v);
    size_t off = 0;
    auto region = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes);
        return o;
    };
    const size_t o_cs = region((size_t)(B + 1) * sizeof(int32_t));
    const size_t o_rec = region(nchunk * 4 * sizeof(int32_t));
    size_t o_qa = 0, o_wa = 0, o_ka = 0, o_ud = 0, o_el = 0, o_ta = 0, o_fac = 0, o_hw = 0;
    if (slim) {
        o_ta = region(blocks * BT * BT * sizeof(float));
        o_fac = region(blocks * 128 * sizeof(float));
        o_hw = region((size_t)B * 3 * ((size_t)2 * H_k * d_k + (size_t)H_v * d_v) * sizeof(uint16_t));
    } else {
        o_qa = region(blocks * BT * d_k * sizeof(float));
        o_wa = region(blocks * BT * d_k * sizeof(float));
        o_ka = region(blocks * BT * d_k * sizeof(float));
        o_ud = region(blocks * BT * d_v * sizeof(float));
        o_el = region(blocks * sizeof(float));
    }
    const size_t o_pa = region(blocks * BT * BT * sizeof(float));
    if (base && ws) {
        char *c = static_cast<char *>(base);
        auto f = [&](size_t o) { return reinterpret_cast<float *>(c + o); };
        *ws = TwoPassWorkspace{};
        ws->chunk_start = reinterpret_cast<int32_t *>(c + o_cs);
        ws->chunk_rec = reinterpret_cast<int32_t *>(c + o_rec);
        ws->pa = f(o_pa);
        if (slim) {
            ws->ta = f(o_ta);
            ws->fac = f(o_fac);
            ws->hw = reinterpret_cast<uint16_t *>(c + o_hw);
        } else {
            ws->qa = f(o_qa);
            ws->wa = f(o_wa);
            ws->ka = f(o_ka);
            ws->ud = f(o_ud);
            ws->el = f(o_el);
        }
        ws->nchunk = (int)nchunk;
        ws->slim = slim ? 1 : 0;
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
