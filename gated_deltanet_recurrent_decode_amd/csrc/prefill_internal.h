// prefill_internal.h -- parameter block and launcher of the chunked prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Chunked prefill over packed sequences, in place.
struct PrefillParams {
    const uint16_t *x;          // [total][C] bf16, rows x_row_stride apart
    int64_t x_row_stride;
    const int32_t *cu_seqlens;  // [B+1]: sequence b owns tokens cu[b] .. cu[b+1]-1
    const uint16_t *conv_w;     // [C][4] bf16
    const uint16_t *conv_b;     // [C] bf16 or null
    uint16_t *conv_state;       // [N][3][C] bf16
    float *state;               // [N][H_v][d_k][d_v] fp32
    const float *g;             // [total][H_v]
    const float *beta;          // [total][H_v]
    const int32_t *slot;        // [B]
    uint16_t *out;              // [total][H_v][d_v] bf16
    float q_scale;
    float l2_eps;
    int B, total, H_k, H_v, G, N, C;
};

hipError_t launch_gdn_prefill(const PrefillParams &p, int d_k, int d_v, hipStream_t stream);

// The two-pass prefill: its workspace, carved by two_pass_layout from one
// caller buffer.  Per value head hv and packed token t (row hv * total + t):
// q~ = e^gamma q^ [d_k], k~ = e^(gamma_last - gamma) k^ [d_k],
// w = ((I + A)^-1 diag(beta e^gamma) K)[t] [d_k], u~ = ((I + A)^-1 diag(beta) V)[t]
// [d_v], p = P[t] [32], and el = e^gamma_last at the chunk's first token.
struct TwoPassWorkspace {
    int32_t *chunk_start; // [B+1]: exclusive scan of each sequence's chunk count
    float *qt, *kt, *ww, *ut, *pp, *el;
};

struct TwoPassParams {
    PrefillParams p;
    TwoPassWorkspace ws;
};

// Bytes of the workspace for B sequences, total tokens, H_v heads, d_k, d_v;
// with a base pointer, also the regions (each 256-byte aligned).
size_t two_pass_layout(int B, int total, int H_v, int d_k, int d_v, void *base, TwoPassWorkspace *ws);

hipError_t launch_gdn_prefill_two_pass(const TwoPassParams &p, int d_k, int d_v, hipStream_t stream);

} // namespace gdn
