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

} // namespace gdn
