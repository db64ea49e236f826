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
// caller buffer.  Chunks are numbered across the call (sequence b's chunks
// start at chunk_start[b]); the workspace holds nchunk = ceil(total / 32) + B
// chunk blocks per value head, block (hv, g) at hv * nchunk + g, each laid out
// as the second pass's matrix-core operands, so it loads them straight into
// registers.  Two layouts, picked by two_pass_slim from the call's shape:
// full (the second pass reads every product of the chunk that does not depend
// on the state):
//   qa, wa  [2 row blocks][d_k / 16][64 lanes][4]: q~ = e^gamma q^ and
//           w = ((I + A)^-1 diag(beta e^gamma) K), element (rb, m, lane) the
//           A operand of k-slice m: row rb * 16 + lane % 16, column 4 m + lane / 16
//   ka      [d_k / 16 row blocks][2][64][4]: k~ = e^(gamma_last - gamma) k^ as
//           the A operand of the state update, element (ib, m, lane) =
//           k~[4 m + lane / 16][ib * 16 + lane % 16]
//   pa      [2][2][64][4]: P as an A operand, like qa
//   ud      [2 row blocks][d_v / 16 column blocks][64][4]: u~ = ((I + A)^-1
//           diag(beta) V) in the accumulator layout, lane j + 16 g holding rows
//           4 g .. 4 g + 3 of column j
//   el      e^gamma_last of the chunk
// slim (the second pass runs the conv itself and forms U from T'):
//   ta      [2][2][64][4]: T' = (I + A)^-1 diag(beta) as an A operand, like pa
//   pa      as above
//   fac     [128] floats: per token t < 32 the row factors k-norm e^gamma
//           ([0, 32)), q-norm q_scale e^gamma ([32, 64)) and
//           k-norm e^(gamma_last - gamma) ([64, 96)), each zero for a padding
//           token; e^gamma_last at [96]
//   hw      [B][3][C] bf16: each prompt's conv window as the call found it
//           (the second pass's first chunk takes its three earlier inputs from
//           here, as another workgroup may already have advanced the slot's)
// and, per chunk of the call, its record [nchunk][4]: first token, tokens
// (at most 32), slot, and for a sequence's first chunk (whose three earlier
// inputs come from the slot's window) the sequence's index + 1, else 0.
struct TwoPassWorkspace {
    int32_t *chunk_start; // [B+1]: exclusive scan of each sequence's chunk count
    int32_t *chunk_rec;   // [nchunk][4]
    float *qa, *wa, *ka, *pa, *ud, *el; // full layout (pa in both)
    float *ta, *fac;                    // slim layout
    uint16_t *hw;                       // slim layout
    int nchunk;
    int slim;
};

struct TwoPassParams {
    PrefillParams p;
    TwoPassWorkspace ws;
};

// Whether a call of B sequences over H_v value heads takes the slim layout and
// its second pass (a workgroup a sequence and value head; at least 256 of
// them, the last round of 256 at least three quarters full).
bool two_pass_slim(int B, int H_v, int d_k, int d_v);

// Bytes of the workspace for B sequences, total tokens, H_k / H_v heads, d_k,
// d_v; with a base pointer, also the regions (each 256-byte aligned).
size_t two_pass_layout(int B, int total, int H_k, int H_v, int d_k, int d_v, void *base, TwoPassWorkspace *ws);

hipError_t launch_gdn_prefill_two_pass(const TwoPassParams &p, int d_k, int d_v, hipStream_t stream);

} // namespace gdn
