// gdn_internal.h -- kernel parameter blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Everything the fused step kernel reads; passed by value as the kernel argument.
struct StepParams {
    const uint16_t *x;       // [B][T][C] bf16, rows x_row_stride apart
    int64_t x_row_stride;
    const uint16_t *conv_w;  // [C][4] bf16
    const uint16_t *conv_b;  // [C] bf16 or null
    uint16_t *conv_state;    // [N][3][C] bf16
    float *state;            // [N][H_v][d_k][d_v] fp32
    const float *g;          // [B][T][H_v]
    const float *beta;       // [B][T][H_v]
    const int32_t *read_slot;
    const int32_t *write_slot; // null in place
    uint16_t *out;           // [B][T][H_v][d_v] bf16
    float q_scale;
    float l2_eps;
    int B, T, H_k, H_v, N, C, G;
    int32_t *next_read_slot;  // fused commit: receives write_slot[r] (null: no commit)
    int32_t *next_write_slot; // fused commit: receives read_slot[r]
    int n_slices; // d_v column slices per head (set by the launcher)
    int twin;     // 1: write to write_slot; 0: in place
    int xcd_groups; // tile kernel: the grid size to give each XCD a contiguous run of tile groups (0: off)
    const int32_t *token_slots; // [B][T]: in-place kernel keeps the state after token t in slot [r][t] (0: not
                                // kept) and leaves the read slot alone; null: plain in place
};

struct ConvParams {
    const uint16_t *x;
    int64_t x_row_stride;
    const uint16_t *conv_w;
    const uint16_t *conv_b;
    uint16_t *conv_state;
    const int32_t *read_slot;
    const int32_t *write_slot;
    uint16_t *out;
    int64_t out_row_stride;
    int B, C, N;
    int activation;
};

struct ProbeParams {
    float *state;
    const int32_t *read_slot;
    const int32_t *write_slot; // null for read-only and in-place traffic
    float *sink;
    float one; // 1.0f, opaque to the compiler (a never-true test on it keeps read-only loads alive)
    int B, H, N;
    int traffic;         // 0 read only, 1 write only, 2 copy, 3 read and write back in place
    int layout;          // 0 the rows' slots, 1 consecutive slots from read_slot[0] / write_slot[0]
    int shape;           // workgroup design (see gdn_probe in gdn.h)
    uint32_t hold_ticks; // 0, or: stores wait until this many 100 MHz ticks after the workgroup started
    int order;           // 0 each store after its own load, 1 a lane's loads first, 2 the workgroup's loads first
    int threads, loads;  // chunk design: workgroup size, 16-byte loads a lane
    int persistent;      // chunk design: 0 one chunk a workgroup, k: k workgroups a CU walking the chunks
    int policy;          // 0 streaming (nt), 1 plain, 2 system scope (sc0 sc1)
};

// Zero (src == null) or copy (src[i] -> dst[i]) whole slots of the pool.
struct SlotOpsParams {
    float *state;         // [N][slot_state] fp32
    uint16_t *conv_state; // [N][slot_conv] bf16
    const int32_t *src;   // [n] or null (reset)
    const int32_t *dst;   // [n]
    size_t slot_state;    // H_v * d_k * d_v
    size_t slot_conv;     // (W - 1) * C
    int N;
};

hipError_t launch_gdn_step(const StepParams &p, int d_k, int d_v, hipStream_t stream);
// key heads a workgroup of the walk kernel for this step (1 unless it groups several)
int walk_key_heads(const StepParams &p, int d_k, int d_v);
int device_cus();
hipError_t launch_gdn_step_tile(const StepParams &p, int d_k, int d_v, hipStream_t stream);
hipError_t launch_conv_decode(const ConvParams &p, hipStream_t stream);
hipError_t launch_slot_commit(int32_t *read_slot, int32_t *write_slot, int B, hipStream_t stream);
hipError_t launch_slot_check(const int32_t *read_slot, const int32_t *write_slot, int B, int N, int32_t *result,
                             hipStream_t stream);
hipError_t launch_slot_ops(const SlotOpsParams &p, int n, hipStream_t stream);
hipError_t launch_traffic_probe(const ProbeParams &p, int d_k, int d_v, hipStream_t stream);

} // namespace gdn
