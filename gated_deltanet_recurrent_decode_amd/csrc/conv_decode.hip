// conv_decode.hip -- pooled conv-window update for one token a row (gfx950).
//
// The standalone form of the conv stage that the fused step runs inline
// (mstar PR #1139, "What changed": causal_conv1d_decode -- one token a row,
// optional bias and activation, strided rows, null slots, and a separate
// write slot that leaves the read slot alone).  One thread per (row,
// channel); the window rows [N][3][C] make every load and store coalesced
// across the channels of a wave.

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {

__global__ __launch_bounds__(256) void conv_decode_kernel(ConvParams p)
{
    const int r = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= p.C)
        return;
    const int rs = p.read_slot[r];
    const int ws = p.write_slot ? p.write_slot[r] : rs;
    uint16_t *o = p.out + (size_t)r * p.out_row_stride + c;
    if (rs == 0) { // padding row: zero output, no slot touched
        *o = 0;
        return;
    }
    // unusable: a slot out of range, or a write into the null slot (which must
    // stay zero): NaN, no slot touched
    if (rs < 0 || rs >= p.N || ws < 0 || ws >= p.N || ws == 0) {
        *o = 0x7fc0;
        return;
    }
    const size_t C = (size_t)p.C;
    const uint16_t *rd = p.conv_state + (size_t)rs * 3 * C + c;
    const uint16_t b1 = rd[C], b2 = rd[2 * C];
    const float w0 = bf16_to_f32(rd[0]), w1 = bf16_to_f32(b1), w2 = bf16_to_f32(b2);
    const uint16_t xb = p.x[(size_t)r * p.x_row_stride + c];
    const uint16_t *wc = p.conv_w + (size_t)c * 4;
    float acc = bf16_to_f32(wc[0]) * w0;
    acc = fmaf(bf16_to_f32(wc[1]), w1, acc);
    acc = fmaf(bf16_to_f32(wc[2]), w2, acc);
    acc = fmaf(bf16_to_f32(wc[3]), bf16_to_f32(xb), acc);
    if (p.conv_b)
        acc += bf16_to_f32(p.conv_b[c]);
    *o = f32_to_bf16_rne(p.activation ? silu(acc) : acc);
    uint16_t *wr = p.conv_state + (size_t)ws * 3 * C + c;
    wr[0] = b1;
    wr[C] = b2;
    wr[2 * C] = xb;
}

hipError_t launch_conv_decode(const ConvParams &p, hipStream_t stream)
{
    if (p.B <= 0 || p.C <= 0)
        return hipSuccess;
    ConvParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&conv_decode_kernel),
                           dim3((unsigned)((p.C + 255) / 256), (unsigned)p.B), dim3(256), args, 0, stream);
}

} // namespace gdn
