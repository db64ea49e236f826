// gdn_abi.hip -- the extern "C" boundary of libgdn.so: host-side validation,
// then one launch on the caller's stream.  Nothing here allocates, synchronises
// or reads device memory, so every entry point can be captured into a graph.
// The contracts are stated in include/gdn.h.

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"
#include "gdn_internal.h"
#include "prefill_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

} // namespace

extern "C" const char *gdn_status_string(gdn_status status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "inconsistent or out-of-range sizes or strides";
    case GDN_ERR_UNSUPPORTED: return "sizes or alignment outside what the kernels are built for";
    case GDN_ERR_REFUSED: return "refused: a twin-slot write takes one token a row (multi-token walks stay in place)";
    case GDN_ERR_HIP: return "the HIP launch failed";
    case GDN_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    }
    return "unknown gdn_status";
}

namespace {

gdn_status step_impl(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride, const gdn_bf16 *conv_w,
                     const gdn_bf16 *conv_b, gdn_bf16 *conv_state, float *state, const float *g, const float *beta,
                     const int32_t *read_slot, const int32_t *write_slot, int32_t *next_read_slot,
                     int32_t *next_write_slot, const int32_t *token_slots, gdn_bf16 *out, float q_scale,
                     float l2_eps, hipStream_t stream)
{
    if (!dims)
        return GDN_ERR_NULL;
    const gdn_dims d = *dims;
    if (d.B == 0) // nothing to do; per-row arrays may be NULL
        return GDN_OK;
    if (!x || !conv_w || !conv_state || !state || !g || !beta || !read_slot || !out)
        return GDN_ERR_NULL;
    if (d.B < 0 || d.T < 1 || d.H_k < 1 || d.H_v < 1 || d.N < 1 || d.H_v % d.H_k != 0)
        return GDN_ERR_SHAPE;
    if (!head_dim_ok(d.d_k) || !head_dim_ok(d.d_v) || d.W != 4)
        return GDN_ERR_UNSUPPORTED;
    const int64_t C = 2LL * d.H_k * d.d_k + (int64_t)d.H_v * d.d_v;
    if (C > INT32_MAX || x_row_stride < (int64_t)d.T * C)
        return GDN_ERR_SHAPE;
    if ((int64_t)d.B * d.H_v * 4 > INT32_MAX) // workgroups in the grid
        return GDN_ERR_SHAPE;
    // the kernels address a row's x (with up to eight tokens of overrun past
    // the last, which read as zero), its outputs and its gates, and the conv
    // weights, through 32-bit byte offsets under 2 GiB
    const int64_t lim = (int64_t)1 << 31;
    if ((d.T + 8LL) * C * 2 >= lim || 8LL * C >= lim || (int64_t)d.T * d.H_v * d.d_v * 2 >= lim ||
        (int64_t)d.T * d.H_v * 4 >= lim)
        return GDN_ERR_SHAPE;
    if (!(l2_eps >= 0.0f) || !isfinite(l2_eps) || !isfinite(q_scale))
        return GDN_ERR_SHAPE;
    const int G = d.H_v / d.H_k;
    if (write_slot && d.T > 1)
        return GDN_ERR_REFUSED;
    if (!write_slot && G != 1 && G != 2 && G != 4)
        return GDN_ERR_UNSUPPORTED;
    // the step reads and writes four channels at a time and whole fp32 rows
    if (!aligned(state, 16) || !aligned(out, 8) || !aligned(conv_w, 16) || !aligned(conv_state, 8) ||
        !aligned(x, 8) || x_row_stride % 4 != 0 || (conv_b && !aligned(conv_b, 8)))
        return GDN_ERR_UNSUPPORTED;

    gdn::StepParams p{};
    p.x = x;
    p.x_row_stride = x_row_stride;
    p.conv_w = conv_w;
    p.conv_b = conv_b;
    p.conv_state = conv_state;
    p.state = state;
    p.g = g;
    p.beta = beta;
    p.read_slot = read_slot;
    p.write_slot = write_slot;
    p.next_read_slot = next_read_slot;
    p.next_write_slot = next_write_slot;
    p.out = out;
    p.q_scale = q_scale;
    p.l2_eps = l2_eps;
    p.B = d.B;
    p.T = d.T;
    p.H_k = d.H_k;
    p.H_v = d.H_v;
    p.N = d.N;
    p.C = (int)C;
    p.G = G;
    p.twin = write_slot ? 1 : 0;
    p.token_slots = token_slots;
    // one head tile a workgroup for every single-token step that allows it (a
    // twin write, or in place with one value head per key head), except the
    // in-place sizes that run faster with four value heads a workgroup; the
    // key-head-group kernel for those, token walks, per-token states and
    // in-place GQA
    const bool tile = d.T == 1 && !token_slots && (write_slot || G == 1) &&
                      !(!write_slot && gdn::walk_key_heads(p, d.d_k, d.d_v) > 1);
    return from_hip(tile ? gdn::launch_gdn_step_tile(p, d.d_k, d.d_v, stream)
                         : gdn::launch_gdn_step(p, d.d_k, d.d_v, stream));
}

} // namespace

extern "C" {

gdn_status gdn_decode_step(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                           const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                           float *state, const float *g, const float *beta,
                           const int32_t *read_slot, const int32_t *write_slot, gdn_bf16 *out,
                           float q_scale, float l2_eps, hipStream_t stream)
{
    return step_impl(dims, x, x_row_stride, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot,
                     nullptr, nullptr, nullptr, out, q_scale, l2_eps, stream);
}

gdn_status gdn_decode_step_tokens(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                  const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                                  float *state, const float *g, const float *beta, const int32_t *read_slot,
                                  const int32_t *token_slots, gdn_bf16 *out, float q_scale, float l2_eps,
                                  hipStream_t stream)
{
    if (dims && dims->B != 0 && !token_slots)
        return GDN_ERR_NULL;
    return step_impl(dims, x, x_row_stride, conv_w, conv_b, conv_state, state, g, beta, read_slot, nullptr,
                     nullptr, nullptr, token_slots, out, q_scale, l2_eps, stream);
}

gdn_status gdn_decode_step_commit(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                  const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state,
                                  float *state, const float *g, const float *beta, const int32_t *read_slot,
                                  const int32_t *write_slot, int32_t *next_read_slot, int32_t *next_write_slot,
                                  gdn_bf16 *out, float q_scale, float l2_eps, hipStream_t stream)
{
    if (dims && dims->B != 0) {
        if (!write_slot || !next_read_slot || !next_write_slot)
            return GDN_ERR_NULL;
        const int32_t *ins[2] = {read_slot, write_slot};
        const int32_t *outs[2] = {next_read_slot, next_write_slot};
        if (next_read_slot == next_write_slot)
            return GDN_ERR_SHAPE;
        for (const int32_t *a : ins)
            for (const int32_t *b : outs)
                if (a == b)
                    return GDN_ERR_SHAPE;
    }
    return step_impl(dims, x, x_row_stride, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot,
                     next_read_slot, next_write_slot, nullptr, out, q_scale, l2_eps, stream);
}

namespace {

// The checks gdn_prefill and gdn_prefill_two_pass share; on GDN_OK with
// *run set, p holds the launch parameters (*run is false when there is
// nothing to do).
gdn_status prefill_setup(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride, const int32_t *cu_seqlens,
                         const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state, float *state,
                         const float *g, const float *beta, const int32_t *slot, gdn_bf16 *out, float q_scale,
                         float l2_eps, gdn::PrefillParams &p, bool *run)
{
    *run = false;
    if (!dims)
        return GDN_ERR_NULL;
    const gdn_dims d = *dims;
    if (d.B == 0) // no sequences; the arrays may be NULL
        return GDN_OK;
    if (!x || !cu_seqlens || !conv_w || !conv_state || !state || !g || !beta || !slot || !out)
        return GDN_ERR_NULL;
    if (d.B < 0 || d.T < 0 || d.H_k < 1 || d.H_v < 1 || d.N < 1 || d.H_v % d.H_k != 0)
        return GDN_ERR_SHAPE;
    if (!head_dim_ok(d.d_k) || !head_dim_ok(d.d_v) || d.W != 4)
        return GDN_ERR_UNSUPPORTED;
    const int64_t C = 2LL * d.H_k * d.d_k + (int64_t)d.H_v * d.d_v;
    if (C > INT32_MAX || x_row_stride < C || (int64_t)d.B * d.H_v * 4 > INT32_MAX || d.H_v > 65535)
        return GDN_ERR_SHAPE;
    if (!(l2_eps >= 0.0f) || !isfinite(l2_eps) || !isfinite(q_scale))
        return GDN_ERR_SHAPE;
    // channel pairs are read and written 4 bytes at a time, the state 16
    if (!aligned(x, 4) || x_row_stride % 2 != 0 || !aligned(conv_state, 4) || !aligned(state, 16) ||
        !aligned(out, 2) || !aligned(conv_w, 2) || (conv_b && !aligned(conv_b, 2)))
        return GDN_ERR_UNSUPPORTED;
    if (d.T == 0) // every sequence is empty
        return GDN_OK;
    p = gdn::PrefillParams{};
    p.x = x;
    p.x_row_stride = x_row_stride;
    p.cu_seqlens = cu_seqlens;
    p.conv_w = conv_w;
    p.conv_b = conv_b;
    p.conv_state = conv_state;
    p.state = state;
    p.g = g;
    p.beta = beta;
    p.slot = slot;
    p.out = out;
    p.q_scale = q_scale;
    p.l2_eps = l2_eps;
    p.B = d.B;
    p.total = d.T;
    p.H_k = d.H_k;
    p.H_v = d.H_v;
    p.G = d.H_v / d.H_k;
    p.N = d.N;
    p.C = (int)C;
    *run = true;
    return GDN_OK;
}

} // namespace

gdn_status gdn_prefill(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride, const int32_t *cu_seqlens,
                       const gdn_bf16 *conv_w, const gdn_bf16 *conv_b, gdn_bf16 *conv_state, float *state,
                       const float *g, const float *beta, const int32_t *slot, gdn_bf16 *out, float q_scale,
                       float l2_eps, hipStream_t stream)
{
    gdn::PrefillParams p;
    bool run;
    const gdn_status st = prefill_setup(dims, x, x_row_stride, cu_seqlens, conv_w, conv_b, conv_state, state, g,
                                        beta, slot, out, q_scale, l2_eps, p, &run);
    if (st != GDN_OK || !run)
        return st;
    return from_hip(gdn::launch_gdn_prefill(p, dims->d_k, dims->d_v, stream));
}

size_t gdn_prefill_two_pass_workspace_bytes(const gdn_dims *dims)
{
    if (!dims)
        return 0;
    const gdn_dims d = *dims;
    if (d.B < 0 || d.T < 0 || d.H_v < 1 || !head_dim_ok(d.d_k) || !head_dim_ok(d.d_v))
        return 0;
    return gdn::two_pass_layout(d.B, d.T, d.H_k, d.H_v, d.d_k, d.d_v, nullptr, nullptr);
}

gdn_status gdn_prefill_two_pass(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                const int32_t *cu_seqlens, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                                gdn_bf16 *conv_state, float *state, const float *g, const float *beta,
                                const int32_t *slot, gdn_bf16 *out, float q_scale, float l2_eps, void *workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    gdn::PrefillParams p;
    bool run;
    const gdn_status st = prefill_setup(dims, x, x_row_stride, cu_seqlens, conv_w, conv_b, conv_state, state, g,
                                        beta, slot, out, q_scale, l2_eps, p, &run);
    if (st != GDN_OK || !run)
        return st;
    if (!workspace)
        return GDN_ERR_NULL;
    if (!aligned(workspace, 256))
        return GDN_ERR_UNSUPPORTED;
    if ((long long)p.total / 32 + p.B + 1 > INT32_MAX)
        return GDN_ERR_SHAPE;
    gdn::TwoPassParams tp{};
    tp.p = p;
    if (workspace_bytes < gdn::two_pass_layout(p.B, p.total, p.H_k, p.H_v, dims->d_k, dims->d_v, workspace, &tp.ws))
        return GDN_ERR_SHAPE;
    return from_hip(gdn::launch_gdn_prefill_two_pass(tp, dims->d_k, dims->d_v, stream));
}

} // extern "C"

// Scratch of gdn_prefill_two_pass_noalloc: a file-scope device array, one copy
// on every GPU the library is loaded on, kept until the process ends.  Host
// code must not pass the array's name to a kernel (on the host it stands for
// a host-side stub, not a device address); the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// The current device's copy of `scratch` (resolved on the first call on each
// device; a race between two first calls resolves the same address twice).
gdn_status scratch_for_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GDN_ERR_HIP;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return GDN_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return GDN_OK;
}

} // namespace

extern "C" {

gdn_status gdn_prefill_two_pass_noalloc(const gdn_dims *dims, const gdn_bf16 *x, int64_t x_row_stride,
                                        const int32_t *cu_seqlens, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                                        gdn_bf16 *conv_state, float *state, const float *g, const float *beta,
                                        const int32_t *slot, gdn_bf16 *out, float q_scale, float l2_eps,
                                        hipStream_t stream)
{
    gdn::PrefillParams p;
    bool run;
    const gdn_status st = prefill_setup(dims, x, x_row_stride, cu_seqlens, conv_w, conv_b, conv_state, state, g,
                                        beta, slot, out, q_scale, l2_eps, p, &run);
    if (st != GDN_OK || !run)
        return st;
    if ((long long)p.total / 32 + p.B + 1 > INT32_MAX)
        return GDN_ERR_SHAPE;
    if (gdn::two_pass_layout(p.B, p.total, p.H_k, p.H_v, dims->d_k, dims->d_v, nullptr, nullptr) > kScratchBytes)
        return GDN_ERR_SCRATCH;
    void *ws = nullptr;
    const gdn_status sst = scratch_for_current_device(&ws);
    if (sst != GDN_OK)
        return sst;
    gdn::TwoPassParams tp{};
    tp.p = p;
    gdn::two_pass_layout(p.B, p.total, p.H_k, p.H_v, dims->d_k, dims->d_v, ws, &tp.ws);
    return from_hip(gdn::launch_gdn_prefill_two_pass(tp, dims->d_k, dims->d_v, stream));
}

gdn_status conv_decode(int32_t B, int32_t C, int32_t W, int32_t N, const gdn_bf16 *x,
                       int64_t x_row_stride, const gdn_bf16 *conv_w, const gdn_bf16 *conv_b,
                       gdn_bf16 *conv_state, const int32_t *read_slot, const int32_t *write_slot,
                       gdn_bf16 *out, int64_t out_row_stride, int32_t activation,
                       hipStream_t stream)
{
    if (B == 0)
        return GDN_OK;
    if (!x || !conv_w || !conv_state || !read_slot || !out)
        return GDN_ERR_NULL;
    if (B < 0 || C < 1 || N < 1 || x_row_stride < C || out_row_stride < C || B > 65535)
        return GDN_ERR_SHAPE;
    if (activation != 0 && activation != 1)
        return GDN_ERR_SHAPE;
    if (W != 4)
        return GDN_ERR_UNSUPPORTED;
    gdn::ConvParams p{};
    p.x = x;
    p.x_row_stride = x_row_stride;
    p.conv_w = conv_w;
    p.conv_b = conv_b;
    p.conv_state = conv_state;
    p.read_slot = read_slot;
    p.write_slot = write_slot;
    p.out = out;
    p.out_row_stride = out_row_stride;
    p.B = B;
    p.C = C;
    p.N = N;
    p.activation = activation;
    return from_hip(gdn::launch_conv_decode(p, stream));
}

gdn_status slot_commit(int32_t *read_slot, int32_t *write_slot, int32_t B, hipStream_t stream)
{
    if (B == 0)
        return GDN_OK;
    if (!read_slot || !write_slot)
        return GDN_ERR_NULL;
    if (B < 0)
        return GDN_ERR_SHAPE;
    return from_hip(gdn::launch_slot_commit(read_slot, write_slot, B, stream));
}

gdn_status gdn_check_slots(const gdn_dims *dims, const int32_t *read_slot, const int32_t *write_slot,
                           int32_t *result, hipStream_t stream)
{
    if (!dims)
        return GDN_ERR_NULL;
    if (dims->B == 0)
        return GDN_OK;
    if (!read_slot || !result)
        return GDN_ERR_NULL;
    if (dims->B < 0 || dims->N < 1)
        return GDN_ERR_SHAPE;
    if (!aligned(read_slot, 4) || !aligned(result, 4) || (write_slot && !aligned(write_slot, 4)))
        return GDN_ERR_UNSUPPORTED;
    return from_hip(gdn::launch_slot_check(read_slot, write_slot, dims->B, dims->N, result, stream));
}

static gdn_status slot_ops_impl(const gdn_dims *dims, float *state, gdn_bf16 *conv_state, const int32_t *src,
                                const int32_t *dst, int32_t n, hipStream_t stream)
{
    if (!dims)
        return GDN_ERR_NULL;
    if (n == 0)
        return GDN_OK;
    const gdn_dims d = *dims;
    if (!state || !conv_state || !dst)
        return GDN_ERR_NULL;
    if (n < 0 || n > 65535 || d.H_k < 1 || d.H_v < 1 || d.d_k < 1 || d.d_v < 1 || d.W < 2 || d.N < 1 ||
        d.H_v % d.H_k != 0)
        return GDN_ERR_SHAPE;
    const int64_t C = 2LL * d.H_k * d.d_k + (int64_t)d.H_v * d.d_v;
    const int64_t slot_state = (int64_t)d.H_v * d.d_k * d.d_v;
    if (slot_state % 4 != 0 || C % 4 != 0 || !aligned(state, 16) || !aligned(conv_state, 8))
        return GDN_ERR_UNSUPPORTED;
    gdn::SlotOpsParams p{};
    p.state = state;
    p.conv_state = conv_state;
    p.src = src;
    p.dst = dst;
    p.slot_state = (size_t)slot_state;
    p.slot_conv = (size_t)((d.W - 1) * C);
    p.N = d.N;
    return from_hip(gdn::launch_slot_ops(p, n, stream));
}

gdn_status gdn_slot_reset(const gdn_dims *dims, float *state, gdn_bf16 *conv_state, const int32_t *slots,
                          int32_t n, hipStream_t stream)
{
    if (n != 0 && !slots)
        return GDN_ERR_NULL;
    return slot_ops_impl(dims, state, conv_state, nullptr, slots, n, stream);
}

gdn_status gdn_slot_copy(const gdn_dims *dims, float *state, gdn_bf16 *conv_state, const int32_t *src_slots,
                         const int32_t *dst_slots, int32_t n, hipStream_t stream)
{
    if (n != 0 && (!src_slots || !dst_slots))
        return GDN_ERR_NULL;
    return slot_ops_impl(dims, state, conv_state, src_slots, dst_slots, n, stream);
}

gdn_status gdn_traffic_probe(const gdn_probe *probe, int32_t B, int32_t H, int32_t d_k, int32_t d_v, int32_t N,
                             float *state, const int32_t *read_slot, const int32_t *write_slot, float *sink,
                             hipStream_t stream)
{
    if (!probe || !state || !read_slot || !sink)
        return GDN_ERR_NULL;
    const gdn_probe pr = *probe;
    if (pr.traffic < 0 || pr.traffic > 3 || pr.layout < 0 || pr.layout > 1 || pr.shape < 0 || pr.shape > 5 ||
        pr.hold_ns < 0 || pr.hold_ns > 1000000 || pr.order < 0 || pr.order > 2 || pr.policy < 0 ||
        pr.policy > 2 || pr.persistent < 0 || pr.persistent > 8 || (pr.persistent > 0 && pr.hold_ns > 0))
        return GDN_ERR_SHAPE;
    const bool uses_write = pr.traffic == 1 || pr.traffic == 2;
    if (uses_write && !write_slot)
        return GDN_ERR_NULL;
    if (B < 0 || H < 1 || N < 1 || (int64_t)B * H * 16 > INT32_MAX)
        return GDN_ERR_SHAPE;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v))
        return GDN_ERR_UNSUPPORTED;
    if ((pr.shape == 1 || pr.shape == 2) && (d_k != 128 || d_v != 128))
        return GDN_ERR_UNSUPPORTED;
    const int64_t tile_bytes = (int64_t)d_k * d_v * 4;
    if (pr.shape == 3) {
        const bool threads_ok = pr.threads == 256 || pr.threads == 512 || pr.threads == 1024;
        const bool loads_ok = pr.loads == 1 || pr.loads == 4 || pr.loads == 8 || pr.loads == 16;
        if (!threads_ok || !loads_ok || (int64_t)pr.threads * pr.loads > 4096)
            return GDN_ERR_SHAPE;
        if (tile_bytes % ((int64_t)pr.threads * pr.loads * 16) != 0)
            return GDN_ERR_UNSUPPORTED;
    }
    if (pr.layout == 1 && (int64_t)B * H * tile_bytes > INT32_MAX)
        return GDN_ERR_SHAPE;
    if (!aligned(state, 16))
        return GDN_ERR_UNSUPPORTED;
    if (B == 0 && pr.shape != 4)
        return GDN_OK;
    gdn::ProbeParams p{};
    p.state = state;
    p.read_slot = read_slot;
    p.write_slot = uses_write ? write_slot : nullptr;
    p.sink = sink;
    p.one = 1.0f;
    p.B = B;
    p.H = H;
    p.N = N;
    p.traffic = pr.traffic;
    p.layout = pr.layout;
    p.shape = pr.shape;
    p.hold_ticks = (uint32_t)(pr.hold_ns / 10); // the constant clock ticks at 100 MHz
    p.order = pr.order;
    p.threads = pr.threads;
    p.loads = pr.loads;
    p.persistent = pr.persistent;
    p.policy = pr.policy;
    return from_hip(gdn::launch_traffic_probe(p, d_k, d_v, stream));
}

} // extern "C"
