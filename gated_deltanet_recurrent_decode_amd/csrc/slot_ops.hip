// slot_ops.hip -- slot lifecycle on the pool (gfx950): zero slots, copy slots.
//
// mstar PR #1139, "Tests": rollback and release zero both slots of a request,
// and decode snapshots and forks must read the right slot.  A slot's contents
// are its fp32 state [H_v][d_k][d_v] and its bf16 conv window [W-1][C]; both
// are moved with 16-byte streaming accesses.  Slot 0 (the null slot) is never
// written; slot indices outside the pool are skipped.

#include "device_common.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// blockIdx.y = pair i; the blocks along x stride over the slot's contents.
__global__ __launch_bounds__(256) void slot_ops_kernel(SlotOpsParams p)
{
    const int i = blockIdx.y;
    const int dst = p.dst[i];
    const int src = p.src ? p.src[i] : 0;
    if (dst <= 0 || dst >= p.N || src < 0 || src >= p.N)
        return;
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t first = (size_t)blockIdx.x * 256 + threadIdx.x;

    f32x4 *sd = reinterpret_cast<f32x4 *>(p.state + (size_t)dst * p.slot_state);
    const f32x4 *ss = reinterpret_cast<const f32x4 *>(p.state + (size_t)src * p.slot_state);
    const size_t n4 = p.slot_state / 4;
    for (size_t e = first; e < n4; e += stride) {
        const f32x4 v = p.src ? __builtin_nontemporal_load(ss + e) : f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_nontemporal_store(v, sd + e);
    }

    u32x2 *cd = reinterpret_cast<u32x2 *>(p.conv_state + (size_t)dst * p.slot_conv);
    const u32x2 *cs = reinterpret_cast<const u32x2 *>(p.conv_state + (size_t)src * p.slot_conv);
    const size_t c4 = p.slot_conv / 4;
    for (size_t e = first; e < c4; e += stride) {
        const u32x2 v = p.src ? __builtin_nontemporal_load(cs + e) : u32x2{0u, 0u};
        __builtin_nontemporal_store(v, cd + e);
    }
}

hipError_t launch_slot_ops(const SlotOpsParams &p, int n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    // enough blocks per slot to keep every slot's contents in flight at once
    const size_t per_slot = (p.slot_state / 4 + 1023) / 1024;
    const unsigned bx = (unsigned)(per_slot < 1 ? 1 : (per_slot > 256 ? 256 : per_slot));
    SlotOpsParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(&slot_ops_kernel), dim3(bx, (unsigned)n), dim3(256), args,
                           0, stream);
}

} // namespace gdn
