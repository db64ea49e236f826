// slot_commit.hip -- commit of a twin-slot step on the device (gfx950).
//
// mstar PR #1139, "What changed": after a decode step that read one slot and
// wrote the other, commit swaps them, so the next step reads what this one
// wrote.  Stream-ordered after the step; nothing is read back to the host.

#include "gdn_internal.h"

namespace gdn {

__global__ __launch_bounds__(256) void slot_commit_kernel(int32_t *read_slot, int32_t *write_slot, int B)
{
    for (int r = blockIdx.x * 256 + threadIdx.x; r < B; r += gridDim.x * 256) {
        const int32_t a = read_slot[r];
        const int32_t b = write_slot[r];
        read_slot[r] = b;
        write_slot[r] = a;
    }
}

hipError_t launch_slot_commit(int32_t *read_slot, int32_t *write_slot, int B, hipStream_t stream)
{
    if (B <= 0)
        return hipSuccess;
    int blocks = (B + 255) / 256;
    if (blocks > 1024)
        blocks = 1024;
    void *args[] = {&read_slot, &write_slot, &B};
    return hipLaunchKernel(reinterpret_cast<const void *>(&slot_commit_kernel), dim3(blocks), dim3(256), args, 0,
                           stream);
}

} // namespace gdn
