// slot_commit.hip -- the slot arrays on the device (gfx950): the commit of a
// twin-slot step, and a debug check of a step's slot preconditions.
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

// The preconditions a step relies on (PR #1139, "What changed": a step reads
// one slot of a row's pair and writes the other; row 0 of the pool is the
// null slot padding rows point at): every slot in [0, N); a real row (read
// slot not 0) shares its read slot with no other real row; for a twin write,
// a real row's write slot is not its own read slot, not 0, and no other row's
// read or write slot other than 0.  One workgroup compares every pair of rows
// (O(B^2): a check for debugging, not for the step's hot loop) and writes the
// number of rows that break a precondition and the first of them.
__global__ __launch_bounds__(1024) void slot_check_kernel(const int32_t *read_slot, const int32_t *write_slot, int B,
                                                          int N, int32_t *result)
{
    __shared__ int nbad, first;
    if (threadIdx.x == 0) {
        nbad = 0;
        first = B;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < B; r += blockDim.x) {
        const int32_t rs = read_slot[r];
        const int32_t ws = write_slot ? write_slot[r] : rs;
        bool bad = rs < 0 || rs >= N || ws < 0 || ws >= N;
        if (!bad && rs != 0) {
            if (write_slot && (ws == rs || ws == 0))
                bad = true;
            for (int j = 0; j < B && !bad; ++j) {
                if (j == r)
                    continue;
                const int32_t rj = read_slot[j];
                const int32_t wj = write_slot ? write_slot[j] : rj;
                if (rj != 0 && rj == rs)
                    bad = true;
                if (write_slot && ((rj != 0 && rj == ws) || (wj != 0 && (wj == ws || wj == rs))))
                    bad = true;
            }
        }
        if (bad) {
            atomicAdd(&nbad, 1);
            atomicMin(&first, r);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        result[0] = nbad;
        result[1] = nbad ? first : -1;
    }
}

hipError_t launch_slot_check(const int32_t *read_slot, const int32_t *write_slot, int B, int N, int32_t *result,
                             hipStream_t stream)
{
    void *args[] = {&read_slot, &write_slot, &B, &N, &result};
    return hipLaunchKernel(reinterpret_cast<const void *>(&slot_check_kernel), dim3(1), dim3(1024), args, 0, stream);
}

} // namespace gdn
