// Ancestor bitmasks of draft trees on the GPU.
//
// Visibility rule ("Validating the Native Engine", section "The Broader Context": the
// verify kernel applies visibility masking to the draft tree): node i sees itself and the
// nodes on its root-to-node path.  With parents numbered before their children (the order
// a best-first builder pops nodes in, "The Capstone Validation", section "What the Test
// Actually Validated"), the walk i -> parent[i] -> ... strictly decreases and ends at -1.
//
// One workgroup per request, one thread per node.  The request's parent array (N <= 256
// entries) is staged in LDS first, so each step of the walk is an LDS read rather than a
// dependent global load.  A thread keeps its W <= 4 words in registers, walks at most i+1
// steps (each step checks parent < current, so it always terminates) and writes its row
// once.  The work is a few thousand words; the kernel is launch-bound.
#include "kdt_internal.h"

namespace kdt {

template <int W>
__global__ __launch_bounds__(256) void visibility_kernel(const int32_t *__restrict__ parents, int N,
                                                         uint64_t *__restrict__ masks,
                                                         int32_t *__restrict__ dev_status) {
    __shared__ int32_t par[kMaxNodes];
    const int64_t b = blockIdx.x;
    for (int i = threadIdx.x; i < N; i += blockDim.x) par[i] = parents[b * N + i];
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        uint64_t w[W];
#pragma unroll
        for (int k = 0; k < W; k++) w[k] = 0;
        bool ok = true;
        int j = i;
        while (j != -1) {
#pragma unroll
            for (int k = 0; k < W; k++)
                if ((j >> 6) == k) w[k] |= 1ull << (j & 63);
            const int p = par[j];
            if (p < -1 || p >= j) { ok = false; break; }
            j = p;
        }
        uint64_t *row = masks + (b * N + i) * W;
#pragma unroll
        for (int k = 0; k < W; k++) row[k] = ok ? w[k] : 0ull;
        if (!ok && dev_status) atomicOr(dev_status, (int32_t)KDT_DEV_BAD_PARENT);
    }
}

hipError_t launch_visibility(const int32_t *parents, int B, int N, uint64_t *masks,
                             int32_t *dev_status, hipStream_t st) {
    const unsigned grid = (unsigned)B;
    const unsigned block = (unsigned)((N + 63) / 64 * 64);
    const int W = (N + 63) / 64;
    switch (W) {
        case 1: visibility_kernel<1><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        case 2: visibility_kernel<2><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        case 3: visibility_kernel<3><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
        default: visibility_kernel<4><<<grid, block, 0, st>>>(parents, N, masks, dev_status); break;
    }
    return hipGetLastError();
}

}  // namespace kdt
