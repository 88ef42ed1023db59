// Ancestor bitmasks of draft trees on the GPU: the per-request walk, shared by the
// visibility kernel and the fused prepare kernel (masks + plan in one launch).
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
#pragma once
#include "kdt_internal.h"

namespace kdt {

// Masks of request b (N nodes, W words per node) by one workgroup; `par` is LDS for N ints.
template <int W>
__device__ __forceinline__ void visibility_rows(const int32_t *__restrict__ parents, int N,
                                                uint64_t *__restrict__ masks, int32_t *__restrict__ dev_status,
                                                int64_t b, int32_t *par) {
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

}  // namespace kdt
