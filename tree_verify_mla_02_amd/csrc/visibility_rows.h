// Ancestor bitmasks of draft trees on the GPU: the per-request builder, shared by the
// visibility kernel and the fused prepare kernel (masks + plan in one launch).
//
// Visibility rule ("Validating the Native Engine", section "The Broader Context": the
// verify kernel applies visibility masking to the draft tree): node i sees itself and the
// nodes on its root-to-node path.  With parents numbered before their children (the order
// a best-first builder pops nodes in, "The Capstone Validation", section "What the Test
// Actually Validated"), the path i -> parent[i] -> ... strictly decreases and ends at -1.
//
// One workgroup per request, one thread per node (the block has at least N threads).  A walk
// of the path costs one dependent LDS read per ancestor, up to N = 256 of them on a chain, so
// the masks are built by pointer jumping instead: node i keeps the mask of the path segment it
// has covered and a jump to the first ancestor past it; each round ORs in the mask of the node
// it jumps to and takes that node's jump, doubling the covered length, so ceil(log2 N) rounds
// (at most 8) cover every path.  A parent link outside [-1, j-1] ends the path at node j and
// marks j bad; badness spreads along the jumps like the mask bits, and a row whose path meets
// a bad node is written as zeros with KDT_DEV_BAD_PARENT raised -- exactly the rows a walk that
// stops at the first bad link would reject.
#pragma once
#include "kdt_internal.h"

namespace kdt {

struct VisLds {
    uint64_t msk[kMaxNodes][4];
    int32_t jmp[kMaxNodes];
    int32_t bad[kMaxNodes];
};

// Masks of request b (N <= blockDim.x nodes, W words per node) by one workgroup.
template <int W>
__device__ __forceinline__ void visibility_rows(const int32_t *__restrict__ parents, int N,
                                                uint64_t *__restrict__ masks, int32_t *__restrict__ dev_status,
                                                int64_t b, VisLds &L) {
    const int i = threadIdx.x;
    const bool node = i < N;
    uint64_t w[W];
#pragma unroll
    for (int k = 0; k < W; k++) w[k] = (i >> 6) == k ? 1ull << (i & 63) : 0ull;
    int jmp = -1, bad = 0;
    if (node) {
        const int p = parents[b * N + i];
        bad = p < -1 || p >= i;
        jmp = bad ? -1 : p;
#pragma unroll
        for (int k = 0; k < W; k++) L.msk[i][k] = w[k];
        L.jmp[i] = jmp;
        L.bad[i] = bad;
    }
    // a round while some node still has an ancestor beyond its covered segment
    while (__syncthreads_or(jmp >= 0)) {
        int nj = -1, nb = 0;
        uint64_t add[W];
#pragma unroll
        for (int k = 0; k < W; k++) add[k] = 0;
        if (jmp >= 0) {
#pragma unroll
            for (int k = 0; k < W; k++) add[k] = L.msk[jmp][k];
            nj = L.jmp[jmp];
            nb = L.bad[jmp];
        }
        __syncthreads();                    // every read of this round before any write
        if (jmp >= 0) {
#pragma unroll
            for (int k = 0; k < W; k++) w[k] |= add[k];
            bad |= nb;
            jmp = nj;
#pragma unroll
            for (int k = 0; k < W; k++) L.msk[i][k] = w[k];
            L.jmp[i] = jmp;
            L.bad[i] = bad;
        }
    }
    if (node) {
        uint64_t *row = masks + (b * N + i) * W;
#pragma unroll
        for (int k = 0; k < W; k++) row[k] = bad ? 0ull : w[k];
        if (bad && dev_status) atomicOr(dev_status, (int32_t)KDT_DEV_BAD_PARENT);
    }
}

}  // namespace kdt
