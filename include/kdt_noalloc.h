/*
 * kdt_noalloc.h -- the allocation-free variant of kdt_tree_verify_attn (include/kdt.h).
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It computes exactly what kdt_tree_verify_attn
 * computes, with the same kernels, arguments, errors and device status, but takes no workspace:
 * the plan and the split partials live in a static device array of KDT_NOALLOC_SCRATCH_BYTES
 * bytes inside libkdt, one per device, held from the first call on that device until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or allocating library call).
 *
 *  - A batch whose workspace (kdt_tree_verify_workspace_size) exceeds the array is rejected
 *    with KDT_ERR_WORKSPACE before anything is enqueued; use kdt_tree_verify_attn with a
 *    workspace of that size instead.  On a 256-CU MI355X the measured workloads fit: a 64-node
 *    tree over 4096 tokens needs 48.3 MiB, a 16-node chain or a 256-node chain over 32768
 *    tokens 48.3 MiB, a one-node decode over 32768 tokens 24.1 MiB, batches that fill the GPU
 *    without splitting keys well under 1 MiB.  The largest one-request need with 64 heads is
 *    71.8 MiB (254 nodes, keys split in three), which is rejected.
 *  - Every call on one device uses that device's array: calls that overlap on one device (on
 *    two streams, or from two threads without ordering) race and give wrong results.  Calls
 *    ordered on one stream are safe; nothing in the array has to start at zero.
 *  - The first call on a device looks the array's address up (hipGetSymbolAddress); a failure
 *    there returns KDT_ERR_HIP.
 */
#ifndef KDT_NOALLOC_H_
#define KDT_NOALLOC_H_

#include "kdt.h"

#ifdef __cplusplus
extern "C" {
#endif

#define KDT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)   /* 64 MiB per device */

int kdt_tree_verify_attn_noalloc(const void *q_lat, const void *q_rope, const void *ckv_cache,
                                 const void *krope_cache, const void *tree_ckv, const void *tree_krope,
                                 const uint64_t *bitmask, const int32_t *cache_lens, float scale, float *out,
                                 const kdt_verify_desc *desc, int32_t *dev_status, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KDT_NOALLOC_H_ */
