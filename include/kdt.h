/*
 * kdt.h -- C ABI of libkdt: tree-verify MLA-absorb attention for AMD MI355X (gfx950).
 *
 * The operation.  A speculative decoder drafts candidate tokens as a tree and the
 * target model verifies every node of that tree in one batched forward pass ("The
 * Capstone Validation: Writing the DDTree Speculative Decode Test", section "Context and
 * Motivation").  Inside that pass the engine runs a tree-verify attention kernel for
 * absorbed MLA, masked by tree visibility ("Validating the Native Engine: The Autoregressive
 * Test Driver for Kimi K2.6 DDTree Inference", section "The Broader Context"): with Multi-head Latent
 * Attention in absorbed form, all heads share one latent KV row per token (a d_latent
 * wide latent plus a d_rope wide rotary key), and every tree node must attend to exactly
 * what an ordinary decode of its own root-to-node path would attend to -- the committed
 * cache of its request, its ancestors and itself, never its siblings or descendants.
 *
 * For request b, node i, head h (row r = i*H + h, node-major), with key set
 * K(b,i) = {committed cache rows of b} U {tree nodes j : bit j of mask[b,i] set}:
 *     s_k          = scale * (q_lat[b,i,h,:] . ckv_k + q_rope[b,i,h,:] . krope_k)
 *     out[b,i,h,:] = sum_k exp(s_k - max s) ckv_k / sum_k exp(s_k - max s)     (fp32)
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library keeps no
 *    reference after the call returns and allocates no device memory; scratch space is
 *    the caller's `workspace`.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = the legacy
 *    default stream).  No call synchronises the host.
 *  - Errors the host can see (null pointers, unsupported sizes, misalignment, a too small
 *    workspace, a failed launch) are returned synchronously as a kdt_status and leave the
 *    outputs untouched; kdt_last_error() then holds a thread-local description.
 *  - Errors that depend on device data (a bad parent index, a cache length above the host
 *    bounds) are OR-ed as KDT_DEV_* bits into *dev_status when dev_status is not NULL.
 *    The caller zeroes *dev_status beforehand.  Masks of rows with a bad parent on their
 *    path are all-zero; when cache lengths are out of bounds the attention calls write
 *    nothing.
 *  - Inputs are assumed finite.  Rows need not be contiguous (strides are in elements),
 *    but every base pointer must be 16-byte aligned and every stride a multiple of
 *    16 bytes / element size.
 *  - No global mutable state besides a per-device cache of the compute-unit count; calls
 *    on different streams may overlap as long as their workspaces differ.
 */
#ifndef KDT_H_
#define KDT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDT_VERSION 1

/* Synchronous return codes. */
typedef enum {
    KDT_OK = 0,
    KDT_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size */
    KDT_ERR_UNSUPPORTED = 2,   /* dims / dtype combination not built, N outside [1, 256],
                                  max_cache_len above 2^30 keys */
    KDT_ERR_MISALIGNED = 3,    /* base pointer not 16-byte aligned or stride not a 16-byte multiple */
    KDT_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than kdt_tree_verify_workspace_size() */
    KDT_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} kdt_status;

/* Device-side error bits, OR-ed into *dev_status. */
enum {
    KDT_DEV_OK = 0,
    KDT_DEV_BAD_PARENT = 1,    /* some parent[b,j] on a walked path is outside [-1, j-1] */
    KDT_DEV_CACHE_LEN = 2,     /* some cache_lens[b] < 0 or > max_cache_len, or their sum > total_cache_len */
    KDT_DEV_BAD_ACCEPT = 4     /* kdt_kv_compact: a length or path entry out of range, or too many rows */
};

/* Element type of q_lat, q_rope and the cache / tree rows; `out` is always fp32. */
typedef enum { KDT_BF16 = 0, KDT_F32 = 1 } kdt_dtype;

/* Shape and layout of one verify batch.  Built combinations (d_latent, d_rope, dtype):
 * (512, 64, BF16) -- the DeepSeekV3 / Kimi MLA head; (64, 16, BF16); (64, 16, F32). */
typedef struct kdt_verify_desc {
    int32_t batch;              /* B >= 1 requests */
    int32_t num_nodes;          /* N in [1, 256] tree nodes per request */
    int32_t num_heads;          /* H >= 1 query heads sharing one latent cache */
    int32_t d_latent;           /* d_c: latent width (value width) */
    int32_t d_rope;             /* d_r: rotary key width */
    int32_t dtype;              /* kdt_dtype */
    int64_t max_cache_len;      /* host bound: every cache_lens[b] <= max_cache_len (at most 2^30) */
    int64_t total_cache_len;    /* rows present in ckv_cache / krope_cache (>= sum cache_lens) */
    int64_t q_lat_stride;       /* elements between consecutive (b,i,h) rows of q_lat  (>= d_c) */
    int64_t q_rope_stride;      /* elements between consecutive (b,i,h) rows of q_rope (>= d_r) */
    int64_t ckv_stride;         /* elements between consecutive cache tokens of ckv_cache   (>= d_c) */
    int64_t krope_stride;       /* elements between consecutive cache tokens of krope_cache (>= d_r) */
    int64_t tree_ckv_stride;    /* elements between consecutive (b,i) rows of tree_ckv   (>= d_c) */
    int64_t tree_krope_stride;  /* elements between consecutive (b,i) rows of tree_krope (>= d_r) */
} kdt_verify_desc;

/*
 * kdt_build_visibility -- ancestor bitmasks of B draft trees (the visibility masking of
 * "Validating the Native Engine", section "The Broader Context").
 *   parents   [B, N] int32, device.  parent[b,i] in [-1, i-1]; -1 = attached to the
 *             committed cache (nodes are numbered parents-first, as a best-first builder
 *             pops them: "The Capstone Validation", section "What the Test Actually
 *             Validated").
 *   bitmask   [B, N, W] uint64, device, W = ceil(N/64).  Bit j%64 of word j/64 of row
 *             (b,i) is set iff node j is i or an ancestor of i.  Bits >= N are 0.
 *   dev_status nullable; KDT_DEV_BAD_PARENT is OR-ed in when a walked parent is invalid
 *             (that row is written as all zeros).
 * N must lie in [1, 256].
 */
int kdt_build_visibility(const int32_t *parents, int32_t batch, int32_t num_nodes,
                         uint64_t *bitmask, int32_t *dev_status, void *stream);

/* Bytes of device workspace kdt_tree_verify_* need for `desc` on the current device
 * (plan, per-request offsets, and split-KV partials when the batch is too small to fill
 * the GPU).  Returns 0 when desc is invalid (see kdt_last_error()).  The pages fix no
 * workspace; it exists because the verify pass of "The Capstone Validation" (section
 * "Broader Significance": verify passes are attention-bound and scale with context length)
 * must spread long caches over the whole GPU. */
size_t kdt_tree_verify_workspace_size(const kdt_verify_desc *desc);

/*
 * kdt_tree_verify_attn -- the whole verify attention: plan + attend + combine.  This is the
 * engine's visibility-masked tree-verify attention for absorbed MLA ("Validating the Native
 * Engine", section "The Broader Context"), applied to the tree of candidates that "The Capstone
 * Validation", section "Context and Motivation", verifies in one batched pass: each node's
 * output is the attention a plain decode of its own root-to-node path would compute (the
 * formula at the top of this file).
 *   q_lat      [B, N, H, d_c] rows at q_lat_stride;  q_rope [B, N, H, d_r] at q_rope_stride.
 *   ckv_cache  [T, d_c], krope_cache [T, d_r]: committed caches of all requests packed in
 *              request order (request b owns rows off_b .. off_b + cache_lens[b] - 1 with
 *              off_b = sum of the earlier lengths).  The two may be views of one [T, 576]
 *              buffer through the strides.
 *   tree_ckv   [B, N, d_c], tree_krope [B, N, d_r]: latent rows of the drafted nodes.
 *   bitmask    [B, N, ceil(N/64)] uint64 from kdt_build_visibility (or equivalent).
 *   cache_lens [B] int32, device; 0 is allowed.
 *   scale      softmax scale applied to the raw dot products.
 *   out        [B, N, H, d_c] fp32, contiguous; must not alias any input.
 *   workspace  >= kdt_tree_verify_workspace_size(desc) bytes, 256-byte aligned.
 * A row with no visible key (possible only with an all-zero mask and L = 0) gets 0.
 */
int kdt_tree_verify_attn(const void *q_lat, const void *q_rope, const void *ckv_cache,
                         const void *krope_cache, const void *tree_ckv, const void *tree_krope,
                         const uint64_t *bitmask, const int32_t *cache_lens, float scale,
                         float *out, const kdt_verify_desc *desc, void *workspace,
                         size_t workspace_bytes, int32_t *dev_status, void *stream);

/*
 * The same operation in three stream-ordered stages, for callers that reuse one plan for
 * every layer of a verify pass (the cache lengths do not change between layers: the verify
 * pass of "The Capstone Validation", section "Context and Motivation", runs every layer of the
 * target over the same drafted tree and the same committed cache).
 *   kdt_tree_verify_plan    validates cache_lens, builds per-request offsets and the
 *                           longest-first work list in `workspace`.
 *   kdt_tree_verify_attend  the attention kernel; needs a plan for the same desc in
 *                           `workspace`.  Writes `out` directly when no request is split,
 *                           else split partials into the workspace.
 *   kdt_tree_verify_combine merges split partials into `out` (does nothing when the plan
 *                           has no split).
 */
int kdt_tree_verify_plan(const int32_t *cache_lens, const kdt_verify_desc *desc, void *workspace,
                         size_t workspace_bytes, int32_t *dev_status, void *stream);
int kdt_tree_verify_attend(const void *q_lat, const void *q_rope, const void *ckv_cache,
                           const void *krope_cache, const void *tree_ckv, const void *tree_krope,
                           const uint64_t *bitmask, float scale, float *out,
                           const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                           void *stream);
int kdt_tree_verify_combine(float *out, const kdt_verify_desc *desc, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * kdt_tree_verify_prepare -- kdt_build_visibility and kdt_tree_verify_plan in one launch
 * (the two are independent; a verify step needs both before the attention: the visibility
 * masks of "Validating the Native Engine", section "The Broader Context", and the ragged work
 * list of the batch).
 *   parents   [B, N] int32, device, with B = desc->batch and N = desc->num_nodes; bitmask
 *             [B, N, ceil(N/64)] uint64 -- exactly as kdt_build_visibility.
 *   cache_lens, workspace, dev_status -- exactly as kdt_tree_verify_plan.
 * Host-side errors are those of the two calls; device-side errors OR the same bits into
 * *dev_status.
 */
int kdt_tree_verify_prepare(const int32_t *parents, uint64_t *bitmask, const int32_t *cache_lens,
                            const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                            int32_t *dev_status, void *stream);

/*
 * kdt_tree_verify_prepare_attend -- kdt_tree_verify_prepare followed by kdt_tree_verify_attend,
 * with their arguments, checks and results (bitmask is written, the workspace holds the plan,
 * out or the split partials hold the attention; kdt_tree_verify_combine follows as after
 * kdt_tree_verify_attend), in one launch where the shape allows.  A verify step needs the
 * visibility masks ("Validating the Native Engine", section "The Broader Context") and the ragged
 * plan before its attention.  For a one-request batch of bf16 512 + 64 inputs
 * (kdt_tree_verify_prepare_attend_launches() == 1) both are made inside the attention launch:
 * each workgroup works out the unit the plan would give its grid slot from cache_lens[0]; on
 * 64-row workgroups (a decode step, small trees, trees of up to 8192 rows over short caches) the
 * workgroups with tree keys walk the root paths of their rows' nodes, on 128-row ones (longer
 * caches, prefill chains) they build all masks by pointer jumping; one workgroup writes bitmask.
 * Other batches run the two stages.
 * Results are bit-identical to the staged calls (the workspace included); a caller that reuses
 * one plan for every layer still uses the staged calls.
 */
int kdt_tree_verify_prepare_attend(const int32_t *parents, uint64_t *bitmask, const int32_t *cache_lens,
                                   const void *q_lat, const void *q_rope, const void *ckv_cache,
                                   const void *krope_cache, const void *tree_ckv, const void *tree_krope, float scale,
                                   float *out, const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                                   int32_t *dev_status, void *stream);
/* Kernel launches kdt_tree_verify_prepare_attend makes for desc: 1 or 2; -1 when desc is invalid
 * (see kdt_last_error()). */
int kdt_tree_verify_prepare_attend_launches(const kdt_verify_desc *desc);

/*
 * kdt_tree_accept -- greedy acceptance closing a verify pass.  Accepted tokens are committed
 * and rejected ones discarded, and the target's prediction at the final accepted node is the
 * bonus token ("The Capstone Validation", sections "Context and Motivation" and "What the
 * Test Actually Validated"); the engine runs a greedy tree-accept kernel ("Validating the
 * Native Engine", section "The Broader Context").
 *   parents     [B, N] int32, device: parent < child, -1 at depth 1 (as kdt_build_visibility).
 *   tokens      [B, N] int32, device: each node's drafted token id.
 *   target_next [B, N] int32, device: the target's greedy token at each node's position.
 *   root_next   [B] int32, device: the target's greedy token after the committed context.
 *   path        [B, N] int32, device, out: accepted node ids in root-to-leaf order, then -1.
 *   accept_len  [B] int32, device, out: number of accepted nodes.
 *   bonus       [B] int32, device, out: the target's token after the last accepted node
 *               (root_next when none is accepted).
 * A node is accepted when its parent is (the committed context at depth 1) and its token is
 * the target's greedy token at the parent's position.  Among children with equal tokens the
 * lowest index is taken; children are looked for only above the parent's index, so a
 * malformed parent array ends the walk rather than looping.  N must lie in [1, 256].
 */
int kdt_tree_accept(const int32_t *parents, const int32_t *tokens, const int32_t *target_next,
                    const int32_t *root_next, int32_t batch, int32_t num_nodes, int32_t *path,
                    int32_t *accept_len, int32_t *bonus, void *stream);

/*
 * kdt_build_tree -- best-first draft-tree construction, the step before verification: the
 * engine's GPU best-first tree builder, which replaced a per-request CPU heap ("Validating the
 * Native Engine", section "The Broader Context").  The drafter gives, per depth and top-k
 * slot, a log probability sorted descending and a token id ("The Capstone Validation",
 * section "What the Test Actually Validated").
 *   logp     [B, D, K] float32, device: row (b, d) holds depth d+1's K log probabilities,
 *            best first.  Must not hold NaN.
 *   cand     [B, D, K] int32, device: the matching token ids.
 *   max_depth D >= 1, topk K >= 1, D * K <= 8192; num_nodes N in [1, 256].
 *   parents  [B, N] int32, device, out: node i's parent (-1 at depth 1); parent < child, ready
 *            for kdt_build_visibility / kdt_tree_verify_prepare.
 *   tokens, depth, rank [B, N] int32, device, out, each nullable: node i's token id, depth
 *            (1-based) and rank within its depth's K slots.
 * A node is a rank path (k_1..k_d) scored by the fp32 sum of its log probabilities, added one
 * depth at a time.  Starting from the depth-1 rank-0 path, each step takes the best frontier
 * path (equal scores: the earliest pushed) as node i, then pushes its next sibling (rank + 1,
 * if below K) and its first child (rank 0 one level deeper, if below D), in that order.  With
 * rows sorted descending the nodes are the N best rank paths, in score order.  A request with
 * fewer than N paths in total (K + K^2 + ... + K^D < N) gets -2 in every output of the rows
 * it cannot fill.  Everything is checked on the host; nothing is written to device status.
 */
int kdt_build_tree(const float *logp, const int32_t *cand, int32_t batch, int32_t max_depth, int32_t topk,
                   int32_t num_nodes, int32_t *parents, int32_t *tokens, int32_t *depth, int32_t *rank,
                   void *stream);

/*
 * kdt_kv_compact -- post-verify compaction of the committed cache ("Validating the Native
 * Engine", section "The Broader Context": a KV cache with post-verify compaction): each
 * request's accepted tree rows are committed right after its committed rows.
 *   ckv_cache, krope_cache, cache_lens: the packed cache exactly as for kdt_tree_verify_attn
 *               (desc gives batch, num_nodes, d_latent, d_rope, dtype, the row strides,
 *               max_cache_len and total_cache_len).
 *   tree_ckv, tree_krope [B, N, d_c], [B, N, d_r] at desc's tree strides.
 *   path, accept_len: as written by kdt_tree_accept.
 *   ckv_out, krope_out: destination rows at the source's strides, room for out_capacity_rows
 *               rows.  Request b's new rows start at the sum of the earlier new lengths: its
 *               committed rows, then its accepted rows in path order.
 *   new_lens    [B] int32, device, out: cache_lens + accept_len.
 * The destination must not overlap an input, except in place (ckv_out == ckv_cache and
 * krope_out == krope_cache) with batch 1, where the committed rows stay and only the
 * accepted rows are written.  Device-side checks: a length outside [0, max_cache_len], an
 * accept_len outside [0, N], more than total_cache_len source rows or more than
 * out_capacity_rows destination rows writes nothing; a path entry that names no node leaves
 * that request (rows and new length) unwritten; both OR KDT_DEV_BAD_ACCEPT into *dev_status.
 */
int kdt_kv_compact(const void *ckv_cache, const void *krope_cache, const int32_t *cache_lens,
                   const void *tree_ckv, const void *tree_krope, const int32_t *path,
                   const int32_t *accept_len, void *ckv_out, void *krope_out, int32_t *new_lens,
                   int64_t out_capacity_rows, const kdt_verify_desc *desc, int32_t *dev_status,
                   void *stream);

/* Number of key splits per request the plan uses for desc on the current device (1 = no
 * split), or -1 for an invalid desc. */
int kdt_tree_verify_num_splits(const kdt_verify_desc *desc);

const char *kdt_status_string(int status);
const char *kdt_last_error(void);   /* thread-local; "" after a successful call */
int kdt_last_status(void);          /* thread-local kdt_status of the last call (KDT_OK after success);
                                       the code behind a 0 from kdt_tree_verify_workspace_size */
int kdt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDT_H_ */
