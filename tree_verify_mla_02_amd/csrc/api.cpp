// C ABI of libkdt: argument validation, launch geometry and dispatch.
//
// Every entry point checks what the host can see (pointers, sizes, alignment, workspace),
// then enqueues kernels on the caller's stream and returns without synchronising.  No
// exception crosses the ABI; errors are a kdt_status plus a thread-local message.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kdt_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local int g_status = KDT_OK;

int fail(int code, const char *fmt, ...) {
    g_status = code;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    g_status = KDT_OK;
    return KDT_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(KDT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, cached per device id.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int current_cus(int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KDT_ERR_HIP, "device id %d out of range", dev);
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        if (n <= 0) n = 1;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return KDT_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elem_size(int dtype) { return dtype == KDT_BF16 ? 2 : 4; }

int check_desc(const kdt_verify_desc *d) {
    if (!d) return fail(KDT_ERR_INVALID_ARG, "desc is NULL");
    if (d->batch < 1) return fail(KDT_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
    if (d->num_nodes < 1 || d->num_nodes > kdt::kMaxNodes)
        return fail(KDT_ERR_UNSUPPORTED, "num_nodes must be in [1, %d] (got %d)", kdt::kMaxNodes, d->num_nodes);
    if (d->num_heads < 1) return fail(KDT_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", d->num_heads);
    if (d->dtype != KDT_BF16 && d->dtype != KDT_F32) return fail(KDT_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
    const bool kimi = d->d_latent == 512 && d->d_rope == 64 && d->dtype == KDT_BF16;
    const bool tiny = d->d_latent == 64 && d->d_rope == 16;
    if (!kimi && !tiny)
        return fail(KDT_ERR_UNSUPPORTED,
                    "(d_latent, d_rope, dtype) = (%d, %d, %s) is not built; built: (512, 64, bf16), (64, 16, bf16), "
                    "(64, 16, f32)",
                    d->d_latent, d->d_rope, d->dtype == KDT_BF16 ? "bf16" : "f32");
    if (d->max_cache_len < 0 || d->total_cache_len < 0)
        return fail(KDT_ERR_INVALID_ARG, "cache length bounds must be >= 0");
    if (d->max_cache_len > (int64_t)INT32_MAX) return fail(KDT_ERR_INVALID_ARG, "max_cache_len exceeds int32");
    // 32-bit key arithmetic of the plan: a split count is (L + tree places + chunk - 1) / chunk
    if (d->max_cache_len > ((int64_t)1 << 30))
        return fail(KDT_ERR_UNSUPPORTED, "max_cache_len above 2^30 keys is not supported");
    const int64_t epc = 16 / elem_size(d->dtype);
    const struct { int64_t stride; int width; const char *name; } s[] = {
        {d->q_lat_stride, d->d_latent, "q_lat_stride"},   {d->q_rope_stride, d->d_rope, "q_rope_stride"},
        {d->ckv_stride, d->d_latent, "ckv_stride"},       {d->krope_stride, d->d_rope, "krope_stride"},
        {d->tree_ckv_stride, d->d_latent, "tree_ckv_stride"}, {d->tree_krope_stride, d->d_rope, "tree_krope_stride"},
    };
    for (const auto &x : s) {
        if (x.stride < x.width) return fail(KDT_ERR_INVALID_ARG, "%s = %lld is below the row width %d", x.name,
                                            (long long)x.stride, x.width);
        // tile addressing uses 32-bit offsets over 64 rows
        if (x.stride > (int64_t)(INT32_MAX / 128) / elem_size(d->dtype))
            return fail(KDT_ERR_UNSUPPORTED, "%s = %lld is too large (row strides up to %d bytes)", x.name,
                        (long long)x.stride, INT32_MAX / 128);
        if (x.stride % epc) return fail(KDT_ERR_MISALIGNED, "%s = %lld is not a multiple of %lld elements (16 bytes)",
                                        x.name, (long long)x.stride, (long long)epc);
    }
    return KDT_OK;
}

int geometry_for(const kdt_verify_desc *d, kdt::Geometry *g) {
    int rc = check_desc(d);
    if (rc) return rc;
    int cus = 0;
    rc = current_cus(&cus);
    if (rc) return rc;
    if (!kdt::make_geometry(*d, cus, g)) return fail(KDT_ERR_INVALID_ARG, "batch too large for one launch");
    return KDT_OK;
}

int check_ws(const kdt::Geometry &g, const void *ws, size_t bytes) {
    if (!ws) return fail(KDT_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)ws & 255u) return fail(KDT_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if (bytes < g.total_bytes)
        return fail(KDT_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", bytes, g.total_bytes);
    return KDT_OK;
}

kdt::AttnArgs make_args(const kdt_verify_desc &d, const kdt::Geometry &g, void *ws) {
    char *w = (char *)ws;
    kdt::AttnArgs a{};
    a.q_lat_stride = d.q_lat_stride;
    a.q_rope_stride = d.q_rope_stride;
    a.ckv_stride = d.ckv_stride;
    a.krope_stride = d.krope_stride;
    a.tckv_stride = d.tree_ckv_stride;
    a.tkrope_stride = d.tree_krope_stride;
    a.B = d.batch;
    a.N = d.num_nodes;
    a.H = d.num_heads;
    a.W = g.mask_words;
    a.R = g.rows;
    a.RT = g.layout_tiles;
    a.tile_rows = g.tile_rows;
    a.S = g.nsplit;
    a.chunk = g.chunk;
    a.tree_keys = g.tree_keys;
    a.hdr = (const kdt::WsHeader *)(w + g.off_header);
    a.offsets = (const int64_t *)(w + g.off_offsets);
    a.lens = (const int32_t *)(w + g.off_lens);
    a.units = (const kdt::Unit *)(w + g.off_units);
    a.part_ml = g.off_ml ? (float2 *)(w + g.off_ml) : nullptr;
    a.part_o = g.off_o ? (uint32_t *)(w + g.off_o) : nullptr;
    return a;
}

}  // namespace

namespace kdt {

int set_error(int code, const char *msg) { return fail(code, "%s", msg); }

bool make_geometry(const kdt_verify_desc &d, int num_cus, Geometry *g) {
    Geometry x{};
    x.rows = (int64_t)d.num_nodes * d.num_heads;
    // 64-row workgroups (bf16, d = 512 + 64 only) when 128-row ones would not fill the GPU:
    // twice the workgroups for the same keys, each wave working on one 32-key block of every
    // tile.  For requests of at most 512 rows (a decode step, small trees) 128-row tiles would
    // be half empty.  Larger requests (up to 8192 rows) take them over short caches (at most
    // 8192 keys), where the key split that fills the GPU makes partials that are large next to
    // the key work: halving the split count halves the partials written and merged, which
    // outweighs the 64-row kernel's less efficient tile loop (the Kimi shape, 4096 rows over
    // 4096 keys: about 5 % less time per step; over 32768 keys, the chain shape, it does not pay).
    const int64_t rt128 = (x.rows + kRowsPerTile - 1) / kRowsPerTile;
    const bool small = d.dtype == KDT_BF16 && d.d_latent == 512 && d.d_rope == 64 &&
                       (x.rows <= 512 || (x.rows <= 8192 && d.max_cache_len <= 8192)) &&
                       (int64_t)d.batch * rt128 < num_cus;
    x.tile_rows = small ? kRowsPerTile / 2 : kRowsPerTile;
    const int64_t rt = (x.rows + x.tile_rows - 1) / x.tile_rows;
    if (rt > (1 << 30)) return false;
    x.row_tiles = (int)rt;
    x.layout_tiles = (int)rt128;
    x.mask_words = (d.num_nodes + 63) / 64;
    const int64_t units0 = (int64_t)d.batch * rt;
    const int64_t maxL = d.max_cache_len;
    // Split the keys only when the batch alone cannot fill the GPU (about two workgroups per
    // CU); keep every split at least kMinChunk keys so partials stay small next to the key
    // traffic.  Split 0 also does the tree's tiles.  A tree of more than one 64-key tile takes
    // Tf = tree_span(N) places in the split range, so that split 0 does no more tiles than the
    // others (a 256-node prefill chunk over 4096 keys: 34 tiles on the longest split against 36,
    // 6 % less time).  A one-tile tree takes none: a place for it measured 1.5-2.7 % slower on
    // the Kimi, 16-node chain and 7-node shapes (2 % faster on a one-node decode step).
    const int64_t T = d.num_nodes > kKeysPerTile ? tree_span(d.num_nodes) : 0;
    const int64_t Lv = maxL + T;
    int64_t S = 1;
    if (units0 < 2 * (int64_t)num_cus && maxL > kMinChunk) {
        const int64_t want = ((int64_t)num_cus + units0 - 1) / units0;
        const int64_t cap = (Lv + kMinChunk - 1) / kMinChunk;
        S = want < cap ? want : cap;
        if (S < 1) S = 1;
    }
    int64_t chunk = Lv > 0 ? (Lv + S - 1) / S : kKeysPerTile;
    chunk = (chunk + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile;
    if (chunk < kKeysPerTile) chunk = kKeysPerTile;
    if (chunk < T) chunk = T;                 // the tree's places fit in split 0
    S = Lv > 0 ? (Lv + chunk - 1) / chunk : 1;
    if (S < 1) S = 1;
    x.nsplit = (int)S;
    x.chunk = chunk;
    x.tree_keys = (int)T;
    // Units are dealt to the 8 XCD lanes of the grid in groups of bt row tiles x bs splits of
    // one request; the row tiles of a group share its splits' keys through one L2, its splits
    // share the row tiles' queries.  By default a group is one split with all RT row tiles.
    // A request with many row tiles and splits (the Kimi shape: 32 x 8) would then have every
    // XCD fetch all of its queries at once when the kernel starts; blocks of RT/4 row tiles x
    // 4 splits cut that burst to a quarter for twice the key traffic, which measured faster
    // (56.8 vs 60.5 us there; 16 x 2 blocks: 57.7 us).  On 64-row tiles (the Kimi shape there
    // is 64 x 4) a query tile is half as large, and blocks of 16 row tiles x 2 splits read a
    // third less from beyond L2 than 8 x 4 (29.0 against 43.5 MB per launch) in the same time;
    // 32 x 1 reads as little but measured 1.6 us slower (the query burst again).
    x.bs = (S >= 4 && rt >= 16) ? (x.tile_rows == kRowsPerTile ? 4 : 2) : 1;
    x.bt = (int)(x.bs > 1 ? (rt + 3) / 4 : rt);
    // A group runs on one XCD, so fewer groups than XCDs would leave XCDs idle (one request
    // of 128 row tiles with 2 splits would run on 2 of the 8): halve the row-tile blocks until
    // every XCD has a group.
    auto ngroups = [&]() { return (int64_t)d.batch * ((rt + x.bt - 1) / x.bt) * ((S + x.bs - 1) / x.bs); };
    while (ngroups() < kXcds && x.bt > 1) x.bt = (x.bt + 1) / 2;
    x.groups = ngroups();
    const int64_t groups = x.groups;
    x.units = (groups + 7) / 8 * 8 * ((int64_t)x.bt * x.bs);
    if (x.units > INT32_MAX) return false;
    const int64_t B = d.batch;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, 256);
        return o;
    };
    x.off_header = take(sizeof(WsHeader));
    x.off_offsets = take(8 * B);
    x.off_lens = take(4 * B);
    x.off_units = take(sizeof(kdt::Unit) * (size_t)x.units);
    if (S > 1) {
        x.off_ml = take(8 * (size_t)B * S * x.rows);
        // whole 128-row tiles; 3 words per 4 values (24-bit) for bf16, 4 for fp32
        x.off_o = take((size_t)partial_words(d.dtype) * B * S * rt128 * kRowsPerTile * d.d_latent);
    } else {
        x.off_ml = x.off_o = 0;
    }
    x.total_bytes = off;
    *g = x;
    return true;
}

}  // namespace kdt

extern "C" {

int kdt_version(void) { return KDT_VERSION; }

const char *kdt_last_error(void) { return g_err; }

int kdt_last_status(void) { return g_status; }

const char *kdt_status_string(int status) {
    switch (status) {
        case KDT_OK: return "KDT_OK";
        case KDT_ERR_INVALID_ARG: return "KDT_ERR_INVALID_ARG";
        case KDT_ERR_UNSUPPORTED: return "KDT_ERR_UNSUPPORTED";
        case KDT_ERR_MISALIGNED: return "KDT_ERR_MISALIGNED";
        case KDT_ERR_WORKSPACE: return "KDT_ERR_WORKSPACE";
        case KDT_ERR_HIP: return "KDT_ERR_HIP";
        default: return "KDT_ERR_UNKNOWN";
    }
}

int kdt_build_visibility(const int32_t *parents, int32_t batch, int32_t num_nodes, uint64_t *bitmask,
                         int32_t *dev_status, void *stream) {
    if (!parents || !bitmask) return fail(KDT_ERR_INVALID_ARG, "parents and bitmask must not be NULL");
    if (batch < 1) return fail(KDT_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (num_nodes < 1 || num_nodes > kdt::kMaxNodes)
        return fail(KDT_ERR_UNSUPPORTED, "num_nodes must be in [1, %d] (got %d)", kdt::kMaxNodes, num_nodes);
    if (((uintptr_t)parents & 3u) || ((uintptr_t)bitmask & 7u))
        return fail(KDT_ERR_MISALIGNED, "parents must be 4-byte and bitmask 8-byte aligned");
    if (batch > INT32_MAX / 2) return fail(KDT_ERR_INVALID_ARG, "batch too large for one launch");
    const hipError_t e = kdt::launch_visibility(parents, batch, num_nodes, bitmask, dev_status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "visibility launch");
    return ok();
}

int kdt_tree_accept(const int32_t *parents, const int32_t *tokens, const int32_t *target_next,
                    const int32_t *root_next, int32_t batch, int32_t num_nodes, int32_t *path, int32_t *accept_len,
                    int32_t *bonus, void *stream) {
    if (!parents || !tokens || !target_next || !root_next || !path || !accept_len || !bonus)
        return fail(KDT_ERR_INVALID_ARG, "no pointer of kdt_tree_accept may be NULL");
    if (batch < 1) return fail(KDT_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (num_nodes < 1 || num_nodes > kdt::kMaxNodes)
        return fail(KDT_ERR_UNSUPPORTED, "num_nodes must be in [1, %d] (got %d)", kdt::kMaxNodes, num_nodes);
    const void *ptrs[] = {parents, tokens, target_next, root_next, path, accept_len, bonus};
    for (const void *q : ptrs)
        if ((uintptr_t)q & 3u) return fail(KDT_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
    if (batch > INT32_MAX / 2) return fail(KDT_ERR_INVALID_ARG, "batch too large for one launch");
    const hipError_t e = kdt::launch_accept(parents, tokens, target_next, root_next, batch, num_nodes, path,
                                            accept_len, bonus, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "accept launch");
    return ok();
}

int kdt_build_tree(const float *logp, const int32_t *cand, int32_t batch, int32_t max_depth, int32_t topk,
                   int32_t num_nodes, int32_t *parents, int32_t *tokens, int32_t *depth, int32_t *rank,
                   void *stream) {
    if (!logp || !cand || !parents) return fail(KDT_ERR_INVALID_ARG, "logp, cand and parents may not be NULL");
    if (batch < 1) return fail(KDT_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (max_depth < 1 || topk < 1) return fail(KDT_ERR_INVALID_ARG, "max_depth and topk must be >= 1");
    if ((int64_t)max_depth * topk > kdt::kMaxTreeTable)
        return fail(KDT_ERR_UNSUPPORTED, "max_depth * topk must be at most %d (got %lld)", kdt::kMaxTreeTable,
                    (long long)max_depth * topk);
    if (num_nodes < 1 || num_nodes > kdt::kMaxNodes)
        return fail(KDT_ERR_UNSUPPORTED, "num_nodes must be in [1, %d] (got %d)", kdt::kMaxNodes, num_nodes);
    const void *ptrs[] = {logp, cand, parents, tokens, depth, rank};
    for (const void *q : ptrs)
        if ((uintptr_t)q & 3u) return fail(KDT_ERR_MISALIGNED, "arrays must be 4-byte aligned");
    if (batch > INT32_MAX / 2) return fail(KDT_ERR_INVALID_ARG, "batch too large for one launch");
    const hipError_t e = kdt::launch_tree_build(logp, cand, batch, max_depth, topk, num_nodes, parents, tokens,
                                                depth, rank, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "tree build launch");
    return ok();
}

int kdt_kv_compact(const void *ckv_cache, const void *krope_cache, const int32_t *cache_lens, const void *tree_ckv,
                   const void *tree_krope, const int32_t *path, const int32_t *accept_len, void *ckv_out,
                   void *krope_out, int32_t *new_lens, int64_t out_capacity_rows, const kdt_verify_desc *desc,
                   int32_t *dev_status, void *stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!ckv_cache || !krope_cache || !cache_lens || !tree_ckv || !tree_krope || !path || !accept_len ||
        !ckv_out || !krope_out || !new_lens)
        return fail(KDT_ERR_INVALID_ARG, "only dev_status of kdt_kv_compact may be NULL");
    if (out_capacity_rows < 0) return fail(KDT_ERR_INVALID_ARG, "out_capacity_rows must be >= 0");
    const void *rows[] = {ckv_cache, krope_cache, tree_ckv, tree_krope, ckv_out, krope_out};
    for (const void *q : rows)
        if (!aligned16(q)) return fail(KDT_ERR_MISALIGNED, "row pointers must be 16-byte aligned");
    const void *ints[] = {cache_lens, path, accept_len, new_lens};
    for (const void *q : ints)
        if ((uintptr_t)q & 3u) return fail(KDT_ERR_MISALIGNED, "int32 arrays must be 4-byte aligned");
    const bool lat_in_place = ckv_out == ckv_cache, rope_in_place = krope_out == krope_cache;
    if (lat_in_place != rope_in_place)
        return fail(KDT_ERR_INVALID_ARG, "compaction is in place for both parts or for neither");
    if (lat_in_place && desc->batch != 1)
        return fail(KDT_ERR_INVALID_ARG, "in-place compaction needs batch 1 (later requests would move)");
    const int64_t rows_max = desc->max_cache_len + desc->num_nodes;
    if ((rows_max + 31) / 32 > 65535) return fail(KDT_ERR_UNSUPPORTED, "max_cache_len too large for one launch");
    const hipError_t e = kdt::launch_compact(ckv_cache, krope_cache, cache_lens, tree_ckv, tree_krope, path,
                                             accept_len, ckv_out, krope_out, new_lens, out_capacity_rows, *desc,
                                             dev_status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "compaction launch");
    return ok();
}

size_t kdt_tree_verify_workspace_size(const kdt_verify_desc *desc) {
    kdt::Geometry g;
    if (geometry_for(desc, &g)) return 0;
    ok();
    return g.total_bytes;
}

int kdt_tree_verify_num_splits(const kdt_verify_desc *desc) {
    kdt::Geometry g;
    if (geometry_for(desc, &g)) return -1;
    ok();
    return g.nsplit;
}

int kdt_tree_verify_plan(const int32_t *cache_lens, const kdt_verify_desc *desc, void *workspace,
                         size_t workspace_bytes, int32_t *dev_status, void *stream) {
    kdt::Geometry g;
    int rc = geometry_for(desc, &g);
    if (rc) return rc;
    if (!cache_lens) return fail(KDT_ERR_INVALID_ARG, "cache_lens is NULL");
    if ((uintptr_t)cache_lens & 3u) return fail(KDT_ERR_MISALIGNED, "cache_lens must be 4-byte aligned");
    rc = check_ws(g, workspace, workspace_bytes);
    if (rc) return rc;
    const hipError_t e = kdt::launch_plan(cache_lens, *desc, g, workspace, dev_status, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return ok();
}

int kdt_tree_verify_prepare(const int32_t *parents, uint64_t *bitmask, const int32_t *cache_lens,
                            const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                            int32_t *dev_status, void *stream) {
    if (!parents || !bitmask || !cache_lens)
        return fail(KDT_ERR_INVALID_ARG, "parents, bitmask and cache_lens must not be NULL");
    if (((uintptr_t)parents & 3u) || ((uintptr_t)bitmask & 7u) || ((uintptr_t)cache_lens & 3u))
        return fail(KDT_ERR_MISALIGNED, "parents and cache_lens must be 4-byte and bitmask 8-byte aligned");
    kdt::Geometry g;
    int rc = geometry_for(desc, &g);
    if (rc) return rc;
    if (desc->batch > INT32_MAX / 2) return fail(KDT_ERR_INVALID_ARG, "batch too large for one launch");
    rc = check_ws(g, workspace, workspace_bytes);
    if (rc) return rc;
    const hipError_t e = kdt::launch_prepare(parents, bitmask, cache_lens, *desc, g, workspace, dev_status,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prepare launch");
    return ok();
}

int kdt_tree_verify_attend(const void *q_lat, const void *q_rope, const void *ckv_cache, const void *krope_cache,
                           const void *tree_ckv, const void *tree_krope, const uint64_t *bitmask, float scale,
                           float *out, const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                           void *stream) {
    kdt::Geometry g;
    int rc = geometry_for(desc, &g);
    if (rc) return rc;
    const void *ptrs[] = {q_lat, q_rope, ckv_cache, krope_cache, tree_ckv, tree_krope, bitmask, out};
    const char *names[] = {"q_lat", "q_rope", "ckv_cache", "krope_cache", "tree_ckv", "tree_krope", "bitmask", "out"};
    for (int k = 0; k < 8; k++) {
        // the cache pointers may be NULL only when there is no committed row at all
        if (!ptrs[k] && !((k == 2 || k == 3) && desc->total_cache_len == 0))
            return fail(KDT_ERR_INVALID_ARG, "%s is NULL", names[k]);
        if (!aligned16(ptrs[k])) return fail(KDT_ERR_MISALIGNED, "%s is not 16-byte aligned", names[k]);
    }
    if (!std::isfinite(scale)) return fail(KDT_ERR_INVALID_ARG, "scale must be finite");
    rc = check_ws(g, workspace, workspace_bytes);
    if (rc) return rc;
    kdt::AttnArgs a = make_args(*desc, g, workspace);
    a.q_lat = q_lat;
    a.q_rope = q_rope;
    a.ckv = ckv_cache;
    a.krope = krope_cache;
    a.tckv = tree_ckv;
    a.tkrope = tree_krope;
    a.masks = bitmask;
    a.out = out;
    a.scale_log2 = scale * 1.4426950408889634f;
    const hipError_t e = kdt::launch_attend(a, desc->d_latent, desc->d_rope, desc->dtype, g.units, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

int kdt_tree_verify_combine(float *out, const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                            void *stream) {
    kdt::Geometry g;
    int rc = geometry_for(desc, &g);
    if (rc) return rc;
    if (!out) return fail(KDT_ERR_INVALID_ARG, "out is NULL");
    if (!aligned16(out)) return fail(KDT_ERR_MISALIGNED, "out is not 16-byte aligned");
    rc = check_ws(g, workspace, workspace_bytes);
    if (rc) return rc;
    if (g.nsplit <= 1) return ok();
    kdt::AttnArgs a = make_args(*desc, g, workspace);
    a.out = out;
    const hipError_t e = kdt::launch_combine(a, desc->d_latent, desc->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

int kdt_tree_verify_prepare_attend(const int32_t *parents, uint64_t *bitmask, const int32_t *cache_lens,
                                   const void *q_lat, const void *q_rope, const void *ckv_cache,
                                   const void *krope_cache, const void *tree_ckv, const void *tree_krope, float scale,
                                   float *out, const kdt_verify_desc *desc, void *workspace, size_t workspace_bytes,
                                   int32_t *dev_status, void *stream) {
    kdt::Geometry g;
    int rc = geometry_for(desc, &g);
    if (rc) return rc;
    if (!kdt::fused_supported(*desc, g)) {
        rc = kdt_tree_verify_prepare(parents, bitmask, cache_lens, desc, workspace, workspace_bytes, dev_status,
                                     stream);
        if (rc) return rc;
        return kdt_tree_verify_attend(q_lat, q_rope, ckv_cache, krope_cache, tree_ckv, tree_krope, bitmask, scale,
                                      out, desc, workspace, workspace_bytes, stream);
    }
    // the checks of kdt_tree_verify_prepare and kdt_tree_verify_attend
    if (!parents || !bitmask || !cache_lens)
        return fail(KDT_ERR_INVALID_ARG, "parents, bitmask and cache_lens must not be NULL");
    if (((uintptr_t)parents & 3u) || ((uintptr_t)bitmask & 7u) || ((uintptr_t)cache_lens & 3u))
        return fail(KDT_ERR_MISALIGNED, "parents and cache_lens must be 4-byte and bitmask 8-byte aligned");
    const void *ptrs[] = {q_lat, q_rope, ckv_cache, krope_cache, tree_ckv, tree_krope, out};
    const char *names[] = {"q_lat", "q_rope", "ckv_cache", "krope_cache", "tree_ckv", "tree_krope", "out"};
    for (int k = 0; k < 7; k++) {
        if (!ptrs[k] && !((k == 2 || k == 3) && desc->total_cache_len == 0))
            return fail(KDT_ERR_INVALID_ARG, "%s is NULL", names[k]);
        if (!aligned16(ptrs[k])) return fail(KDT_ERR_MISALIGNED, "%s is not 16-byte aligned", names[k]);
    }
    if (!std::isfinite(scale)) return fail(KDT_ERR_INVALID_ARG, "scale must be finite");
    rc = check_ws(g, workspace, workspace_bytes);
    if (rc) return rc;
    kdt::AttnArgs a = make_args(*desc, g, workspace);
    a.q_lat = q_lat;
    a.q_rope = q_rope;
    a.ckv = ckv_cache;
    a.krope = krope_cache;
    a.tckv = tree_ckv;
    a.tkrope = tree_krope;
    a.masks = bitmask;
    a.out = out;
    a.scale_log2 = scale * 1.4426950408889634f;
    const hipError_t e = kdt::launch_attend_fused(a, *desc, g, parents, bitmask, cache_lens, workspace, dev_status,
                                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prepare + attention launch");
    return ok();
}

int kdt_tree_verify_prepare_attend_launches(const kdt_verify_desc *desc) {
    kdt::Geometry g;
    if (geometry_for(desc, &g)) return -1;
    ok();
    return kdt::fused_supported(*desc, g) ? 1 : 2;
}

int kdt_tree_verify_attn(const void *q_lat, const void *q_rope, const void *ckv_cache, const void *krope_cache,
                         const void *tree_ckv, const void *tree_krope, const uint64_t *bitmask,
                         const int32_t *cache_lens, float scale, float *out, const kdt_verify_desc *desc,
                         void *workspace, size_t workspace_bytes, int32_t *dev_status, void *stream) {
    int rc = kdt_tree_verify_plan(cache_lens, desc, workspace, workspace_bytes, dev_status, stream);
    if (rc) return rc;
    rc = kdt_tree_verify_attend(q_lat, q_rope, ckv_cache, krope_cache, tree_ckv, tree_krope, bitmask, scale, out,
                                desc, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return kdt_tree_verify_combine(out, desc, workspace, workspace_bytes, stream);
}

}  // extern "C"
