// Greedy tree-accept and post-verify KV compaction: the two steps that close a verify pass.
//
// The engine ends each verify pass with a greedy tree-accept kernel and commits the accepted
// nodes' KV with a post-verify compaction ("Validating the Native Engine", section "The
// Broader Context"); accepted tokens are committed, rejected ones discarded, and the
// target's prediction at the final accepted node is a bonus token ("The Capstone
// Validation", sections "Context and Motivation" and "What the Test Actually Validated").
//
// Acceptance walks the tree from the committed context: a node is accepted when its token
// equals the target's greedy token at its parent's position (root_next for depth 1), then the
// walk continues from it.  Siblings of a well-formed tree carry distinct tokens; otherwise
// the lowest-index match wins.  Children are looked for only above the current node (parents
// come before children), which also bounds the walk by N steps.
#include "kdt_internal.h"

namespace kdt {

// One wave per request.  The request's arrays go to LDS; each step of the walk is one ballot
// per 64 nodes over "parent == cur and token == want and j > cur", the lowest set lane wins.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *__restrict__ parents,
                                                    const int32_t *__restrict__ tokens,
                                                    const int32_t *__restrict__ target_next,
                                                    const int32_t *__restrict__ root_next, int N,
                                                    int32_t *__restrict__ path, int32_t *__restrict__ accept_len,
                                                    int32_t *__restrict__ bonus) {
    __shared__ int32_t s_par[kMaxNodes], s_tok[kMaxNodes], s_nxt[kMaxNodes];
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    for (int i = lane; i < N; i += 64) {
        s_par[i] = parents[b * N + i];
        s_tok[i] = tokens[b * N + i];
        s_nxt[i] = target_next[b * N + i];
    }
    int want = root_next[b];
    __syncthreads();
    int cur = -1, k = 0;
    while (true) {
        int found = -1;
        for (int j0 = 0; j0 < N; j0 += 64) {
            const int j = j0 + lane;
            const bool hit = j < N && j > cur && s_par[j] == cur && s_tok[j] == want;
            const uint64_t m = __ballot(hit);
            if (m) {
                found = j0 + __builtin_ctzll(m);
                break;
            }
        }
        if (found < 0) break;                 // uniform: every lane saw the same ballot
        if (lane == 0) path[b * N + k] = found;
        k++;
        cur = found;
        want = s_nxt[found];
    }
    for (int i = k + lane; i < N; i += 64) path[b * N + i] = -1;
    if (lane == 0) {
        accept_len[b] = k;
        bonus[b] = want;
    }
}

hipError_t launch_accept(const int32_t *parents, const int32_t *tokens, const int32_t *target_next,
                         const int32_t *root_next, int B, int N, int32_t *path, int32_t *accept_len,
                         int32_t *bonus, hipStream_t st) {
    accept_kernel<<<(unsigned)B, 64, 0, st>>>(parents, tokens, target_next, root_next, N, path, accept_len, bonus);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------ compaction
// New packed cache: request b's committed rows, then its accepted rows in path order, requests
// packed in request order.  Workgroup (b, c) copies rows [32pc, 32p(c + 1)) of request b's
// new range in p passes of 32 rows (p = 1 for small grids, up to 4 for large ones, which
// spreads each workgroup's length scan over more rows).  Each first computes, from all of cache_lens and accept_len, the request's
// old and new offsets and whether the lengths are valid.  A bad length anywhere, or more rows
// than the source bound or the destination capacity, writes nothing; a path entry that names
// no node leaves that request unwritten; both set KDT_DEV_BAD_ACCEPT.  Rows move as 16-byte
// chunks: a wave copies whole rows, so every load and store instruction covers 1 KB of one
// row.
constexpr int kCompactWindow = 32;                 // rows copied per pass of a workgroup
constexpr int kCompactMaxPasses = 4;               // passes per workgroup at most

struct CompactArgs {
    const char *ckv, *krope;             // source rows (element strides below)
    const char *tckv, *tkrope;           // tree rows [B, N]
    char *ockv, *okrope;                 // destination rows, same strides as the source
    const int32_t *lens, *path, *acc;
    int32_t *new_lens, *dev_status;
    int64_t ckv_stride, krope_stride, tckv_stride, tkrope_stride;   // bytes
    int B, N;
    int lat_chunks, rope_chunks;         // 16-byte chunks per row of each part
    int64_t max_len, total_len, capacity;
    int in_place;                        // destination == source (one request): copy appended rows only
    int passes;                          // 32-row passes per workgroup
};

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
    __shared__ int64_t s_red[4][4];
    __shared__ int s_bad_len, s_bad_path;
    const int b = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    if (tid == 0) {
        s_bad_len = 0;
        s_bad_path = 0;
    }
    __syncthreads();
    // over all requests: old rows and accepted rows before b, and in total; any bad length
    int64_t v[4] = {0, 0, 0, 0};
    for (int i = tid; i < a.B; i += blockDim.x) {
        const int64_t L = a.lens[i], A = a.acc[i];
        if (L < 0 || L > a.max_len || A < 0 || A > a.N) s_bad_len = 1;
        const int64_t Lc = L < 0 ? 0 : L, Ac = A < 0 ? 0 : A;
        v[2] += Lc;
        v[3] += Ac;
        if (i < b) {
            v[0] += Lc;
            v[1] += Ac;
        }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) v[k] += __shfl_xor(v[k], d, 64);
        if (lane == 0) s_red[k][wave] = v[k];
    }
    // this request's path entries must name nodes
    const int64_t L = a.lens[b], A = a.acc[b];
    for (int k = tid; k < a.N; k += blockDim.x)
        if (k < A) {
            const int32_t node = a.path[(int64_t)b * a.N + k];
            if (node < 0 || node >= a.N) s_bad_path = 1;
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = s_red[k][0] + s_red[k][1] + s_red[k][2] + s_red[k][3];
    const int64_t old_off = v[0], new_off = v[0] + v[1], tot_old = v[2], tot_new = v[2] + v[3];
    // a bad length anywhere, or too many rows: nothing is written
    if (s_bad_len || tot_old > a.total_len || tot_new > a.capacity) {
        if (b == 0 && c == 0 && tid == 0 && a.dev_status) atomicOr(a.dev_status, (int32_t)KDT_DEV_BAD_ACCEPT);
        return;
    }
    // a bad path entry: this request is not written (neither rows nor its new length)
    if (s_bad_path) {
        if (c == 0 && tid == 0 && a.dev_status) atomicOr(a.dev_status, (int32_t)KDT_DEV_BAD_ACCEPT);
        return;
    }
    if (c == 0 && tid == 0) a.new_lens[b] = (int32_t)(L + A);
    const int cpr = a.lat_chunks + a.rope_chunks;
    for (int pass = 0; pass < a.passes; pass++) {
        const int64_t r0 = ((int64_t)c * a.passes + pass) * kCompactWindow;
        if (r0 >= L + A) break;
        const int64_t r_end = (r0 + kCompactWindow < L + A) ? r0 + kCompactWindow : L + A;
        const int64_t first = a.in_place ? (r0 > L ? r0 : L) : r0;   // in place: committed rows stay
        // Wave w copies rows first + w, first + w + 4, ... (kWaveRows of them at most); lane l
        // moves 16-byte chunks l, l + 64, ... of each row.  All of a wave's loads are issued before
        // its stores, so every lane keeps up to kWaveRows * kChunksPerLane loads in flight.
        constexpr int kWaveRows = kCompactWindow / 4;
        constexpr int kChunksPerLane = 3;                  // rows of at most 192 chunks (3 KB)
        // Row bases are wave-uniform: the path entries of the wave's accepted rows are read
        // before any data load, so the data loads are issued back to back with no wait between.
        const int w = __builtin_amdgcn_readfirstlane(wave);
        const char *sl[kWaveRows], *sr[kWaveRows];
        char *dl[kWaveRows], *dr[kWaveRows];
        bool live[kWaveRows];
        int32_t node[kWaveRows];
    #pragma unroll
        for (int i = 0; i < kWaveRows; i++) {
            const int64_t r = first + w + 4 * i;
            live[i] = r < r_end;
            node[i] = (live[i] && r >= L) ? a.path[(int64_t)b * a.N + (r - L)] : 0;
        }
    #pragma unroll
        for (int i = 0; i < kWaveRows; i++) {
            const int64_t r = first + w + 4 * i;
            const int64_t crow = old_off + r, trow = (int64_t)b * a.N + node[i], drow = new_off + r;
            const bool cached = r < L;
            sl[i] = cached ? a.ckv + crow * a.ckv_stride : a.tckv + trow * a.tckv_stride;
            sr[i] = cached ? a.krope + crow * a.krope_stride : a.tkrope + trow * a.tkrope_stride;
            dl[i] = a.ockv + drow * a.ckv_stride;
            dr[i] = a.okrope + drow * a.krope_stride;
        }
        uint4 x[kWaveRows][kChunksPerLane];
    #pragma unroll
        for (int i = 0; i < kWaveRows; i++)
    #pragma unroll
            for (int j = 0; j < kChunksPerLane; j++) {
                const int ch = lane + 64 * j;
                const bool lat = ch < a.lat_chunks;
                const char *src = lat ? sl[i] + ch * 16 : sr[i] + (ch - a.lat_chunks) * 16;
                x[i][j] = make_uint4(0u, 0u, 0u, 0u);
                if (live[i] && ch < cpr) x[i][j] = *(const uint4 *)src;
            }
    #pragma unroll
        for (int i = 0; i < kWaveRows; i++)
    #pragma unroll
            for (int j = 0; j < kChunksPerLane; j++) {
                const int ch = lane + 64 * j;
                const bool lat = ch < a.lat_chunks;
                char *dst = lat ? dl[i] + ch * 16 : dr[i] + (ch - a.lat_chunks) * 16;
                if (live[i] && ch < cpr) *(uint4 *)dst = x[i][j];
            }
    }
}

hipError_t launch_compact(const void *ckv, const void *krope, const int32_t *cache_lens, const void *tree_ckv,
                          const void *tree_krope, const int32_t *path, const int32_t *accept_len, void *ckv_out,
                          void *krope_out, int32_t *new_lens, int64_t capacity, const kdt_verify_desc &d,
                          int32_t *dev_status, hipStream_t st) {
    const int es = d.dtype == KDT_BF16 ? 2 : 4;
    CompactArgs a;
    a.ckv = (const char *)ckv;
    a.krope = (const char *)krope;
    a.tckv = (const char *)tree_ckv;
    a.tkrope = (const char *)tree_krope;
    a.ockv = (char *)ckv_out;
    a.okrope = (char *)krope_out;
    a.lens = cache_lens;
    a.path = path;
    a.acc = accept_len;
    a.new_lens = new_lens;
    a.dev_status = dev_status;
    a.ckv_stride = d.ckv_stride * es;
    a.krope_stride = d.krope_stride * es;
    a.tckv_stride = d.tree_ckv_stride * es;
    a.tkrope_stride = d.tree_krope_stride * es;
    a.B = d.batch;
    a.N = d.num_nodes;
    a.lat_chunks = d.d_latent * es / 16;
    a.rope_chunks = d.d_rope * es / 16;
    a.max_len = d.max_cache_len;
    a.total_len = d.total_cache_len;
    a.capacity = capacity;
    a.in_place = ckv_out == ckv;
    if (a.lat_chunks + a.rope_chunks > 192) return hipErrorInvalidValue;   // 3 chunks per lane and row
    const int64_t rows_max = d.max_cache_len + d.num_nodes;
    const int64_t windows = (rows_max + kCompactWindow - 1) / kCompactWindow;
    int64_t p = (int64_t)d.batch * windows / 2048;           // keep about 2048 workgroups or more
    a.passes = (int)(p < 1 ? 1 : p > kCompactMaxPasses ? kCompactMaxPasses : p);
    const dim3 grid((unsigned)d.batch, (unsigned)((windows + a.passes - 1) / a.passes));
    compact_kernel<<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace kdt
