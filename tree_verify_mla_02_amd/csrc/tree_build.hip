// Best-first draft-tree construction on the GPU: the step right before verification.
//
// The engine builds the draft tree with a GPU best-first builder that replaced a per-request
// CPU heap ("Validating the Native Engine", section "The Broader Context").  The drafter
// gives, for each depth d < D and each of K slots, a log probability (sorted descending per
// depth) and a token id ("The Capstone Validation", section "What the Test Actually
// Validated").  A node is a rank path (k_1..k_d) scored by the sum of its per-depth log
// probabilities.  The frontier starts with the depth-1 rank-0 path; each step takes the best
// frontier entry (equal scores: the one pushed first) as the next node, then pushes its next
// sibling (same prefix, rank + 1, if below K) and its first child (rank 0 one level deeper, if
// below D), in that order.  A path's score is its prefix's score plus one fp32 log
// probability, rounded once per step.
//
// The search is sequential per request, so one wave builds one request.  Frontier entries are
// numbered in push order (entry e = the e-th push; at most 1 + 2N of them) and entry e belongs
// to lane e % 64, slot e / 64.  Each lane keeps its slots' order keys in registers and its own
// best; a pop is a wave arg-max over the 64 lane bests (DPP inside rows of 16 lanes, lane reads
// across rows), so no step touches memory on the way to the next decision.  The order key is
// the score's fp32 pattern mapped to an unsigned integer that sorts like the float (zeroes of
// either sign map to one key); equal keys go to the lower entry number = the earlier push.
#include "kdt_internal.h"

namespace kdt {

constexpr int kTreeSlots = (1 + 2 * kMaxNodes + 63) / 64;   // 9 entries per lane at most

// Unsigned key that orders like the float value (-0 and +0 equal); 0 is below every score.
__device__ __forceinline__ uint32_t order_key(float s) {
    if (s == 0.0f) s = 0.0f;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Reductions over a wave of 64: within each row of 16 lanes by DPP (quad swaps, then row
// rotations by 4 and 8), then across the four rows by lane reads.  Results are uniform.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
    auto op = [](uint32_t a, uint32_t b) { return kMax ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
    v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return op(op(r0, r1), op(r2, r3));
}

struct TreeEntry {          // one frontier entry, in LDS
    float score;            // the path's score
    float base;             // its prefix node's score (0 at depth 1): a next sibling adds to it
    int32_t prefix;         // prefix node index, -1 at depth 1
    int32_t dk;             // depth index d (0-based) << 16 | rank k
};

__global__ __launch_bounds__(64) void tree_build_kernel(const float *__restrict__ logp,
                                                        const int32_t *__restrict__ cand, int D, int K,
                                                        int N, int32_t *__restrict__ parents,
                                                        int32_t *__restrict__ tokens,
                                                        int32_t *__restrict__ depth,
                                                        int32_t *__restrict__ rank) {
    extern __shared__ float s_lp[];                     // [D*K] this request's log probabilities
    __shared__ TreeEntry s_ent[64 * kTreeSlots];
    __shared__ int32_t s_npar[kMaxNodes], s_ndk[kMaxNodes];
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int DK = D * K;
    for (int i = lane; i < DK; i += 64) s_lp[i] = logp[b * DK + i];
    __syncthreads();

    // keys of this lane's entries (entry e lives in lane e % 64, slot e / 64), as scalars so
    // that they stay in registers; 0 = no entry
    uint32_t k0 = 0, k1 = 0, k2 = 0, k3 = 0, k4 = 0, k5 = 0, k6 = 0, k7 = 0, k8 = 0;
    static_assert(kTreeSlots == 9, "one register per slot");
    uint32_t best_key = 0u;          // this lane's best entry key and slot
    int best_slot = 0;
    int count = 0;                   // entries pushed so far (uniform)

#define KDT_SET_SLOT(slot, v)                                                                   \
    do {                                                                                        \
        const int s_ = (slot);                                                                  \
        const uint32_t v_ = (v);                                                                \
        k0 = s_ == 0 ? v_ : k0; k1 = s_ == 1 ? v_ : k1; k2 = s_ == 2 ? v_ : k2;                 \
        k3 = s_ == 3 ? v_ : k3; k4 = s_ == 4 ? v_ : k4; k5 = s_ == 5 ? v_ : k5;                 \
        k6 = s_ == 6 ? v_ : k6; k7 = s_ == 7 ? v_ : k7; k8 = s_ == 8 ? v_ : k8;                 \
    } while (0)
    // push entry number `count` (uniform); its owner lane records the key
#define KDT_PUSH(score_, base_, prefix_, d_, k_)                                                \
    do {                                                                                        \
        const float sc_ = (score_);                                                             \
        const int e_ = count++;                                                                 \
        const uint32_t kk_ = order_key(sc_);                                                    \
        if (lane == 0) s_ent[e_] = TreeEntry{sc_, (base_), (prefix_), ((d_) << 16) | (k_)};     \
        if (lane == (e_ & 63)) {                                                                \
            KDT_SET_SLOT(e_ >> 6, kk_);                                                         \
            if (kk_ > best_key) { /* a later push never beats an equal earlier one */           \
                best_key = kk_;                                                                 \
                best_slot = e_ >> 6;                                                            \
            }                                                                                   \
        }                                                                                       \
    } while (0)

    KDT_PUSH(s_lp[0], 0.0f, -1, 0, 0);
    int n = 0;
    for (; n < N; n++) {
        const uint32_t top = wave_reduce_u32<true>(best_key);
        if (top == 0u) break;                                       // the frontier is empty
        const uint32_t cand_e = best_key == top ? (uint32_t)(best_slot * 64 + lane) : 0xFFFFFFFFu;
        const int e = (int)wave_reduce_u32<false>(cand_e);          // earliest push among the best
        __syncthreads();                                            // lane 0's entry write is visible
        const TreeEntry t = s_ent[e];
        const int d = t.dk >> 16, k = t.dk & 0xFFFF;
        if (lane == 0) {
            s_npar[n] = t.prefix;
            s_ndk[n] = t.dk;
        }
        if (lane == (e & 63)) {                                     // retire the entry, rescan the lane
            KDT_SET_SLOT(e >> 6, 0u);
            const uint32_t ks[kTreeSlots] = {k0, k1, k2, k3, k4, k5, k6, k7, k8};
            best_key = 0u;
            best_slot = 0;
#pragma unroll
            for (int s = 0; s < kTreeSlots; s++)
                if (ks[s] > best_key) {
                    best_key = ks[s];
                    best_slot = s;
                }
        }
        if (k + 1 < K) KDT_PUSH(t.base + s_lp[d * K + k + 1], t.base, t.prefix, d, k + 1);
        if (d + 1 < D) KDT_PUSH(t.score + s_lp[(d + 1) * K], t.score, n, d + 1, 0);
    }
#undef KDT_PUSH
#undef KDT_SET_SLOT
    __syncthreads();
    // outputs: nodes [0, n), then -2 for the rows a too small tree could not fill
    for (int i = lane; i < N; i += 64) {
        int32_t p = -2, tk = -2, dd = -2, rk = -2;
        if (i < n) {
            const int dk = s_ndk[i], d = dk >> 16, k = dk & 0xFFFF;
            p = s_npar[i];
            tk = cand[b * DK + d * K + k];
            dd = d + 1;
            rk = k;
        }
        parents[b * N + i] = p;
        if (tokens) tokens[b * N + i] = tk;
        if (depth) depth[b * N + i] = dd;
        if (rank) rank[b * N + i] = rk;
    }
}

hipError_t launch_tree_build(const float *logp, const int32_t *cand, int B, int D, int K, int N,
                             int32_t *parents, int32_t *tokens, int32_t *depth, int32_t *rank, hipStream_t st) {
    const size_t lds = (size_t)D * K * sizeof(float);
    tree_build_kernel<<<(unsigned)B, 64, lds, st>>>(logp, cand, D, K, N, parents, tokens, depth, rank);
    return hipGetLastError();
}

}  // namespace kdt
