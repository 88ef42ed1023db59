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
// The search is sequential per request, so one wave builds one request.  A prefix's child of
// rank r + 1 is pushed only when its child of rank r is popped (rank 0: when the prefix itself
// is), so the frontier holds at most one entry per prefix: its next unpopped child.  It is
// therefore kept as one slot per prefix p (p = -1 for depth 1, else a popped node), holding
// that child's rank r, the prefix's score and the entry's score; a pop moves the slot of the
// popped child's prefix on to rank r + 1 and opens the slot of the new node (its rank-0
// child).  Slot j = p + 1 lives in lane j % 64, register slot j / 64; the last node opens no
// slot (nothing is popped after it), so slots 0 .. N-1 suffice: at most 4 per lane for
// N <= 256.  Equal scores go to the earlier push; an entry's push number is counted exactly
// as a heap would count it (a next sibling is pushed before the first child).  A pop is a wave
// max over the 64 lane bests (DPP inside rows of 16 lanes and row broadcasts across them) and
// a ballot for the lane that holds it; the winner's fields come back by lane reads, and one LDS
// read of the log-probability table gives the two new entry scores.  The order key is the
// score's fp32 pattern mapped to an unsigned integer that sorts like the float (zeroes of
// either sign map to one key).
#include "kdt_internal.h"

namespace kdt {

// Unsigned key that orders like the float value (-0 and +0 equal); 0 is below every score.
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v == 0.0f) v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Max over a wave of 64: within each row of 16 lanes by DPP (quad swaps, row rotations by 4
// and 8), then row 0 into row 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows
// 2-3 (row_bcast:31); lane 63 then holds the maximum.  Uniform result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    // lanes a move does not write read 0, the identity of an unsigned max, so each move can
    // fold into the max instruction
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));    // quad_perm 1,0,3,2
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));    // quad_perm 2,3,0,1
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, true));   // row_ror 4
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, true));   // row_ror 8
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, true));   // row_bcast:15
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, true));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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

// f(0), ..., f(S-1) with compile-time indices (keeps per-slot arrays in registers).
template <int I, int S, class F>
__device__ __forceinline__ void each_slot(F &&f) {
    if constexpr (I < S) {
        f(std::integral_constant<int, I>{});
        each_slot<I + 1, S>(f);
    }
}

// Value of register slot `slot` (uniform) of lane `lane` (uniform), for every lane.
template <int S>
__device__ __forceinline__ uint32_t fetch(const uint32_t (&v)[S], int slot, int lane) {
    uint32_t x = v[0];
    each_slot<1, S>([&](auto I) { x = slot == I.value ? v[I.value] : x; });
    return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}

// S = register slots per lane: ceil(N / 64).
template <int S>
__global__ __launch_bounds__(64) void tree_build_kernel(const float *__restrict__ logp,
                                                        const int32_t *__restrict__ cand, int D, int K,
                                                        int N, int32_t *__restrict__ parents,
                                                        int32_t *__restrict__ tokens,
                                                        int32_t *__restrict__ depth,
                                                        int32_t *__restrict__ rank) {
    extern __shared__ float s_lp[];                     // [D*K] this request's log probabilities
    __shared__ int32_t s_npar[kMaxNodes], s_ndk[kMaxNodes];
    const int64_t b = blockIdx.x;
    const int lane = threadIdx.x;
    const int DK = D * K;
    for (int i = lane; i < DK; i += 64) s_lp[i] = logp[b * DK + i];
    __syncthreads();

    // this lane's slots: entry order key (0 = none), push number, entry score, prefix score,
    // and (children's depth index << 16 | next rank)
    uint32_t key[S], tie[S], esc[S], base[S], dr[S];
    each_slot<0, S>([&](auto I) { key[I.value] = tie[I.value] = esc[I.value] = base[I.value] = dr[I.value] = 0u; });
    uint32_t best_key = 0u, best_tie = 0u;   // this lane's best slot by (key desc, push asc)
    int best_slot = 0;
    if (lane == 0) {                          // slot 0: prefix -1, entry = depth-1 rank 0
        const float e = s_lp[0];
        key[0] = best_key = order_key(e);
        esc[0] = __float_as_uint(e);
    }
    int pushes = 1;

    int n = 0;
    for (; n < N; n++) {
        const uint32_t top = wave_max_u32(best_key);
        if (top == 0u) break;                                       // the frontier is empty
        // the lane holding the best entry; only equal best scores in several lanes (rare)
        // need the push numbers compared
        uint64_t m = __ballot(best_key == top);
        if (__builtin_popcountll(m) > 1) {
            const uint32_t t_min = wave_reduce_u32<false>(best_key == top ? best_tie : 0xFFFFFFFFu);
            m = __ballot(best_key == top && best_tie == t_min);   // push numbers are unique
        }
        const int jl = __builtin_ctzll(m);
        const int js = __builtin_amdgcn_readlane(best_slot, jl);
        const int j = js * 64 + jl;
        const float score = __uint_as_float(fetch<S>(esc, js, jl));
        const float pbase = __uint_as_float(fetch<S>(base, js, jl));
        const uint32_t pdr = fetch<S>(dr, js, jl);
        const int d = (int)(pdr >> 16), r = (int)(pdr & 0xFFFFu);
        // the two entries this pop pushes: the next sibling, then the first child
        const bool sib = r + 1 < K, child = d + 1 < D;
        const float lp_sib = s_lp[d * K + (sib ? r + 1 : r)];
        const float lp_child = s_lp[(child ? d + 1 : d) * K];
        if (lane == 0) {
            s_npar[n] = j - 1;
            s_ndk[n] = (int)pdr;
        }
        const uint32_t t_sib = (uint32_t)pushes;
        pushes += sib ? 1 : 0;
        const uint32_t t_child = (uint32_t)pushes;
        pushes += child ? 1 : 0;
        const float e_sib = pbase + lp_sib;
        const float e_child = score + lp_child;
        const uint32_t k_sib = sib ? order_key(e_sib) : 0u;
        const uint32_t k_child = child ? order_key(e_child) : 0u;
        // slot j moves on to rank r + 1; slot n + 1 opens with the new node's rank-0 child (not
        // for the last node: nothing is popped after it, so slots 0 .. N-1 suffice)
        const int jn = n + 1 < N ? n + 1 : -1, jnl = jn & 63, jns = jn < 0 ? -1 : jn >> 6;
        each_slot<0, S>([&](auto I) {
            constexpr int i = I.value;
            if (lane == jl && i == js) {
                key[i] = k_sib;
                tie[i] = t_sib;
                esc[i] = __float_as_uint(e_sib);
                dr[i] = pdr + 1u;
            }
            if (lane == jnl && i == jns) {
                key[i] = k_child;
                tie[i] = t_child;
                esc[i] = __float_as_uint(e_child);
                base[i] = __float_as_uint(score);
                dr[i] = (uint32_t)(d + 1) << 16;
            }
        });
        {                                   // rescan (only lanes jl and jnl changed; the others
            best_key = 0u;                  // recompute the same best, with no branch)
            best_tie = 0u;
            best_slot = 0;
            each_slot<0, S>([&](auto I) {
                constexpr int i = I.value;
                if (key[i] > best_key || (key[i] == best_key && key[i] != 0u && tie[i] < best_tie)) {
                    best_key = key[i];
                    best_tie = tie[i];
                    best_slot = i;
                }
            });
        }
    }
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
    const int slots = (N + 63) / 64;
    auto go = [&](auto kernel) {
        kernel<<<(unsigned)B, 64, lds, st>>>(logp, cand, D, K, N, parents, tokens, depth, rank);
    };
    switch (slots) {
        case 1: go(tree_build_kernel<1>); break;
        case 2: go(tree_build_kernel<2>); break;
        case 3: go(tree_build_kernel<3>); break;
        case 4: go(tree_build_kernel<4>); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kdt
