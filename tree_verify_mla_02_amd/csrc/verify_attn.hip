// Tree-verify MLA-absorb attention for gfx950 (MI355X).
//
// What is computed ("Validating the Native Engine", section "The Broader Context": a
// tree-verify MLA-absorb attention kernel with visibility masking; "The Capstone
// Validation", section "Context and Motivation": all drafted continuations are verified in
// one batched pass): for request b, tree node i and head h,
//     out[b,i,h] = softmax_k(scale * (q_lat.ckv_k + q_rope.krope_k)) . ckv_k
// over the request's committed cache and the tree nodes on i's root-to-node path.
//
// How it maps to CDNA4.  In absorbed MLA every head reads the same latent rows, so the
// (node x head) query rows of a request form the M dimension of one dense contraction
// against shared 576-wide key rows -- exactly the shape bf16 MFMA is built for.
//   * A workgroup is 4 waves x 32 query rows (128 rows).  A wave keeps its queries in
//     VGPRs (B operand of S^T = K Q^T) and its 32 x d_c fp32 output accumulator O^T in the
//     MFMA result registers for the whole key loop.
//   * Key rows stream HBM -> LDS in 64-key tiles with global_load_lds_dwordx4 (no VGPR
//     staging), double buffered.  The LDS tile is stored in 1 KB blocks of (keys x 16-byte
//     chunks) with an XOR swizzle of the chunk index by the key, so that both the row-wise
//     K reads of S^T = K Q^T and the column-wise V reads of O^T = V^T P^T are free of bank
//     conflicts.
//   * Scores come out of the MFMA transposed (one query row per lane pair), so the online
//     softmax needs one cross-lane exchange per tile; P^T feeds the P.V MFMA directly from
//     the score registers, and V^T comes from LDS through ds_read_b64_tr_b16.
//   * P is split into bf16 hi + lo parts, both multiplied by V (fp32 accumulate): this
//     keeps the probability weights ~16 bits accurate, which a single bf16 rounding of P
//     is not when a few keys with large latent values dominate a row.
//   * The tree segment is one more tile (or up to four for 256 nodes) whose scores are
//     masked with the row's 64-bit ancestor word.
//   * Small batches split the committed keys over workgroups; partial (O, max, sum) are
//     merged by a log-sum-exp combine.
//   * Requests that 128-row workgroups cannot spread over the GPU take 64-row ones
//     (decode_attn_kernel: waves split the rows and the keys of each tile).
//   * For a one-request batch both kernels can also make the visibility masks and the plan
//     unit inside the attention launch (their FUSED instantiations), saving a launch.
#include "kdt_internal.h"
#include "visibility_rows.h"

namespace kdt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

template <int I>
struct IntC {
    static constexpr int value = I;
};
// Compile-time loop: f(IntC<B>), ..., f(IntC<E-1>).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

// Splits used for request b: those that cut its Tf + L virtual keys (Tf committed-key places
// given to the tree; see kdt_internal.h).  Split 0 always exists (it owns the tree keys).
__device__ __forceinline__ int splits_of(int L, int Tf, int64_t chunk, int S) {
    const int64_t n = ((L > 0 ? L : 0) + Tf + chunk - 1) / chunk;
    return (int)(n < 1 ? 1 : n < S ? n : S);
}

// ------------------------------------------------------------------------------ plan
// One workgroup.  Validates cache_lens, writes per-request offsets (exclusive scan) and the
// unit list the attention grid reads.
//
// Unit order.  The dispatcher deals workgroups to the kXcds XCDs round-robin (grid slot u runs
// on XCD u % kXcds), and each XCD has its own L2.  The row tiles of one (request, key split)
// "group" all read the same key rows, so a group's units are given grid slots x + kXcds*k on
// a single XCD x: its key tiles come from HBM once and from that L2 for the other row tiles.
// Groups are sorted by work (keys), dealt to XCDs in snake order (0..7, 7..0, ...) to balance
// the XCDs, and each XCD runs its groups longest first.
constexpr int kMaxSortGroups = 2048;    // above this the groups keep request order

// Division of 32-bit unsigned integers by a divisor d (1 <= d <= 2^31) fixed for the launch, as
// a high multiply and shifts (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// t = mulhi(m, n), n / d = (t + ((n - t) >> 1)) >> (l - 1), and n / 1 = n.  The host sets the
// constants; a hardware-less 32-bit division is a dependent chain of about forty instructions.
static inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) l++;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    const uint32_t t = __umulhi(n, f.m);
    return f.l == 0 ? n : (t + ((n - t) >> 1)) >> (f.l - 1);
}

struct PlanArgs {
    const int32_t *cache_lens;
    int B, N;
    int64_t max_len, total_len;
    int RT, S, bt, bs;
    int tree_keys;         // Tf: committed-key places of the tree in split 0
    int64_t chunk, U;
    WsHeader *hdr;
    int64_t *offsets;
    int32_t *lens;
    Unit *units;
    int32_t *dev_status;
    FastDiv fd_chunk, fd_per, fd_grgs, fd_gs, fd_gr, fd_bs;
};

// LDS of the plan: the lengths and offsets of up to kMaxLdsReq requests, and the sort keys and
// work order of up to kMaxSortGroups groups, so that every step after the first load of
// cache_lens reads LDS (more requests read the workspace copies of lengths and offsets; more
// groups keep request order).
constexpr int kMaxLdsReq = 1024;
struct alignas(16) PlanLds {
    uint32_t key[kMaxSortGroups];       // sort key of each group (see plan_body); 16-byte reads
    int32_t order[kMaxSortGroups];
    int64_t offs[kMaxLdsReq];
    int64_t wsum[16];                   // per-wave totals of the offsets scan (<= 1024 threads)
    int32_t lens[kMaxLdsReq];
    int32_t sb[kMaxLdsReq];             // splits of each request
    int ok;
};
static_assert(kMaxSortGroups % 4 == 0, "whole 16-byte key reads");

// Barrier for data exchanged through LDS only: waits for this wave's LDS traffic, not for
// its global stores (a full __syncthreads also waits for every store to reach memory).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The plan, by one workgroup whose size is a multiple of 64 (at most 1024).  Index
// arithmetic is 32-bit: the host bounds the grid (every group index and unit slot) below 2^31,
// and divides by the launch's fixed divisors through FastDiv.
__device__ __forceinline__ void plan_body(const PlanArgs &pa, PlanLds &L) {
    const int32_t *__restrict__ cache_lens = pa.cache_lens;
    const int B = pa.B, N = pa.N, RT = pa.RT, S = pa.S, bt = pa.bt, bs = pa.bs;
    const int64_t max_len = pa.max_len, total_len = pa.total_len;
    const uint32_t chunk = (uint32_t)pa.chunk;
    const int U = (int)pa.U;
    const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wave = tid >> 6, nwaves = nth >> 6;
    const bool req_lds = B <= kMaxLdsReq;
    int32_t *lens = req_lds ? L.lens : pa.lens;
    int64_t *offs = req_lds ? L.offs : pa.offsets;
    // virtual keys before the committed ones: the tree's places (0 or its whole tiles)
    const uint32_t T = (uint32_t)pa.tree_keys;
    // splits of a request of len committed keys: ceil((len + T) / chunk), at least 1, at most S
    auto splits = [&](int len) {
        const uint32_t n = fdiv((uint32_t)(len > 0 ? len : 0) + T + chunk - 1u, pa.fd_chunk);   // < 2^32
        return (int)(n < 1u ? 1u : n < (uint32_t)S ? n : (uint32_t)S);
    };
    if (tid == 0) L.ok = 1;
    lds_sync();
    for (int b = tid; b < B; b += nth) {
        const int len = cache_lens[b];
        lens[b] = len;
        if (req_lds) {
            pa.lens[b] = len;
            L.sb[b] = splits(len);
        }
        if (len < 0 || (int64_t)len > max_len) L.ok = 0;
    }
    if (req_lds) lds_sync(); else __syncthreads();
    // offsets: exclusive scan of max(len, 0).  Up to 64 requests one thread adds them up
    // (a chain of adds is shorter than a scan's chain of lane shuffles); more go nth at a
    // time through wave scans and the wave totals.
    int64_t carry = 0;
    if (B <= 64) {
        if (tid == 0) {
            for (int b = 0; b < B; b++) {
                offs[b] = carry;
                if (req_lds) pa.offsets[b] = carry;
                carry += lens[b] > 0 ? lens[b] : 0;
            }
        }
    } else {
        for (int base = 0; base < B; base += nth) {
            const int b = base + tid;
            const int64_t v = b < B && lens[b] > 0 ? lens[b] : 0;
            int64_t x = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int64_t y = __shfl_up(x, d, 64);
                if (lane >= d) x += y;
            }
            if (lane == 63) L.wsum[wave] = x;
            lds_sync();
            int64_t pre = carry, tot = 0;
            for (int w = 0; w < nwaves; w++) {
                if (w < wave) pre += L.wsum[w];
                tot += L.wsum[w];
            }
            if (b < B) {
                offs[b] = pre + x - v;
                if (req_lds) pa.offsets[b] = pre + x - v;
            }
            carry += tot;
            lds_sync();                  // wsum is rewritten by the next round
        }
    }
    if (tid == 0) {
        if (carry > total_len) L.ok = 0;
        pa.hdr->ok = L.ok;
        if (!L.ok && pa.dev_status) atomicOr(pa.dev_status, (int32_t)KDT_DEV_CACHE_LEN);
    }
    if (req_lds) lds_sync(); else __syncthreads();
    const int ok = L.ok;
    // Groups: bt row tiles x bs splits of one request, (request, row-tile block, split block)
    // with the split block fastest.  A group's work is the virtual keys of its splits, plus the
    // N tree keys for split 0 when they have no place among them (its row tiles all cost the
    // same).  With G <= kMaxSortGroups groups are ranked by a unique 32-bit key:
    // bit 31 = the group has a split (a request's lengths may leave a split block empty, and
    // rejected lengths leave every group empty), bits 30..11 = its 64-key tiles (saturated),
    // bits 10..0 = 2047 - g (ties by index).  Larger keys go first.
    const int GR = (RT + bt - 1) / bt, GS = (S + bs - 1) / bs;
    const int G = B * GR * GS;
    const int per = bt * bs;
    const bool grp_lds = G <= kMaxSortGroups;
    if (grp_lds) {
        uint32_t *key = L.key;
        for (int g = tid; g < G; g += nth) {
            const uint32_t q = fdiv((uint32_t)g, pa.fd_gs);
            const int b = (int)fdiv((uint32_t)g, pa.fd_grgs), gs = g - (int)q * GS;
            const int len = lens[b];
            int64_t w = -1;
            if (ok) {
                const int sbr = req_lds ? L.sb[b] : splits(len);
                const int64_t lv = (int64_t)(len > 0 ? len : 0) + T;
                for (int sp = gs * bs; sp < gs * bs + bs && sp < sbr; sp++) {
                    const int64_t left = lv - (int64_t)sp * chunk;
                    w = (w < 0 ? 0 : w) + (left < chunk ? (left > 0 ? left : 0) : chunk) + (sp == 0 && T == 0u ? N : 0);
                }
            }
            const int64_t tiles = w < 0 ? 0 : (w + kKeysPerTile - 1) / kKeysPerTile;
            key[g] = (w < 0 ? 0u : 0x80000000u) | ((uint32_t)(tiles < 0xfffff ? tiles : 0xfffff) << 11) |
                     (uint32_t)(2047 - g);
        }
        for (int g = G + tid; g < ((G + 3) & ~3); g += nth) key[g] = 0u;   // whole 4-key reads: 0 ranks last
        lds_sync();
        // rank = #{h : key[h] > key[g]}: every thread reads the same keys (LDS broadcasts), four
        // per read, eight reads in flight
        const int G4 = (G + 3) >> 2;
        const uint4 *key4 = (const uint4 *)key;
        for (int g = tid; g < G; g += nth) {
            const uint32_t kg = key[g];
            int rank = 0;
            int h = 0;
            for (; h + 8 <= G4; h += 8) {
                uint4 v[8];
#pragma unroll
                for (int k = 0; k < 8; k++) v[k] = key4[h + k];
#pragma unroll
                for (int k = 0; k < 8; k++) rank += (v[k].x > kg) + (v[k].y > kg) + (v[k].z > kg) + (v[k].w > kg);
            }
            for (; h < G4; h++) {
                const uint4 v = key4[h];
                rank += (v.x > kg) + (v.y > kg) + (v.z > kg) + (v.w > kg);
            }
            L.order[rank] = g;
        }
        lds_sync();
    }
    // Group p (in work order; request order above kMaxSortGroups groups) goes to XCD lane x in
    // snake order over rounds of 8 groups, and its unit i takes grid slot x + 8 * (round * per + i).
    // Slots are dealt to the XCDs round-robin, so a group runs on one XCD.  The loop runs over the
    // slots and inverts that map, so that every slot is stored exactly once: a slot no unit takes
    // (padding, a split past the request's keys, a row tile past its rows, rejected lengths) gets
    // the empty record.  A group with no work has no split below its request's split count, so
    // the per-slot test covers it.
    for (int u = tid; u < U; u += nth) {
        const int x = u & (kXcds - 1);
        const int k = u >> 3;                 // kXcds = 8
        const int round = (int)fdiv((uint32_t)k, pa.fd_per);
        const int i = k - round * per;
        const int p = round * kXcds + ((round & 1) ? kXcds - 1 - x : x);
        Unit un{-1, 0, 0, 0, 0, 0, 0};
        if (ok && p < G) {
            const int g = grp_lds ? L.order[p] : p;
            const uint32_t q = fdiv((uint32_t)g, pa.fd_gs);
            const int b = (int)fdiv((uint32_t)g, pa.fd_grgs);
            const int gs = g - (int)q * GS, gr = (int)q - (int)fdiv(q, pa.fd_gr) * GR;
            const int ib = (int)fdiv((uint32_t)i, pa.fd_bs);
            const int rt = gr * bt + ib, sp = gs * bs + (i - ib * bs);
            const int len = lens[b];
            const int sb = req_lds ? L.sb[b] : splits(len);
            if (rt < RT && sp < sb) {
                // committed keys [k0, k1): virtual [sp*chunk, (sp+1)*chunk) less the tree's places
                const int64_t v0 = (int64_t)sp * chunk - T, v1 = v0 + chunk;
                const int64_t k0 = v0 > 0 ? v0 : 0;
                const int64_t k1 = v1 < (int64_t)len ? v1 : (int64_t)len;
                un = Unit{b, rt, sp, sb, (int32_t)k0, (int32_t)(k1 > k0 ? k1 : k0), offs[b] + k0};
            }
        }
        pa.units[u] = un;
    }
}

__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs pa) {
    __shared__ PlanLds lds;
    plan_body(pa, lds);
}

// Masks and plan in one launch (they are independent): workgroups 0 .. B-1 build the masks
// of one request each, workgroup B runs the plan.  Saves a kernel launch per verify step.
template <int W>
__global__ __launch_bounds__(256) void prepare_kernel(const int32_t *__restrict__ parents,
                                                      uint64_t *__restrict__ masks, PlanArgs pa) {
    __shared__ VisLds vis;
    __shared__ PlanLds lds;
    if ((int)blockIdx.x < pa.B)
        visibility_rows<W>(parents, pa.N, masks, pa.dev_status, blockIdx.x, vis);   // 256 threads >= N
    else
        plan_body(pa, lds);
}

// ------------------------------------------------------------------------------ attention
template <typename T, int DC, int DR>
struct Shape {
    static constexpr int D = DC + DR;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int EPC = 16 / ES;             // elements per 16-byte chunk
    static constexpr int CH = D / EPC;              // chunks per key row
    static constexpr int CH_LAT = DC / EPC;         // chunks of the latent part
    static constexpr int CB = (CH % 8 == 0) ? 8 : (CH % 4 == 0) ? 4 : 2;   // chunks per LDS block row
    static constexpr int KB = 64 / CB;              // keys per 1 KB LDS block
    static constexpr int NKG = kKeysPerTile / KB;   // key groups per tile
    static constexpr int NCG = CH / CB;             // chunk groups per key row
    static constexpr int TILE_BYTES = kKeysPerTile * D * ES;
    static constexpr bool BF16 = (ES == 2);
    // XOR applied to the 16-byte chunk index of a key row inside its 1 KB block.  gfx950 LDS
    // serves a 16-byte-per-lane read 16 lanes at a time over 64 four-byte banks (256 B).
    // With 8-chunk rows (CB = 8) the 16 lanes of an S^T fragment read keys k..k+15 at one
    // chunk: rows of even / odd key land in the two 128-byte bank halves, and bits 1..3 of
    // the key pick distinct chunk slots within a half.  Bit 1 drives the top bit of the XOR,
    // so the transposed V^T reads (keys r and r+2 of a 4-key group, 4 chunks each) also fall
    // in opposite slot halves.  Both read patterns are conflict-free.  Only key % 16 matters.
    static __host__ __device__ constexpr int swz(int key) {
        return CB == 8 ? ((((key >> 1) & 1) << 2) | (((key >> 2) & 1) << 1) | ((key >> 3) & 1)) : (key % KB) % CB;
    }
    static_assert(D % EPC == 0 && CH % CB == 0 && CH_LAT % CB == 0, "row must split into blocks");
    static_assert(TILE_BYTES == NKG * NCG * 1024, "tile = whole 1 KB blocks");
    static_assert(DC % 32 == 0, "latent width must be a multiple of 32");
    static_assert(!BF16 || (DC % 16 == 0 && DR % 16 == 0), "bf16 K steps are 16 wide");
    static_assert(BF16 || (DC % 4 == 0 && DR % 4 == 0), "fp32 rows are whole chunks");
};

// Byte offset of logical 16-byte chunk c of tile key `key` inside one LDS tile buffer.
template <class Sh>
__device__ __forceinline__ int lds_off(int key, int c) {
    const int kg = key / Sh::KB, kr = key % Sh::KB;
    const int cg = c / Sh::CB, cc = c % Sh::CB;
    return ((kg * Sh::NCG + cg) << 10) + kr * (Sh::CB * 16) + ((cc ^ Sh::swz(key)) << 4);
}

// Offset of tile key `k` (a multiple of 16) relative to key k % 16 with the same chunk: the
// swizzle only looks at key % 16, so it is unchanged.
template <class Sh>
__host__ __device__ constexpr int key_off(int k) {
    return (k / Sh::KB) * Sh::NCG * 1024 + (k % Sh::KB) * Sh::CB * 16;
}

// One 16-byte-per-lane HBM -> LDS copy (lane l writes bytes 16l..16l+15 at lds_addr) from
// base + voff, with base a wave-uniform 64-bit pointer in SGPRs and voff this lane's 32-bit
// byte offset (the global "saddr" form: no 64-bit address arithmetic per copy in VALU).  The
// instruction's immediate offset is left at 0: for LDS-DMA loads it also moves the LDS
// destination, so the per-chunk offset goes into the scalar base instead.  The copy is issued
// as asm: as a compiler intrinsic it counts as an LDS store of unknown address, and the
// compiler then waits for it (vmcnt) before every later LDS read -- a full memory latency
// after each batch of copies.  The copies only ever target the tile buffer that is not being
// read, and the wait that makes them visible is explicit (s_waitcnt vmcnt(0) + barrier at the
// top of the next tile).
// The LDS destination goes in M0, set inside the asm.  The compiler warns that M0 is a reserved
// register it may not preserve across the statement; it uses M0 for nothing else in these
// kernels (the generated code sets M0 only before these copies), and binding M0 as an operand
// instead measured about 0.2 % slower.
__device__ __forceinline__ void lds_dma16(const char *base, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 : : "v"(voff), "s"(base), "s"(lds_addr) : "m0");
}

// Copy of one key tile (kKeysPerTile rows of D elements, latent and rope parts from separate
// bases) into the LDS layout of lds_off.  Each copy moves a 1 KB block: KB keys x CB chunks,
// lane -> (key kr = lane / CB, stored chunk lane % CB), so the swizzle is applied by choosing
// which logical chunk of the row a lane fetches.  Keys past the end of a partial tile re-read
// the last valid row (their scores are masked).  Wave w copies key groups w, w + 4, ...
template <class Sh, typename T>
struct TileDma {
    static constexpr int KGW = (Sh::NKG + kWaves - 1) / kWaves;   // key groups per wave (max)
    static constexpr int NINST = KGW * Sh::NCG;                     // loads per wave per tile
    const char *lat, *rope;      // wave-uniform bases: key row 0 of the tile
    LDS_AS char *dst;            // the tile buffer
    uint32_t off_lat[KGW], off_rope[KGW];
    int wave;

    __device__ __forceinline__ void setup(LDS_AS char *buf, const T *lat_base, int64_t lat_stride,
                                          const T *rope_base, int64_t rope_stride, int64_t row0, int nvalid,
                                          int wave_, int lane) {
        wave = wave_;
        dst = buf;
        lat = (const char *)(lat_base + row0 * lat_stride);
        rope = (const char *)(rope_base + row0 * rope_stride);
        const int kr = lane / Sh::CB;
        const uint32_t lsb = (uint32_t)(lat_stride * (int64_t)sizeof(T));
        const uint32_t rsb = (uint32_t)(rope_stride * (int64_t)sizeof(T));
#pragma unroll
        for (int g = 0; g < KGW; g++) {
            const int slot_key = (wave + kWaves * g) * Sh::KB + kr;    // the key this LDS slot holds
            const uint32_t cc = (uint32_t)((lane % Sh::CB) ^ Sh::swz(slot_key));   // its logical chunk
            const uint32_t key = (uint32_t)(slot_key < nvalid ? slot_key : nvalid - 1);
            off_lat[g] = key * lsb + cc * 16u;
            off_rope[g] = key * rsb + cc * 16u;
        }
    }

    // loads [J0, J1) of this wave's NINST (key group major, chunk group minor)
    template <int J0, int J1>
    __device__ __forceinline__ void issue() const {
        static_for<J0, (J1 < NINST ? J1 : NINST)>([&](auto J) {
            constexpr int j = decltype(J)::value;
            constexpr int g = j / Sh::NCG, cg = j % Sh::NCG;
            const int kg = wave + kWaves * g;
            // every wave has KGW groups when they divide evenly: no test (and no branch)
            if (Sh::NKG % kWaves == 0 || kg < Sh::NKG) {
                const uint32_t lds = (uint32_t)(uintptr_t)(dst + ((kg * Sh::NCG + cg) << 10));
                if constexpr (cg * Sh::CB < Sh::CH_LAT)
                    lds_dma16(lat + cg * Sh::CB * 16, off_lat[g], lds);
                else
                    lds_dma16(rope + (cg * Sh::CB - Sh::CH_LAT) * 16, off_rope[g], lds);
            }
        });
    }
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// O^T *= alpha (one scale per lane = per query row), done in place in the accumulation
// registers.  Written as AGPR read / VALU multiply / AGPR write so the 32 x d_c accumulator
// never needs a VGPR home: a plain `o *= alpha` makes the register allocator move the whole
// accumulator into VGPRs and spill.  The leading s_nops cover the wait states between an
// MFMA writing an accumulator and a v_accvgpr_read of it, the trailing one those between
// v_accvgpr_write and the next MFMA reading it as srcC.
template <int NT>
__device__ __forceinline__ void rescale_acc(f32x16 (&o)[NT], float alpha) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
            float tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(o[t][i]), "=&v"(tmp)
                         : "v"(alpha));
        }
    asm volatile("s_nop 7" ::: "memory");
}

// ------------------------------------------------------------------------------ softmax
// Online softmax of one query row over 32-key blocks, in base 2 (scores times scale*log2 e).
// Probabilities are taken relative to a reference m_ref rather than the running max m_max: P
// may exceed 1, and fp32 and the bf16 hi/lo pair keep the same relative accuracy at any
// magnitude, so the result is the same softmax.  The reference moves only when a block max
// passes it by more than kLazy; O and l are then rescaled by 2^(old - new) -- for the whole
// wave, since each lane holds its row's accumulator, whichever of the 32 rows needed it.  So
// when one row must move, every row of the wave moves, to its own running max + kHead: the
// rescale is paid once for all, and a row next forces one only when its max has risen by more
// than kHead + kLazy.  On inputs with large outliers (scores spread over hundreds, base 2)
// this cuts wave rescales from a quarter of the 32-key blocks to a few percent.
// Bounds: P <= 2^kLazy and, for the row's running max, P >= 2^-kHead, so keys more than
// 126 - kHead below the max underflow (weight below 2^-94: nothing); O <= keys * 2^kLazy * max|v|
// stays finite for latent magnitudes below 2^60.
constexpr float kLazy = 32.f;
constexpr float kHead = 32.f;

struct Update {
    float m_use;    // reference the block's probabilities are taken against (0 if none yet)
    float alpha;    // factor for O and l accumulated so far (1 = unchanged)
};

// Visibility of the 16 keys a lane holds in one 32-key block: bit (i/4)*8 + i%4 of
// `w` is key kb*32 + (i/4)*8 + 4*half + i%4.  `vis` is the tile's 64-bit visibility word
// (ancestor word of the row's node for tree tiles, all ones for cache tiles) with the keys at
// or beyond the valid count already cleared.
__device__ __forceinline__ uint32_t block_bits(uint64_t vis, int kb, int half) {
    return (uint32_t)(vis >> (kb * 32 + 4 * half));
}
__device__ __forceinline__ bool bit_of(uint32_t w, int i) { return (w >> ((i >> 2) * 8 + (i & 3))) & 1u; }

// Value of the other half of this lane's row combined with this one: lanes l and l+32 hold
// the same query row.  v_permlane32_swap exchanges the two 32-lane halves between its two
// operands; fed the same value twice, one result holds the low half's value and the other
// the high half's in every lane, so a symmetric op of the two is the row-wide result
// whichever way the swap goes.
__device__ __forceinline__ float row_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Masked keys get score -inf (rare tiles only: partial cache tiles and tree tiles).
__device__ __forceinline__ void mask_scores(f32x16 &s, uint32_t w) {
#pragma unroll
    for (int i = 0; i < 16; i++) s[i] = bit_of(w, i) ? s[i] : -INFINITY;
}

// c = scale * log2(e) is made positive once per workgroup (see normalise_scale), so the row
// max of the raw scores gives the max of the scaled ones and -inf scores map to P = 0.
struct SoftmaxRow {
    float m_ref;    // reference (base-2 domain), -inf until the row sees a key
    float m_max;    // running max of the row's scaled scores, -inf until it sees a key
    float l;        // running sum of probabilities relative to m_ref (this lane's keys only)
    float c;        // scale * log2(e), > 0

    // Called by every lane of the wave together (the move decision is a wave ballot).
    __device__ __forceinline__ Update update_from_max(float e) {
        const float bm = e * c;                                // -inf stays -inf
        const float mm = fmaxf(m_max, bm);
        // also true for the first visible key (m_ref = -inf); -inf stays -inf
        const bool any = __ballot(bm > m_ref + kLazy) != 0;
        const float m_new = any ? mm + kHead : m_ref;
        // exponent 0 (alpha = 1) unless an existing reference moves; no branch
        const float alpha = __builtin_amdgcn_exp2f((m_new != m_ref && m_ref != -INFINITY) ? m_ref - m_new : 0.f);
        m_ref = m_new;
        m_max = mm;
        return Update{m_new == -INFINITY ? 0.f : m_new, alpha};
    }

    __device__ __forceinline__ Update update(const f32x16 &s) {
        float e = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; i++) e = fmaxf(e, s[i]);
        return update_from_max(row_max(e));
    }

    // P = 2^(s*c - m) as bf16 hi + lo pairs (B operands of the two P.V MFMAs); returns sum P
    __device__ __forceinline__ float probs(const f32x16 &s, const Update &u, bf16x8 (&phi)[2],
                                           bf16x8 (&plo)[2]) const {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -u.m_use));
            sum += p;
            const __bf16 hi = (__bf16)p;
            phi[i >> 3][i & 7] = hi;
            plo[i >> 3][i & 7] = (__bf16)(p - (float)hi);
        }
        return sum;
    }

    __device__ __forceinline__ float probs_f32(f32x16 &s, const Update &u) const {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -u.m_use));
            s[i] = p;
            sum += p;
        }
        return sum;
    }
};

// The softmax of one 32-key block cut into kSmStages micro-steps of at most four VALU
// instructions (an exp counts double), so that an MFMA pipeline can issue one of them after
// each MFMA.  A wave issues in order and an MFMA holds the issue port for about half of its 32
// cycles, so only work placed between two MFMAs runs in the matrix core's shadow: a larger
// group stalls the next MFMA.  Steps: partial maxima (4), cross-lane max and reference update
// (4), then per pair of probabilities (8 pairs) exp2, sum, and the exact split into bf16 hi +
// lo (4 each): p = hi + lo_exact with hi = bf16(p) (round to nearest) and lo_exact = p - hi
// exact in fp32, then lo = bf16(lo_exact).
constexpr int kSmPre = 8;
constexpr int kSmStages = kSmPre + 8 * 4;
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
// Empty asm that takes a value as an in/out operand: the value must be computed at this point
// of the program.  Without it the compiler sinks the softmax arithmetic towards its later uses
// (the next P.V chain), out of the MFMA shadow it was placed in.
template <typename V>
__device__ __forceinline__ void pin(V &x) { asm volatile("" : "+v"(x)); }

struct BlockSm {
    f32x16 s;          // raw scores (masked keys -inf)
    float m0, m1, m2, m3, m4;   // partial maxima
    float bm, mm, thr; // block max, new running max, move threshold
    float mx;          // new reference
    float sum;         // sum of this lane's probabilities
    Update u;
    float x1, p0, p1, h0f;
    uint32_t hp;
    u32x4 phi[2], plo[2];   // P as bf16 pairs: dword k of phi[h] holds keys 8h + 2k, 8h + 2k + 1

    template <int ST>
    __device__ __forceinline__ void stage(SoftmaxRow &sm) {
        if constexpr (ST == 0) {
            m0 = fmax3(s[0], s[1], s[2]);
            m1 = fmax3(s[3], s[4], s[5]);
            pin(m0), pin(m1);
        } else if constexpr (ST == 1) {
            m2 = fmax3(s[6], s[7], s[8]);
            m3 = fmax3(s[9], s[10], s[11]);
            pin(m2), pin(m3);
        } else if constexpr (ST == 2) {
            m4 = fmax3(s[12], s[13], s[14]);
            m0 = fmax3(m0, m1, m2);
            pin(m4), pin(m0);
        } else if constexpr (ST == 3) {
            m0 = fmaxf(fmax3(m0, m3, m4), s[15]);
            pin(m0);
        } else if constexpr (ST == 4) {
            m0 = row_max(m0);
            pin(m0);
        } else if constexpr (ST == 5) {
            bm = m0 * sm.c;
            mm = fmaxf(sm.m_max, bm);
            thr = sm.m_ref + kLazy;
            pin(bm), pin(mm), pin(thr);
        } else if constexpr (ST == 6) {
            // every row of the wave moves when some row's block max passes its reference by
            // more than kLazy (also for the first visible key); -inf stays -inf
            mx = __ballot(bm > thr) != 0 ? mm + kHead : sm.m_ref;
            pin(mx);
        } else if constexpr (ST == 7) {
            // alpha = 1 unless an existing reference moves; no branch
            u.alpha = __builtin_amdgcn_exp2f((mx != sm.m_ref && sm.m_ref != -INFINITY) ? sm.m_ref - mx : 0.f);
            sm.m_ref = mx;
            sm.m_max = mm;
            u.m_use = mx == -INFINITY ? 0.f : mx;
            sum = 0.f;
            pin(u.alpha), pin(u.m_use), pin(sm.m_ref), pin(sm.m_max), pin(sum);
        } else if constexpr (ST < kSmStages) {
            constexpr int k = (ST - kSmPre) / 4, r = (ST - kSmPre) % 4;
            if constexpr (r == 0) {
                const float x0 = __builtin_fmaf(s[2 * k], sm.c, -u.m_use);
                x1 = __builtin_fmaf(s[2 * k + 1], sm.c, -u.m_use);
                p0 = __builtin_amdgcn_exp2f(x0);
                pin(x1), pin(p0);
            } else if constexpr (r == 1) {
                p1 = __builtin_amdgcn_exp2f(x1);
                sum += p0;
                pin(p1), pin(sum);
            } else if constexpr (r == 2) {
                sum += p1;
                hp = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
                h0f = __uint_as_float(hp << 16);
                pin(sum), pin(hp), pin(h0f);
            } else {
                const float l0 = p0 - h0f, l1 = p1 - __uint_as_float(hp & 0xffff0000u);
                uint32_t lp = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){l0, l1}, bf16x2));
                pin(lp);
                phi[k >> 2][k & 3] = hp;
                plo[k >> 2][k & 3] = lp;
            }
        }
    }

};

// Compile-time placement of items [LO, HI) into the steps of a pipeline: item LO + n goes to
// step FIRST + n*EVERY.  `at<K, NSTEPS>` runs the item placed at step K; `tail<NSTEPS>` runs,
// in order, the items whose step would be NSTEPS or later, so every item runs exactly once
// and in order whatever the pipeline length.
template <int LO, int HI, int FIRST, int EVERY>
struct Spread {
    static constexpr int step_of(int n) { return FIRST + n * EVERY; }
    template <int K, int NSTEPS, class F>
    __device__ __forceinline__ static void at(F &&f) {
        constexpr int rel = K - FIRST;
        if constexpr (K < NSTEPS && rel >= 0 && rel % EVERY == 0 && LO + rel / EVERY < HI)
            f(IntC<LO + rel / EVERY>{});
    }
    template <int NSTEPS, class F>
    __device__ __forceinline__ static void tail(F &&f) {
        static_for<LO, HI>([&](auto J) {
            constexpr int n = decltype(J)::value - LO;
            if constexpr (step_of(n) >= NSTEPS) f(J);
        });
    }
};

struct NoFill {
    template <class K>
    __device__ __forceinline__ void operator()(K) const {}
};

// ------------------------------------------------------------------------------ MFMA blocks
// The S^T chain keeps its accumulator in VGPRs (the softmax reads it with VALU ops) while the
// 256 AGPRs hold O^T.  Compiler-selected MFMAs in a kernel that uses AGPRs all write AGPRs,
// which would push part of O^T out, so these MFMAs are written out with explicit register
// classes.  The wait states the compiler would insert are spelled out: none between dependent
// 32x32x16 MFMAs on the same accumulator (also with LDS reads between them; the compiler's own
// chains of the builtin have none), 12 before a VALU instruction reads the result (s_nop 7 +
// s_nop 4 after the last one: 13).  The first MFMA takes srcC = 0.
template <int WAIT>
__device__ __forceinline__ void mfma_s_first(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                 : "=&v"(acc) : "v"(a), "v"(b), "i"(WAIT));
}
template <int WAIT>
__device__ __forceinline__ void mfma_s_next(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+v"(acc) : "v"(a), "v"(b), "i"(WAIT));
}
template <int WAIT>
__device__ __forceinline__ void mfma_s_last(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 4"
                 : "+v"(acc) : "v"(a), "v"(b), "i"(WAIT));
}
// K fragment read for the chain above.  Issued as asm so that the compiler does not add its
// own (full) LDS wait in front of each asm MFMA; the MFMA that consumes the fragment waits
// for it with an exact lgkmcnt.  LDS reads complete in order, so any LDS or scalar-memory
// operation the compiler places in between only makes that count more conservative.
template <int OFF>
__device__ __forceinline__ void ds_read_k(bf16x8 &dst, const LDS_AS char *base) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(base), "i"(OFF));
}

// S^T of both 32-key blocks of a tile x this wave's 32 rows: one chain of 2*NQ MFMA 32x32x16,
// block 0's accumulator first, then block 1's.  The K fragment of step g is read QD steps
// ahead into slot g % (QD+1) -- across the block boundary too, so block 1 starts without
// refilling the pipeline -- and a slot is refilled one MFMA after the one that last read it.
// mid() runs once block 0's scores are final, before the first fill; fill(K) runs after
// block 1's MFMA K.
template <class Sh, int NQ, class Mid, class F>
__device__ __forceinline__ void qk_pair(const LDS_AS char *buf, const bf16x8 (&q)[NQ],
                                        const int (&qk_base)[Sh::CB / 2], f32x16 &s0, f32x16 &s1, Mid &&mid,
                                        F &&fill) {
    constexpr int PAT = Sh::CB / 2;
    constexpr int NG = 2 * NQ;
    constexpr int QD = NQ > 5 ? 5 : NQ - 1, NS = QD + 1;
    static_assert(QD >= 1, "chain of at least two MFMAs per block");
    const LDS_AS char *pq[PAT];
#pragma unroll
    for (int j = 0; j < PAT; j++) pq[j] = buf + qk_base[j];
    bf16x8 kf[NS];
    auto read = [&](auto G) {
        constexpr int g = decltype(G)::value, kb = g / NQ, kk = g % NQ;
        ds_read_k<key_off<Sh>(kb * 32) + (kk / PAT) * 1024>(kf[g % NS], pq[kk % PAT]);
    };
    static_for<0, QD>(read);
    static_for<0, NG>([&](auto G) {
        constexpr int g = decltype(G)::value, kb = g / NQ, kk = g % NQ;
        // loads issued so far: steps < min(NG, g + QD); those after step g may stay in flight
        constexpr int issued = (g + QD < NG) ? g + QD : NG;
        constexpr int after = issued - g - 1;
        f32x16 &acc = kb == 0 ? s0 : s1;
        if constexpr (kk == 0)
            mfma_s_first<after>(acc, kf[g % NS], q[kk]);
        else if constexpr (kk == NQ - 1)
            mfma_s_last<after>(acc, kf[g % NS], q[kk]);
        else
            mfma_s_next<after>(acc, kf[g % NS], q[kk]);
        if constexpr (g + QD < NG) read(IntC<g + QD>{});
        if constexpr (kb == 1) {
            if constexpr (kk == 0) mid();
            fill(IntC<kk>{});                      // independent work for the MFMA shadow
        }
        __builtin_amdgcn_sched_barrier(0);         // keep each step's instructions together
    });
}

// O^T += V^T P^T over both 32-key blocks of a tile: one chain of 2 x 4*NT16 MFMAs.  For each
// 16-key step and 32-column tile, one V^T fragment (two ds_read_b64_tr_b16) feeds the hi and
// the lo MFMA.  Fragments are read PD steps ahead -- across the block boundary too, so block 1
// starts without refilling the pipeline; column tiles go in pairs so consecutive MFMAs use
// different accumulators.  mid() runs between the blocks (after block 0's last MFMA, before
// block 1's first); fill(m) runs after MFMA m (0 .. 8*NT16-1).  P is read at the MFMA that
// uses it, so fill may still be producing keys 16..31 of a block during the first half of
// that block's MFMAs.
template <class Sh, int NT16, class Mid, class F>
__device__ __forceinline__ void pv_pair(const LDS_AS char *buf, const u32x4 (&phi0)[2], const u32x4 (&plo0)[2],
                                        const u32x4 (&phi1)[2], const u32x4 (&plo1)[2], f32x16 (&o)[NT16],
                                        const int (&pv_base)[Sh::CB >= 8 ? Sh::CB / 4 : 1][2], Mid &&mid,
                                        F &&fill) {
    constexpr int NSTEP = 2 * NT16;     // (h16, t16) pairs per block
    constexpr int PD = 4;
    auto load = [&](int st) {
        const int kb = st / NSTEP, sl = st % NSTEP;
        const int h16 = sl / NT16, t16 = sl % NT16;
        const int kbase = kb * 32 + 16 * h16;
        const int j = (4 * t16 % Sh::CB) / 4, cg_off = (4 * t16 / Sh::CB) * 1024 + key_off<Sh>(kbase);
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(buf + pv_base[j][0] + cg_off));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(buf + pv_base[j][1] + cg_off));
        return (bf16x8)__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vf[PD];
#pragma unroll
    for (int j = 0; j < PD; j++) vf[j] = load(j);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NSTEP>([&](auto S2) {     // NSTEP pairs of steps over the two blocks
        constexpr int st = 2 * decltype(S2)::value;
        constexpr int kb = st / NSTEP, sl = st % NSTEP;
        constexpr int h16 = sl / NT16, t16 = sl % NT16, m = 2 * st;
        const u32x4(&phi)[2] = kb == 0 ? phi0 : phi1;
        const u32x4(&plo)[2] = kb == 0 ? plo0 : plo1;
        if constexpr (sl == 0 && kb == 1) {
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
        o[t16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % PD], __builtin_bit_cast(bf16x8, phi[h16]), o[t16], 0, 0, 0);
        fill(IntC<m>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[(st + 1) % PD], __builtin_bit_cast(bf16x8, phi[h16]), o[t16 + 1], 0, 0, 0);
        fill(IntC<m + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % PD], __builtin_bit_cast(bf16x8, plo[h16]), o[t16], 0, 0, 0);
        if constexpr (st + PD < 2 * NSTEP) vf[st % PD] = load(st + PD);
        fill(IntC<m + 2>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[(st + 1) % PD], __builtin_bit_cast(bf16x8, plo[h16]), o[t16 + 1], 0, 0, 0);
        if constexpr (st + 1 + PD < 2 * NSTEP) vf[(st + 1) % PD] = load(st + 1 + PD);
        fill(IntC<m + 3>{});
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Split partials of bf16 requests are stored as 24-bit floats: the top 24 bits of the fp32
// value (sign, exponent, 15 mantissa bits), the magnitude rounded half away from zero by adding
// 0x80 before the low byte is dropped -- relative error <= 2^-16, far inside the 2e-3 output
// tolerance -- 4 values in 3 words, so the partial round trip through memory (the cost of
// splitting keys over workgroups) is a quarter smaller.  Packing is one add per value and one
// v_perm_b32 byte select per word; unpacking one byte select per value.  fp32 requests keep
// plain fp32 partials: 2^-16 of an output of magnitude 1 is already above their 1e-5 tolerance.
// (A finite value cannot carry into infinity: that needs a magnitude above 3.4e38.)
__device__ __forceinline__ void pack24x4(uint32_t *dst, float a, float b, float c, float d) {
    const uint32_t x = __float_as_uint(a) + 0x80u, y = __float_as_uint(b) + 0x80u;
    const uint32_t z = __float_as_uint(c) + 0x80u, w = __float_as_uint(d) + 0x80u;
    // __builtin_amdgcn_perm(hi, lo, sel): byte k of the result is byte sel_k of the 8-byte value
    // hi:lo (0-3 from lo, 4-7 from hi; 12 gives 0)
    dst[0] = __builtin_amdgcn_perm(y, x, 0x05030201u);      // x1 x2 x3 y1
    dst[1] = __builtin_amdgcn_perm(z, y, 0x06050302u);      // y2 y3 z1 z2
    dst[2] = __builtin_amdgcn_perm(w, z, 0x07060503u);      // z3 w1 w2 w3
}
__device__ __forceinline__ float4 unpack24x4(const uint32_t *src) {
    const uint32_t p = src[0], q = src[1], r = src[2];
    return make_float4(__uint_as_float(__builtin_amdgcn_perm(0u, p, 0x0201000Cu)),    // 0 x1 x2 x3
                       __uint_as_float(__builtin_amdgcn_perm(q, p, 0x0504030Cu)),     // 0 y1 y2 y3
                       __uint_as_float(__builtin_amdgcn_perm(r, q, 0x0403020Cu)),     // 0 z1 z2 z3
                       __uint_as_float(__builtin_amdgcn_perm(0u, r, 0x0302010Cu)));   // 0 w1 w2 w3
}

// Store / load of 4 partial values in the format of the input type: kPartWords<T> words each.
template <typename T>
constexpr int kPartWords = std::is_same<T, float>::value ? 4 : 3;
template <typename T>
__device__ __forceinline__ void store_part4(uint32_t *dst, float a, float b, float c, float d) {
    if constexpr (kPartWords<T> == 4)
        *(float4 *)dst = make_float4(a, b, c, d);
    else
        pack24x4(dst, a, b, c, d);
}
template <bool F32>
__device__ __forceinline__ float4 load_part4(const uint32_t *src) {
    if constexpr (F32)
        return *(const float4 *)src;
    else
        return unpack24x4(src);
}

// ---- one-launch path of a one-request batch: plan unit and masks inside the attention
// workgroups (the plan and visibility kernels' results, computed where they are used)

// Work unit the plan kernel gives grid slot u when the batch is one request of L committed
// keys (plan_body with B = 1).  The plan ranks its groups by work, longest first, ties by
// index.  With one request a group's work depends only on its split block gs and never grows
// with gs.  When the tree has Tf places in the split range (see kdt_internal.h) the blocks whose
// bs splits are all full come first, block 0 among them; with none, block 0 (its tree keys on
// top of its share) comes alone before them.  Then come at most one partly filled block, then
// the blocks past the last split.  So the groups of equal work form runs of consecutive gs, and
// within a run the plan's order is the index order (row block major).  Slot -> rank p follows
// the plan's snake dealing; rank p lies in the run that contains gs = p / GR.
// Branch-free, so that the kernel-argument loads it needs go out together at the start.
__device__ __forceinline__ Unit fused_unit(const FusedPlan &f, int64_t chunk, int S, int Tf, int L, uint32_t u) {
    // splits_of without its 64-bit division: lv + chunk - 1 < 2^32 (the host bounds the cache
    // length by 2^30 keys)
    const int64_t lv = (int64_t)(L > 0 ? L : 0) + Tf;
    const uint32_t nsp = fdiv((uint32_t)(lv > 0 ? lv : 1) + (uint32_t)chunk - 1u, f.fd_chunk);
    const int sb = nsp < (uint32_t)S ? (int)nsp : S;
    const uint32_t x = u & (kXcds - 1), k = u >> 3;       // kXcds = 8
    const uint32_t round = fdiv(k, f.fd_per);
    const uint32_t i = k - round * (uint32_t)f.per;
    const uint32_t p = round * kXcds + ((round & 1) ? kXcds - 1 - x : x);
    const int E = (int)fdiv((uint32_t)(sb + f.bs - 1), f.fd_bs);     // blocks with a split
    const int c = (int)fdiv(p, f.fd_gr);
    // blocks 0 .. E-2 are full; block E-1 holds lv - (E-1)*span virtual keys, at least 1 and at
    // most span, as many 64-key tiles as a full block when more than span - 64.  With Tf = 0
    // block 0 is a run of its own.
    const int64_t span = (int64_t)f.bs * chunk;           // a multiple of 64
    const int fe = (lv - (int64_t)(E - 1) * span > span - kKeysPerTile) ? E - 1 : E - 2;   // last full block
    const bool alone = Tf == 0, first = alone && c == 0, in_full = c <= fe, mid = c < E;
    const int lo = first ? 0 : in_full ? (alone ? 1 : 0) : mid ? E - 1 : E;
    const int hi = first ? 0 : in_full ? fe : mid ? E - 1 : f.GS - 1;
    const uint32_t m = (uint32_t)(hi - lo + 1), q = p - (uint32_t)f.GR * (uint32_t)lo;
    // q / m through a float reciprocal: q < G <= 2048, so the estimate is off by at most one
    uint32_t gr = (uint32_t)((float)q * __builtin_amdgcn_rcpf((float)m));
    gr = gr * m > q ? gr - 1 : gr;
    gr = (gr + 1) * m <= q ? gr + 1 : gr;
    const uint32_t gs = (uint32_t)lo + (q - gr * m);
    const uint32_t ib = fdiv(i, f.fd_bs);
    const int rt = (int)(gr * (uint32_t)f.bt + ib), sp = (int)(gs * (uint32_t)f.bs + (i - ib * (uint32_t)f.bs));
    // committed keys [k0, k1): virtual [sp*chunk, (sp+1)*chunk) less the tree's places
    const int64_t v0 = (int64_t)sp * chunk - Tf, v1 = v0 + chunk;
    const int64_t k0 = v0 > 0 ? v0 : 0;
    const int64_t k1e = v1 < (int64_t)L ? v1 : (int64_t)L;
    const int64_t k1 = k1e > k0 ? k1e : k0;
    const bool valid = p < (uint32_t)f.G && rt < f.RT && sp < sb;
    return valid ? Unit{0, rt, sp, sb, (int32_t)k0, (int32_t)k1, k0} : Unit{-1, 0, 0, 0, 0, 0, 0};
}

// One 4-byte-per-lane HBM -> LDS copy: lane l writes its dword at lds_addr + 4l (see lds_dma16).
__device__ __forceinline__ void lds_dma4(const char *base, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 : : "v"(voff), "s"(base), "s"(lds_addr) : "m0");
}

// The masks of the request's N nodes in LDS (msk[k][n] holds word k of node n's final row: zero
// for a node whose path meets a bad parent link), built by fused_masks_wave while the
// workgroup's first copies are in flight.  Word-major, so that the lanes of a wave, which hold
// consecutive nodes, touch consecutive 8-byte words (node-major rows 32 bytes apart put every
// eight lanes on the same banks).
struct FusedVis {
    uint64_t msk[4][kMaxNodes];
    int32_t jmp[kMaxNodes], bad[kMaxNodes];
    int32_t par[kWaves][kMaxNodes];   // each wave's copy of parents[0 .. 255] (past N: the last)
};

// Copies parents[0 .. 64*ceil(N/64)) of request 0 into `par` (entries past N repeat the last),
// one dword copy per 64 nodes, by the calling wave.  Completion is the caller's vmcnt wait.
__device__ __forceinline__ void fused_parents_copy(int32_t *par, const int32_t *parents, int N, int lane) {
    for (int j = 0; j < (N + 63) / 64; j++) {
        const int idx = lane + 64 * j;
        lds_dma4((const char *)parents, (uint32_t)(idx < N ? idx : N - 1) * 4u, (uint32_t)(uintptr_t)&par[64 * j]);
    }
}

// All N masks from V.par[0] by wave 0 alone, which copied it (lane l holds nodes l + 64j, j < 4),
// while the other waves go on; the caller has waited for that copy.  The pointer jumping of visibility_rows, ceil(log2 N) rounds
// through V, in which LDS serves this wave's reads and writes in program order: no barrier.  A
// node keeps its own words in registers; V holds them for the nodes that jump to it.  Nodes
// whose path meets a bad parent link get a zero row.  With masks_out, also writes the [N, W]
// bitmask rows and raises KDT_DEV_BAD_PARENT as kdt_build_visibility does.
__device__ __forceinline__ void fused_masks_wave(FusedVis &V, int N, int W, uint64_t *masks_out, int32_t *dev_status,
                                                 int lane) {
    constexpr int NS = kMaxNodes / 64;
    uint64_t w[NS][4];
    int jmp[NS], bad[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int i = lane + 64 * j;
        jmp[j] = -1;
        bad[j] = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) w[j][k] = k == j ? 1ull << lane : 0ull;
        if (i < N) {
            const int p = V.par[0][i];
            bad[j] = p < -1 || p >= i;
            jmp[j] = bad[j] ? -1 : p;
#pragma unroll
            for (int k = 0; k < 4; k++) V.msk[k][i] = w[j][k];
            V.jmp[i] = jmp[j];
            V.bad[i] = bad[j];
        }
    }
    // after r rounds a node covers 2^r nodes of its path (or all of it); paths have <= N nodes
    for (int n = 1; n < N; n <<= 1) {
        uint64_t add[NS][4];
        int nj[NS], nb[NS];
#pragma unroll
        for (int j = 0; j < NS; j++) {
            nj[j] = -1;
            nb[j] = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) add[j][k] = 0ull;
            if (jmp[j] >= 0) {
#pragma unroll
                for (int k = 0; k < 4; k++) add[j][k] = V.msk[k][jmp[j]];
                nj[j] = V.jmp[jmp[j]];
                nb[j] = V.bad[jmp[j]];
            }
        }
#pragma unroll
        for (int j = 0; j < NS; j++) {
            const int i = lane + 64 * j;
            if (jmp[j] >= 0) {
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    w[j][k] |= add[j][k];
                    V.msk[k][i] = w[j][k];
                }
                bad[j] |= nb[j];
                jmp[j] = nj[j];
                V.jmp[i] = jmp[j];
                V.bad[i] = bad[j];
            }
        }
    }
    bool any_bad = false;
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int i = lane + 64 * j;
        if (i < N) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint64_t v = bad[j] ? 0ull : w[j][k];
                V.msk[k][i] = v;
                if (masks_out && k < W) masks_out[(int64_t)i * W + k] = v;
            }
            any_bad |= bad[j] != 0;
        }
    }
    if (masks_out && dev_status && any_bad) atomicOr(dev_status, (int32_t)KDT_DEV_BAD_PARENT);
}

// All masks of a tree of N <= 64 nodes by pointer jumping in registers, every lane at once: lane
// l holds node l's parent and its own mask word; each round a lane ORs in the word of the node it
// jumps to and takes over that node's jump and bad flag, read with ds_bpermute (a cross-lane
// read through the LDS crossbar, no LDS memory).  ceil(log2 N) rounds cover any path, however
// deep.  Returns lane l's word (zero when its path meets a parent link outside [-1, j-1], the rows
// visibility_rows rejects; zero for lanes >= N).
__device__ __forceinline__ uint64_t masks64_jump(int par, int N, int lane) {
    const bool in = lane < N;
    int bad = in && (par < -1 || par >= lane);
    int jmp = in && !bad ? par : -1;
    uint64_t m = in ? 1ull << lane : 0ull;
    for (int n = 1; n < N; n <<= 1) {
        const int addr = (jmp >= 0 ? jmp : lane) * 4;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)m);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)(uint32_t)(m >> 32));
        const int nj = __builtin_amdgcn_ds_bpermute(addr, jmp);
        const int nb = __builtin_amdgcn_ds_bpermute(addr, bad);
        if (jmp >= 0) {
            m |= ((uint64_t)hi << 32) | lo;
            bad |= nb;
            jmp = nj;
        }
    }
    return bad ? 0ull : m;
}

template <typename T, int DC, int DR, bool FUSED = false>
__global__ __launch_bounds__(256, 1) void verify_attn_kernel(AttnArgs a) {
    using Sh = Shape<T, DC, DR>;
    constexpr int D = Sh::D;
    constexpr int NT16 = DC / 32;                       // 32-wide output column tiles
    constexpr int NQ = Sh::BF16 ? D / 16 : D / 2;       // query fragments per lane
    __shared__ __attribute__((aligned(1024))) char smem[2 * Sh::TILE_BYTES];
    __shared__ std::conditional_t<FUSED, FusedVis, char> fvis;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps LDS bases in SGPRs

    Unit unit;
    bool vis_full = false;          // builds all N masks: every workgroup with tree keys, and the writer
    bool writer = false;            // writes the masks and the plan's device status
    if constexpr (FUSED) {
        // One request: this slot's plan unit from cache_lens[0], as in the 64-row kernel.  Chains
        // (a prefill chunk) make root paths as long as the tree, so the workgroups with tree keys
        // build all masks by pointer jumping (log2 N rounds) rather than walking their nodes' paths.
        fused_parents_copy(fvis.par[wave], a.fp.parents, a.N, lane);
        const int L = a.fp.cache_lens[0];
        const bool ok = L >= 0 && (int64_t)L <= a.fp.max_len && (int64_t)L <= a.fp.total_len;
        unit = ok ? fused_unit(a.fp, a.chunk, a.S, a.tree_keys, L, blockIdx.x) : Unit{-1, 0, 0, 0, 0, 0, 0};
        if (threadIdx.x == 0) {
            a.fp.units[blockIdx.x] = unit;
            if (blockIdx.x == 0) {
                a.fp.hdr->ok = ok ? 1 : 0;
                a.fp.lens[0] = L;
                a.fp.offsets[0] = 0;
                if (!ok && a.fp.dev_status) atomicOr(a.fp.dev_status, (int32_t)KDT_DEV_CACHE_LEN);
            }
        }
        writer = ok ? unit.rt == 0 && unit.s == unit.sb - 1 : blockIdx.x == 0;
        vis_full = writer || (unit.b >= 0 && unit.s == 0);
        if (unit.b < 0) {
            wait_vm_all();          // the parents copy; no copy may still be landing when a workgroup exits
            if (vis_full && wave == 0) fused_masks_wave(fvis, a.N, a.W, a.fp.masks_out, a.fp.dev_status, lane);
            return;
        }
    } else {
        // One scalar load: a slot the plan left empty (or every slot, when it rejected the
        // cache lengths) has b < 0.
        unit = a.units[blockIdx.x];
        if (unit.b < 0) return;
    }
    const int b = unit.b, rt = unit.rt, s = unit.s, sb = unit.sb;
    const int half = lane >> 5;                          // 0: lanes 0-31, 1: lanes 32-63
    const int64_t R = a.R;

    // ---- this lane's query row (lanes l and l+32 share row l%32 of the wave)
    const int64_t r = (int64_t)rt * kRowsPerTile + wave * kRowsPerWave + (lane & 31);
    const bool row_ok = r < R;
    const int64_t rc = row_ok ? r : R - 1;
    const int node = (int)(rc / a.H);
    const T *qlat = (const T *)a.q_lat + ((int64_t)b * R + rc) * a.q_lat_stride;
    const T *qrope = (const T *)a.q_rope + ((int64_t)b * R + rc) * a.q_rope_stride;

    // ---- key ranges: cache keys [k0, k1) of this split, then the tree keys if s == 0
    const int64_t k0 = unit.k0, k1 = unit.k1;
    const int n_cache = k1 > k0 ? (int)(((k1 - k0) + kKeysPerTile - 1) / kKeysPerTile) : 0;
    const int n_tree = (s == 0) ? (a.N + kKeysPerTile - 1) / kKeysPerTile : 0;
    const int n_tiles = n_cache + n_tree;
    const int64_t cache_row0 = unit.row0;

    using Dma = TileDma<Sh, T>;
    auto dma_setup = [&](Dma &d, int t, int bsel) {
        LDS_AS char *buf = (LDS_AS char *)smem + bsel * Sh::TILE_BYTES;
        if (t < n_cache) {
            const int64_t left = k1 - k0 - (int64_t)t * kKeysPerTile;
            d.setup(buf, (const T *)a.ckv, a.ckv_stride, (const T *)a.krope, a.krope_stride,
                    cache_row0 + (int64_t)t * kKeysPerTile, left < kKeysPerTile ? (int)left : kKeysPerTile, wave,
                    lane);
        } else {
            const int tt = t - n_cache;
            const int left = a.N - tt * kKeysPerTile;
            d.setup(buf, (const T *)a.tckv, a.tckv_stride, (const T *)a.tkrope, a.tkrope_stride,
                    (int64_t)b * a.N + (int64_t)tt * kKeysPerTile, left < kKeysPerTile ? left : kKeysPerTile, wave,
                    lane);
        }
    };
    {
        Dma d0;
        dma_setup(d0, 0, 0);
        d0.template issue<0, Dma::NINST>();
    }

    // per-lane LDS byte offsets (see lds_off) of the few swizzle patterns this lane reads
    constexpr int QK_PAT = Sh::CB / 2;                       // K reads: chunk 2kk + half
    constexpr int PV_PAT = Sh::CB >= 8 ? Sh::CB / 4 : 1;     // V^T reads: chunk 4*t16 + y
    int qk_base[QK_PAT], pv_base[PV_PAT][2];
#pragma unroll
    for (int j = 0; j < QK_PAT; j++) qk_base[j] = lds_off<Sh>(lane & 31, 2 * j + half);
    {
        const int w = 4 * half + ((lane & 15) >> 2);              // key within an 8-key group
        const int y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within 4 chunks (32 columns)
#pragma unroll
        for (int j = 0; j < PV_PAT; j++)
#pragma unroll
            for (int e = 0; e < 2; e++) pv_base[j][e] = lds_off<Sh>(w + 8 * e, 4 * j + y) + 8 * (lane & 1);
    }

    // ---- queries to registers: B operand of S^T = K Q^T
    typedef typename std::conditional<Sh::BF16, bf16x8, float>::type QFrag;
    QFrag q[NQ];
    if constexpr (Sh::BF16) {
        // The workgroup's 128 query rows go through LDS: each half (64 rows) is copied into
        // buffer 1 exactly like a key tile (full 128-byte row segments per copy, swizzled 1 KB
        // blocks) while tile 0 lands in buffer 0, and the two waves owning those rows read
        // their fragments with the K-fragment pattern.  Loading the fragments straight from
        // HBM touches 32 rows x 32 bytes per instruction, a quarter of each fetched line.
        LDS_AS char *qbuf = (LDS_AS char *)smem + Sh::TILE_BYTES;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            int64_t first = (int64_t)rt * kRowsPerTile + 64 * h;
            int64_t nrows = R - first;
            if (nrows <= 0) {                  // no row of this half exists: copy a valid one
                first = R - 1;
                nrows = 1;
            }
            Dma dq;
            dq.setup(qbuf, (const T *)a.q_lat, a.q_lat_stride, (const T *)a.q_rope, a.q_rope_stride,
                     (int64_t)b * R + first, nrows < 64 ? (int)nrows : 64, wave, lane);
            if (h == 1) __syncthreads();       // waves 0 and 1 are done reading half 0
            dq.template issue<0, Dma::NINST>();
            if constexpr (FUSED) {
                // the masks while tile 0 and the first query rows land: the parents copy went
                // out before their 2 * NINST copies (loads complete in order).  Up to 64 nodes
                // every wave works them out in registers (the tree tile reads word 0); the
                // writer and larger trees build them in LDS with wave 0.
                const bool regs = !writer && a.N <= 64;
                if (h == 0 && vis_full && (regs || wave == 0)) {
                    asm volatile("s_waitcnt vmcnt(%0)" : : "i"(2 * Dma::NINST) : "memory");
                    if (regs) {
                        const uint64_t mine = masks64_jump(fvis.par[wave][lane], a.N, lane);
                        if (lane < a.N) fvis.msk[0][lane] = mine;
                    } else {
                        fused_masks_wave(fvis, a.N, a.W, writer ? a.fp.masks_out : nullptr,
                                         writer ? a.fp.dev_status : nullptr, lane);
                    }
                }
            }
            wait_vm_all();
            __syncthreads();
            if (wave / 2 == h) {
                const LDS_AS char *src = qbuf + key_off<Sh>(32 * (wave % 2));
#pragma unroll
                for (int kk = 0; kk < NQ; kk++)
                    q[kk] = *(const LDS_AS bf16x8 *)(src + qk_base[kk % QK_PAT] + (kk / QK_PAT) * 1024);
            }
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < NQ; kk++) {
            const int d = 2 * kk + half;
            q[kk] = (2 * kk < DC) ? (float)qlat[d] : (float)qrope[d - DC];
        }
    }

    // Make c = scale*log2(e) positive: a negative scale negates the queries (exact: a sign
    // flip), a zero scale zeroes them (every score is then exactly 0 as with scale 0) and
    // uses c = 1.  Scores then order like scaled scores and masked -inf scores give P = 0.
    float c_pos = a.scale_log2;
    if (c_pos <= 0.f) {
        const bool zero = c_pos == 0.f;
#pragma unroll
        for (int kk = 0; kk < NQ; kk++) q[kk] = zero ? q[kk] * (T)0.f : -q[kk];
        c_pos = zero ? 1.f : -c_pos;
    }

    f32x16 o[NT16];
#pragma unroll
    for (int t = 0; t < NT16; t++) o[t] = (f32x16){};
    SoftmaxRow sm{-INFINITY, -INFINITY, 0.f, c_pos};

    for (int t = 0; t < n_tiles; t++) {
        wait_vm_all();
        __syncthreads();                 // tile t is in LDS; every wave is done with tile t-1
        const LDS_AS char *buf = (const LDS_AS char *)smem + (t & 1) * Sh::TILE_BYTES;

        // ---- which keys of this tile the row sees: a full cache tile needs no mask.  The tree
        // tile's ancestor word is loaded and consumed here, before any copy of tile t+1 is
        // issued: a later first use would make its vmcnt wait cover those copies as well.
        const bool is_tree = t >= n_cache;
        bool need_mask;
        uint32_t w0 = ~0u, w1 = ~0u;
        if (!is_tree) {
            const int64_t left = k1 - k0 - (int64_t)t * kKeysPerTile;
            need_mask = left < kKeysPerTile;
            if (need_mask) {
                const uint64_t vis = (1ull << left) - 1ull;
                w0 = block_bits(vis, 0, half);
                w1 = block_bits(vis, 1, half);
            }
        } else {
            const int tt = t - n_cache;
            const int nvalid = a.N - tt * kKeysPerTile;
            uint64_t vis;
            if constexpr (FUSED)
                vis = fvis.msk[tt][node];
            else
                vis = a.masks[((int64_t)b * a.N + node) * a.W + tt];
            if (nvalid < kKeysPerTile) vis &= (1ull << nvalid) - 1ull;
            w0 = block_bits(vis, 0, half);
            w1 = block_bits(vis, 1, half);
            need_mask = true;
        }
        __builtin_amdgcn_sched_barrier(0);
        // tile t+1 goes into the other buffer
        const bool more = t + 1 < n_tiles;
        Dma dn;

        if constexpr (Sh::BF16) {
            // Two 32-key blocks; every step of the softmax is placed between two MFMAs (see
            // BlockSm).  The first half of a block's softmax (maxima, reference update, keys
            // 0..15) must be done before its P.V chain starts; the second half (keys 16..31)
            // only before the chain's MFMA 2*NT16, so it runs in the first slots of that chain.
            //   QK0, QK1 (one chain)                  QK1 slots: block 0, first half
            //                                         (QK0 is LDS-bound: nothing else)
            //   P.V0: block 0 second half | block 1 first half | copy set-up | copies 0..NINST/2
            //   P.V1: block 1 second half | copies NINST/2..NINST
            // The copy of tile t+1 goes into P.V chains (which leave LDS bandwidth to spare for
            // the copied data to land), at most one per two MFMAs: faster, the copies outrun
            // what one CU can fetch and stall the wave that issues them.  They are issued on
            // every tile so that the chains have no branch: after the last tile they copy that
            // tile again into the idle buffer, and the kernel waits for them before it exits.
            constexpr int NPVM = 4 * NT16;                  // MFMAs per P.V chain
            constexpr int H1 = kSmPre + 16;                 // steps of a softmax first half
            constexpr int NC = Dma::NINST;
            BlockSm b0, b1;
            using A0 = Spread<0, H1, 0, 1>;
            qk_pair<Sh, NQ>(
                buf, q, qk_base, b0.s, b1.s, [&]() { if (need_mask) mask_scores(b0.s, w0); },
                [&](auto K) { A0::template at<decltype(K)::value, NQ>([&](auto J) { b0.template stage<J.value>(sm); }); });
            A0::template tail<NQ>([&](auto J) { b0.template stage<J.value>(sm); });
            if (need_mask) mask_scores(b1.s, w1);
            if (__ballot(b0.u.alpha != 1.f)) rescale_acc<NT16>(o, b0.u.alpha);
            // The second half goes into the chain only if it is done by MFMA 2*NT16 (short
            // chains, small d_c: it runs before the chain instead).
            constexpr bool kIn = kSmStages - H1 <= 2 * NT16;
            constexpr int H1e = kIn ? kSmStages : H1;
            if constexpr (!kIn) static_for<H1, kSmStages>([&](auto J) { b0.template stage<J.value>(sm); });
            using B0 = Spread<H1, H1e, 0, 1>;
            using A1 = Spread<0, H1, kSmStages - H1, 1>;
            constexpr int kSetup = kSmStages;
            using C0 = Spread<0, NC / 2, kSetup + 1, 2>;
            using B1 = Spread<H1, H1e, 0, 1>;
            using C1 = Spread<NC / 2, NC, kSmStages - H1, 2>;
            pv_pair<Sh, NT16>(
                buf, b0.phi, b0.plo, b1.phi, b1.plo, o, pv_base,
                [&]() {
                    // what block 0's slots could not hold (block 1's first half, and its second
                    // half for short chains), then the rare rescale of O for block 1
                    B0::template tail<NPVM>([&](auto J) { b0.template stage<J.value>(sm); });
                    A1::template tail<NPVM>([&](auto J) { b1.template stage<J.value>(sm); });
                    if constexpr (!kIn) static_for<H1, kSmStages>([&](auto J) { b1.template stage<J.value>(sm); });
                    if constexpr (kSetup >= NPVM) dma_setup(dn, more ? t + 1 : t, (t + 1) & 1);
                    C0::template tail<NPVM>([&](auto J) { dn.template issue<J.value, J.value + 1>(); });
                    if (__ballot(b1.u.alpha != 1.f)) rescale_acc<NT16>(o, b1.u.alpha);
                },
                [&](auto K) {
                    constexpr int k = decltype(K)::value;
                    if constexpr (k < NPVM) {           // block 0's P.V
                        B0::template at<k, NPVM>([&](auto J) { b0.template stage<J.value>(sm); });
                        A1::template at<k, NPVM>([&](auto J) { b1.template stage<J.value>(sm); });
                        if constexpr (k == kSetup) dma_setup(dn, more ? t + 1 : t, (t + 1) & 1);
                        C0::template at<k, NPVM>([&](auto J) { dn.template issue<J.value, J.value + 1>(); });
                    } else {                            // block 1's P.V
                        constexpr int k1 = k - NPVM;
                        B1::template at<k1, NPVM>([&](auto J) { b1.template stage<J.value>(sm); });
                        C1::template at<k1, NPVM>([&](auto J) { dn.template issue<J.value, J.value + 1>(); });
                    }
                });
            B1::template tail<NPVM>([&](auto J) { b1.template stage<J.value>(sm); });
            C1::template tail<NPVM>([&](auto J) { dn.template issue<J.value, J.value + 1>(); });
            sm.l = (sm.l * b0.u.alpha + b0.sum) * b1.u.alpha + b1.sum;
        } else {
            if (more) {
                dma_setup(dn, t + 1, (t + 1) & 1);
                dn.template issue<0, Dma::NINST>();
            }
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                // A block that no row of the wave sees (past the last key of a partial tile, or
                // tree keys off every row's path) would add nothing: all its scores are -inf, so
                // P = 0 and the reference stays.  The half-0 lanes' words hold all 32 of its keys.
                if (need_mask && __ballot((kb ? w1 : w0) != 0u) == 0) continue;
                f32x16 sc = (f32x16){};
#pragma unroll
                for (int kk = 0; kk < NQ; kk++) {
                    const int d = 2 * kk + half;
                    const float ka =
                        *(const LDS_AS float *)(buf + lds_off<Sh>(kb * 32 + (lane & 31), d >> 2) + ((d & 3) << 2));
                    sc = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, q[kk], sc, 0, 0, 0);
                }
                if (need_mask) mask_scores(sc, kb ? w1 : w0);
                const Update u = sm.update(sc);
                const float lsum = sm.probs_f32(sc, u);
                sm.l = sm.l * u.alpha + lsum;
                if (__ballot(u.alpha != 1.f)) rescale_acc<NT16>(o, u.alpha);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int key = kb * 32 + (i >> 2) * 8 + 4 * half + (i & 3);
#pragma unroll
                    for (int t16 = 0; t16 < NT16; t16++) {
                        const int dc = t16 * 32 + (lane & 31);
                        const float va =
                            *(const LDS_AS float *)(buf + lds_off<Sh>(key, dc >> 2) + ((dc & 3) << 2));
                        o[t16] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, sc[i], o[t16], 0, 0, 0);
                    }
                }
            }
        }
    }
    wait_vm_all();                       // no copy may still be landing when the workgroup exits
    const float m_run = sm.m_ref, l_run = sm.l;

    // ---- epilogue: lane holds O^T[dc = t16*32 + (i/4)*8 + 4*half + i%4][row]
    const float l_tot = row_sum(l_run);
    if (!row_ok) return;
    if (sb == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *dst = a.out + ((int64_t)b * R + r) * DC;
#pragma unroll
        for (int t16 = 0; t16 < NT16; t16++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 v = make_float4(o[t16][4 * g] * inv, o[t16][4 * g + 1] * inv, o[t16][4 * g + 2] * inv,
                                             o[t16][4 * g + 3] * inv);
                *(float4 *)(dst + t16 * 32 + g * 8 + 4 * half) = v;
            }
    } else {
        // Partials keep the wave's register order: block ((b*S + s)*RT + rt)*4 + wave holds the
        // wave's 32 rows, and the 4 values (t16, g) of lane l, in PW words, sit at words
        // ((t16*4 + g)*64 + l)*PW, so every store instruction writes 64*PW*4 contiguous bytes
        // (the row-major order would write 32 rows x 32 bytes).  The combine reads the same order.
        constexpr int PW = kPartWords<T>;
        const int64_t prow = ((int64_t)b * a.S + s) * R + r;
        const int64_t blk = (((int64_t)b * a.S + s) * a.RT + rt) * kWaves + wave;
        uint32_t *dst = a.part_o + blk * (kRowsPerWave * DC / 4 * PW) + lane * PW;
#pragma unroll
        for (int t16 = 0; t16 < NT16; t16++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                store_part4<T>(dst + (t16 * 4 + g) * 64 * PW, o[t16][4 * g], o[t16][4 * g + 1], o[t16][4 * g + 2],
                               o[t16][4 * g + 3]);
        if (half == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
    }
}

// ------------------------------------------------------------------------------ 64-row workgroups
// Requests that cannot fill the GPU with 128-row workgroups: a decode step (one node x up to 64
// heads), a small tree, or a tree of up to 8192 rows over a short cache (the host's geometry
// picks them).  With the 128-row workgroup above a 64-row request would leave half of the rows empty, and
// every wave would still issue the 200 MFMAs of a 64-key tile: one CU's matrix pipes, not HBM,
// would bound the key stream.  Here a workgroup takes 64 rows and wave w = (key half kh, row
// half rh) takes rows 32*rh .. +31 and keys 32*kh .. +31 of every tile: 36 QK + 64 P.V MFMAs
// per tile and wave instead of 72 + 128, and twice the workgroups for a small tree.  Each wave
// keeps its own online softmax (m, l, O) over its key half; at the end the two key halves of a
// row half are merged through LDS, and the merged wave writes the output or the split partial
// exactly as the 128-row kernel's wave would (the partial layout stays in 128-row tiles and the
// combine is shared).  Same unit records, tile copies, LDS layout, fragment patterns and
// precision (P as bf16 hi + lo) as the 128-row kernel.

// S^T of one 32-key block x this wave's 32 rows: a chain of NQ MFMA 32x32x16 on one
// accumulator, K fragments read QD steps ahead (pq already points at the wave's block).
template <class Sh, int NQ>
__device__ __forceinline__ void qk_block(const LDS_AS char *const (&pq)[Sh::CB / 2], const bf16x8 (&q)[NQ],
                                         f32x16 &acc) {
    constexpr int PAT = Sh::CB / 2;
    constexpr int QD = NQ > 5 ? 5 : NQ - 1, NS = QD + 1;
    static_assert(QD >= 1, "chain of at least two MFMAs");
    bf16x8 kf[NS];
    auto read = [&](auto G) {
        constexpr int g = decltype(G)::value;
        ds_read_k<(g / PAT) * 1024>(kf[g % NS], pq[g % PAT]);
    };
    static_for<0, QD>(read);
    static_for<0, NQ>([&](auto G) {
        constexpr int g = decltype(G)::value;
        constexpr int issued = (g + QD < NQ) ? g + QD : NQ;
        constexpr int after = issued - g - 1;
        if constexpr (g == 0)
            mfma_s_first<after>(acc, kf[g % NS], q[g]);
        else if constexpr (g == NQ - 1)
            mfma_s_last<after>(acc, kf[g % NS], q[g]);
        else
            mfma_s_next<after>(acc, kf[g % NS], q[g]);
        if constexpr (g + QD < NQ) read(IntC<g + QD>{});
        __builtin_amdgcn_sched_barrier(0);
    });
}

// S^T of the same block with MFMA 16x16x32, in two 16-key halves of two 16-row blocks.  A
// 16x16x32 MFMA gives lane l the keys 4*(l/16) + i (i = 0..3) of a half for query row l % 16 of
// a row block: the wave's 32 rows are two row blocks, two accumulators sharing each K fragment.
// With the half's keys taken in the A operand with bits 2 and 3 swapped, the four lane groups
// hold keys 0-3, 8-11, 4-7 and 12-15, and one v_permlane16_swap of the two row blocks'
// registers (odd 16-lane rows of the first operand exchanged with even rows of the second)
// leaves every lane its row l % 32 and keys 8*(i/4) + 4*(l/32) + i%4: the 32x32x16 chain's
// layout, with the same scores bit for bit (checked on the GPU on the Kimi, decode, 7-node,
// outlier, ragged and 128-node shapes).  Used for long key splits, where it measured faster (a
// Kimi-shape launch, 16 tiles per workgroup: 51.4 against 52.3 us, 53.8 against 54.4 us on
// another GPU, 54.2 against 54.9 us against the chain without wait states between its MFMAs);
// on 4-tile splits (a decode step, the 7-node block) the 32x32x16 chain measured
// faster (21.7 against 22.2 us).  Running the first half's softmax steps in the shadow of the
// second half's MFMAs measured slower than both, one step per MFMA or per two: a 16-cycle MFMA
// leaves too few issue slots for them.

// The VGPR-accumulator MFMA of this chain (see the S^T chain above for why asm).  A chain
// alternating two accumulators needs no wait states between MFMAs; WAIT < 0: no LDS wait.
template <int WAIT, bool FIRST>
__device__ __forceinline__ void mfma16_s(f32x4 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (FIRST && WAIT >= 0)
        asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                     : "=&v"(acc) : "v"(a), "v"(b), "i"(WAIT));
    else if constexpr (FIRST)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
    else if constexpr (WAIT >= 0)
        asm volatile("s_waitcnt lgkmcnt(%3)\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                     : "+v"(acc) : "v"(a), "v"(b), "i"(WAIT));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Both halves in one chain of 2*NQ MFMAs: per 32-dim step g of half h, row block 0 then 1 on
// the K fragment of (h, g) (q[2g + rb]); fragments are read QD steps ahead across the half
// boundary.  The scores land in s as the 32x32x16 chain leaves them; a VALU instruction may
// read a 16x16x32 result 8 wait states after the MFMA, 10 are spelled out.
template <class Sh, int NQ>
__device__ __forceinline__ void qk16_block(const LDS_AS char *const (&pk)[2][2], const bf16x8 (&q)[NQ],
                                           f32x16 &s) {
    constexpr int NG = NQ / 2, NT = 2 * NG;
    constexpr int QD = 5, NS = QD + 1;
    static_assert(NQ % 2 == 0 && NG > QD, "whole 32-dim steps, more than the read-ahead");
    bf16x8 kf[NS];
    f32x4 acc[2][2];                    // [half][row block]
    auto read = [&](auto F_) {
        constexpr int f = decltype(F_)::value, h = f / NG, g = f % NG;
        ds_read_k<(g / 2) * 1024>(kf[f % NS], pk[h][g % 2]);
    };
    static_for<0, QD>(read);
    static_for<0, NT>([&](auto F_) {
        constexpr int f = decltype(F_)::value, h = f / NG, g = f % NG;
        constexpr int issued = (f + QD < NT) ? f + QD : NT;      // fragments read before step f
        mfma16_s<issued - f - 1, g == 0>(acc[h][0], kf[f % NS], q[2 * g]);
        // the slot step f-1 read: its last reader was the MFMA before the one just issued
        if constexpr (f + QD < NT) read(IntC<f + QD>{});
        __builtin_amdgcn_sched_barrier(0);
        mfma16_s<-1, g == 0>(acc[h][1], kf[f % NS], q[2 * g + 1]);
        __builtin_amdgcn_sched_barrier(0);
    });
    asm volatile("s_nop 7\n\ts_nop 1" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[h][0][i]),
                                                            __float_as_uint(acc[h][1][i]), false, false);
            s[8 * h + i] = __uint_as_float(x[0]);
            s[8 * h + 4 + i] = __uint_as_float(x[1]);
        }
}

// O^T += V^T P^T over one 32-key block: 2 x 16-key steps x NT16 column tiles x (hi, lo) = 4*NT16
// MFMAs; vbuf already points at the wave's block.  fill(m) runs after MFMA m.  The column tiles
// are taken rotated by NT16/2 when `rot` is the byte distance between column tiles 0 and NT16/2
// (0: not rotated): accumulator t then holds column tile (t + NT16/2) % NT16.
template <class Sh, int NT16, class F>
__device__ __forceinline__ void pv_block(const LDS_AS char *vbuf, int rot, const u32x4 (&phi)[2],
                                         const u32x4 (&plo)[2], f32x16 (&o)[NT16],
                                         const int (&pv_base)[Sh::CB >= 8 ? Sh::CB / 4 : 1][2], F &&fill) {
    constexpr int NSTEP = 2 * NT16;     // (h16, t16) pairs
    constexpr int PD = 4;
    static_assert((2 * NT16) % Sh::CB == 0, "half the column tiles are whole chunk groups");
    const LDS_AS char *vlo = vbuf + rot, *vhi = vbuf - rot;
    auto load = [&](int st) {
        const int h16 = st / NT16, t16 = st % NT16;
        const int j = (4 * t16 % Sh::CB) / 4, cg_off = (4 * t16 / Sh::CB) * 1024 + key_off<Sh>(16 * h16);
        const LDS_AS char *vb = t16 < NT16 / 2 ? vlo : vhi;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(vb + pv_base[j][0] + cg_off));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(vb + pv_base[j][1] + cg_off));
        return (bf16x8)__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vf[PD];
#pragma unroll
    for (int j = 0; j < PD; j++) vf[j] = load(j);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NSTEP / 2>([&](auto S2) {
        constexpr int st = 2 * decltype(S2)::value;
        constexpr int h16 = st / NT16, t16 = st % NT16, m = 2 * st;
        o[t16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % PD], __builtin_bit_cast(bf16x8, phi[h16]), o[t16], 0, 0, 0);
        fill(IntC<m>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[(st + 1) % PD], __builtin_bit_cast(bf16x8, phi[h16]), o[t16 + 1], 0, 0, 0);
        fill(IntC<m + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % PD], __builtin_bit_cast(bf16x8, plo[h16]), o[t16], 0, 0, 0);
        if constexpr (st + PD < NSTEP) vf[st % PD] = load(st + PD);
        fill(IntC<m + 2>{});
        __builtin_amdgcn_sched_barrier(0);
        o[t16 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[(st + 1) % PD], __builtin_bit_cast(bf16x8, plo[h16]), o[t16 + 1], 0, 0, 0);
        if constexpr (st + 1 + PD < NSTEP) vf[(st + 1) % PD] = load(st + 1 + PD);
        fill(IntC<m + 3>{});
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int DC, int DR, bool FUSED = false, bool QK16 = false>
__global__ __launch_bounds__(256, 1) void decode_attn_kernel(AttnArgs a) {
    using T = __bf16;
    using Sh = Shape<T, DC, DR>;
    constexpr int NT16 = DC / 32;
    constexpr int NQ = Sh::D / 16;
    static_assert(Sh::BF16 && Sh::CB == 8, "bf16 rows of 8-chunk LDS blocks");
    __shared__ __attribute__((aligned(1024))) char smem[2 * Sh::TILE_BYTES];
    static_assert(2 * 64 * 256 * 4 + 2 * 64 * 8 <= 2 * Sh::TILE_BYTES, "merge buffers fit in the tile buffers");
    __shared__ std::conditional_t<FUSED, FusedVis, char> fvis;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int64_t R = a.R;
    using Dma = TileDma<Sh, T>;
    // The workgroup's first copies for unit u: tile 0 (its first cache tile, or the tree's
    // first) into buffer 0 and the workgroup's rows (at most 64) into buffer 1, one round trip.
    auto issue_first = [&](const Unit &u) {
        const int64_t q0 = (int64_t)(a.tile_rows == 2 * kRowsPerWave ? u.rt : 0) * 2 * kRowsPerWave;
        const int64_t nq = R - q0 < 2 * kRowsPerWave ? R - q0 : 2 * kRowsPerWave;
        Dma d0, dq;
        LDS_AS char *buf0 = (LDS_AS char *)smem, *buf1 = (LDS_AS char *)smem + Sh::TILE_BYTES;
        if (u.k1 > u.k0) {
            const int64_t left = (int64_t)u.k1 - u.k0;
            d0.setup(buf0, (const T *)a.ckv, a.ckv_stride, (const T *)a.krope, a.krope_stride, u.row0,
                     left < kKeysPerTile ? (int)left : kKeysPerTile, wave, lane);
        } else {
            d0.setup(buf0, (const T *)a.tckv, a.tckv_stride, (const T *)a.tkrope, a.tkrope_stride, (int64_t)u.b * a.N,
                     a.N < kKeysPerTile ? a.N : kKeysPerTile, wave, lane);
        }
        d0.template issue<0, Dma::NINST>();
        dq.setup(buf1, (const T *)a.q_lat, a.q_lat_stride, (const T *)a.q_rope, a.q_rope_stride, (int64_t)u.b * R + q0,
                 (int)nq, wave, lane);
        dq.template issue<0, Dma::NINST>();
    };

    Unit unit;
    bool vis_full = false;          // builds all N masks (see below)
    bool own = false;               // takes tree keys: works out the masks in registers (N <= 64)
    bool writer = false;            // writes the masks and the plan's device status
    if constexpr (FUSED) {
        // the parents go out first (each wave its own copy): they arrive while the plan unit is
        // worked out
        fused_parents_copy(fvis.par[wave], a.fp.parents, a.N, lane);
        // the plan, for this workgroup's slot only (one request: cache_lens[0] is all it reads)
        const int L = a.fp.cache_lens[0];
        const bool ok = L >= 0 && (int64_t)L <= a.fp.max_len && (int64_t)L <= a.fp.total_len;
        unit = ok ? fused_unit(a.fp, a.chunk, a.S, a.tree_keys, L, blockIdx.x) : Unit{-1, 0, 0, 0, 0, 0, 0};
        if (threadIdx.x == 0) {
            a.fp.units[blockIdx.x] = unit;
            if (blockIdx.x == 0) {
                a.fp.hdr->ok = ok ? 1 : 0;
                a.fp.lens[0] = L;
                a.fp.offsets[0] = 0;
                if (!ok && a.fp.dev_status) atomicOr(a.fp.dev_status, (int32_t)KDT_DEV_CACHE_LEN);
            }
        }
        // One workgroup builds all N masks and writes them out: that of row tile 0 and the last
        // split (without tree keys when there are several splits, so it has a tile to spare),
        // or workgroup 0 of a rejected plan; its wave 0 jumps through LDS.  The others with tree
        // keys need them for the tree tiles: for N <= 64 every wave works them out in registers
        // (masks64_jump), for larger trees their wave 0 builds them in LDS too.  Pointer jumping
        // takes log2 N rounds: a walk of each row's path took up to N dependent steps (18 us
        // more for a 128-node chain).
        writer = ok ? unit.rt == 0 && unit.s == unit.sb - 1 : blockIdx.x == 0;
        vis_full = writer || (unit.b >= 0 && unit.s == 0 && a.N > 64);
        own = !vis_full && unit.b >= 0 && unit.s == 0;
        if (unit.b < 0) {
            wait_vm_all();          // the parents copy; no copy may still be landing when a workgroup exits
            if (vis_full && wave == 0) fused_masks_wave(fvis, a.N, a.W, a.fp.masks_out, a.fp.dev_status, lane);
            return;
        }
    } else {
        unit = a.units[blockIdx.x];
        if (unit.b < 0) return;
    }
    const int b = unit.b, s = unit.s, sb = unit.sb;
    // 64-row tile of the unit: unit.rt counts 64-row tiles when the plan was made for them, and
    // is 0 for a request of at most 64 rows under 128-row tiles
    const int rt64 = a.tile_rows == 2 * kRowsPerWave ? unit.rt : 0;
    const int rh = wave & 1, kh = wave >> 1;            // row half, key half
    const int half = lane >> 5;
    const int64_t row0 = (int64_t)rt64 * 2 * kRowsPerWave;          // the workgroup's first row

    const int64_t r = row0 + (int64_t)rh * kRowsPerWave + (lane & 31);
    const bool row_ok = r < R;
    const int64_t rc = row_ok ? r : R - 1;
    const int node = (int)(rc / a.H);

    const int64_t k0 = unit.k0, k1 = unit.k1;
    const int n_cache = k1 > k0 ? (int)(((k1 - k0) + kKeysPerTile - 1) / kKeysPerTile) : 0;
    const int n_tree = (s == 0) ? (a.N + kKeysPerTile - 1) / kKeysPerTile : 0;
    const int n_tiles = n_cache + n_tree;
    const int64_t cache_row0 = unit.row0;

    // copy setup of tile t into buffer bsel
    auto dma_setup = [&](Dma &d, int t, int bsel) {
        LDS_AS char *buf = (LDS_AS char *)smem + bsel * Sh::TILE_BYTES;
        if (t < n_cache) {
            const int64_t left = k1 - k0 - (int64_t)t * kKeysPerTile;
            d.setup(buf, (const T *)a.ckv, a.ckv_stride, (const T *)a.krope, a.krope_stride,
                    cache_row0 + (int64_t)t * kKeysPerTile, left < kKeysPerTile ? (int)left : kKeysPerTile, wave,
                    lane);
        } else {
            const int tt = t - n_cache;
            const int left = a.N - tt * kKeysPerTile;
            d.setup(buf, (const T *)a.tckv, a.tckv_stride, (const T *)a.tkrope, a.tkrope_stride,
                    (int64_t)b * a.N + (int64_t)tt * kKeysPerTile, left < kKeysPerTile ? left : kKeysPerTile, wave,
                    lane);
        }
    };
    LDS_AS char *qbuf = (LDS_AS char *)smem + Sh::TILE_BYTES;
    issue_first(unit);
    if constexpr (FUSED) {
        if (vis_full) {
            // while the copies land: the parents copy went out before the 2*NINST copies of
            // issue_first (loads complete in order)
            if (wave == 0) {
                asm volatile("s_waitcnt vmcnt(%0)" : : "i"(2 * Dma::NINST) : "memory");
                fused_masks_wave(fvis, a.N, a.W, writer ? a.fp.masks_out : nullptr, writer ? a.fp.dev_status : nullptr,
                                 lane);
            }
        } else if (own) {
            // the masks of all N <= 64 nodes (the tree tile reads word 0) while the copies land.
            // This wave's parents copy went out before its last 2*NINST copies (loads complete in
            // order).  Every wave writes the same words.
            asm volatile("s_waitcnt vmcnt(%0)" : : "i"(2 * Dma::NINST) : "memory");
            const uint64_t mine = masks64_jump(fvis.par[wave][lane], a.N, lane);
            if (lane < a.N) fvis.msk[0][lane] = mine;
        }
    }

    constexpr int QK_PAT = Sh::CB / 2;
    constexpr int PV_PAT = Sh::CB / 4;
    // K and Q reads: 32x32x16 chain, lane l reads key (row) l % 32 at 16-byte chunk 2kk + l/32
    // for 16-dim step kk; 16x16x32 chain (qk16_block), lane l reads key l % 16 with bits 2 and
    // 3 swapped (Q: row 16*rb + l % 16 of row block rb) at chunk 4g + l/16 for 32-dim step g
    int qk_base[QK_PAT], k16_base[2], q16_base[2][2], pv_base[PV_PAT][2];
    if constexpr (QK16) {
        const int kperm = (lane & 3) | ((lane & 4) << 1) | ((lane & 8) >> 1);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            k16_base[j] = lds_off<Sh>(kperm, 4 * j + ((lane >> 4) & 3));
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
                q16_base[rb][j] = lds_off<Sh>(16 * rb + (lane & 15), 4 * j + ((lane >> 4) & 3));
        }
    } else {
#pragma unroll
        for (int j = 0; j < QK_PAT; j++) qk_base[j] = lds_off<Sh>(lane & 31, 2 * j + half);
    }
    {
        const int w = 4 * half + ((lane & 15) >> 2);
        const int y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int j = 0; j < PV_PAT; j++)
#pragma unroll
            for (int e = 0; e < 2; e++) pv_base[j][e] = lds_off<Sh>(w + 8 * e, 4 * j + y) + 8 * (lane & 1);
    }
    const int blk_off = kh * key_off<Sh>(32);          // this wave's 32-key block inside a tile
    // key half 1 takes its column tiles rotated by NT16/2 (see the epilogue)
    const int rot = kh * (2 * NT16 / Sh::CB) * 1024;

    bf16x8 q[NQ];                       // 16x16x32 chain: q[2g + rb] for row block rb, 32-dim step g
    wait_vm_all();
    __syncthreads();
    {
        const LDS_AS char *src = qbuf + key_off<Sh>(32 * rh);
#pragma unroll
        for (int kk = 0; kk < NQ; kk++) {
            const int g = kk / 2, rb = kk % 2;
            q[kk] = QK16 ? *(const LDS_AS bf16x8 *)(src + q16_base[rb][g % 2] + (g / 2) * 1024)
                         : *(const LDS_AS bf16x8 *)(src + qk_base[kk % QK_PAT] + (kk / QK_PAT) * 1024);
        }
    }
    float c_pos = a.scale_log2;
    if (c_pos <= 0.f) {
        const bool zero = c_pos == 0.f;
#pragma unroll
        for (int kk = 0; kk < NQ; kk++) q[kk] = zero ? q[kk] * (T)0.f : -q[kk];
        c_pos = zero ? 1.f : -c_pos;
    }

    f32x16 o[NT16];
#pragma unroll
    for (int t = 0; t < NT16; t++) o[t] = (f32x16){};
    SoftmaxRow sm{-INFINITY, -INFINITY, 0.f, c_pos};

    for (int t = 0; t < n_tiles; t++) {
        wait_vm_all();
        __syncthreads();                 // tile t is in LDS; every wave is done with tile t-1 (and Q)
        const LDS_AS char *buf = (const LDS_AS char *)smem + (t & 1) * Sh::TILE_BYTES;
        const bool is_tree = t >= n_cache;
        bool need_mask;
        uint32_t wv = ~0u;
        if (!is_tree) {
            const int64_t left = k1 - k0 - (int64_t)t * kKeysPerTile;
            need_mask = left < kKeysPerTile;
            if (need_mask) wv = block_bits((1ull << left) - 1ull, kh, half);
        } else {
            const int tt = t - n_cache;
            const int nvalid = a.N - tt * kKeysPerTile;
            uint64_t vis;
            if constexpr (FUSED)
                vis = fvis.msk[tt][node];
            else
                vis = a.masks[((int64_t)b * a.N + node) * a.W + tt];
            if (nvalid < kKeysPerTile) vis &= (1ull << nvalid) - 1ull;
            wv = block_bits(vis, kh, half);
            need_mask = true;
        }
        __builtin_amdgcn_sched_barrier(0);
        // tile t+1 goes into the other buffer (after the last tile: tile t again, as a no-op
        // for the result, so that the chain below has no branch)
        const bool more = t + 1 < n_tiles;
        Dma dn;
        dma_setup(dn, more ? t + 1 : t, (t + 1) & 1);

        BlockSm bs;
        if constexpr (QK16) {
            const LDS_AS char *pk[2][2];
#pragma unroll
            for (int j = 0; j < 2; j++) {
                pk[0][j] = buf + blk_off + k16_base[j];
                pk[1][j] = pk[0][j] + key_off<Sh>(16);
            }
            qk16_block<Sh, NQ>(pk, q, bs.s);
        } else {
            const LDS_AS char *pq[QK_PAT];
#pragma unroll
            for (int j = 0; j < QK_PAT; j++) pq[j] = buf + blk_off + qk_base[j];
            qk_block<Sh, NQ>(pq, q, bs.s);
        }
        if (need_mask) mask_scores(bs.s, wv);
        // the first half of the softmax (maxima, reference, keys 0..15) before the P.V chain;
        // keys 16..31 are only read from MFMA 2*NT16 on, so their steps go into the chain
        constexpr int H1 = kSmPre + 16;
        static_for<0, H1>([&](auto J) { bs.template stage<J.value>(sm); });
        if (__ballot(bs.u.alpha != 1.f)) rescale_acc<NT16>(o, bs.u.alpha);
        constexpr int NC = Dma::NINST;
        static_assert(2 * (kSmStages - H1) <= 2 * NT16 && 2 * NC <= 4 * NT16, "steps fit in the chain");
        pv_block<Sh, NT16>(buf + blk_off, rot, bs.phi, bs.plo, o, pv_base, [&](auto M) {
            constexpr int m = decltype(M)::value;
            if constexpr (m % 2 == 1 && H1 + m / 2 < kSmStages) bs.template stage<H1 + m / 2>(sm);
            if constexpr (m % 2 == 0 && m / 2 < NC) dn.template issue<m / 2, m / 2 + 1>();
        });
        sm.l = sm.l * bs.u.alpha + bs.sum;
    }
    wait_vm_all();                       // no copy may still be landing
    __syncthreads();                     // every wave is done with the tile buffers

    // ---- merge the two key halves of each row half.  Wave (rh, kh) accumulated its column tiles
    // rotated by kh * NT16/2: o[0 .. HT) are column tiles kh*HT .. +HT-1, its own half of the
    // output, and o[HT .. NT16) the other wave's half.  Each wave hands that other half and its
    // (m, l) over through LDS, merges its own half, and writes it: all four waves share the
    // epilogue, with register indices fixed at compile time.
    constexpr int HT = NT16 / 2;
    // [rh][sender kh][t][g][lane] float4: each store and load moves 16 contiguous bytes per lane
    float4 *xo = (float4 *)smem;
    float2 *xml = (float2 *)((char *)smem + 2 * 2 * HT * 4 * 64 * 16);     // [rh][kh][64]
    static_assert(2 * 2 * HT * 4 * 64 * 16 + 2 * 2 * 64 * 8 <= 2 * Sh::TILE_BYTES, "exchange fits in the tiles");
#pragma unroll
    for (int t = 0; t < HT; t++)
#pragma unroll
        for (int g = 0; g < 4; g++)
            xo[(((rh * 2 + kh) * HT + t) * 4 + g) * 64 + lane] =
                make_float4(o[HT + t][4 * g], o[HT + t][4 * g + 1], o[HT + t][4 * g + 2], o[HT + t][4 * g + 3]);
    xml[(rh * 2 + kh) * 64 + lane] = make_float2(sm.m_ref, sm.l);
    __syncthreads();
    float m_run, l_run;
    {
        // (m, l) of key halves 0 and 1 in that order in both waves, so both get the same bits
        const float2 ml0 = xml[(rh * 2 + 0) * 64 + lane], ml1 = xml[(rh * 2 + 1) * 64 + lane];
        const float M = fmaxf(ml0.x, ml1.x);
        const float c0 = ml0.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml0.x - M);
        const float c1 = ml1.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml1.x - M);
        l_run = ml0.y * c0 + ml1.y * c1;
        m_run = M;
        const float cs = kh ? c1 : c0, cp = kh ? c0 : c1;       // own half, other half
        const int pk = kh ^ 1;
#pragma unroll
        for (int t = 0; t < HT; t++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 x = xo[(((rh * 2 + pk) * HT + t) * 4 + g) * 64 + lane];
                o[t][4 * g] = o[t][4 * g] * cs + x.x * cp;
                o[t][4 * g + 1] = o[t][4 * g + 1] * cs + x.y * cp;
                o[t][4 * g + 2] = o[t][4 * g + 2] * cs + x.z * cp;
                o[t][4 * g + 3] = o[t][4 * g + 3] * cs + x.w * cp;
            }
    }

    // ---- epilogue of the own half, as the 128-row kernel's wave rh for column tiles
    // kh*HT .. +HT-1: lane holds O^T[(kh*HT + t)*32 + (i/4)*8 + 4*half + i%4][row]
    const float l_tot = row_sum(l_run);
    if (!row_ok) return;
    if (sb == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *dst = a.out + ((int64_t)b * R + r) * DC + kh * HT * 32;
#pragma unroll
        for (int t = 0; t < HT; t++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 v = make_float4(o[t][4 * g] * inv, o[t][4 * g + 1] * inv, o[t][4 * g + 2] * inv,
                                             o[t][4 * g + 3] * inv);
                *(float4 *)(dst + t * 32 + g * 8 + 4 * half) = v;
            }
    } else {
        const int64_t prow = ((int64_t)b * a.S + s) * R + r;
        // 32-row group 2*rt64 + rh of the request = group (rt64 & 1)*2 + rh of 128-row tile rt64/2
        const int64_t blk = (((int64_t)b * a.S + s) * a.RT + (rt64 >> 1)) * kWaves + (rt64 & 1) * 2 + rh;
        constexpr int PW = kPartWords<T>;
        uint32_t *dst = a.part_o + blk * (kRowsPerWave * DC / 4 * PW) + lane * PW + kh * HT * 4 * 64 * PW;
#pragma unroll
        for (int t = 0; t < HT; t++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                store_part4<T>(dst + (t * 4 + g) * 64 * PW, o[t][4 * g], o[t][4 * g + 1], o[t][4 * g + 2],
                               o[t][4 * g + 3]);
        if (half == 0 && kh == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
    }
}

// ------------------------------------------------------------------------------ combine
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s, for rows of split
// requests.  A tile is (request, 32-row group, 32-column tile).  Lane l holds row l % 32 and
// columns 4*(l/32) + 8g .. +3 of the tile (g = 0..3) -- the attention wave's register order,
// so each partial load (4 packed values per lane) is 768 bytes contiguous.  Splits are merged with a running max, U of them in
// flight.  With WS = 1 each wave of a workgroup takes its own tile; with WS = 2 or 4 (more
// splits) WS waves share one tile, wave w of them taking splits w, w+WS, ..., and their
// results are merged in LDS: more waves, fewer loads each, for the same bytes.
template <int DC, int WS, int GC, bool F32P>
__global__ __launch_bounds__(64 * (WS > kWaves ? WS : kWaves)) void combine_kernel(AttnArgs a) {
    constexpr int NT16 = DC / 32;
    constexpr int PW = F32P ? 4 : 3;                  // partial words per 4 values
    constexpr int NSUB = 4 / GC;                      // waves over one tile's 4 column groups
    constexpr int NW = WS > kWaves ? WS : kWaves;     // waves per workgroup
    static_assert((NW % WS == 0 && (NT16 * NSUB) % (NW / WS) == 0) || WS == 1, "tiles of a workgroup share a row group");
    __shared__ float s_m[NW][64], s_den[NW][64], s_acc[NW][4 * GC][64];
    const int lane = threadIdx.x & 63, half = lane >> 5;
    const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wv = wave_id % WS;                      // position among the waves sharing the tile
    const int64_t groups = (a.R + kRowsPerWave - 1) / kRowsPerWave;     // 32-row groups per request
    // a workgroup's NW / WS (sub-)tiles are consecutive column tiles of one row group, so with
    // WS > 1 the exits below are uniform over the workgroup (no wave skips the barrier)
    const int64_t tile = (int64_t)blockIdx.x * (NW / WS) + wave_id / WS;
    if (tile >= (int64_t)a.B * groups * NT16 * NSUB) return;
    const int sub = (int)(tile % NSUB);
    const int t16 = (int)((tile / NSUB) % NT16);
    const int64_t grp = (tile / (NSUB * NT16)) % groups;
    const int b = (int)(tile / (NSUB * NT16 * groups));
    const int64_t r = grp * kRowsPerWave + (lane & 31);
    const bool valid = r < a.R;
    const int64_t rc = valid ? r : a.R - 1;
    const int rt = (int)(grp / kWaves), wave = (int)(grp % kWaves);
    constexpr int U = 8;                              // splits in flight per wave
    float2 ml[U];
    float4 x[U][GC];
    // The first U splits' loads go out before the plan's validity flag and the request's split count
    // arrive (splits the request does not have are read from the workspace and ignored): the
    // merge waits for one memory round trip instead of two.
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int sp = wv + u * WS;
        if (sp < a.S) {
            ml[u] = a.part_ml[((int64_t)b * a.S + sp) * a.R + rc];
            const int64_t blk = (((int64_t)b * a.S + sp) * a.RT + rt) * kWaves + wave;
            const uint32_t *src = a.part_o + blk * (kRowsPerWave * DC / 4 * PW) + lane * PW;
#pragma unroll
            for (int g = 0; g < GC; g++) x[u][g] = load_part4<F32P>(src + (t16 * 4 + sub * GC + g) * 64 * PW);
        }
    }
    const int ok = a.hdr->ok;
    const int sb = splits_of(a.lens[b], a.tree_keys, a.chunk, a.S);
    if (!ok || sb <= 1) return;                       // uniform over the workgroup
    float acc[GC][4];
#pragma unroll
    for (int g = 0; g < GC; g++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[g][j] = 0.f;
    float M = -INFINITY, den = 0.f;
    for (int s0 = wv; s0 < sb; s0 += U * WS) {
        if (s0 != wv) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int sp = s0 + u * WS;
                if (sp < sb) {
                    ml[u] = a.part_ml[((int64_t)b * a.S + sp) * a.R + rc];
                    const int64_t blk = (((int64_t)b * a.S + sp) * a.RT + rt) * kWaves + wave;
                    const uint32_t *src = a.part_o + blk * (kRowsPerWave * DC / 4 * PW) + lane * PW;
#pragma unroll
                    for (int g = 0; g < GC; g++)
                        x[u][g] = load_part4<F32P>(src + (t16 * 4 + sub * GC + g) * 64 * PW);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (s0 + u * WS < sb && ml[u].x != -INFINITY) {   // a split with no visible key adds nothing
                const float mn = fmaxf(M, ml[u].x);
                const float c = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
                const float w = __builtin_amdgcn_exp2f(ml[u].x - mn);
                den = den * c + w * ml[u].y;
#pragma unroll
                for (int g = 0; g < GC; g++) {
                    acc[g][0] = acc[g][0] * c + w * x[u][g].x;
                    acc[g][1] = acc[g][1] * c + w * x[u][g].y;
                    acc[g][2] = acc[g][2] * c + w * x[u][g].z;
                    acc[g][3] = acc[g][3] * c + w * x[u][g].w;
                }
                M = mn;
            }
        }
    }
    float tot = den, o[4 * GC];
#pragma unroll
    for (int g = 0; g < GC; g++)
#pragma unroll
        for (int j = 0; j < 4; j++) o[4 * g + j] = acc[g][j];
    if constexpr (WS > 1) {
        s_m[wave_id][lane] = M;
        s_den[wave_id][lane] = den;
#pragma unroll
        for (int k = 0; k < 4 * GC; k++) s_acc[wave_id][k][lane] = o[k];
        __syncthreads();
        if (wv != 0) return;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = wave_id; w < wave_id + WS; w++) Mx = fmaxf(Mx, s_m[w][lane]);
        tot = 0.f;
#pragma unroll
        for (int k = 0; k < 4 * GC; k++) o[k] = 0.f;
        if (Mx != -INFINITY) {
#pragma unroll
            for (int w = wave_id; w < wave_id + WS; w++) {
                const float mw = s_m[w][lane];
                const float c = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
                tot += c * s_den[w][lane];
#pragma unroll
                for (int k = 0; k < 4 * GC; k++) o[k] += c * s_acc[w][k][lane];
            }
        }
    }
    if (!valid) return;
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    float *dst = a.out + ((int64_t)b * a.R + r) * DC + t16 * 32 + 4 * half;
#pragma unroll
    for (int g = 0; g < GC; g++)
        *(float4 *)(dst + 8 * (sub * GC + g)) =
            make_float4(o[4 * g] * inv, o[4 * g + 1] * inv, o[4 * g + 2] * inv, o[4 * g + 3] * inv);
}

// ------------------------------------------------------------------------------ launchers
static PlanArgs plan_args(const int32_t *cache_lens, const kdt_verify_desc &d, const Geometry &g, void *ws,
                          int32_t *dev_status) {
    char *w = (char *)ws;
    PlanArgs pa;
    pa.cache_lens = cache_lens;
    pa.B = d.batch;
    pa.N = d.num_nodes;
    pa.max_len = d.max_cache_len;
    pa.total_len = d.total_cache_len;
    pa.RT = g.row_tiles;
    pa.S = g.nsplit;
    pa.bt = g.bt;
    pa.bs = g.bs;
    pa.chunk = g.chunk;
    pa.tree_keys = g.tree_keys;
    pa.U = g.units;
    pa.hdr = (WsHeader *)(w + g.off_header);
    pa.offsets = (int64_t *)(w + g.off_offsets);
    pa.lens = (int32_t *)(w + g.off_lens);
    pa.units = (Unit *)(w + g.off_units);
    pa.dev_status = dev_status;
    const int GR = (g.row_tiles + g.bt - 1) / g.bt, GS = (g.nsplit + g.bs - 1) / g.bs;
    pa.fd_chunk = make_fastdiv((uint32_t)g.chunk);
    pa.fd_per = make_fastdiv((uint32_t)(g.bt * g.bs));
    pa.fd_grgs = make_fastdiv((uint32_t)GR * (uint32_t)GS);
    pa.fd_gs = make_fastdiv((uint32_t)GS);
    pa.fd_gr = make_fastdiv((uint32_t)GR);
    pa.fd_bs = make_fastdiv((uint32_t)g.bs);
    return pa;
}

hipError_t launch_plan(const int32_t *cache_lens, const kdt_verify_desc &d, const Geometry &g, void *ws,
                       int32_t *dev_status, hipStream_t st) {
    plan_kernel<<<1, 1024, 0, st>>>(plan_args(cache_lens, d, g, ws, dev_status));
    return hipGetLastError();
}

hipError_t launch_prepare(const int32_t *parents, uint64_t *masks, const int32_t *cache_lens,
                          const kdt_verify_desc &d, const Geometry &g, void *ws, int32_t *dev_status,
                          hipStream_t st) {
    const PlanArgs pa = plan_args(cache_lens, d, g, ws, dev_status);
    const unsigned grid = (unsigned)d.batch + 1;
    switch ((d.num_nodes + 63) / 64) {
        case 1: prepare_kernel<1><<<grid, 256, 0, st>>>(parents, masks, pa); break;
        case 2: prepare_kernel<2><<<grid, 256, 0, st>>>(parents, masks, pa); break;
        case 3: prepare_kernel<3><<<grid, 256, 0, st>>>(parents, masks, pa); break;
        default: prepare_kernel<4><<<grid, 256, 0, st>>>(parents, masks, pa); break;
    }
    return hipGetLastError();
}

// The 64-row kernel's S^T chain: 16x16x32 MFMAs for key splits of at least this many keys (a
// request that splits, so that every unit streams that many), 32x32x16 for shorter ones and
// for requests that do not split (see qk16_block).
constexpr int64_t kQk16MinChunk = 1024;
static bool use_qk16(const AttnArgs &a) { return a.S > 1 && a.chunk >= kQk16MinChunk; }

hipError_t launch_attend(const AttnArgs &a, int d_latent, int d_rope, int dtype, int64_t units, hipStream_t st) {
    const dim3 grid((unsigned)units), block(256);
    const bool kimi_dims = dtype == KDT_BF16 && d_latent == 512 && d_rope == 64;
    // 64-row workgroups: the plan made 64-row tiles, or (128-row tiles of a batch that fills the
    // GPU) a request has at most 64 rows, its one tile at rt = 0
    if (a.tile_rows == 2 * kRowsPerWave) {
        if (!kimi_dims) return hipErrorInvalidValue;
        if (use_qk16(a))
            decode_attn_kernel<512, 64, false, true><<<grid, block, 0, st>>>(a);
        else
            decode_attn_kernel<512, 64><<<grid, block, 0, st>>>(a);
    } else if (kimi_dims && a.R <= 2 * kRowsPerWave)
        decode_attn_kernel<512, 64><<<grid, block, 0, st>>>(a);
    else if (kimi_dims)
        verify_attn_kernel<__bf16, 512, 64><<<grid, block, 0, st>>>(a);
    else if (dtype == KDT_BF16 && d_latent == 64 && d_rope == 16)
        verify_attn_kernel<__bf16, 64, 16><<<grid, block, 0, st>>>(a);
    else if (dtype == KDT_F32 && d_latent == 64 && d_rope == 16)
        verify_attn_kernel<float, 64, 16><<<grid, block, 0, st>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

bool fused_supported(const kdt_verify_desc &d, const Geometry &g) {
    // one bf16 512 + 64 request (either tile size), groups the plan sorts (<= kMaxSortGroups)
    // and work keys that do not saturate (fewer than 0xfffff tiles per group)
    return d.batch == 1 && d.dtype == KDT_BF16 && d.d_latent == 512 && d.d_rope == 64 &&
           g.groups <= kMaxSortGroups && g.units <= INT32_MAX &&
           d.max_cache_len + tree_span(d.num_nodes) < (int64_t)0xfffff * kKeysPerTile;
}

hipError_t launch_attend_fused(AttnArgs a, const kdt_verify_desc &d, const Geometry &g, const int32_t *parents,
                               uint64_t *masks_out, const int32_t *cache_lens, void *ws, int32_t *dev_status,
                               hipStream_t st) {
    if (!fused_supported(d, g)) return hipErrorInvalidValue;
    char *w = (char *)ws;
    FusedPlan &f = a.fp;
    f.parents = parents;
    f.cache_lens = cache_lens;
    f.masks_out = masks_out;
    f.dev_status = dev_status;
    f.hdr = (WsHeader *)(w + g.off_header);
    f.offsets = (int64_t *)(w + g.off_offsets);
    f.lens = (int32_t *)(w + g.off_lens);
    f.units = (Unit *)(w + g.off_units);
    f.max_len = d.max_cache_len;
    f.total_len = d.total_cache_len;
    f.RT = g.row_tiles;
    f.bt = g.bt;
    f.bs = g.bs;
    f.GR = (g.row_tiles + g.bt - 1) / g.bt;
    f.GS = (g.nsplit + g.bs - 1) / g.bs;
    f.G = (int)g.groups;
    f.per = g.bt * g.bs;
    f.fd_chunk = make_fastdiv((uint32_t)g.chunk);
    f.fd_per = make_fastdiv((uint32_t)f.per);
    f.fd_bs = make_fastdiv((uint32_t)f.bs);
    f.fd_gr = make_fastdiv((uint32_t)f.GR);
    if (g.tile_rows == 2 * kRowsPerWave && use_qk16(a))
        decode_attn_kernel<512, 64, true, true><<<dim3((unsigned)g.units), dim3(256), 0, st>>>(a);
    else if (g.tile_rows == 2 * kRowsPerWave)
        decode_attn_kernel<512, 64, true><<<dim3((unsigned)g.units), dim3(256), 0, st>>>(a);
    else
        verify_attn_kernel<__bf16, 512, 64, true><<<dim3((unsigned)g.units), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs &a, int d_latent, int dtype, hipStream_t st) {
    const int64_t tiles = (int64_t)a.B * ((a.R + kRowsPerWave - 1) / kRowsPerWave) * (d_latent / 32);
    // Waves per tile: first more waves share a tile (each keeping at least 4 splits), then a
    // tile's four column groups go to 2 or 4 waves, while the grid stays within about 8 waves
    // per CU (2048 on 256 CUs).  Measured best on the split counts 8, 16 and 32 (the Kimi,
    // 7-node and 16-node shapes): 1 x 4, 4 x 2 and 4 x 4 waves x groups; decode (128 splits,
    // 32 tiles) takes 16 x 1, 1.2 us faster than 8 x 1.
    int ws = 1, gc = 4;
    while (ws < 16 && tiles * ws * 2 <= 2048 && ws * 2 * 4 <= a.S) ws *= 2;
    while (gc > 1 && tiles * ws * (4 / gc) * 2 <= 2048) gc /= 2;
    const int64_t subs = tiles * (4 / gc);
    const int nw = ws > kWaves ? ws : kWaves;
    const int64_t tpb = nw / ws;
    const unsigned grid = (unsigned)((subs + tpb - 1) / tpb);
    const unsigned block = (unsigned)(64 * nw);
    auto go = [&](auto dc, auto gcv, auto f32p) {
        constexpr int DCv = decltype(dc)::value, GC = decltype(gcv)::value;
        constexpr bool F = decltype(f32p)::value;
        switch (ws) {
            case 16: combine_kernel<DCv, 16, GC, F><<<grid, block, 0, st>>>(a); break;
            case 8: combine_kernel<DCv, 8, GC, F><<<grid, block, 0, st>>>(a); break;
            case 4: combine_kernel<DCv, 4, GC, F><<<grid, block, 0, st>>>(a); break;
            case 2: combine_kernel<DCv, 2, GC, F><<<grid, block, 0, st>>>(a); break;
            default: combine_kernel<DCv, 1, GC, F><<<grid, block, 0, st>>>(a); break;
        }
    };
    auto go_dc = [&](auto dc, auto f32p) {
        if (gc == 4) go(dc, std::integral_constant<int, 4>{}, f32p);
        else if (gc == 2) go(dc, std::integral_constant<int, 2>{}, f32p);
        else go(dc, std::integral_constant<int, 1>{}, f32p);
    };
    if (d_latent == 512 && dtype == KDT_BF16) {
        go_dc(std::integral_constant<int, 512>{}, std::false_type{});
    } else if (d_latent == 64 && dtype == KDT_BF16) {
        go_dc(std::integral_constant<int, 64>{}, std::false_type{});
    } else if (d_latent == 64 && dtype == KDT_F32) {
        go_dc(std::integral_constant<int, 64>{}, std::true_type{});
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kdt
