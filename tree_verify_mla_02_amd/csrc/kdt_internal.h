// Internal declarations of libkdt shared by the C-ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "kdt.h"

namespace kdt {

// Work decomposition of the verify attention.
//   A work unit is (request b, row tile rt, key split s).  A row tile is 128 query rows
//   (4 waves x 32 rows, rows node-major r = i*H + h).  Split 0 of every request also owns its
//   tree segment.  The keys of a request are split as one range of L + Tf "virtual" keys, Tf
//   committed-key places given to the tree, then its L committed-cache keys: split s takes
//   virtual keys [s*chunk, (s+1)*chunk), that is cache keys [s*chunk - Tf, (s+1)*chunk - Tf)
//   (from 0 for split 0).  Tf = tree_span(N) for trees of more than one 64-key tile, so that
//   split 0, tree included, does no more tiles than the others; 0 for one-tile trees, whose
//   tile split 0 does on top of its share (chunk >= Tf always).
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerTile = kWaves * kRowsPerWave;   // 128
constexpr int kKeysPerTile = 64;                       // one LDS tile = 64 keys
constexpr int kMaxNodes = 256;                         // 4 mask words
#ifndef KDT_MIN_CHUNK
#define KDT_MIN_CHUNK 256
#endif
constexpr int kMinChunk = KDT_MIN_CHUNK;               // keys per split at least (a multiple of 64)
static_assert(kMinChunk % 64 == 0 && kMinChunk >= 64, "whole key tiles per split");
constexpr int kMaxTreeTable = 8192;                    // tree builder: D * K log probabilities in LDS
constexpr int kXcds = 8;                               // MI355X: 8 XCDs, each with its own L2

// Keys of the tree segment as the attention takes them: whole 64-key tiles.
constexpr int64_t tree_span(int N) { return (int64_t)kKeysPerTile * ((N + kKeysPerTile - 1) / kKeysPerTile); }

struct Geometry {
    int64_t rows;          // R = N * H query rows per request
    int tile_rows;         // query rows per workgroup: 128, or 64 for small requests (see make_geometry)
    int row_tiles;         // RT = ceil(R / tile_rows): row tiles of the unit list
    int layout_tiles;      // ceil(R / 128): 128-row tiles of the split-partial layout
    int nsplit;            // S: splits per request at most (1 = no split)
    int64_t chunk;         // virtual keys (tree places, then committed keys) per split
    int tree_keys;         // Tf: committed-key places the tree takes in split 0
    int64_t units;         // grid size of the attention kernel: 8 * ceil(G / 8) * bt * bs slots
    int bt, bs;            // a plan group: bt row tiles x bs splits of one request
    int64_t groups;        // G = B * ceil(RT / bt) * ceil(S / bs)
    int mask_words;        // W = ceil(N / 64)
    // workspace layout (byte offsets, 256-aligned)
    size_t off_header, off_offsets, off_lens, off_units, off_ml, off_o, total_bytes;
};

// Records `code` and `msg` as the calling thread's last status and error (kdt_last_status,
// kdt_last_error) and returns code.
int set_error(int code, const char *msg);

// Fills g from desc for a device with `num_cus` compute units.  Returns false on overflow.
bool make_geometry(const kdt_verify_desc &d, int num_cus, Geometry *g);

// Workspace header written by the plan kernel.
struct WsHeader {
    int32_t ok;            // 1 when cache_lens passed the device checks
    int32_t pad[63];
};

// One workgroup's share of the attention, written by the plan: everything the kernel needs
// to start, in one 32-byte scalar load.  b < 0 marks an empty grid slot (also every slot
// when the plan rejected cache_lens).
struct Unit {
    int32_t b, rt, s, sb;      // request, row tile, split, splits of that request
    int32_t k0, k1;            // cache keys [k0, k1) of this split, request-relative
    int64_t row0;              // packed-cache row of key k0
};
static_assert(sizeof(Unit) == 32, "one 32-byte record");

// Division by a divisor fixed for the launch (see fdiv in verify_attn.hip).
struct FastDiv {
    uint32_t d, m, l;
};

// What the one-launch path (masks, plan and attention of a one-request batch in one attention
// launch) needs beyond AttnArgs: the inputs of the masks and the plan, where the plan kernel
// would have written its results, and the plan's group shape (see make_geometry).
struct FusedPlan {
    const int32_t *parents, *cache_lens;
    uint64_t *masks_out;
    int32_t *dev_status;
    WsHeader *hdr;
    int64_t *offsets;
    int32_t *lens;
    Unit *units;
    int64_t max_len, total_len;
    int RT, bt, bs, GR, GS, G, per;     // RT: row tiles of the unit list
    FastDiv fd_chunk, fd_per, fd_bs, fd_gr;
};

struct AttnArgs {
    const void *q_lat, *q_rope, *ckv, *krope, *tckv, *tkrope;
    const uint64_t *masks;
    float *out;
    int64_t q_lat_stride, q_rope_stride, ckv_stride, krope_stride, tckv_stride, tkrope_stride;
    int B, N, H, W;
    int64_t R;
    int RT, S;             // RT: 128-row tiles of the partial layout
    int tile_rows;         // 128: verify_attn_kernel; 64: the 64-row kernel (unit rt counts 64-row tiles)
    int64_t chunk;
    int tree_keys;         // Tf (see above)
    float scale_log2;      // scale * log2(e): scores are kept in the base-2 domain
    const WsHeader *hdr;
    const int64_t *offsets;
    const int32_t *lens;
    const Unit *units;     // one per grid slot
    float2 *part_ml;       // [B][S][R] (running max in log2 domain, sum)
    uint32_t *part_o;      // un-normalised partial outputs, per wave in register order: block
                           // ((b*S + s)*RT + rt)*4 + wave of 32 rows x d_c values, as packed
                           // 24-bit floats (bf16 inputs) or plain fp32 (fp32 inputs)
    FusedPlan fp;          // one-launch path only
};

hipError_t launch_visibility(const int32_t *parents, int B, int N, uint64_t *masks,
                             int32_t *dev_status, hipStream_t st);
hipError_t launch_plan(const int32_t *cache_lens, const kdt_verify_desc &d, const Geometry &g,
                       void *ws, int32_t *dev_status, hipStream_t st);
hipError_t launch_prepare(const int32_t *parents, uint64_t *masks, const int32_t *cache_lens,
                          const kdt_verify_desc &d, const Geometry &g, void *ws, int32_t *dev_status,
                          hipStream_t st);
hipError_t launch_attend(const AttnArgs &a, int d_latent, int d_rope, int dtype, int64_t units,
                         hipStream_t st);
hipError_t launch_combine(const AttnArgs &a, int d_latent, int dtype, hipStream_t st);
// Masks, plan and attention of a one-request batch in one launch (64- or 128-row workgroups, as
// the geometry says); `a` as for launch_attend.  fused_supported says whether desc and g allow it.
bool fused_supported(const kdt_verify_desc &d, const Geometry &g);
hipError_t launch_attend_fused(AttnArgs a, const kdt_verify_desc &d, const Geometry &g, const int32_t *parents,
                               uint64_t *masks_out, const int32_t *cache_lens, void *ws, int32_t *dev_status,
                               hipStream_t st);

// 32-bit words of split-partial storage per 4 output values: 3 (24-bit floats) for bf16
// inputs, 4 (fp32) for fp32 inputs.
constexpr int partial_words(int dtype) { return dtype == KDT_F32 ? 4 : 3; }
hipError_t launch_accept(const int32_t *parents, const int32_t *tokens, const int32_t *target_next,
                         const int32_t *root_next, int B, int N, int32_t *path, int32_t *accept_len,
                         int32_t *bonus, hipStream_t st);
hipError_t launch_tree_build(const float *logp, const int32_t *cand, int B, int D, int K, int N,
                             int32_t *parents, int32_t *tokens, int32_t *depth, int32_t *rank, hipStream_t st);
hipError_t launch_compact(const void *ckv, const void *krope, const int32_t *cache_lens, const void *tree_ckv,
                          const void *tree_krope, const int32_t *path, const int32_t *accept_len, void *ckv_out,
                          void *krope_out, int32_t *new_lens, int64_t capacity, const kdt_verify_desc &d,
                          int32_t *dev_status, hipStream_t st);

}  // namespace kdt
