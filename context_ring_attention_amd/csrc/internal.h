// Internal declarations shared by the host side of libcpattn and its kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "cpattn.h"

namespace cpattn {

// Tile geometry of each kernel.  The bf16 kernel runs 4 waves per work-group
// (one per SIMD), each wave owning 32 query tokens of one head; heads_per_tile
// waves share a token block, so a tile covers 32 * 4 / heads_per_tile tokens.
// The fp32 kernel runs one head and 64 tokens per work-group.
constexpr int kBf16Waves = 4;
constexpr int kBf16RowsPerWave = 32;
constexpr int kBf16BlockN = 64;
constexpr int kF32TokensPerTile = 64;
constexpr int kF32BlockN = 32;
// Smallest token block of any geometry (bounds the number of plan entries).
constexpr int kMinTileTokens = kBf16RowsPerWave < kF32TokensPerTile ? kBf16RowsPerWave : kF32TokensPerTile;

struct Geometry {
  int tokens_per_tile;
  int heads_per_tile;
  int block_n;
};

Geometry geometry_for(cpattn_dtype dtype, int hq, int hkv);

// Validate metadata of nchunks chunks (host arrays; cu_k is [nchunks][nseq + 1],
// k_off [nchunks][nseq] or null).  On failure sets the thread's error text.
cpattn_status validate_metadata(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                                const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t hq,
                                int32_t hkv, int32_t d);

// Number of (sequence, token block) tiles for these query lengths and this geometry.
int64_t count_tiles(const int32_t* cu_q, int32_t nseq, int tokens_per_tile);

// Fill `out` (n_tiles * nchunks entries, tile-major, tiles sorted by total cost,
// longest first; may be null) and optionally the stats.
void build_entries(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                   const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                   const Geometry& g, cpattn_plan_entry* out, int64_t n_tiles,
                   cpattn_plan_info* info);

// Backward, key-stationary kernel (dK, dV): a work-group owns kBwdKeysPerTile keys of one
// kv head (kBwdWaves waves in two pairs, kPairKeys keys a pair) and streams the query tokens
// that see them, in blocks of kBwdQueryBlock, for every query head of the kv head's group.
constexpr int kBwdWaves = 4;
constexpr int kPairKeys = 48;
constexpr int kBwdKeysPerTile = kPairKeys * kBwdWaves / 2;
constexpr int kBwdQueryBlock = 32;

// One tile of the key-stationary plan: kBwdKeysPerTile keys of one sequence in one chunk
// (the record cpattn_key_plan_build exports).
using KeyTile = cpattn_key_tile;
static_assert(sizeof(KeyTile) == 32, "plan records are 32 bytes");

// One work-group's share of a key tile in the dK/dV launch: query heads [h_begin, h_end) of
// the kv head's group (the whole group, or half of it when the tile is split).  The two halves
// of a split tile each leave their partial dK/dV in scratch slot `part` of split unit
// split * hkv + kvh, and the second to finish adds both and folds them into dK/dV.
constexpr int kMinSplitSteps = 1024;
struct KeyPart {
  int32_t row0, nrows, q_start, q_len, delta, cost, chunk;
  int32_t h_begin, h_end, split, part, reserved;
};
static_assert(sizeof(KeyPart) == 48, "key parts are 48 bytes");

// Number of (chunk, sequence, key block) tiles of the key-stationary plan (cu_k is
// [nchunks][nseq + 1]).
int64_t count_key_tiles(const int32_t* cu_k, int32_t nchunks, int32_t nseq);

// The dK/dV launch's parts from the key plan (tiles sorted longest first): a tile of at least
// kMinSplitSteps steps (cost x group) that exceeds a quarter of the ideal per-slot share of all
// steps (slots = work-groups the GPU runs at once) is split into its group's two halves of
// query heads, up to max_split tiles; parts sorted by steps, longest first.  Writes at most 2 n_tiles parts,
// returns their number and the number of split tiles in *n_split.
int64_t build_key_parts(const KeyTile* tiles, int64_t n_tiles, int group, int hkv, int slots,
                        int64_t max_split, KeyPart* out, int64_t* n_split);

// Key-stationary plan over nchunks chunks, sorted by cost, longest first.
void build_key_entries(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                       const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                       KeyTile* out, int64_t n_tiles);

// Metadata of a forward call passed by value to the device planner: cu_q [nseq + 1], q_off
// [nseq], then per chunk cu_k [nseq + 1] and k_off [nseq].  Calls whose metadata does not fit,
// or whose plan has more than kPlanDeviceMaxTiles token tiles, build their plan on the host and
// copy it instead.
constexpr int kPlanMetaInts = 480;
constexpr int kPlanDeviceMaxTiles = 4096;
struct PlanMeta {
  int32_t nseq, nchunks, causal, tt, bn, n_tiles;
  int32_t v[kPlanMetaInts];
};
// Fill m for these arguments; false if they do not fit (or nseq == 0, or n_tiles is too large).
bool fill_plan_meta(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                    const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                    const Geometry& g, int64_t n_tiles, PlanMeta* m);
// Writes build_entries' plan (n_tiles * nchunks entries) into device memory `out` on `stream`.
hipError_t launch_plan_device(const PlanMeta& m, cpattn_plan_entry* out, hipStream_t stream);

// Device pointers of the chunks of one launch (passed by value as a kernel argument).
template <class T>
struct ChunkPtrs {
  const T* k[CPATTN_MAX_CHUNKS];
  const T* v[CPATTN_MAX_CHUNKS];
};

cpattn_status set_error(cpattn_status s, const char* fmt, ...);

// Body of the forward entry points (api.cpp): validation, plan, upload into `workspace` on
// `stream`, launch.  The plan is built into host_buf (host_cap bytes) if one is given, else
// into a buffer of the call's own.
cpattn_status fwd_impl(const void* q, const void* const* ks, const void* const* vs,
                       int32_t nchunks, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       const int32_t* q_pos_offset, const int32_t* k_pos_offset, int32_t nseq,
                       int32_t hq, int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                       int32_t accumulate, float* o, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, char* host_buf,
                       size_t host_cap);

// The Dynamic CP scheduler behind cpattn_dcp_schedule (dcp.cpp).
cpattn_status dcp_schedule(const int32_t* lengths, int32_t n, int32_t world, int32_t limit,
                           int32_t* cp_size, int32_t* micro_batch, int32_t* group_rank,
                           int32_t* slot, int32_t* n_micro_batches);

// Kernel launchers (defined in the .hip files).  They assume validated input.
// plan holds n_tiles * nchunks entries (tile-major); accumulate folds the result
// into (o, lse) instead of overwriting them.
hipError_t launch_attn_fwd_bf16(const void* q, const ChunkPtrs<__bf16>& kv, int nchunks,
                                const cpattn_plan_entry* plan, int n_tiles, int head_groups,
                                int heads_per_tile, int hq, int hkv, int d, int tq_total,
                                bool accumulate, float* o, float* lse, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const float* q, const ChunkPtrs<float>& kv, int nchunks,
                               const cpattn_plan_entry* plan, int n_tiles, int hq, int hkv, int d,
                               int tq_total, bool accumulate, float* o, float* lse,
                               hipStream_t stream);
// Backward launchers: delta = rowsum(dO * O) into delta [hq, tq] (and the LSE in log2 units);
// then one gradient launch with dQ over the query plan (tile-major over nchunks chunks, as the
// forward's) and dK, dV over the key parts.
hipError_t launch_bwd_delta(const void* do_, const float* o, const float* lse, int tq, int hq,
                            int d, float* delta, float* lse2, hipStream_t stream);
// Arguments of the gradient launch (dQ and dK/dV work-groups in one grid).  qplan holds n_tiles
// * nchunks entries (tile-major, as the forward's); kplan the key parts; counters (one int per
// split unit, zero on entry) and scratch (two slots of bwd_part_floats(d) floats per split
// unit) serve the split key tiles.
struct BwdArgs {
  const void* q;
  const void* dout;
  ChunkPtrs<__bf16> kv;
  ChunkPtrs<float> dkv;
  const float* lse;
  const float* lse2;
  const float* delta;
  const cpattn_plan_entry* qplan;
  const KeyPart* kplan;
  int* counters;
  float* scratch;
  float* dq;
  int nchunks, head_groups, heads_per_tile, hq, hkv, tq;
};
// order[b] names work-group b of the launch: a dQ work-group (tile * head_groups + head
// group), or a dK/dV work-group (part * hkv + kv head) with kDkdvBit set.
constexpr uint32_t kDkdvBit = 0x80000000u;
hipError_t launch_bwd_fused(const BwdArgs& a, const uint32_t* order, int n_wg, bool split, int d,
                            hipStream_t stream);
// Floats of one partial dK/dV slot (a work-group's 96 keys x d, both gradients).
constexpr int64_t bwd_part_floats(int d) { return int64_t(2) * kBwdKeysPerTile * d; }
hipError_t launch_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                        int64_t t, int hq, int d, hipStream_t stream);

}  // namespace cpattn
