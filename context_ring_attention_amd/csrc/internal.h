// Internal declarations shared by the host side of libcpattn and its kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "cpattn.h"

namespace cpattn {

// Tile geometry of each kernel.  The bf16 kernel runs 4 waves per work-group
// (one per SIMD), each wave owning 64 query tokens of one head; heads_per_tile
// waves share a token block, so a tile covers 64 * 4 / heads_per_tile tokens.
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

// Validate metadata (host arrays).  On failure sets the thread's error text.
cpattn_status validate_metadata(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                                const int32_t* k_off, int32_t nseq, int32_t hq, int32_t hkv,
                                int32_t d);

// Number of plan entries for these query lengths and this geometry.
int64_t count_entries(const int32_t* cu_q, int32_t nseq, int tokens_per_tile);

// Fill `out` (n entries, sorted longest first) and optionally the stats.
void build_entries(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                   const int32_t* k_off, int32_t nseq, int32_t causal, const Geometry& g,
                   cpattn_plan_entry* out, int64_t n, cpattn_plan_info* info);

cpattn_status set_error(cpattn_status s, const char* fmt, ...);

// Kernel launchers (defined in the .hip files).  They assume validated input.
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v,
                                const cpattn_plan_entry* plan, int n_entries, int head_groups,
                                int heads_per_tile, int hq, int hkv, int d, int tq_total,
                                float* o, float* lse, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v,
                               const cpattn_plan_entry* plan, int n_entries, int hq, int hkv,
                               int d, int tq_total, float* o, float* lse, hipStream_t stream);
hipError_t launch_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                        int64_t t, int hq, int d, hipStream_t stream);

}  // namespace cpattn
