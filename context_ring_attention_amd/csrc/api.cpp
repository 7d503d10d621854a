// C ABI of libcpattn: argument checks, plan upload, kernel dispatch.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

namespace cpattn {
const char* last_error_text();
void clear_error();

namespace {

// Every call builds its plan on the host and copies it into the caller's device workspace on
// the caller's stream, ahead of the launches that read it; the library holds no memory and no
// state between calls.  The host copy is pageable: the runtime has taken the bytes when
// hipMemcpyAsync returns, so the buffer can go at once.  A stream being captured into a graph
// is refused, since a captured copy would re-read that freed host buffer on every replay.
cpattn_status stage_plan(void* dst, const char* host, size_t bytes, hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "hipStreamIsCapturing failed");
  if (cap != hipStreamCaptureStatusNone)
    return set_error(CPATTN_ERR_UNSUPPORTED,
                     "the stream is being captured: the plan upload reads host memory that is "
                     "freed when the call returns");
  if (bytes == 0) return CPATTN_OK;
  const hipError_t err = hipMemcpyAsync(dst, host, bytes, hipMemcpyHostToDevice, stream);
  if (err != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "plan upload failed: %s", hipGetErrorString(err));
  return CPATTN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" {

const char* cpattn_status_string(cpattn_status s) {
  switch (s) {
    case CPATTN_OK: return "ok";
    case CPATTN_ERR_INVALID_ARG: return "invalid argument";
    case CPATTN_ERR_UNSUPPORTED: return "unsupported";
    case CPATTN_ERR_WORKSPACE: return "workspace too small";
    case CPATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* cpattn_last_error(void) { return last_error_text(); }

size_t cpattn_workspace_size_chunks(int32_t nseq, const int32_t* cu_seqlens_q, int32_t hq,
                                    int32_t hkv, int32_t d, int32_t nchunks) {
  (void)d;
  if (nseq < 0 || hq < 1 || hkv < 1 || (nseq > 0 && !cu_seqlens_q)) return 0;
  if (nchunks < 1 || nchunks > CPATTN_MAX_CHUNKS) return 0;
  for (int32_t i = 0; i < nseq; ++i)
    if (cu_seqlens_q[i + 1] < cu_seqlens_q[i]) return 0;
  // The smallest token block of any geometry bounds the tile count.
  const int64_t n = count_tiles(cu_seqlens_q, nseq, kMinTileTokens);
  return std::max<size_t>(256, size_t(n) * nchunks * sizeof(cpattn_plan_entry));
}

size_t cpattn_workspace_size(int32_t nseq, const int32_t* cu_seqlens_q, int32_t hq, int32_t hkv,
                             int32_t d) {
  return cpattn_workspace_size_chunks(nseq, cu_seqlens_q, hq, hkv, d, 1);
}

cpattn_status cpattn_plan_build_chunks(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                       int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                       int32_t d, cpattn_dtype dtype, int32_t causal,
                                       cpattn_plan_entry* plan, size_t plan_bytes,
                                       cpattn_plan_info* info) {
  clear_error();
  if (dtype != CPATTN_BF16 && dtype != CPATTN_FP32)
    return set_error(CPATTN_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  cpattn_status st = validate_metadata(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset,
                                       nchunks, nseq, hq, hkv, d);
  if (st != CPATTN_OK) return st;
  const Geometry g = geometry_for(dtype, hq, hkv);
  const int64_t n = count_tiles(cu_seqlens_q, nseq, g.tokens_per_tile);
  if (n * nchunks > int64_t(INT32_MAX))
    return set_error(CPATTN_ERR_UNSUPPORTED, "too many plan entries");
  const size_t need = size_t(n) * nchunks * sizeof(cpattn_plan_entry);
  if (plan && plan_bytes < need)
    return set_error(CPATTN_ERR_WORKSPACE, "plan buffer of %zu bytes, need %zu", plan_bytes, need);
  build_entries(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal, g,
                plan, n, info);
  if (info) {
    info->head_groups = hq / g.heads_per_tile;
    info->n_tiles = int32_t(n * info->head_groups);
  }
  return CPATTN_OK;
}

cpattn_status cpattn_key_plan_build(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                    int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                    int32_t d, int32_t causal, cpattn_key_tile* plan,
                                    size_t plan_bytes, cpattn_key_plan_info* info) {
  clear_error();
  cpattn_status st = validate_metadata(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset,
                                       nchunks, nseq, hq, hkv, d);
  if (st != CPATTN_OK) return st;
  const int64_t n = count_key_tiles(cu_seqlens_k, nchunks, nseq);
  if (n > int64_t(INT32_MAX)) return set_error(CPATTN_ERR_UNSUPPORTED, "too many key tiles");
  const size_t need = size_t(n) * sizeof(cpattn_key_tile);
  if (plan && plan_bytes < need)
    return set_error(CPATTN_ERR_WORKSPACE, "plan buffer of %zu bytes, need %zu", plan_bytes, need);
  if (plan)
    build_key_entries(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq,
                      causal, plan, n);
  if (info) {
    info->n_tiles = int32_t(n);
    info->keys_per_tile = kBwdKeysPerTile;
    info->query_block = kBwdQueryBlock;
    info->reserved = 0;
  }
  return CPATTN_OK;
}

cpattn_status cpattn_plan_build_device(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                       int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                       int32_t d, cpattn_dtype dtype, int32_t causal,
                                       cpattn_plan_entry* plan, size_t plan_bytes,
                                       hipStream_t stream) {
  clear_error();
  if (dtype != CPATTN_BF16 && dtype != CPATTN_FP32)
    return set_error(CPATTN_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  cpattn_status st = validate_metadata(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset,
                                       nchunks, nseq, hq, hkv, d);
  if (st != CPATTN_OK) return st;
  const Geometry g = geometry_for(dtype, hq, hkv);
  const int64_t n = count_tiles(cu_seqlens_q, nseq, g.tokens_per_tile);
  const size_t need = size_t(n) * nchunks * sizeof(cpattn_plan_entry);
  if (!plan || plan_bytes < need || !aligned(plan, 16))
    return set_error(CPATTN_ERR_WORKSPACE, "plan buffer of %zu bytes, need %zu (16-byte aligned)",
                     plan_bytes, need);
  PlanMeta meta;
  if (!fill_plan_meta(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal,
                      g, n, &meta))
    return set_error(CPATTN_ERR_UNSUPPORTED, "%d sequences x %d chunks (%lld token tiles) exceed the "
                     "device planner's limits", nseq, nchunks, (long long)n);
  const hipError_t err = launch_plan_device(meta, plan, stream);
  if (err != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "plan kernel launch failed: %s", hipGetErrorString(err));
  return CPATTN_OK;
}

cpattn_status cpattn_dcp_schedule(const int32_t* lengths, int32_t n, int32_t world,
                                  int32_t max_seqlen_per_rank, int32_t* cp_size,
                                  int32_t* micro_batch, int32_t* group_rank, int32_t* slot,
                                  int32_t* n_micro_batches) {
  clear_error();
  return dcp_schedule(lengths, n, world, max_seqlen_per_rank, cp_size, micro_batch, group_rank,
                      slot, n_micro_batches);
}

cpattn_status cpattn_plan_build(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                                cpattn_dtype dtype, int32_t causal, cpattn_plan_entry* plan,
                                size_t plan_bytes, cpattn_plan_info* info) {
  return cpattn_plan_build_chunks(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, 1, nseq,
                                  hq, hkv, d, dtype, causal, plan, plan_bytes, info);
}

}  // extern "C"

namespace cpattn {

// Shared body of the attention entry points.  The plan is built into host_buf (host_cap bytes)
// when one is given, else into a buffer of its own.
cpattn_status fwd_impl(const void* q, const void* const* ks, const void* const* vs,
                       int32_t nchunks, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       const int32_t* q_pos_offset, const int32_t* k_pos_offset, int32_t nseq,
                       int32_t hq, int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                       int32_t accumulate, float* o, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, char* host_buf,
                       size_t host_cap) {
  clear_error();
  if (dtype != CPATTN_BF16 && dtype != CPATTN_FP32)
    return set_error(CPATTN_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (accumulate != 0 && accumulate != 1)
    return set_error(CPATTN_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (nchunks >= 1 && nchunks <= CPATTN_MAX_CHUNKS && (!ks || !vs))
    return set_error(CPATTN_ERR_INVALID_ARG, "chunk pointer arrays must be non-null");
  cpattn_status st = validate_metadata(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset,
                                       nchunks, nseq, hq, hkv, d);
  if (st != CPATTN_OK) return st;
  const int64_t tq = cu_seqlens_q[nseq];
  if (tq == 0) return CPATTN_OK;  // nothing to write
  const size_t esz = dtype == CPATTN_BF16 ? 2 : 4;
  if (!q || !o || !lse) return set_error(CPATTN_ERR_INVALID_ARG, "q, o and lse must be non-null");
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return set_error(CPATTN_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned and lse 4-byte aligned");
  const size_t q_bytes = size_t(tq) * hq * d * esz;
  const size_t o_bytes = size_t(tq) * hq * d * 4, lse_bytes = size_t(tq) * hq * 4;
  if (overlaps(o, o_bytes, q, q_bytes) || overlaps(lse, lse_bytes, o, o_bytes) ||
      overlaps(lse, lse_bytes, q, q_bytes))
    return set_error(CPATTN_ERR_INVALID_ARG, "o/lse must not overlap q, k, v or each other");
  for (int32_t c = 0; c < nchunks; ++c) {
    const int64_t tk = cu_seqlens_k[int64_t(c) * (nseq + 1) + nseq];
    if (tk == 0) continue;
    if (!ks[c] || !vs[c])
      return set_error(CPATTN_ERR_INVALID_ARG, "k and v must be non-null (chunk %d)", c);
    if (!aligned(ks[c], 16) || !aligned(vs[c], 16))
      return set_error(CPATTN_ERR_INVALID_ARG, "q/k/v/o must be 16-byte aligned and lse 4-byte aligned");
    const size_t kv_bytes = size_t(tk) * hkv * d * esz;
    if (overlaps(o, o_bytes, ks[c], kv_bytes) || overlaps(o, o_bytes, vs[c], kv_bytes) ||
        overlaps(lse, lse_bytes, ks[c], kv_bytes) || overlaps(lse, lse_bytes, vs[c], kv_bytes))
      return set_error(CPATTN_ERR_INVALID_ARG, "o/lse must not overlap q, k, v or each other");
  }

  const Geometry g = geometry_for(dtype, hq, hkv);
  const int64_t n = count_tiles(cu_seqlens_q, nseq, g.tokens_per_tile);
  const size_t plan_bytes = size_t(n) * nchunks * sizeof(cpattn_plan_entry);
  if (!workspace || workspace_bytes < plan_bytes || !aligned(workspace, 256))
    return set_error(CPATTN_ERR_WORKSPACE, "workspace of %zu bytes (need %zu, 256-byte aligned)",
                     workspace_bytes, plan_bytes);
  const int head_groups = hq / g.heads_per_tile;
  if (n * head_groups > int64_t(INT32_MAX) || n * nchunks > int64_t(INT32_MAX))
    return set_error(CPATTN_ERR_UNSUPPORTED, "too many tiles for one launch");

  // The plan region of the workspace is written by the upload: it must not overlap a tensor.
  if (overlaps(workspace, plan_bytes, q, q_bytes) || overlaps(workspace, plan_bytes, o, o_bytes) ||
      overlaps(workspace, plan_bytes, lse, lse_bytes))
    return set_error(CPATTN_ERR_INVALID_ARG, "the workspace must not overlap q, o or lse");
  for (int32_t c = 0; c < nchunks; ++c) {
    const int64_t tk = cu_seqlens_k[int64_t(c) * (nseq + 1) + nseq];
    const size_t kv_bytes = size_t(tk) * hkv * d * esz;
    if (overlaps(workspace, plan_bytes, ks[c], kv_bytes) ||
        overlaps(workspace, plan_bytes, vs[c], kv_bytes))
      return set_error(CPATTN_ERR_INVALID_ARG, "the workspace must not overlap k or v (chunk %d)", c);
  }

  // The plan: built on the device from the metadata passed by value when it fits the planner's
  // kernel argument (nothing crosses from host memory at run time, so the call also works under
  // graph capture), else built here and copied.
  PlanMeta meta;
  hipError_t err;
  if (fill_plan_meta(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal,
                     g, n, &meta)) {
    err = launch_plan_device(meta, static_cast<cpattn_plan_entry*>(workspace), stream);
    if (err != hipSuccess)
      return set_error(CPATTN_ERR_HIP, "plan kernel launch failed: %s", hipGetErrorString(err));
  } else {
    std::vector<char> own;
    if (!host_buf) {
      own.resize(plan_bytes);
      host_buf = own.data();
    } else if (host_cap < plan_bytes) {
      return set_error(CPATTN_ERR_WORKSPACE, "plan of %zu bytes exceeds the %zu-byte staging buffer",
                       plan_bytes, host_cap);
    }
    build_entries(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal, g,
                  reinterpret_cast<cpattn_plan_entry*>(host_buf), n, nullptr);
    st = stage_plan(workspace, host_buf, plan_bytes, stream);
    if (st != CPATTN_OK) return st;
  }
  const auto* plan = static_cast<const cpattn_plan_entry*>(workspace);
  if (dtype == CPATTN_BF16) {
    ChunkPtrs<__bf16> kv{};
    for (int32_t c = 0; c < nchunks; ++c) {
      kv.k[c] = static_cast<const __bf16*>(ks[c]);
      kv.v[c] = static_cast<const __bf16*>(vs[c]);
    }
    err = launch_attn_fwd_bf16(q, kv, nchunks, plan, int(n), head_groups, g.heads_per_tile, hq,
                               hkv, d, int(tq), accumulate != 0, o, lse, stream);
  } else {
    ChunkPtrs<float> kv{};
    for (int32_t c = 0; c < nchunks; ++c) {
      kv.k[c] = static_cast<const float*>(ks[c]);
      kv.v[c] = static_cast<const float*>(vs[c]);
    }
    err = launch_attn_fwd_f32(static_cast<const float*>(q), kv, nchunks, plan, int(n), hq, hkv, d,
                              int(tq), accumulate != 0, o, lse, stream);
  }
  if (err != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "attention launch failed: %s", hipGetErrorString(err));
  return CPATTN_OK;
}

}  // namespace cpattn

extern "C" {

cpattn_status cpattn_fwd_chunk(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                               int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                               cpattn_dtype dtype, int32_t causal, float* o, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(q, &k, &v, 1, cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nseq, hq,
                  hkv, d, dtype, causal, 0, o, lse, workspace, workspace_bytes, stream, nullptr, 0);
}

cpattn_status cpattn_fwd_chunk_accum(const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                     int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                                     cpattn_dtype dtype, int32_t causal, float* o, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(q, &k, &v, 1, cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nseq, hq,
                  hkv, d, dtype, causal, 1, o, lse, workspace, workspace_bytes, stream, nullptr, 0);
}

cpattn_status cpattn_fwd_chunks(const void* q, const void* const* ks, const void* const* vs,
                                int32_t nchunks, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                                const int32_t* k_pos_offset, int32_t nseq, int32_t hq, int32_t hkv,
                                int32_t d, cpattn_dtype dtype, int32_t causal, int32_t accumulate,
                                float* o, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return fwd_impl(q, ks, vs, nchunks, cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nseq,
                  hq, hkv, d, dtype, causal, accumulate, o, lse, workspace, workspace_bytes, stream,
                  nullptr, 0);
}

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the backward, each region 256-byte aligned: the query plan, the dK/dV launch's
// key parts (at most two per key tile) and the split tiles' counters (one per split unit,
// zeroed), all uploaded by the call; delta and the log2-scaled LSE (written by the delta
// kernel); and the split tiles' partial dK/dV (two slots per split unit), sized for every tile
// being split.
struct BwdLayout {
  int64_t n_q, n_k, units, n_wg;    // query plan entries, key tiles, split units (n_k * hkv),
                                    // work-groups of the gradient launch (bounds)
  size_t key_plan_at, counters_at, order_at, plan_bytes;   // uploaded: [0, plan_bytes)
  size_t delta_at, lse2_at, scratch_at, total;
};

// n_q32: query tiles of 32 tokens (the smallest tile), which bounds the dQ work-groups by
// n_q32 * hq.
BwdLayout bwd_layout(int64_t n_q32, int32_t nchunks, int64_t n_k, int64_t tq, int32_t hq,
                     int32_t hkv, int32_t d) {
  BwdLayout l;
  l.n_q = n_q32 * nchunks;
  l.n_k = n_k;
  l.units = n_k * hkv;
  l.n_wg = n_q32 * hq + 2 * n_k * hkv;
  l.key_plan_at = align256(size_t(l.n_q) * sizeof(cpattn_plan_entry));
  l.counters_at = align256(l.key_plan_at + size_t(2 * n_k) * sizeof(KeyPart));
  l.order_at = align256(l.counters_at + size_t(l.units) * sizeof(int32_t));
  l.plan_bytes = l.order_at + size_t(l.n_wg) * sizeof(uint32_t);
  l.delta_at = align256(l.plan_bytes);
  l.lse2_at = align256(l.delta_at + size_t(tq) * hq * sizeof(float));
  l.scratch_at = align256(l.lse2_at + size_t(tq) * hq * sizeof(float));
  l.total = std::max<size_t>(256, l.scratch_at + size_t(l.units) * 2 * bwd_part_floats(d) * sizeof(float));
  return l;
}
}  // namespace

size_t cpattn_bwd_workspace_size_chunks(int32_t nseq, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k, int32_t nchunks, int32_t hq,
                                        int32_t hkv, int32_t d) {
  if (nseq < 0 || hq < 1 || hkv < 1 || nchunks < 1 || nchunks > CPATTN_MAX_CHUNKS) return 0;
  if (d != 64 && d != 128) return 0;
  if (nseq > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return 0;
  for (int32_t i = 0; i < nseq; ++i)
    if (cu_seqlens_q[i + 1] < cu_seqlens_q[i]) return 0;
  for (int32_t c = 0; c < nchunks; ++c)
    for (int32_t i = 0; i < nseq; ++i)
      if (cu_seqlens_k[int64_t(c) * (nseq + 1) + i + 1] < cu_seqlens_k[int64_t(c) * (nseq + 1) + i])
        return 0;
  const int64_t tq = nseq > 0 ? cu_seqlens_q[nseq] : 0;
  return bwd_layout(count_tiles(cu_seqlens_q, nseq, kMinTileTokens), nchunks,
                    count_key_tiles(cu_seqlens_k, nchunks, nseq), tq, hq, hkv, d).total;
}

size_t cpattn_bwd_workspace_size(int32_t nseq, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t hq, int32_t hkv, int32_t d) {
  return cpattn_bwd_workspace_size_chunks(nseq, cu_seqlens_q, cu_seqlens_k, 1, hq, hkv, d);
}

cpattn_status cpattn_bwd_chunks(const void* q, const void* const* ks, const void* const* vs,
                                int32_t nchunks, const float* o, const void* do_,
                                const float* lse, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                                const int32_t* k_pos_offset, int32_t nseq, int32_t hq,
                                int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                                float* dq, float* const* dks, float* const* dvs, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (dtype != CPATTN_BF16 && dtype != CPATTN_FP32)
    return set_error(CPATTN_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (nchunks >= 1 && nchunks <= CPATTN_MAX_CHUNKS && (!ks || !vs || !dks || !dvs))
    return set_error(CPATTN_ERR_INVALID_ARG, "chunk pointer arrays must be non-null");
  cpattn_status st = validate_metadata(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset,
                                       nchunks, nseq, hq, hkv, d);
  if (st != CPATTN_OK) return st;
  if (dtype != CPATTN_BF16)
    return set_error(CPATTN_ERR_UNSUPPORTED, "the backward takes bf16 inputs only");
  const int64_t tq = cu_seqlens_q[nseq];
  if (tq == 0) return CPATTN_OK;  // no query, nothing to add
  if (!q || !o || !do_ || !lse || !dq)
    return set_error(CPATTN_ERR_INVALID_ARG, "every tensor must be non-null");
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(do_, 16) || !aligned(lse, 4) || !aligned(dq, 16))
    return set_error(CPATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned and lse 4-byte aligned");
  const size_t qb = size_t(tq) * hq * d * 2;
  const size_t of = size_t(tq) * hq * d * 4, lb = size_t(tq) * hq * 4;
  // Every output region against every input region and every other output region.
  std::vector<const void*> in_p = {q, o, do_, lse};
  std::vector<size_t> in_b = {qb, of, qb, lb};
  std::vector<const void*> out_p = {dq};
  std::vector<size_t> out_b = {of};
  for (int32_t c = 0; c < nchunks; ++c) {
    const int64_t tk = cu_seqlens_k[int64_t(c) * (nseq + 1) + nseq];
    if (tk == 0) continue;
    if (!ks[c] || !vs[c] || !dks[c] || !dvs[c])
      return set_error(CPATTN_ERR_INVALID_ARG, "chunk %d: k, v, dk and dv must be non-null", c);
    if (!aligned(ks[c], 16) || !aligned(vs[c], 16) || !aligned(dks[c], 16) || !aligned(dvs[c], 16))
      return set_error(CPATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned and lse 4-byte aligned");
    const size_t kb = size_t(tk) * hkv * d * 2, kf = size_t(tk) * hkv * d * 4;
    in_p.push_back(ks[c]); in_b.push_back(kb);
    in_p.push_back(vs[c]); in_b.push_back(kb);
    out_p.push_back(dks[c]); out_b.push_back(kf);
    out_p.push_back(dvs[c]); out_b.push_back(kf);
  }
  for (size_t a = 0; a < out_p.size(); ++a) {
    for (size_t b = 0; b < in_p.size(); ++b)
      if (overlaps(out_p[a], out_b[a], in_p[b], in_b[b]))
        return set_error(CPATTN_ERR_INVALID_ARG, "gradients must not overlap any input");
    for (size_t b = a + 1; b < out_p.size(); ++b)
      if (overlaps(out_p[a], out_b[a], out_p[b], out_b[b]))
        return set_error(CPATTN_ERR_INVALID_ARG, "gradients must not overlap each other");
  }
  const Geometry g = geometry_for(CPATTN_BF16, hq, hkv);
  const int64_t n_qt = count_tiles(cu_seqlens_q, nseq, g.tokens_per_tile);
  const BwdLayout lay = bwd_layout(count_tiles(cu_seqlens_q, nseq, kMinTileTokens), nchunks,
                                   count_key_tiles(cu_seqlens_k, nchunks, nseq), tq, hq, hkv, d);
  if (!workspace || workspace_bytes < lay.total || !aligned(workspace, 256))
    return set_error(CPATTN_ERR_WORKSPACE, "workspace of %zu bytes (need %zu, 256-byte aligned)",
                     workspace_bytes, lay.total);
  const int head_groups = hq / g.heads_per_tile;
  if (n_qt * head_groups > int64_t(INT32_MAX) || lay.n_k * hkv > int64_t(INT32_MAX) ||
      n_qt * nchunks > int64_t(INT32_MAX))
    return set_error(CPATTN_ERR_UNSUPPORTED, "too many tiles for one launch");
  char* ws = static_cast<char*>(workspace);
  for (size_t a = 0; a < out_p.size(); ++a)
    if (overlaps(out_p[a], out_b[a], ws, lay.total))
      return set_error(CPATTN_ERR_INVALID_ARG, "the workspace must not overlap the gradients");

  for (size_t b = 0; b < in_p.size(); ++b)
    if (overlaps(in_p[b], in_b[b], ws, lay.total))
      return set_error(CPATTN_ERR_INVALID_ARG, "the workspace must not overlap an input");

  // Work-groups the GPU runs at once in the dK/dV launch (two per CU), for its balance.
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return set_error(CPATTN_ERR_HIP, "cannot read the device's compute-unit count");
  std::vector<char> host(lay.plan_bytes, 0);   // counters start at zero
  build_entries(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal, g,
                reinterpret_cast<cpattn_plan_entry*>(host.data()), n_qt, nullptr);
  std::vector<KeyTile> tiles(size_t(lay.n_k));
  build_key_entries(cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nchunks, nseq, causal,
                    tiles.data(), lay.n_k);
  int64_t n_split = 0;
  const int64_t n_parts =
      build_key_parts(tiles.data(), lay.n_k, hq / hkv, hkv, 2 * cus, lay.n_k,
                      reinterpret_cast<KeyPart*>(host.data() + lay.key_plan_at), &n_split);
  if (n_parts * hkv > int64_t(INT32_MAX))
    return set_error(CPATTN_ERR_UNSUPPORTED, "too many tiles for one launch");
  // The gradient launch's order: dQ tiles (head_groups work-groups each) and dK/dV parts (hkv
  // work-groups each), both plans already longest first, merged by estimated work per
  // work-group: a dQ block is 3 products over 64 keys x 128 query rows, a dK/dV step 4
  // products over 32 queries x 96 keys (in units of 2 D FLOPs).
  const auto* qents = reinterpret_cast<const cpattn_plan_entry*>(host.data());
  const auto* kps = reinterpret_cast<const KeyPart*>(host.data() + lay.key_plan_at);
  auto* order = reinterpret_cast<uint32_t*>(host.data() + lay.order_at);
  auto dq_work = [&](int64_t e) {
    int64_t blocks = 0;
    for (int32_t c = 0; c < nchunks; ++c) blocks += qents[e * nchunks + c].cost;
    return double(blocks) * 3.0 * kBf16BlockN * kBf16RowsPerWave * kBf16Waves;
  };
  auto kv_work = [&](int64_t p) {
    return double(kps[p].cost) * (kps[p].h_end - kps[p].h_begin) * 4.0 * kBwdQueryBlock *
           kBwdKeysPerTile;
  };
  int64_t n_wg = 0;
  for (int64_t e = 0, p = 0; e < n_qt || p < n_parts;) {
    if (p >= n_parts || (e < n_qt && dq_work(e) >= kv_work(p))) {
      for (int h = 0; h < head_groups; ++h) order[n_wg++] = uint32_t(e * head_groups + h);
      ++e;
    } else {
      for (int h = 0; h < hkv; ++h) order[n_wg++] = kDkdvBit | uint32_t(p * hkv + h);
      ++p;
    }
  }
  if (n_wg > int64_t(INT32_MAX) || n_qt * head_groups >= int64_t(kDkdvBit) ||
      n_parts * hkv >= int64_t(kDkdvBit))
    return set_error(CPATTN_ERR_UNSUPPORTED, "too many tiles for one launch");
  st = stage_plan(ws, host.data(), host.size(), stream);
  if (st != CPATTN_OK) return st;
  BwdArgs a{};
  a.q = q;
  a.dout = do_;
  for (int32_t c = 0; c < nchunks; ++c) {
    a.kv.k[c] = static_cast<const __bf16*>(ks[c]);
    a.kv.v[c] = static_cast<const __bf16*>(vs[c]);
    a.dkv.k[c] = dks[c];
    a.dkv.v[c] = dvs[c];
  }
  a.lse = lse;
  a.lse2 = reinterpret_cast<float*>(ws + lay.lse2_at);
  a.delta = reinterpret_cast<float*>(ws + lay.delta_at);
  a.qplan = reinterpret_cast<const cpattn_plan_entry*>(ws);
  a.kplan = reinterpret_cast<const KeyPart*>(ws + lay.key_plan_at);
  a.counters = reinterpret_cast<int*>(ws + lay.counters_at);
  a.scratch = reinterpret_cast<float*>(ws + lay.scratch_at);
  a.dq = dq;
  a.nchunks = nchunks;
  a.head_groups = head_groups;
  a.heads_per_tile = g.heads_per_tile;
  a.hq = hq;
  a.hkv = hkv;
  a.tq = int(tq);
  hipError_t err = launch_bwd_delta(do_, o, lse, int(tq), hq, d, reinterpret_cast<float*>(ws + lay.delta_at),
                                    reinterpret_cast<float*>(ws + lay.lse2_at), stream);
  if (err == hipSuccess)
    err = launch_bwd_fused(a, reinterpret_cast<const uint32_t*>(ws + lay.order_at), int(n_wg),
                           n_split > 0, d, stream);
  if (err != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(err));
  return CPATTN_OK;
}

cpattn_status cpattn_bwd_chunk(const void* q, const void* k, const void* v, const float* o,
                               const void* do_, const float* lse, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                               const int32_t* k_pos_offset, int32_t nseq, int32_t hq,
                               int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                               float* dq, float* dk, float* dv, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return cpattn_bwd_chunks(q, &k, &v, 1, o, do_, lse, cu_seqlens_q, cu_seqlens_k, q_pos_offset,
                           k_pos_offset, nseq, hq, hkv, d, dtype, causal, dq, &dk, &dv, workspace,
                           workspace_bytes, stream);
}

cpattn_status cpattn_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                           int64_t t, int32_t hq, int32_t d, hipStream_t stream) {
  clear_error();
  if (t < 0 || hq < 1 || d < 4 || d > 256 || (d & (d - 1)) != 0)
    return set_error(CPATTN_ERR_INVALID_ARG, "merge needs t >= 0, hq >= 1, d a power of two in [4, 256]");
  if (t == 0) return CPATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b)
    return set_error(CPATTN_ERR_INVALID_ARG, "merge buffers must be non-null");
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(lse_a, 4) || !aligned(lse_b, 4))
    return set_error(CPATTN_ERR_INVALID_ARG, "o must be 16-byte and lse 4-byte aligned");
  const size_t ob = size_t(t) * hq * d * 4, lb = size_t(t) * hq * 4;
  if (overlaps(o_a, ob, o_b, ob) || overlaps(o_a, ob, lse_b, lb) || overlaps(lse_a, lb, o_b, ob) ||
      overlaps(lse_a, lb, lse_b, lb) || overlaps(o_a, ob, lse_a, lb))
    return set_error(CPATTN_ERR_INVALID_ARG, "merge inputs must not overlap");
  if (t * int64_t(hq) * (d / 4) > (int64_t(1) << 40))
    return set_error(CPATTN_ERR_UNSUPPORTED, "merge too large");
  hipError_t err = launch_merge(o_a, lse_a, o_b, lse_b, t, hq, d, stream);
  if (err != hipSuccess)
    return set_error(CPATTN_ERR_HIP, "merge launch failed: %s", hipGetErrorString(err));
  return CPATTN_OK;
}

}  // extern "C"
