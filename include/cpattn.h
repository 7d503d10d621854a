/*
 * cpattn: chunked causal attention over packed variable-length sequences, and the
 * log-sum-exp merge of partial results, on AMD Instinct MI355X (gfx950).
 *
 * This is the per-GPU compute of ring-style context parallelism as described in
 * the "Megatron 6D parallelism guide", section 6 (context parallelism): each
 * rank holds a 1/CP slice of a sequence's queries, computes a partial attention
 * result against one KV chunk at a time, and folds each partial into a running
 * result by the online-softmax rule (both sides rescaled to a common maximum,
 * then added), normalising at the end.  Inputs are
 * "remove-padding / THD" packs (verl docs, "Dynamic Context Parallelism"): the
 * sequences of a micro-batch are concatenated without padding and described by
 * prefix sums of their lengths (cu_seqlens).
 *
 * Conventions shared by every call:
 *   - THD tensors are row-major [T, H, D] with D fastest; element (t, h, d) is at
 *     ((t * H) + h) * D + d.  They are contiguous and 16-byte aligned.
 *   - LSE tensors are row-major [H, T] fp32, natural log.
 *   - cu_seqlens arrays are int32 [nseq + 1], cu[0] == 0, non-decreasing; the
 *     tensor holds cu[nseq] rows.  Sequence i owns rows cu[i] .. cu[i+1]-1.
 *   - Query token t of sequence i has global position q_pos_offset[i] + t; key u
 *     has k_pos_offset[i] + u.  With causal != 0 a query sees a key of the SAME
 *     sequence iff key position <= query position (diagonal included).  Sequences
 *     never see each other.  Without causal it sees every key of its sequence.
 *   - Query head h reads kv head floor(h * hkv / hq) (contiguous GQA groups).
 *   - Scores are scaled by 1/sqrt(d).
 *   - A query with no visible key gets O = 0 and LSE = -inf (the empty partial:
 *     the pages' initial state O = 0, m = -inf, l = 0, normalised).
 *   - All device work is asynchronous on `stream`.  Device faults surface at the
 *     caller's next synchronisation.  The library never aborts: invalid arguments
 *     return a status code and leave every output untouched.
 *   - Metadata arrays (cu_seqlens, offsets) live in HOST memory; all tensors live
 *     in device memory of the current device.
 */
#ifndef CPATTN_H_
#define CPATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CPATTN_OK = 0,
  CPATTN_ERR_INVALID_ARG = 1,   /* malformed metadata, null or misaligned pointer, bad sizes */
  CPATTN_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement (e.g. d not in {64,128}) */
  CPATTN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than cpattn_workspace_size() */
  CPATTN_ERR_HIP = 4            /* a HIP runtime call failed; see cpattn_last_error() */
} cpattn_status;

typedef enum {
  CPATTN_BF16 = 0,              /* q, k, v are bfloat16; fp32 accumulation and softmax */
  CPATTN_FP32 = 1               /* q, k, v are float32; fp32 throughout */
} cpattn_dtype;

/*
 * Bytes of device workspace one cpattn_fwd_chunk call takes for these query
 * sequences: the size of the call's work plan.  cu_seqlens_q is host int32
 * [nseq + 1].  The value depends only on nseq, the query lengths and the head
 * counts, so one workspace serves every KV chunk of a rank's share.  Returns 0 if
 * the arguments are invalid (nseq < 0, null cu_seqlens_q with nseq > 0, hq or
 * hkv < 1).
 *
 * Work plans: every call writes its plan into the first bytes of the caller's workspace on
 * `stream`, ahead of the kernels that read it.  When the call's metadata is small (see
 * cpattn_plan_build_device) a planner kernel builds it on the device from the metadata passed
 * by value; otherwise it is built on the host and copied.  The library allocates no device
 * memory and keeps no state between calls; consecutive calls on one stream may reuse one
 * workspace (stream order keeps a plan until its kernels have run).  Calls on different
 * streams need different workspaces.  A stream that is being captured into a graph is refused
 * (CPATTN_ERR_UNSUPPORTED) when the plan would be copied from host memory (that host buffer is
 * freed when the call returns); device-planned calls may be captured.
 */
size_t cpattn_workspace_size(int32_t nseq, const int32_t* cu_seqlens_q, int32_t hq, int32_t hkv,
                             int32_t d);

/* Most KV chunks one cpattn_fwd_chunks call takes (the pages' CP sizes are 1..8). */
#define CPATTN_MAX_CHUNKS 16

/*
 * Bytes of device workspace one cpattn_fwd_chunks call with nchunks chunks needs
 * (the size of its work plan: one record per tile and chunk).  nchunks == 1 gives
 * cpattn_workspace_size().  Returns 0 for invalid arguments, including nchunks
 * outside 1 .. CPATTN_MAX_CHUNKS.
 */
size_t cpattn_workspace_size_chunks(int32_t nseq, const int32_t* cu_seqlens_q, int32_t hq,
                                    int32_t hkv, int32_t d, int32_t nchunks);

/*
 * One KV chunk: the per-step partial result of the ring loop ("Megatron 6D
 * parallelism guide", section 6: one attention call per KV chunk, returning an
 * unnormalised output with its row maximum and row sum), here in normalised form:
 *     o   [Tq, hq, d] fp32 = softmax over the chunk's visible keys, times V
 *     lse [hq, Tq]    fp32 = ln of the row's sum of exp(score) over those keys
 * with Tq = cu_seqlens_q[nseq].
 *
 *   q       device [Tq, hq, d], dtype            (read)
 *   k, v    device [Tk, hkv, d], dtype, Tk = cu_seqlens_k[nseq]  (read)
 *   cu_seqlens_q, cu_seqlens_k   host int32 [nseq + 1]
 *   q_pos_offset, k_pos_offset   host int32 [nseq], >= 0, or NULL for all zeros
 *   hq % hkv == 0; d in {64, 128}
 *   workspace        device, >= cpattn_workspace_size(...) bytes, 256-byte aligned;
 *                    owned by the caller; the call uploads its plan into it (see
 *                    above); it must not overlap q, k, v, o or lse.
 * The caller owns every buffer; o must not overlap q, k or v.  Rows of o/lse for
 * queries of zero-length key sequences are written as (0, -inf).
 * Returns CPATTN_OK, or an error code: invalid arguments (every code but CPATTN_ERR_HIP)
 * return before anything is enqueued; a failed launch (CPATTN_ERR_HIP) may leave the plan's
 * upload or planner kernel enqueued.
 */
cpattn_status cpattn_fwd_chunk(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                               int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                               cpattn_dtype dtype, int32_t causal, float* o, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Accumulating form of cpattn_fwd_chunk: the chunk's partial is folded into the
 * running result in the kernel's epilogue instead of being written out,
 *     (o, lse) <- merge((o, lse), partial of this chunk)
 * with the merge of cpattn_merge below ("Megatron 6D parallelism guide", section
 * 6: the combination applied once per ring step).  o and lse are read
 * and written (device, same shapes as cpattn_fwd_chunk); a first call on a fresh
 * result starts from O = 0, LSE = -inf everywhere.  Rows the chunk shows no key
 * keep their values exactly; rows whose running LSE is -inf take the partial
 * exactly.  Other arguments, ownership and errors as cpattn_fwd_chunk.
 */
cpattn_status cpattn_fwd_chunk_accum(const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                     int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                                     cpattn_dtype dtype, int32_t causal, float* o, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Every KV chunk of a rank's share in ONE launch: the ring loop of the pages
 * ("Megatron 6D parallelism guide", section 6) for chunks that are all resident,
 * with the running max, running sum and accumulator of each query row carried
 * across chunks in registers, so no partial is written and no merge pass runs.
 * The result equals merging the nchunks partials of cpattn_fwd_chunk (up to
 * rounding), i.e. attention of each query over the union of its keys in all
 * chunks.
 *
 *   q            device [Tq, hq, d], dtype                       (read)
 *   ks, vs       HOST arrays of nchunks device pointers; chunk c's keys and values are
 *                [Tk_c, hkv, d], dtype, Tk_c = cu_seqlens_k[c * (nseq + 1) + nseq]  (read)
 *   nchunks      1 .. CPATTN_MAX_CHUNKS
 *   cu_seqlens_q host int32 [nseq + 1]
 *   cu_seqlens_k host int32 [nchunks][nseq + 1], row c = chunk c's prefix sums
 *   q_pos_offset host int32 [nseq] or NULL;  k_pos_offset host int32 [nchunks][nseq] or NULL
 *   accumulate   0: write (o, lse);  1: fold the share into (o, lse) as cpattn_fwd_chunk_accum
 *   o, lse       device [Tq, hq, d] / [hq, Tq] fp32 (written; read too if accumulate)
 *   workspace    device, >= cpattn_workspace_size_chunks(..., nchunks) bytes, 256-byte aligned
 * The chunks may differ in length per sequence (zero allowed).  o must not
 * overlap q or any chunk.  Returns and errors as cpattn_fwd_chunk.
 */
cpattn_status cpattn_fwd_chunks(const void* q, const void* const* ks, const void* const* vs,
                                int32_t nchunks, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                                const int32_t* k_pos_offset, int32_t nseq, int32_t hq, int32_t hkv,
                                int32_t d, cpattn_dtype dtype, int32_t causal, int32_t accumulate,
                                float* o, float* lse, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * cpattn_fwd_chunks without a workspace argument, for callers that cannot allocate device
 * memory (code under graph capture of its own allocations, tight serving loops, harnesses
 * that forbid hipMalloc): the work plan goes into a static device array of 4 MiB that the
 * library holds on every GPU it runs on until the process ends (131,072 plan records: e.g.
 * 4 chunks of a 1M-token query pack in 32-token tiles).  A plan larger than that returns
 * CPATTN_ERR_UNSUPPORTED with nothing enqueued.  The call allocates nothing, host or device.
 * All calls on one GPU share that array: calls that overlap on one GPU (different streams,
 * or threads that do not order their streams) race on it and must not be issued.  The
 * results equal cpattn_fwd_chunks's for the same arguments.  Other arguments, ownership and
 * errors as cpattn_fwd_chunks (a stream under capture is refused).
 */
cpattn_status cpattn_fwd_chunks_noalloc(const void* q, const void* const* ks,
                                        const void* const* vs, int32_t nchunks,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                        const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                        int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                                        cpattn_dtype dtype, int32_t causal, int32_t accumulate,
                                        float* o, float* lse, hipStream_t stream);

/*
 * Backward of one KV chunk: the gradients of the attention the forward computes,
 * i.e. of O = softmax(Q K^T / sqrt(d) + mask) V over all keys of the share, for
 * an upstream gradient dO ("Megatron 6D parallelism guide", section 6: the
 * ring loop is the forward of a training step; its backward is the gradient of
 * the same function).  With P the share's probabilities (from the forward's
 * final LSE), dP = dO V^T and dS = P * (dP - delta), delta = rowsum(dO * O),
 * this call ADDS the chunk's contributions:
 *     dq [Tq, hq, d]  += dS K / sqrt(d)     (sum over the chunks: call once per chunk)
 *     dk [Tk, hkv, d] += dS^T Q / sqrt(d)   (summed over the query heads of each kv head)
 *     dv [Tk, hkv, d] += P^T dO
 * The caller zero-fills dq, dk, dv before the first call.
 *
 *   q, do_    device [Tq, hq, d] bf16           (read; do_ is the gradient of o)
 *   k, v      device [Tk, hkv, d] bf16          (read)
 *   o         device [Tq, hq, d] fp32           (read; the share's final forward output)
 *   lse       device [hq, Tq] fp32              (read; the share's final forward LSE)
 *   dq        device [Tq, hq, d] fp32; dk, dv device [Tk, hkv, d] fp32   (read and written)
 *   metadata  as cpattn_fwd_chunk (host); dtype must be CPATTN_BF16; d in {64, 128}
 *   workspace device, >= cpattn_bwd_workspace_size(...) bytes, 256-byte aligned; it holds
 *             the call's two plans (uploaded as for the forward, see
 *             cpattn_workspace_size), delta and the log2-scaled LSE, and the split key
 *             tiles' partial dK/dV, until the kernels have run; it must not overlap any
 *             tensor
 * Rows whose LSE is -inf (no visible key in the share) contribute nothing.  No output may
 * overlap an input or another output.  Returns CPATTN_OK, or an error code with nothing
 * enqueued (CPATTN_ERR_UNSUPPORTED for fp32 inputs).
 */
cpattn_status cpattn_bwd_chunk(const void* q, const void* k, const void* v, const float* o,
                               const void* do_, const float* lse, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                               const int32_t* k_pos_offset, int32_t nseq, int32_t hq,
                               int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                               float* dq, float* dk, float* dv, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of every KV chunk of a share in one pass (the backward of cpattn_fwd_chunks):
 * delta is formed once, then one gradient launch runs the dQ work-groups (each walks all
 * chunks, so dq gets the whole share's gradient in one write) and the dK/dV work-groups (the
 * key tiles of every chunk), interleaved longest first.
 * ADDS to dq, dks[c], dvs[c] exactly what nchunks cpattn_bwd_chunk calls would (up to
 * rounding order).
 *   ks, vs      HOST arrays of nchunks device pointers, chunk c [Tk_c, hkv, d] bf16
 *   dks, dvs    HOST arrays of nchunks device pointers, chunk c [Tk_c, hkv, d] fp32
 *   cu_seqlens_k, k_pos_offset   laid out as for cpattn_fwd_chunks
 *   workspace   >= cpattn_bwd_workspace_size_chunks(...) bytes, 256-byte aligned
 * Other arguments as cpattn_bwd_chunk.
 */
cpattn_status cpattn_bwd_chunks(const void* q, const void* const* ks, const void* const* vs,
                                int32_t nchunks, const float* o, const void* do_,
                                const float* lse, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
                                const int32_t* k_pos_offset, int32_t nseq, int32_t hq,
                                int32_t hkv, int32_t d, cpattn_dtype dtype, int32_t causal,
                                float* dq, float* const* dks, float* const* dvs, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace one cpattn_bwd_chunk call needs. It holds:
 *   - the query plan, the key plan and the launch order of the gradient launch's
 *     work-groups, with a counter per split key tile;
 *   - delta [hq, Tq] and the LSE in log2 units [hq, Tq], fp32;
 *   - scratch for the partial dK/dV of split key tiles. The dK/dV launch splits a long key
 *     tile between two work-groups (half of the query heads of its GQA group each), so that
 *     a few long tiles do not leave the launch's last round part-filled. Each half keeps a
 *     partial of 2 x 96 x d fp32 values here, and the second to finish adds both.
 * The scratch is sized for every key tile being split: 2 x 2 x 96 x d x 4 bytes per key tile
 * and kv head, e.g. ~270 MB for the 128K-context CP=4 share (4 x 32,768 keys, one kv head, D = 128). Returns 0 for invalid
 * arguments.
 */
size_t cpattn_bwd_workspace_size(int32_t nseq, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t hq, int32_t hkv, int32_t d);

/* The same for cpattn_bwd_chunks with nchunks chunks (cu_seqlens_k [nchunks][nseq + 1]). */
size_t cpattn_bwd_workspace_size_chunks(int32_t nseq, const int32_t* cu_seqlens_q,
                                        const int32_t* cu_seqlens_k, int32_t nchunks, int32_t hq,
                                        int32_t hkv, int32_t d);

/*
 * The merge of two partial results over disjoint key sets, the combination step
 * of the ring loop ("Megatron 6D parallelism guide", section 6: the running
 * result is rescaled to a common maximum and summed with each step's partial).
 * For normalised partials it reads
 *     lse = ln(exp(lse_a) + exp(lse_b))
 *     o   = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b
 * i.e. each side is weighted by its share of the total softmax mass.  In place:
 *     (o_a, lse_a) <- merge((o_a, lse_a), (o_b, lse_b))
 *   o_a, o_b     device fp32 [t, hq, d]
 *   lse_a, lse_b device fp32 [hq, t]
 *   d a power of two in [4, 256].
 * An empty side (LSE = -inf) leaves the other side unchanged exactly; two empty
 * sides stay (O_a, -inf).  The b buffers must not overlap the a buffers.
 */
cpattn_status cpattn_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b,
                           int64_t t, int32_t hq, int32_t d, hipStream_t stream);

/* Static text for a status code. */
const char* cpattn_status_string(cpattn_status s);

/* Text of the last failure on the calling thread ("" if none). */
const char* cpattn_last_error(void);

/* ---------------------------------------------------------------------------
 * Work plan (host only; exposed so the planner can be checked without a GPU).
 *
 * The kernels process "tiles": a run of consecutive query tokens of one
 * sequence, for a group of query heads that share one kv head.  The planner
 * turns host cu_seqlens and position offsets into one entry per (sequence,
 * token block) and KV chunk, orders the tiles by descending cost (number of key
 * blocks the tile must visit under the causal mask, summed over the chunks;
 * longest first), and the launch walks them in that order, all head groups of
 * a tile back to back.
 *
 * Plan layout: an array of cpattn_plan_entry (32 bytes each), tile-major: the
 * entry of tile t and chunk c is at index t * nchunks + c (one entry per tile
 * for a single chunk).  Entries of one tile share row0, nrows, seq and tblock.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t row0;     /* first query row (index into Q's T dimension) of the tile */
  int32_t nrows;    /* valid query tokens in the tile, 1 .. tokens_per_tile */
  int32_t k_start;  /* first key row of the sequence in this chunk */
  int32_t k_len;    /* keys of the sequence in this chunk */
  int32_t delta;    /* tile row r sees key u iff u <= delta + r (clamped to [-tokens_per_tile, k_len]) */
  int32_t cost;     /* key blocks the tile's last row must visit */
  int32_t seq;      /* sequence index */
  int32_t tblock;   /* token-block index within the sequence */
} cpattn_plan_entry;

typedef struct {
  int32_t n_entries;        /* plan entries = (sequence, token block) tiles x n_chunks */
  int32_t n_tiles;          /* work-groups launched = n_entries / n_chunks * head_groups */
  int32_t tokens_per_tile;
  int32_t heads_per_tile;
  int32_t head_groups;      /* hq / heads_per_tile */
  int32_t block_n;          /* keys per inner-loop block */
  int64_t visible_pairs;    /* exact visible (query, key) pairs per query head */
  int64_t key_blocks;       /* sum over entries of cost (key blocks visited per head group) */
  size_t plan_bytes;        /* n_entries * sizeof(cpattn_plan_entry) */
  int32_t n_chunks;         /* KV chunks the plan covers */
  int32_t reserved;
} cpattn_plan_info;

/*
 * Validate metadata and build the plan cpattn_fwd_chunk would launch.
 * plan: host buffer of plan_bytes, or NULL to only fill *info.  Returns
 * CPATTN_ERR_WORKSPACE if plan is non-NULL and plan_bytes is too small.
 */
cpattn_status cpattn_plan_build(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
                                cpattn_dtype dtype, int32_t causal,
                                cpattn_plan_entry* plan, size_t plan_bytes, cpattn_plan_info* info);

/*
 * The plan cpattn_fwd_chunks would launch for nchunks chunks (metadata laid out
 * as for cpattn_fwd_chunks).  nchunks == 1 gives cpattn_plan_build's plan.
 */
cpattn_status cpattn_plan_build_chunks(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                       int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                       int32_t d, cpattn_dtype dtype, int32_t causal,
                                       cpattn_plan_entry* plan, size_t plan_bytes,
                                       cpattn_plan_info* info);

/*
 * Key-stationary plan of the backward (host only; exposed so the planner can be
 * checked without a GPU).  The dK/dV kernel processes "key tiles": up to
 * keys_per_tile consecutive keys of one sequence in one chunk, for one kv head;
 * it streams, in blocks of query_block queries, the queries of the sequence that
 * see at least one of the tile's keys.  Tiles are ordered by descending cost
 * (query blocks to visit), ties in (chunk, sequence, key block) order.
 */
typedef struct {
  int32_t row0;     /* first key row of the tile (index into its chunk's K / V) */
  int32_t nrows;    /* keys in the tile, 1 .. keys_per_tile */
  int32_t q_start;  /* first query row of the tile's sequence */
  int32_t q_len;    /* queries of the sequence */
  int32_t delta;    /* query t of the sequence sees tile key r iff t >= delta + r
                       (causal; clamped to [-keys_per_tile, q_len]); -keys_per_tile when not causal */
  int32_t cost;     /* query blocks from query max(delta, 0) to the sequence's last query */
  int32_t chunk;    /* chunk of the tile's keys */
  int32_t reserved;
} cpattn_key_tile;

typedef struct {
  int32_t n_tiles;        /* key tiles (work-groups per kv head) */
  int32_t keys_per_tile;
  int32_t query_block;    /* queries per inner-loop block */
  int32_t reserved;
} cpattn_key_plan_info;

/*
 * Validate metadata (laid out as for cpattn_bwd_chunks) and build the key plan
 * cpattn_bwd_chunks would launch.  plan: host buffer of plan_bytes, or NULL to
 * only fill *info.  Returns CPATTN_ERR_WORKSPACE if plan is non-NULL and
 * plan_bytes < n_tiles * sizeof(cpattn_key_tile).
 */
cpattn_status cpattn_key_plan_build(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                    int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                    int32_t d, int32_t causal, cpattn_key_tile* plan,
                                    size_t plan_bytes, cpattn_key_plan_info* info);

/*
 * The same plan as cpattn_plan_build_chunks, built on the device into `plan` (device, at least
 * the plan's bytes, 16-byte aligned) on `stream` from the metadata passed by value.  This is
 * how the forward entry points build their plan when the metadata is small enough:
 * (2 nseq + 1) (nchunks + 1) <= 480 int32 values, e.g. up to 47 sequences at 4 chunks or 119
 * sequences in one chunk, and the plan has at most 4096 token tiles (131,072 bf16 query tokens
 * at 32 per tile); larger calls are planned on the host and copied.  Returns
 * CPATTN_ERR_UNSUPPORTED for calls beyond these limits (or nseq == 0).  Exposed so the two
 * planners can be compared.
 */
cpattn_status cpattn_plan_build_device(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       const int32_t* q_pos_offset, const int32_t* k_pos_offset,
                                       int32_t nchunks, int32_t nseq, int32_t hq, int32_t hkv,
                                       int32_t d, cpattn_dtype dtype, int32_t causal,
                                       cpattn_plan_entry* plan, size_t plan_bytes,
                                       hipStream_t stream);

/* -------------------------------------------------------------------------
 * Dynamic Context Parallelism scheduler (host only, no device work).
 *
 * Chooses a CP group size for every sample of a mini-batch and places the
 * samples into micro-batches of CP groups, under the constraints of the verl
 * page "Dynamic Context Parallelism": every DP x CP rank sees the whole
 * mini-batch; a per-rank token limit max_seqlen_per_dp_cp_rank (e.g. 16384 / 4
 * = 4096 for a static CP4 run with a 16,384-token budget); CP groups are the
 * power-of-two subgroups of the `world` = DP x CP ranks plus the full group, and
 * world must be an even integer of at least two.  The pages do not print the
 * assignment rule; this one (see csrc/dcp.cpp) is:
 *   - cp_size[i] = the smallest allowed group size g with ceil(L_i / g) <= limit;
 *   - sample i is split into g contiguous pieces of ceil(L_i / g) tokens (the
 *     last one the remainder); rank group_rank[i] + r holds piece r;
 *   - samples are placed in decreasing (g, L) order, first fit over the
 *     micro-batches: into an existing group of size g if every rank stays within
 *     the limit, else into a new group at the lowest free aligned rank (a
 *     multiple of g; the full group at rank 0), else into a new micro-batch.
 * Every rank of a micro-batch belongs to at most one group.
 *
 *   lengths        host int32 [n], >= 0
 *   cp_size        host int32 [n] out: group size of sample i
 *   micro_batch    host int32 [n] out: micro-batch of sample i (0-based)
 *   group_rank     host int32 [n] out: first rank of sample i's group
 *   slot           host int32 [n] out: position of sample i in its group's THD pack
 *   n_micro_batches host int32 out
 * Returns CPATTN_ERR_INVALID_ARG (and writes nothing meaningful) for an odd or
 * too small world, a limit < 1, a negative length, or a sample longer than
 * world x limit.  Deterministic; thread-safe.
 * ------------------------------------------------------------------------- */
cpattn_status cpattn_dcp_schedule(const int32_t* lengths, int32_t n, int32_t world,
                                  int32_t max_seqlen_per_rank, int32_t* cp_size,
                                  int32_t* micro_batch, int32_t* group_rank, int32_t* slot,
                                  int32_t* n_micro_batches);

#ifdef __cplusplus
}
#endif

#endif  /* CPATTN_H_ */
