// Work plan built on the device from metadata passed by value (the host planner's plan, entry
// for entry), so a forward call needs no host-to-device copy before its kernel.
//
// The plan is the one build_entries (plan.cpp) writes: one entry per (sequence, token tile) and
// chunk, tiles ordered by their total cost over the chunks, longest first, ties in (sequence,
// tile) order.  One work-group of 1024 threads builds it: the metadata goes to LDS, every
// thread forms the total of some tiles and packs it with the tile's index into one 64-bit key
// (INT32_MAX - total above the index, so ascending keys are the plan's order).  Up to
// kRankDirect tiles, each thread counts the keys below its own (its rank) and writes its
// entries there; larger plans bitonic-sort the keys in LDS (log2(n) (log2(n) + 1) / 2
// barrier-separated stages) and write the entries of the sorted order.  Every step reads LDS
// only, so the kernel takes a few microseconds for the plans it accepts (at most
// kPlanDeviceMaxTiles tiles).
#include "internal.h"

namespace cpattn {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxSeq = (kPlanMetaInts / 2 - 1) / 2;   // (2 nseq + 1) * 2 <= kPlanMetaInts
constexpr int kRankDirect = 256;   // direct ranking: n steps per thread instead of the sort's barriers
static_assert(kRankDirect <= kPlanThreads, "one thread per tile when ranking directly");

// Metadata accessors over the LDS copy of PlanMeta::v.  Tile and block sizes are powers of two
// (their logarithms tt_log, bn_log), so the divisions are shifts.
struct Meta {
  const int32_t* v;
  int nseq, nchunks, causal, tt, bn, tt_log, bn_log;
  __device__ int cu_q(int i) const { return v[i]; }
  __device__ int q_off(int i) const { return v[nseq + 1 + i]; }
  __device__ const int32_t* chunk(int c) const { return v + (2 * nseq + 1) * (c + 1); }
  __device__ int cu_k(int c, int i) const { return chunk(c)[i]; }
  __device__ int k_off(int c, int i) const { return chunk(c)[nseq + 1 + i]; }
  __device__ int tiles(int i) const { return int((int64_t(cu_q(i + 1) - cu_q(i)) + tt - 1) >> tt_log); }

  // Entry of sequence i, tile tb, chunk c (as build_entries forms it).
  __device__ cpattn_plan_entry entry(int i, int tb, int c) const {
    const int nq = cu_q(i + 1) - cu_q(i);
    const int nk = cu_k(c, i + 1) - cu_k(c, i);
    cpattn_plan_entry p;
    p.row0 = cu_q(i) + tb * tt;
    p.nrows = min(tt, nq - tb * tt);
    p.k_start = cu_k(c, i);
    p.k_len = nk;
    int64_t delta = causal ? (int64_t(q_off(i)) + int64_t(tb) * tt - k_off(c, i)) : int64_t(nk);
    delta = max(int64_t(-tt), min(delta, int64_t(nk)));
    p.delta = int32_t(delta);
    const int64_t kend = max(int64_t(0), min(int64_t(nk), delta + p.nrows));
    p.cost = int32_t((kend + bn - 1) >> bn_log);
    p.seq = i;
    p.tblock = tb;
    return p;
  }
};

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const PlanMeta meta,
                                                            cpattn_plan_entry* out) {
  __shared__ int32_t sv[kPlanMetaInts];
  __shared__ int32_t first[kPlanMaxSeq + 1];   // first tile of each sequence, then n_tiles
  __shared__ uint64_t key[kPlanDeviceMaxTiles];
  const int tid = threadIdx.x;
  const int nseq = meta.nseq, nch = meta.nchunks, n = meta.n_tiles;
  const int used = (2 * nseq + 1) * (nch + 1);
  for (int i = tid; i < used; i += kPlanThreads) sv[i] = meta.v[i];
  __syncthreads();
  const Meta M{sv, nseq, nch, meta.causal, meta.tt, meta.bn, __builtin_ctz(unsigned(meta.tt)),
               __builtin_ctz(unsigned(meta.bn))};
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < nseq; ++i) {
      first[i] = acc;
      acc += M.tiles(i);
    }
    first[nseq] = acc;
  }
  __syncthreads();
  // sequence of tile t: the last i with first[i] <= t (empty sequences share their first)
  auto seq_of = [&](int t) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };

  int N = 1;
  while (N < n) N <<= 1;
  for (int t = tid; t < N; t += kPlanThreads) {
    uint64_t k = ~uint64_t(0);   // padding sorts last
    if (t < n) {
      const int i = seq_of(t), tb = t - first[i];
      int32_t total = 0;
      for (int c = 0; c < nch; ++c) total += M.entry(i, tb, c).cost;
      k = (uint64_t(uint32_t(INT32_MAX - total)) << 32) | uint32_t(t);
    }
    key[t] = k;
  }
  __syncthreads();
  if (n <= kRankDirect) {   // keys are distinct (the index is part of them)
    if (tid < n) {
      const uint64_t mine = key[tid];
      int rank = 0;
      for (int u = 0; u < n; ++u) rank += key[u] < mine ? 1 : 0;
      const int i = seq_of(tid), tb = tid - first[i];
      for (int c = 0; c < nch; ++c) out[int64_t(rank) * nch + c] = M.entry(i, tb, c);
    }
    return;
  }
  // bitonic sort of key[0, N), ascending
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += kPlanThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t a = key[i], b = key[l];
          if ((a > b) == ((i & k) == 0)) {
            key[i] = b;
            key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < n; r += kPlanThreads) {
    const int t = int(uint32_t(key[r]));
    const int i = seq_of(t), tb = t - first[i];
    for (int c = 0; c < nch; ++c) out[int64_t(r) * nch + c] = M.entry(i, tb, c);
  }
}

}  // namespace

bool fill_plan_meta(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                    const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                    const Geometry& g, int64_t n_tiles, PlanMeta* m) {
  const int64_t need = int64_t(2 * int64_t(nseq) + 1) * (nchunks + 1);
  if (nseq < 1 || need > kPlanMetaInts || n_tiles > kPlanDeviceMaxTiles) return false;
  const auto pow2 = [](int x) { return x > 0 && (x & (x - 1)) == 0; };
  if (!pow2(g.tokens_per_tile) || !pow2(g.block_n)) return false;
  static_assert(kPlanMaxSeq >= 1, "metadata too small for one sequence");
  m->nseq = nseq;
  m->nchunks = nchunks;
  m->causal = causal != 0;
  m->tt = g.tokens_per_tile;
  m->bn = g.block_n;
  m->n_tiles = int32_t(n_tiles);
  int32_t* v = m->v;
  for (int32_t i = 0; i <= nseq; ++i) *v++ = cu_q[i];
  for (int32_t i = 0; i < nseq; ++i) *v++ = q_off ? q_off[i] : 0;
  for (int32_t c = 0; c < nchunks; ++c) {
    for (int32_t i = 0; i <= nseq; ++i) *v++ = cu_k[int64_t(c) * (nseq + 1) + i];
    for (int32_t i = 0; i < nseq; ++i) *v++ = k_off ? k_off[int64_t(c) * nseq + i] : 0;
  }
  return true;
}

hipError_t launch_plan_device(const PlanMeta& m, cpattn_plan_entry* out, hipStream_t stream) {
  if (m.n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, m, out);
  return hipGetLastError();
}

}  // namespace cpattn
