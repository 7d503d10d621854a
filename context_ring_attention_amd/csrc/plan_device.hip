// Work plan built on the device from metadata passed by value (the host planner's plan, entry
// for entry), so a forward call needs no host-to-device copy before its kernel.
//
// The plan is the one build_entries (plan.cpp) writes: one entry per (sequence, token tile) and
// chunk, tiles ordered by their total cost over the chunks, longest first, ties in (sequence,
// tile) order.  Here every thread owns one tile: it finds its sequence and tile from the
// per-sequence tile counts, forms its entries, and computes its position in that order by
// counting the tiles that precede it.  Within one sequence a tile's cost never decreases with
// its index (each chunk's visible key range only grows, and the ragged last tile ends at the
// sequence's last query), so the count over each sequence is two binary searches.
#include "internal.h"

namespace cpattn {
namespace {

struct Meta {
  const PlanMeta& m;
  __device__ int cu_q(int i) const { return m.v[i]; }
  __device__ int q_off(int i) const { return m.v[m.nseq + 1 + i]; }
  __device__ const int32_t* chunk(int c) const { return m.v + (2 * m.nseq + 1) * (c + 1); }
  __device__ int cu_k(int c, int i) const { return chunk(c)[i]; }
  __device__ int k_off(int c, int i) const { return chunk(c)[m.nseq + 1 + i]; }
  __device__ int tiles(int i) const { return (cu_q(i + 1) - cu_q(i) + m.tt - 1) / m.tt; }

  // Entry of sequence i, tile tb, chunk c (as build_entries forms it).
  __device__ cpattn_plan_entry entry(int i, int tb, int c) const {
    const int nq = cu_q(i + 1) - cu_q(i);
    const int nk = cu_k(c, i + 1) - cu_k(c, i);
    cpattn_plan_entry p;
    p.row0 = cu_q(i) + tb * m.tt;
    p.nrows = min(m.tt, nq - tb * m.tt);
    p.k_start = cu_k(c, i);
    p.k_len = nk;
    int64_t delta = m.causal ? (int64_t(q_off(i)) + int64_t(tb) * m.tt - k_off(c, i)) : int64_t(nk);
    delta = max(int64_t(-m.tt), min(delta, int64_t(nk)));
    p.delta = int32_t(delta);
    const int64_t kend = max(int64_t(0), min(int64_t(nk), delta + p.nrows));
    p.cost = int32_t((kend + m.bn - 1) / m.bn);
    p.seq = i;
    p.tblock = tb;
    return p;
  }
  __device__ int64_t total(int i, int tb) const {
    int64_t s = 0;
    for (int c = 0; c < m.nchunks; ++c) s += entry(i, tb, c).cost;
    return s;
  }
  // Number of tiles of sequence i whose total is < x (strict) or <= x.
  __device__ int count_below(int i, int64_t x, bool inclusive) const {
    int lo = 0, hi = tiles(i);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int64_t t = total(i, mid);
      if (inclusive ? (t <= x) : (t < x)) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  }
};

__global__ __launch_bounds__(256) void plan_kernel(const PlanMeta meta, cpattn_plan_entry* out) {
  const Meta M{meta};
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= meta.n_tiles) return;
  // sequence and tile of global tile t
  int i = 0, first = 0;
  while (first + M.tiles(i) <= t) first += M.tiles(i++);
  const int tb = t - first;
  const int64_t mine = M.total(i, tb);
  // tiles before t in the longest-first order: every tile with a larger total, and the
  // earlier tiles (in sequence, tile order) with the same total
  int64_t rank = 0;
  for (int j = 0; j < meta.nseq; ++j) {
    const int le = M.count_below(j, mine, true);
    rank += M.tiles(j) - le;
    if (j < i) rank += le - M.count_below(j, mine, false);
    else if (j == i) rank += tb - M.count_below(j, mine, false);
  }
  for (int c = 0; c < meta.nchunks; ++c) out[rank * meta.nchunks + c] = M.entry(i, tb, c);
}

}  // namespace

bool fill_plan_meta(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                    const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                    const Geometry& g, int64_t n_tiles, PlanMeta* m) {
  const int64_t need = int64_t(2 * int64_t(nseq) + 1) * (nchunks + 1);
  if (nseq < 1 || need > kPlanMetaInts || n_tiles > INT32_MAX / 2) return false;
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
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned((m.n_tiles + 255) / 256)), dim3(256), 0, stream, m,
                     out);
  return hipGetLastError();
}

}  // namespace cpattn
