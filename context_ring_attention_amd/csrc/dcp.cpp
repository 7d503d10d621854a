// Host scheduler for Dynamic Context Parallelism: per-sample CP size and the
// placement of samples into micro-batches of CP groups.
//
// The verl documentation page "Dynamic Context Parallelism" fixes the
// constraints this follows: every DP x CP rank sees the same mini-batch and
// selects its own samples; the scheduler packs under a per-rank token limit
// (max_seqlen_per_dp_cp_rank, e.g. 16384 / 4 = 4096 for a static CP4 run with a
// 16,384-token budget); CP groups are power-of-two subgroups of the DP x CP
// ranks, plus the full DP x CP group when it is needed, so non-power-of-two
// world sizes leave no rank out; the world size must be even and at least two.
// The "Megatron 6D parallelism guide" (section 6.1) adds that the CP size follows
// the sequence lengths of the batch so that short sequences are not split.
// The pages do not print the assignment rule itself.  This file takes the
// plainest rule those constraints support:
//
//   1. CP size of a sample: the smallest allowed group size g (powers of two up
//      to the world size, and the world size) whose largest per-rank piece,
//      ceil(L / g), fits the limit.  A sample of zero tokens gets g = 1.
//   2. A sample of size g is split into g contiguous pieces of ceil(L / g)
//      tokens, the last one the remainder (the ring's per-rank split); rank
//      first + r of its group holds piece r.
//   3. Samples are placed in decreasing (g, L) order (index order among
//      equals), each into the first micro-batch where it fits: first into an
//      existing group of its size whose ranks all stay within the limit, else
//      into a new group at the lowest free aligned position (a multiple of g;
//      the full group starts at rank 0 and needs every rank free).  A sample
//      that fits no micro-batch opens a new one.
//
// Each rank of a micro-batch belongs to at most one group.  The result is a
// deterministic function of (lengths, world, limit).
#include <algorithm>
#include <numeric>
#include <vector>

#include "internal.h"

namespace cpattn {
namespace {

int64_t piece_tokens(int64_t len, int g, int r) {
  const int64_t p = (len + g - 1) / g;
  return std::max<int64_t>(0, std::min<int64_t>(p, len - int64_t(r) * p));
}

struct Group {
  int first, size;
};

struct MicroBatch {
  std::vector<int64_t> load;     // tokens per rank
  std::vector<int> owner;        // group index per rank, -1 if free
  std::vector<Group> groups;
  std::vector<int> group_fill;   // samples placed in each group
};

}  // namespace

cpattn_status dcp_schedule(const int32_t* lengths, int32_t n, int32_t world, int32_t limit,
                           int32_t* cp_size, int32_t* micro_batch, int32_t* group_rank,
                           int32_t* slot, int32_t* n_micro_batches) {
  if (n < 0) return set_error(CPATTN_ERR_INVALID_ARG, "sample count must be >= 0 (got %d)", n);
  if (world < 2 || world % 2 != 0)
    return set_error(CPATTN_ERR_INVALID_ARG,
                     "the DP x CP world size must be an even integer of at least two (got %d)", world);
  if (limit < 1) return set_error(CPATTN_ERR_INVALID_ARG, "the per-rank limit must be >= 1 (got %d)", limit);
  if (n > 0 && (!lengths || !cp_size || !micro_batch || !group_rank || !slot))
    return set_error(CPATTN_ERR_INVALID_ARG, "lengths and the output arrays must be non-null");
  if (!n_micro_batches) return set_error(CPATTN_ERR_INVALID_ARG, "n_micro_batches must be non-null");

  // Allowed group sizes, ascending: powers of two up to the world size, then the world size.
  std::vector<int> sizes;
  for (int g = 1; g <= world; g *= 2) sizes.push_back(g);
  if (sizes.back() != world) sizes.push_back(world);

  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = lengths[i];
    if (len < 0) return set_error(CPATTN_ERR_INVALID_ARG, "sample %d has a negative length", i);
    int g = 0;
    for (int s : sizes)
      if ((len + s - 1) / s <= limit) {
        g = s;
        break;
      }
    if (g == 0)
      return set_error(CPATTN_ERR_INVALID_ARG,
                       "sample %d (%lld tokens) exceeds world x limit = %d x %d", i,
                       static_cast<long long>(len), world, limit);
    cp_size[i] = g;
  }

  std::vector<int32_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (cp_size[a] != cp_size[b]) return cp_size[a] > cp_size[b];
    return lengths[a] > lengths[b];
  });

  std::vector<MicroBatch> mbs;
  auto fits = [&](const MicroBatch& mb, int first, int g, int64_t len) {
    for (int r = 0; r < g; ++r)
      if (mb.load[size_t(first + r)] + piece_tokens(len, g, r) > limit) return false;
    return true;
  };
  auto place = [&](int32_t i, int b, int gi) {
    MicroBatch& mb = mbs[size_t(b)];
    const Group& gr = mb.groups[size_t(gi)];
    for (int r = 0; r < gr.size; ++r) mb.load[size_t(gr.first + r)] += piece_tokens(lengths[i], gr.size, r);
    micro_batch[i] = b;
    group_rank[i] = gr.first;
    slot[i] = mb.group_fill[size_t(gi)]++;
  };
  auto new_group = [&](MicroBatch& mb, int first, int g) {
    for (int r = 0; r < g; ++r) mb.owner[size_t(first + r)] = int(mb.groups.size());
    mb.groups.push_back(Group{first, g});
    mb.group_fill.push_back(0);
    return int(mb.groups.size()) - 1;
  };

  for (int32_t i : order) {
    const int g = cp_size[i];
    const int64_t len = lengths[i];
    bool done = false;
    for (size_t b = 0; b < mbs.size() && !done; ++b) {
      MicroBatch& mb = mbs[b];
      for (size_t gi = 0; gi < mb.groups.size(); ++gi) {
        if (mb.groups[gi].size == g && fits(mb, mb.groups[gi].first, g, len)) {
          place(i, int(b), int(gi));
          done = true;
          break;
        }
      }
      if (done) break;
      // a new group at the lowest free aligned position (the full group only at rank 0)
      const int step = (g & (g - 1)) == 0 ? g : world;
      for (int first = 0; first + g <= world; first += step) {
        bool free_ranks = true;
        for (int r = 0; r < g && free_ranks; ++r) free_ranks = mb.owner[size_t(first + r)] < 0;
        if (free_ranks && fits(mb, first, g, len)) {
          place(i, int(b), new_group(mb, first, g));
          done = true;
          break;
        }
      }
    }
    if (!done) {
      mbs.push_back(MicroBatch{std::vector<int64_t>(size_t(world), 0), std::vector<int>(size_t(world), -1), {}, {}});
      place(i, int(mbs.size()) - 1, new_group(mbs.back(), 0, g));
    }
  }
  *n_micro_batches = int32_t(mbs.size());
  return CPATTN_OK;
}

}  // namespace cpattn
