// Host-side work planner: cu_seqlens + global position offsets -> ordered tiles.
//
// The causal mask is by global position (a query at q_pos sees keys with
// k_pos <= q_pos of its own sequence), so under a KV chunk at offset k_off a
// tile of query rows starting at q_off + row0 sees keys u <= delta + r with
// delta = q_off + row0 - k_off.  The number of key blocks a tile visits in each
// chunk is therefore known on the host, and tiles are ordered by their total
// over the chunks, longest first, so that the hardware's in-order work-group
// dispatch approximates longest-processing-time scheduling of the causally
// unbalanced work (diagonal chunks give tiles of 1..n blocks; sequences of a
// pack differ in length).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <string>
#include <vector>

#include "internal.h"

namespace cpattn {

namespace {
thread_local std::string g_last_error;
}

cpattn_status set_error(cpattn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

const char* last_error_text() { return g_last_error.c_str(); }
void clear_error() { g_last_error.clear(); }

Geometry geometry_for(cpattn_dtype dtype, int hq, int hkv) {
  if (dtype == CPATTN_FP32) return Geometry{kF32TokensPerTile, 1, kF32BlockN};
  const int group = hq / hkv;
  const int hpt = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  return Geometry{kBf16RowsPerWave * kBf16Waves / hpt, hpt, kBf16BlockN};
}

cpattn_status validate_metadata(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                                const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t hq,
                                int32_t hkv, int32_t d) {
  if (nseq < 0) return set_error(CPATTN_ERR_INVALID_ARG, "nseq must be >= 0 (got %d)", nseq);
  if (nchunks < 1 || nchunks > CPATTN_MAX_CHUNKS)
    return set_error(CPATTN_ERR_INVALID_ARG, "nchunks must be in 1..%d (got %d)", CPATTN_MAX_CHUNKS,
                     nchunks);
  if (hq < 1 || hkv < 1) return set_error(CPATTN_ERR_INVALID_ARG, "hq and hkv must be >= 1");
  if (hq % hkv != 0)
    return set_error(CPATTN_ERR_INVALID_ARG, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (d != 64 && d != 128)
    return set_error(CPATTN_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", d);
  if (!cu_q || !cu_k)
    return set_error(CPATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-null");
  if (cu_q[0] != 0) return set_error(CPATTN_ERR_INVALID_ARG, "cu_seqlens must start at 0");
  for (int32_t i = 0; i < nseq; ++i) {
    if (cu_q[i + 1] < cu_q[i])
      return set_error(CPATTN_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing (sequence %d)", i);
    const int64_t qo = q_off ? q_off[i] : 0;
    if (qo < 0) return set_error(CPATTN_ERR_INVALID_ARG, "position offsets must be >= 0 (sequence %d)", i);
    if (qo + (cu_q[i + 1] - cu_q[i]) > INT32_MAX)
      return set_error(CPATTN_ERR_INVALID_ARG, "positions of sequence %d overflow int32", i);
  }
  for (int32_t c = 0; c < nchunks; ++c) {
    const int32_t* ck = cu_k + int64_t(c) * (nseq + 1);
    const int32_t* ko_c = k_off ? k_off + int64_t(c) * nseq : nullptr;
    if (ck[0] != 0) return set_error(CPATTN_ERR_INVALID_ARG, "cu_seqlens must start at 0 (chunk %d)", c);
    for (int32_t i = 0; i < nseq; ++i) {
      if (ck[i + 1] < ck[i])
        return set_error(CPATTN_ERR_INVALID_ARG,
                         "cu_seqlens must be non-decreasing (chunk %d, sequence %d)", c, i);
      const int64_t ko = ko_c ? ko_c[i] : 0;
      if (ko < 0)
        return set_error(CPATTN_ERR_INVALID_ARG, "position offsets must be >= 0 (chunk %d, sequence %d)",
                         c, i);
      if (ko + (ck[i + 1] - ck[i]) > INT32_MAX)
        return set_error(CPATTN_ERR_INVALID_ARG, "positions of chunk %d, sequence %d overflow int32", c, i);
    }
  }
  // Element indices are computed in 64-bit inside the kernels; rows stay int32.
  return CPATTN_OK;
}

int64_t count_tiles(const int32_t* cu_q, int32_t nseq, int tokens_per_tile) {
  int64_t n = 0;
  for (int32_t i = 0; i < nseq; ++i) {
    const int64_t len = int64_t(cu_q[i + 1]) - cu_q[i];
    n += (len + tokens_per_tile - 1) / tokens_per_tile;
  }
  return n;
}

// Visible pairs of one sequence: sum over query rows t of clamp(delta0 + t + 1, 0, nk).
static int64_t visible_pairs(int64_t nq, int64_t nk, int64_t delta0, bool causal) {
  if (!causal) return nq * nk;
  int64_t total = 0;
  // rows where the count grows linearly: delta0 + t + 1 in (0, nk)
  const int64_t t_lo = std::max<int64_t>(0, -delta0);               // first row seeing >= 1 key
  const int64_t t_full = std::max<int64_t>(0, nk - 1 - delta0);     // first row seeing all keys
  const int64_t a = std::min(t_lo, nq), b = std::min(std::max(t_full, a), nq);
  // rows a .. b-1 see delta0 + t + 1 keys
  if (b > a) total += (b - a) * (delta0 + 1) + (b - 1 + a) * (b - a) / 2;
  total += (nq - b) * nk;
  return total;
}

void build_entries(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                   const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                   const Geometry& g, cpattn_plan_entry* out, int64_t n_tiles,
                   cpattn_plan_info* info) {
  const int tt = g.tokens_per_tile, bn = g.block_n;
  // Entries in (sequence, token block) order, chunk fastest.
  std::vector<cpattn_plan_entry> ent(size_t(n_tiles) * nchunks);
  std::vector<int64_t> total(size_t(n_tiles), 0);
  int64_t t = 0, pairs = 0, blocks = 0;
  for (int32_t i = 0; i < nseq; ++i) {
    const int32_t nq = cu_q[i + 1] - cu_q[i];
    const int64_t qo = q_off ? q_off[i] : 0;
    for (int32_t c = 0; c < nchunks; ++c) {
      const int32_t* ck = cu_k + int64_t(c) * (nseq + 1);
      const int64_t ko = k_off ? k_off[int64_t(c) * nseq + i] : 0;
      if (info) pairs += visible_pairs(nq, ck[i + 1] - ck[i], qo - ko, causal != 0);
    }
    for (int32_t tb = 0; tb * int64_t(tt) < nq; ++tb, ++t) {
      for (int32_t c = 0; c < nchunks; ++c) {
        const int32_t* ck = cu_k + int64_t(c) * (nseq + 1);
        const int32_t nk = ck[i + 1] - ck[i];
        const int64_t ko = k_off ? k_off[int64_t(c) * nseq + i] : 0;
        cpattn_plan_entry p;
        p.row0 = cu_q[i] + tb * tt;
        p.nrows = std::min<int32_t>(tt, nq - tb * tt);
        p.k_start = ck[i];
        p.k_len = nk;
        int64_t delta = causal ? (qo + int64_t(tb) * tt - ko) : int64_t(nk);
        delta = std::max<int64_t>(-tt, std::min<int64_t>(delta, nk));
        p.delta = int32_t(delta);
        const int64_t kend = std::max<int64_t>(0, std::min<int64_t>(nk, delta + p.nrows));
        p.cost = int32_t((kend + bn - 1) / bn);
        p.seq = i;
        p.tblock = tb;
        ent[size_t(t) * nchunks + c] = p;
        total[size_t(t)] += p.cost;
        blocks += p.cost;
      }
    }
  }
  if (out) {
    // Longest first; ties keep (sequence, token block) order so plans are deterministic.
    std::vector<int64_t> order(static_cast<size_t>(n_tiles));
    std::iota(order.begin(), order.end(), int64_t(0));
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return total[size_t(a)] > total[size_t(b)]; });
    for (int64_t k = 0; k < n_tiles; ++k)
      std::copy_n(ent.begin() + order[size_t(k)] * nchunks, nchunks, out + k * nchunks);
  }
  if (info) {
    info->n_entries = int32_t(n_tiles * nchunks);
    info->n_chunks = nchunks;
    info->reserved = 0;
    info->tokens_per_tile = tt;
    info->heads_per_tile = g.heads_per_tile;
    info->block_n = bn;
    info->visible_pairs = pairs;
    info->key_blocks = blocks;
    info->plan_bytes = size_t(n_tiles) * nchunks * sizeof(cpattn_plan_entry);
  }
}

int64_t count_key_tiles(const int32_t* cu_k, int32_t nchunks, int32_t nseq) {
  int64_t n = 0;
  for (int32_t c = 0; c < nchunks; ++c) {
    const int32_t* ck = cu_k + int64_t(c) * (nseq + 1);
    for (int32_t i = 0; i < nseq; ++i) {
      const int64_t len = int64_t(ck[i + 1]) - ck[i];
      n += (len + kBwdKeysPerTile - 1) / kBwdKeysPerTile;
    }
  }
  return n;
}

void build_key_entries(const int32_t* cu_q, const int32_t* cu_k, const int32_t* q_off,
                       const int32_t* k_off, int32_t nchunks, int32_t nseq, int32_t causal,
                       KeyTile* out, int64_t n_tiles) {
  const int kt = kBwdKeysPerTile, qb = kBwdQueryBlock;
  int64_t e = 0;
  for (int32_t c = 0; c < nchunks; ++c) {
    const int32_t* ck = cu_k + int64_t(c) * (nseq + 1);
    for (int32_t i = 0; i < nseq; ++i) {
      const int32_t nq = cu_q[i + 1] - cu_q[i], nk = ck[i + 1] - ck[i];
      const int64_t qo = q_off ? q_off[i] : 0, ko = k_off ? k_off[int64_t(c) * nseq + i] : 0;
      for (int32_t tb = 0; tb * int64_t(kt) < nk; ++tb) {
        KeyTile p;
        p.row0 = ck[i] + tb * kt;
        p.nrows = std::min<int32_t>(kt, nk - tb * kt);
        p.q_start = cu_q[i];
        p.q_len = nq;
        // key u = kt tb + r sits at ko + u; query t at qo + t sees it iff t >= ko + u - qo
        int64_t delta = causal ? (ko + int64_t(tb) * kt - qo) : int64_t(-kt);
        delta = std::max<int64_t>(-kt, std::min<int64_t>(delta, nq));
        p.delta = int32_t(delta);
        const int64_t first = std::max<int64_t>(0, delta);
        p.cost = int32_t((nq - first + qb - 1) / qb);
        p.chunk = c;
        p.reserved = 0;
        out[e++] = p;
      }
    }
  }
  // Longest first; ties keep (chunk, sequence, block) order.
  std::stable_sort(out, out + n_tiles,
                   [](const KeyTile& a, const KeyTile& b) { return a.cost > b.cost; });
}

int64_t build_key_parts(const KeyTile* tiles, int64_t n_tiles, int group, int hkv, int slots,
                        int64_t max_split, KeyPart* out, int64_t* n_split) {
  // Tiles run as (tile, kv head) work-groups, longest first; with one step per (query block,
  // head), a tile of a few times the ideal per-slot share of the steps leaves the last round
  // of the launch part-filled (e.g. 1,026 equal tiles on 512 slots take three rounds).  Halving
  // the longest tiles by query head gives the longest-first order units to balance with.  Each
  // split costs its halves a device-scope release and acquire (an L2 write-back and
  // invalidate on their XCD), so only tiles of at least kMinSplitSteps steps are split: on the
  // CP4 share (tiles of at most 448 steps) splitting measured 11% slower, on the 128K share
  // (8,192) 8.5% faster.
  int64_t total = 0;
  for (int64_t t = 0; t < n_tiles; ++t) total += int64_t(tiles[t].cost) * group * hkv;
  const int64_t thresh = total / std::max(1, slots) / 4;
  int64_t n = 0, s = 0;
  for (int64_t t = 0; t < n_tiles; ++t) {
    const KeyTile& k = tiles[t];
    const int64_t steps = int64_t(k.cost) * group;
    KeyPart p;
    p.row0 = k.row0;
    p.nrows = k.nrows;
    p.q_start = k.q_start;
    p.q_len = k.q_len;
    p.delta = k.delta;
    p.cost = k.cost;
    p.chunk = k.chunk;
    p.reserved = 0;
    if (group >= 2 && steps > thresh && steps >= kMinSplitSteps && s < max_split) {
      for (int h = 0; h < 2; ++h) {
        p.h_begin = h == 0 ? 0 : group / 2;
        p.h_end = h == 0 ? group / 2 : group;
        p.split = int32_t(s);
        p.part = h;
        out[n++] = p;
      }
      ++s;
    } else {
      p.h_begin = 0;
      p.h_end = group;
      p.split = -1;
      p.part = 0;
      out[n++] = p;
    }
  }
  // longest first by steps; ties keep the tile order (deterministic)
  std::stable_sort(out, out + n, [](const KeyPart& a, const KeyPart& b) {
    return int64_t(a.cost) * (a.h_end - a.h_begin) > int64_t(b.cost) * (b.h_end - b.h_begin);
  });
  *n_split = s;
  return n;
}

}  // namespace cpattn
