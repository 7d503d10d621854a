// Chunked causal attention forward, bf16 inputs, fp32 accumulation (gfx950).
//
// One work-group = 4 waves = one tile of the host plan: up to 32 query tokens
// per wave, for heads_per_tile query heads of one GQA group (the waves of a
// tile share one kv head, so every K/V block staged in LDS serves all of them).
// The kernel walks the tile's key blocks (64 keys each) of each of its KV
// chunks in turn, keeps a running max m and running sum l per query row (online
// softmax: the update of the ring loop of the "Megatron 6D parallelism guide",
// section 6, applied across key blocks and across chunks alike) and at the end
// writes the normalised O = acc / l and LSE = m + ln l of the tile's rows over
// all those keys.  With one chunk that is the partial of that chunk.  In
// accumulate mode the epilogue instead folds (O, LSE) into the running result
// already in memory with the merge of two partials (each side weighted by its
// share of the softmax mass), so a ring step needs no separate merge pass.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64): the score tile is
// computed transposed, S^T[key][token] = K * Q^T, so the 32x32 accumulator puts
// one query token per lane column (lane % 32) and 16 of its keys per lane; lane
// l and lane l^32 together hold all 32 keys of that token.  Row statistics thus
// need one cross-half swap (v_permlane32_swap) per key block and no LDS.  The
// output is accumulated transposed too, O^T[d][token] = V^T * P^T: P comes
// straight from the score registers (bf16-rounded) as the B operand, and V^T
// is the A operand, gathered from row-major V in LDS by the gfx950 transpose
// read (ds_read_b64_tr_b16 hands each lane 4 consecutive keys of its own d
// column).  Both operands of each MFMA use the same (lane-group, element) -> k
// index mapping, so the contraction pairs the right keys.
//
// Data movement: K and V blocks go from HBM straight into LDS
// (buffer_load_dwordx4 ... lds, 16 bytes per lane), through buffer resources
// whose range ends at the sequence's last key, so rows past the end read as
// zero with no branches.  16-byte chunks are XOR-swizzled by row (one pattern
// for the K reads, another for the V transpose reads) against bank conflicts;
// the swizzle is applied by choosing which global chunk each lane fetches.  Two
// LDS stages: the next block (of the same chunk, or the first of the next chunk
// the tile sees) is in flight while the current one is computed; one barrier per
// block.  The tile's blocks are walked as one flat sequence over its chunks, two
// per loop trip, so the stage of each is a compile-time constant and every LDS
// read address is a per-lane base plus an immediate offset (no per-block address
// arithmetic on the VALU, which this kernel is short of).
//
// Softmax: scores stay in raw units s = q.k; p = exp2(s * c - m * c) with
// c = log2(e)/sqrt(D).  The running max m is only moved when a row's block max
// exceeds it by more than 8/c (a factor 2^8 in p): until then p <= 2^8, which
// fp32 sums and bf16 P carry without loss of relative precision, and the final
// O / l cancels the common factor exactly.  This skips the 64-register rescale
// of the accumulator on almost every block.
//
// Two row sums are kept: over the fp32 probabilities (for the LSE, which then
// carries fp32 rounding only; a sum over bf16-rounded values would be off by up
// to 2^-9 of each term, which moves the LSE of rows with few keys by more than
// 1e-3), and over their bf16 roundings with v_dot2_f32_bf16 (for O, which is then
// an exact convex combination of the weights the PV product multiplied; dividing
// by the fp32 sum instead would scale O by the rounding of the largest weight,
// which under the lazy max below need not be 1).  Most blocks skip the row max
// altogether: once a reference max is set, P is formed against it directly, and a
// lane sum <= 2^8 proves no score passed the threshold (every p >= 0), which is
// all the max was needed for; otherwise the block is redone with the max (and
// rescale) first.  Both paths give the same bits as always taking the max.
//
// Scheduling: the two waves of a SIMD (one from each of the CU's two
// work-groups) run the same block loop; a wave raises its issue priority for
// its matrix-core runs (scores, PV) and drops it for the softmax, so when the
// two meet, the MFMA stream is the one that keeps issuing.
//
// Masking: the host classifies blocks by global position, so only blocks on the
// causal diagonal or past the sequence end pay for per-element masking.  A row
// with no visible key keeps m = -inf and l = 0 and is written as (0, -inf).
//
// This file is compiled with -fno-honor-nans: no value here is ever NaN (scores
// are finite or -inf, exp2(-inf) = 0), and without the flag every max over an
// MFMA result is preceded by a canonicalising v_max_f32 x, x.  Infinities keep
// their IEEE meaning.
#include <type_traits>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kThreads = kBf16Waves * 64;
constexpr int BN = kBf16BlockN;          // keys per block
constexpr float kRescaleLog2 = 8.0f;     // move the running max only past 2^8 growth
constexpr int kBufferWord3 = 0x00020000; // raw buffer, 32-bit data format

template <int D>
struct Layout {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = BN * kRowBytes;     // one K or V block
  static constexpr int kRowsPerKB = 1024 / kRowBytes;   // rows one wave-wide load fills
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kBf16Waves;

  // K is read 16 bytes per lane along a column of 32 rows: spread rows over chunks.
  __device__ static __forceinline__ int k_swz(int row) {
    return (D == 128) ? (row & 15) : ((row >> 1) & 7);
  }
  // V is read by 16-lane groups, 4 rows x 32 bytes each: spread the 4 rows.
  __device__ static __forceinline__ int v_swz(int row) {
    return (D == 128) ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
  }
  __device__ static __forceinline__ int k_off(int row, int c) {
    return row * kRowBytes + ((c ^ k_swz(row)) << 4);
  }
  __device__ static __forceinline__ int v_off(int row, int c) {
    return row * kRowBytes + ((c ^ v_swz(row)) << 4);
  }
};

// v_permlane32_swap with both operands = x leaves x of lanes 0..31 in the first
// result and x of lanes 32..63 in the second, each broadcast to both halves, so
// r[0] op r[1] combines lane l with lane l ^ 32 identically in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

#if defined(__HIP_DEVICE_COMPILE__)
// Buffer resources are a device-only type: the host pass of this file only
// needs the kernel's launch stub, so device helpers and the kernel body are
// compiled in the device pass alone.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const __bf16* base, int64_t rows_left,
                                                           int64_t stride_bytes, int row_bytes) {
  // Bytes from `base` to the end of the last valid row (0 if none).
  const int64_t n = rows_left > 0 ? (rows_left - 1) * stride_bytes + row_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base), (short)0,
                                           int(n > 0x7fffffff ? 0x7fffffff : n), kBufferWord3);
}
#endif

template <int D, bool ACCUM>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const ChunkPtrs<__bf16> kv, int nchunks,
    const cpattn_plan_entry* __restrict__ plan, int head_groups, int heads_per_tile, int hq,
    int hkv, int tq_total, float scale, float scale_log2, float* __restrict__ o,
    float* __restrict__ lse) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Layout<D>;
  constexpr int KS = D / 16;      // k-steps of the score MFMA
  constexpr int DT = D / 32;      // 32-row tiles of O^T
  constexpr int NPV = 4 * DT;     // PV MFMAs per block: 4 key groups of 16 x DT tiles
  constexpr int EPS = 32 / NPV;   // softmax elements (per lane) formed beside each PV MFMA
  // LDS: K stages 0 and 1, then V stages 0 and 1 (one block each).
  __shared__ __attribute__((aligned(1024))) char smem[4 * L::kTileBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;  // token column of the MFMA tiles
  const int g = lane >> 5;  // lane half

  const int b = blockIdx.x;
  const int e = b / head_groups;
  const int hg = b - e * head_groups;
  const cpattn_plan_entry* tile = plan + int64_t(e) * nchunks;  // one entry per chunk
  const int row0 = tile[0].row0, nrows = tile[0].nrows;
  const int head = hg * heads_per_tile + (wave % heads_per_tile);
  const int tok0 = (wave / heads_per_tile) * kBf16RowsPerWave;
  const int kvh = (hg * heads_per_tile) / (hq / hkv);  // shared by every head of the tile
  const int rows_w = min(max(nrows - tok0, 0), kBf16RowsPerWave);  // this wave's rows

  // Q fragment: B operand of S^T = K Q^T; lane holds Q[token n][16 ks + 8 g .. +7].
  bf16x8 qf[KS];
  {
    const bool ok = n < rows_w;
    const __bf16* qp = q + (int64_t(row0 + tok0 + n) * hq + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks) : bf16x8{};
  }

  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running reference max of raw scores (row n)
  float l_run = 0.f;        // running sum of this lane's fp32 weights (for the LSE)
  float lb_run = 0.f;       // running sum of the same weights rounded to bf16 (for O)
  const float thr = kRescaleLog2 / scale_log2;

  // ---- HBM -> LDS block loads (each wave fills kLoadsPerWave KB of the block) ----
  // Block j of chunk c: rows k_start + 64 j .. of that chunk's K or V.
  const int64_t stride_bytes = int64_t(hkv) * D * 2;
  auto issue = [&](const __bf16* src, int c, int j, char* dst, bool is_v) {
    const cpattn_plan_entry& pc_e = tile[c];
    const int64_t first = (int64_t(pc_e.k_start) + int64_t(j) * BN) * hkv + kvh;
    const int64_t rows_left = int64_t(pc_e.k_len) - int64_t(j) * BN;
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(src + first * D, rows_left, stride_bytes, D * 2);
#pragma unroll
    for (int i = 0; i < L::kLoadsPerWave; ++i) {
      // this wave fills the i-th of its 1 KB pieces; lane l fills bytes [16 l, 16 l + 16)
      const int blk = wave * L::kLoadsPerWave + i;
      const int row = blk * L::kRowsPerKB + lane / L::kChunks;
      const int pc = lane % L::kChunks;                  // physical chunk this lane fills
      const int swz = is_v ? L::v_swz(row) : L::k_swz(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + blk * 1024), 16,
                                               row * int(stride_bytes) + ((pc ^ swz) << 4), 0, 0, 0);
    }
  };
  auto kstage = [&](int st) { return smem + st * L::kTileBytes; };
  auto vstage = [&](int st) { return smem + (2 + st) * L::kTileBytes; };

  // Lane-constant parts of the LDS read addresses.
  int k_rd[2][KS];  // S^T A operand: K row 32 kt + n, chunk 2 ks + g
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[kt][ks] = L::k_off(32 * kt + n, 2 * ks + g);
  // O^T A operand via transpose reads: lane (n, g) in 16-lane group (g, h = n / 16) supplies the
  // address of V row 16 kk + 4 g + jr (+ 8 for the second half) at columns 32 dt + 16 h + 4 q.
  // The row swizzle depends only on the row bits that 16 kk and + 8 leave alone, so a lane's
  // addresses are one base per dt plus immediate offsets.
  const int jr = (n & 15) >> 2, qq = n & 3, hh = n >> 4;
  int v_rd[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    v_rd[dt] = L::v_off(4 * g + jr, 4 * dt + 2 * hh + (qq >> 1)) + 8 * (qq & 1);
  // V^T fragment of PV MFMA i (key group i / DT, 32-row tile i % DT) from one V stage.
  auto vread = [&](const char* vs, int i) {
    const int kk = i / DT, dt = i % DT;
    const char* base = vs + v_rd[dt] + 16 * kk * L::kRowBytes;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * L::kRowBytes));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // Chunks the tile sees keys of (cost > 0), in order, and the tile's block count.
  auto next_chunk = [&](int c) {
    ++c;
    while (c < nchunks && tile[c].cost == 0) ++c;
    return c;
  };
  int nblk_tile = 0;
  for (int c = 0; c < nchunks; ++c) nblk_tile += tile[c].cost;
  // This wave's key blocks in chunk c (a prefix of the tile's) and the unmasked ones among them.
  auto wave_range = [&](int c, int& nb, int& nf) {
    nb = 0;
    nf = 0;
    if (rows_w > 0 && c < nchunks) {
      const cpattn_plan_entry pe = tile[c];
      const int kend = max(0, min(pe.k_len, pe.delta + tok0 + rows_w));
      nb = (kend + BN - 1) / BN;
      nf = min(min(pe.k_len / BN, max(0, pe.delta + tok0 + 1) / BN), nb);
    }
  };

  // P = exp2(s c - m c) as bf16 B operands of the PV product (key group kk = registers
  // 8 (kk % 2) .. +7 of score tile kk / 2) and this lane's sum of the fp32 values.
  f32x16 s0, s1;
  bf16x8 pcur[4];
  struct Sums {
    float p, b;  // the lane's sum of the fp32 weights and of their bf16 roundings
  };
  auto exp_block = [&](float neg) {
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[jj], scale_log2, neg));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s0[8 + jj], scale_log2, neg));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(s1[jj], scale_log2, neg));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(s1[8 + jj], scale_log2, neg));
      pcur[0][jj] = (__bf16)p0;
      pcur[1][jj] = (__bf16)p1;
      pcur[2][jj] = (__bf16)p2;
      pcur[3][jj] = (__bf16)p3;
      part[0] += p0;
      part[1] += p1;
      part[2] += p2;
      part[3] += p3;
    }
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float pb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      pb[kk] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pb[kk] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pcur[kk][2 * i], pcur[kk][2 * i + 1]}, ones,
                                                 pb[kk], false);
    }
    return Sums{(part[0] + part[1]) + (part[2] + part[3]), (pb[0] + pb[1]) + (pb[2] + pb[3])};
  };
  // ---- the block loop ----
  // Block p's K and V are staged together; block p + 1's are in flight while p is computed.
  int lc = next_chunk(-1), lj = 0;  // the next block to load
  int cc = lc, cj = 0;              // block p
  int nblk_w = 0, nfull_w = 0;
  wave_range(cc, nblk_w, nfull_w);
  if (nblk_tile > 0) {
    issue(kv.k[lc], lc, lj, kstage(0), false);
    issue(kv.v[lc], lc, lj, vstage(0), true);
    if (++lj == tile[lc].cost) lc = next_chunk(lc), lj = 0;
  }
  auto step = [&](const int p, auto ST) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (p + 1 < nblk_tile) {
      issue(kv.k[lc], lc, lj, kstage(1 - ST), false);
      issue(kv.v[lc], lc, lj, vstage(1 - ST), true);
      if (++lj == tile[lc].cost) lc = next_chunk(lc), lj = 0;
    }
    if (cj < nblk_w) {
      const char* ks = kstage(ST);
      const char* vs = vstage(ST);
      __builtin_amdgcn_s_setprio(1);
      s0 = f32x16{};
      s1 = f32x16{};
      bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ks + k_rd[0][0]);
      bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ks + k_rd[1][0]);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        bf16x8 n0, n1;
        if (k + 1 < KS) {
          n0 = *reinterpret_cast<const bf16x8*>(ks + k_rd[0][k + 1]);
          n1 = *reinterpret_cast<const bf16x8*>(ks + k_rd[1][k + 1]);
        }
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[k], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[k], s1, 0, 0, 0);
        if (k + 1 < KS) {
          a0 = n0;
          a1 = n1;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (cj >= nfull_w) {
        const cpattn_plan_entry pe = tile[cc];
        const int lim = min(pe.k_len - 1, pe.delta + tok0 + n) - cj * BN - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kin = 8 * (r >> 2) + (r & 3);
          if (kin > lim) s0[r] = -INFINITY;
          if (32 + kin > lim) s1[r] = -INFINITY;
        }
      }
      // V^T fragments of the first key group, read before the softmax (LDS latency under VALU).
      bf16x8 va[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) va[dt] = vread(vs, dt);
      __builtin_amdgcn_sched_barrier(0);
      bool slow = __any(m_run == -INFINITY);
      Sums lane_sum = {0.f, 0.f};
      if (!slow) {
        lane_sum = exp_block(-m_run * scale_log2);
        slow = __any(!(lane_sum.p <= 256.0f));
      }
      if (slow) {
        float mx;
        {
          float t[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = __builtin_elementwise_max(s0[r], s1[r]);
#pragma unroll
          for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
            for (int r = 0; r < w; ++r) t[r] = __builtin_elementwise_max(t[r], t[r + w]);
          mx = pair_max(t[0]);
        }
        if (__any(mx > m_run + thr)) {
          const float m_new = __builtin_elementwise_max(m_run, mx);
          const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f((m_run - m_ref) * scale_log2);
#pragma unroll
          for (int i = 0; i < DT; ++i) acc[i] *= alpha;
          l_run *= alpha;
          lb_run *= alpha;
          m_run = m_new;
        }
        lane_sum = exp_block(-((m_run == -INFINITY) ? 0.f : m_run) * scale_log2);
      }
      l_run += lane_sum.p;
      lb_run += lane_sum.b;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const bf16x8 a = i < DT ? va[i] : vread(vs, i);
        acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pcur[i / DT], acc[i % DT], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (++cj == tile[cc].cost) {
      cc = next_chunk(cc);
      cj = 0;
      wave_range(cc, nblk_w, nfull_w);
    }
  };
  for (int p = 0; p < nblk_tile; p += 2) {
    step(p, std::integral_constant<int, 0>{});
    if (p + 1 < nblk_tile) step(p + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = acc / l_b, LSE = m * scale + ln l (or their merge into o, lse) ----
  // O is divided by the sum of the bf16 weights the PV product multiplied (an exact convex
  // combination of the values, whatever the rounding of the largest weight under the lazy
  // max), the LSE is taken from the sum of the fp32 weights.
  const float l_tot = pair_sum(l_run);
  const float lb_tot = pair_sum(lb_run);
  if (n < rows_w) {
    const int64_t row = row0 + tok0 + n;
    float* op = o + (row * hq + head) * D + 4 * g;
    float* lp = lse + int64_t(head) * tq_total + row;
    const float lse_new = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
    float wa = 0.f, wb = l_tot > 0.f ? 1.0f / lb_tot : 0.f, lse_out = lse_new;
    bool write = true;
    if (ACCUM) {
      // (O, LSE) <- merge((O, LSE), (acc / l, lse_new)); an empty side leaves the other exact.
      const float lse_old = *lp;
      if (l_tot == 0.f) {
        write = false;
      } else if (lse_old != -INFINITY) {
        const float mm = fmaxf(lse_old, lse_new);
        const float ea = expf(lse_old - mm), eb = expf(lse_new - mm);
        const float inv = 1.0f / (ea + eb);
        wa = ea * inv;
        wb = eb * inv / lb_tot;
        lse_out = mm + logf(ea + eb);
      }
    }
    if (write) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float4* dst = reinterpret_cast<float4*>(op + 32 * dt + 8 * rq);
          float4 val = make_float4(acc[dt][4 * rq] * wb, acc[dt][4 * rq + 1] * wb,
                                   acc[dt][4 * rq + 2] * wb, acc[dt][4 * rq + 3] * wb);
          if (ACCUM && wa != 0.f) {
            const float4 old = *dst;
            val = make_float4(fmaf(wa, old.x, val.x), fmaf(wa, old.y, val.y), fmaf(wa, old.z, val.z),
                              fmaf(wa, old.w, val.w));
          }
          *dst = val;
        }
      }
      if (g == 0) *lp = lse_out;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const ChunkPtrs<__bf16>& kv, int nchunks,
                                const cpattn_plan_entry* plan, int n_tiles, int head_groups,
                                int heads_per_tile, int hq, int hkv, int d, int tq_total,
                                bool accumulate, float* o, float* lse, hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid(unsigned(n_tiles) * unsigned(head_groups));
  const float scale = 1.0f / sqrtf(float(d));
  const float scale_log2 = scale * 1.4426950408889634f;
  const auto* qb = static_cast<const __bf16*>(q);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, qb, kv, nchunks, plan, head_groups,
                       heads_per_tile, hq, hkv, tq_total, scale, scale_log2, o, lse);
  };
  if (d == 128) {
    if (accumulate) launch(attn_fwd_bf16_kernel<128, true>);
    else launch(attn_fwd_bf16_kernel<128, false>);
  } else if (d == 64) {
    if (accumulate) launch(attn_fwd_bf16_kernel<64, true>);
    else launch(attn_fwd_bf16_kernel<64, false>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
