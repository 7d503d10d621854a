// Chunked causal attention backward, bf16 inputs, fp32 accumulation (gfx950).
//
// Gradients of O = softmax(Q K^T / sqrt(D) + mask) V for an upstream gradient dO,
// with the share's probabilities P = exp(S - LSE) rebuilt from the forward's final
// LSE (the online softmax of the "Megatron 6D parallelism guide", section 6, leaves
// exactly that LSE), dP = dO V^T and dS = P * (dP - delta), delta = rowsum(dO * O):
//   dQ += dS K / sqrt(D),   dK += dS^T Q / sqrt(D),   dV += P^T dO.
// Three kernels, no atomics (results are deterministic):
//   bwd_delta   delta [hq, Tq] = rowsum(dO * O), HBM-bound, and the LSE in log2 units
//               (+inf for rows with no visible key) for bwd_dkdv;
//   bwd_dq      query-stationary, the forward's tiling and its walk over the KV
//               chunks: per 64-key block S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, then
//               dQ^T += K^T dS^T; dQ is written once per launch;
//   bwd_dkdv    key-stationary: a work-group owns 128 keys of one kv head in one
//               chunk (32 per wave, K and V fragments held in registers) and streams
//               the query tokens that see them, 64 at a time, for every query head
//               of the group: S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P,
//               dK^T += Q^T dS.  One launch covers the key tiles of every chunk,
//               longest first.  Query blocks that see every key of the tile (all but
//               the causal diagonal and the ragged end) run in a loop of their own over
//               a copy of the step without the per-element mask; with one loop body per
//               case the accumulators stay in the matrix-core registers.
// Matrix-core mapping: every product is a v_mfma_f32_32x32x16_bf16 whose result
// keeps one column index per lane (lane % 32) and 16 row indices per lane, like the
// forward's S^T tile; the probability-like results (P, dS) are rounded to bf16 and
// used directly as the B operand of the next product, with the A operand gathered
// from LDS by the transpose read (ds_read_b64_tr_b16) in the same (lane group,
// element) -> k order.  Tiles that are read both by rows (16-byte reads) and
// transposed share one XOR swizzle that is conflict-free for both patterns.
//
// This file is compiled with -fno-honor-nans: rows with no visible key use an
// effective LSE of +inf, so every exponent is finite or -inf and no NaN arises.
#include <type_traits>

#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kThreads = 256;              // 4 waves in every backward kernel
constexpr int BN = kBf16BlockN;            // keys per block of the dQ kernel
constexpr int QB = kBwdQueryBlock;         // query tokens per block of the dK/dV kernel
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
static_assert(QB == 64 && BN == 64, "both kernels move 64-row tiles");

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = 64 * kRowBytes;         // one 64-row bf16 tile
  static constexpr int kRowsPerKB = 1024 / kRowBytes;   // rows one wave-wide load fills
  static constexpr int kLoadsPerWave = kBytes / 1024 / 4;
  // Swizzle for tiles read by rows only (16 consecutive rows, one chunk).
  __device__ static __forceinline__ int swz_rows(int row) {
    return (D == 128) ? (row & 15) : ((row >> 1) & 7);
  }
  // Swizzle for tiles read by rows AND transposed (4 consecutive rows, two adjacent
  // chunks): a bit permutation of the row index, a bijection over 16 rows that gives
  // every aligned group of 4 rows distinct chunk pairs.
  __device__ static __forceinline__ int swz_both(int row) {
    return (D == 128) ? ((row & 8) | ((row & 3) << 1) | ((row >> 2) & 1)) : ((row >> 1) & 7);
  }
  template <bool BOTH>
  __device__ static __forceinline__ int off(int row, int c) {
    return row * kRowBytes + ((c ^ (BOTH ? swz_both(row) : swz_rows(row))) << 4);
  }
};

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           int(bytes > 0x7fffffff ? 0x7fffffff : (bytes > 0 ? bytes : 0)),
                                           kBufferWord3);
}

// Rows [first, first + 64) of a [T, H, D] bf16 tensor for head h, rows past `rows_left` reading
// as zero, into an LDS tile (this wave's share of the 16 KB / 8 KB).
template <int D, bool BOTH>
__device__ __forceinline__ void load_tile(const __bf16* base, int64_t first, int h, int nh,
                                          int64_t rows_left, char* lds, int wave, int lane) {
  using T = Tile<D>;
  const int64_t stride = int64_t(nh) * D * 2;
  const int64_t n = rows_left > 0 ? (rows_left - 1) * stride + D * 2 : 0;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (first * nh + h) * D, n);
#pragma unroll
  for (int i = 0; i < T::kLoadsPerWave; ++i) {
    const int blk = wave * T::kLoadsPerWave + i;
    const int row = blk * T::kRowsPerKB + lane / T::kChunks;
    const int pc = lane % T::kChunks;
    const int sw = BOTH ? T::swz_both(row) : T::swz_rows(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + blk * 1024), 16,
                                             row * int(stride) + ((pc ^ sw) << 4), 0, 0, 0);
  }
}

// Two S-like products at once: C[32 rows][32 cols] over d for rows 0-31 and 32-63 of an LDS
// tile (row n of the lane's tile, lane % 32) against B fragments in registers, for tile_a x
// bf_a into c0, c1 and tile_b x bf_b into e0, e1; the k-steps are interleaved so that four
// independent accumulation chains keep the matrix core busy.
template <int D, bool BOTH_A, bool BOTH_B>
__device__ __forceinline__ void rows_product2(const char* tile_a, const bf16x8* bf_a,
                                              const char* tile_b, const bf16x8* bf_b, int n, int g,
                                              f32x16& c0, f32x16& c1, f32x16& e0, f32x16& e1) {
  using T = Tile<D>;
  constexpr int KS = D / 16;
  c0 = f32x16{};
  c1 = f32x16{};
  e0 = f32x16{};
  e1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(tile_a + T::template off<BOTH_A>(n, 2 * ks + g));
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(tile_a + T::template off<BOTH_A>(32 + n, 2 * ks + g));
    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(tile_b + T::template off<BOTH_B>(n, 2 * ks + g));
    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(tile_b + T::template off<BOTH_B>(32 + n, 2 * ks + g));
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bf_a[ks], c0, 0, 0, 0);
    e0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, bf_b[ks], e0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bf_a[ks], c1, 0, 0, 0);
    e1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, bf_b[ks], e1, 0, 0, 0);
  }
}

// Transposed product: acc^T[d][col] += Tile^T[d][row] * B[row][col] over the tile's 64 rows,
// the tile's columns gathered by transpose reads, B as bf16 fragments pb[4] (rows 16 kk ..).
template <int D>
__device__ __forceinline__ void transposed_product(const char* tile, const bf16x8* pb, int n, int g,
                                                   f32x16* acc) {
  using T = Tile<D>;
  constexpr int DT = D / 32;
  const int jr = (n & 15) >> 2, qq = n & 3, hh = n >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int row = 16 * kk + 4 * g + jr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int c16 = 4 * dt + 2 * hh + (qq >> 1);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(tile + T::template off<true>(row, c16) + 8 * (qq & 1)));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(tile + T::template off<true>(row + 8, c16) + 8 * (qq & 1)));
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], acc[dt], 0, 0, 0);
    }
  }
}

// bf16 B operand of a transposed product from two 32-row result tiles: rows 16 kk .. 16 kk + 15
// are registers 8 (kk % 2) .. + 7 of tile kk / 2.
__device__ __forceinline__ void pack_b(const f32x16& t0, const f32x16& t1, bf16x8* pb) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    pb[0][jj] = (__bf16)t0[jj];
    pb[1][jj] = (__bf16)t0[8 + jj];
    pb[2][jj] = (__bf16)t1[jj];
    pb[3][jj] = (__bf16)t1[8 + jj];
  }
}
#endif  // __HIP_DEVICE_COMPILE__

// ---------------------------------------------------------------------------
// delta[h][t] = sum_d dO[t, h, d] * O[t, h, d]: 16 lanes per (t, h) row; alongside, the row's
// LSE in log2 units, lse2[h][t] = LSE * log2(e), or +inf for a row with no visible key, so
// that P = exp2(S * scale * log2(e) - lse2) is one FMA and one exp2 (and 0 for such rows).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const __bf16* __restrict__ dout,
                                                             const float* __restrict__ o,
                                                             const float* __restrict__ lse, int tq,
                                                             int hq, float* __restrict__ delta,
                                                             float* __restrict__ lse2) {
  constexpr int EL = D / 16;  // elements per lane
  const int64_t rows = int64_t(tq) * hq;
  const int sub = threadIdx.x & 15;
  for (int64_t r = (int64_t(blockIdx.x) * kThreads + threadIdx.x) >> 4; r < rows;
       r += (int64_t(gridDim.x) * kThreads) >> 4) {
    const __bf16* dp = dout + r * D + sub * EL;
    const float* op = o + r * D + sub * EL;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < EL; e += 4) {
      const float4 ov = *reinterpret_cast<const float4*>(op + e);
      const bf16x4 dv = *reinterpret_cast<const bf16x4*>(dp + e);
      acc = fmaf(float(dv[0]), ov.x, acc);
      acc = fmaf(float(dv[1]), ov.y, acc);
      acc = fmaf(float(dv[2]), ov.z, acc);
      acc = fmaf(float(dv[3]), ov.w, acc);
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (sub == 0) {
      const int64_t t = r / hq;
      const int h = int(r - t * hq);
      delta[int64_t(h) * tq + t] = acc;
      const float l = lse[int64_t(h) * tq + t];
      lse2[int64_t(h) * tq + t] = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary.  Work-group = one tile of the forward's query plan.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ q, const ChunkPtrs<__bf16> kv, int nchunks,
    const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const cpattn_plan_entry* __restrict__ plan,
    int head_groups, int heads_per_tile, int hq, int hkv, int tq, float scale, float scale_log2,
    float* __restrict__ dq) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int kStage = 2 * T::kBytes;  // K tile (rows and transposed), then V tile (rows)
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int b = blockIdx.x;
  const int e = b / head_groups;
  const int hg = b - e * head_groups;
  const cpattn_plan_entry* tile = plan + int64_t(e) * nchunks;  // one entry per chunk
  const int head = hg * heads_per_tile + (wave % heads_per_tile);
  const int tok0 = (wave / heads_per_tile) * kBf16RowsPerWave;
  const int kvh = (hg * heads_per_tile) / (hq / hkv);
  const int rows_w = min(max(tile[0].nrows - tok0, 0), kBf16RowsPerWave);

  // B operands (token n's row of Q and of dO), the row's effective LSE (log2 units; +inf
  // for rows outside the tile or with no visible key: their P is 0) and delta.
  bf16x8 qf[KS], dof[KS];
  const bool ok = n < rows_w;
  const int64_t row = tile[0].row0 + tok0 + n;
  {
    const __bf16* qp = q + (row * hq + head) * D + 8 * g;
    const __bf16* dp = dout + (row * hq + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks) : bf16x8{};
      dof[ks] = ok ? *reinterpret_cast<const bf16x8*>(dp + 16 * ks) : bf16x8{};
    }
  }
  const float lse_row = ok ? lse[int64_t(head) * tq + row] : -INFINITY;
  const float lse_eff = lse_row == -INFINITY ? INFINITY : lse_row * 1.4426950408889634f;
  const float delta_row = ok ? delta[int64_t(head) * tq + row] : 0.f;

  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};

  // Block j of chunk c into LDS stage `stage`: K (read by rows and transposed), then V.
  auto issue = [&](int c, int j, int stage) {
    char* s = smem + stage * kStage;
    const int64_t first = int64_t(tile[c].k_start) + int64_t(j) * BN;
    const int64_t left = int64_t(tile[c].k_len) - int64_t(j) * BN;
    load_tile<D, true>(kv.k[c], first, kvh, hkv, left, s, wave, lane);
    load_tile<D, false>(kv.v[c], first, kvh, hkv, left, s + T::kBytes, wave, lane);
  };
  auto next_chunk = [&](int c) {
    ++c;
    while (c < nchunks && tile[c].cost == 0) ++c;
    return c;
  };

  int stage = 0;
  int c = next_chunk(-1);
  if (c < nchunks) issue(c, 0, 0);
  for (; c < nchunks;) {
    const cpattn_plan_entry pe = tile[c];
    const int cn = next_chunk(c);
    int nblk_w = 0, nfull_w = 0;
    if (rows_w > 0) {
      const int kend = max(0, min(pe.k_len, pe.delta + tok0 + rows_w));
      nblk_w = (kend + BN - 1) / BN;
      nfull_w = min(min(pe.k_len / BN, max(0, pe.delta + tok0 + 1) / BN), nblk_w);
    }
    const int nblk = pe.cost;
    auto run_block = [&](int j, auto masked) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 1 < nblk) issue(c, j + 1, stage ^ 1);
      else if (cn < nchunks) issue(cn, 0, stage ^ 1);
      if (j < nblk_w) {
        const char* kt = smem + stage * kStage;
        const char* vt = kt + T::kBytes;
        f32x16 s0, s1, p0, p1;
        // S^T = K Q^T and dP^T = V dO^T
        rows_product2<D, true, false>(kt, qf, vt, dof, n, g, s0, s1, p0, p1);
        const int lim = (decltype(masked)::value && j >= nfull_w)
                            ? min(pe.k_len - 1, pe.delta + tok0 + n) - j * BN - 4 * g
                            : BN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kin = 8 * (r >> 2) + (r & 3);
          float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, -lse_eff));
          float e1 = __builtin_amdgcn_exp2f(fmaf(s1[r], scale_log2, -lse_eff));
          if (decltype(masked)::value) {
            e0 = kin > lim ? 0.f : e0;
            e1 = 32 + kin > lim ? 0.f : e1;
          }
          s0[r] = e0 * (p0[r] - delta_row);                  // dS^T
          s1[r] = e1 * (p1[r] - delta_row);
        }
        bf16x8 dsb[4];
        pack_b(s0, s1, dsb);
        transposed_product<D>(kt, dsb, n, g, acc);           // dQ^T += K^T dS^T
      }
      stage ^= 1;
    };
    // Blocks below every wave's diagonal (the first wave's unmasked count bounds the others')
    // run a copy of the step without the mask, in a loop of their own.
    const int nfull_tile =
        min(min(pe.k_len / BN, max(0, pe.delta + 1) / BN), nblk);
    for (int j = 0; j < nfull_tile; ++j) run_block(j, std::false_type{});
    for (int j = nfull_tile; j < nblk; ++j) run_block(j, std::true_type{});
    c = cn;
  }

  if (ok) {
    float* op = dq + (row * hq + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4* dst = reinterpret_cast<float4*>(op + 32 * dt + 8 * rq);
        const float4 old = *dst;
        *dst = make_float4(fmaf(acc[dt][4 * rq], scale, old.x), fmaf(acc[dt][4 * rq + 1], scale, old.y),
                           fmaf(acc[dt][4 * rq + 2], scale, old.z), fmaf(acc[dt][4 * rq + 3], scale, old.w));
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// dK, dV: key-stationary.  Work-group = one tile of the key plan, all query heads of the
// kv head's group; wave w owns keys 32 w .. 32 w + 31 of the tile.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const ChunkPtrs<__bf16> kv, const __bf16* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ delta,
    const KeyTile* __restrict__ plan, int hq, int hkv, int tq, float scale, float scale_log2,
    const ChunkPtrs<float> dkv) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int kStage = 2 * T::kBytes + 512;  // Q tile, dO tile, lse2[64], delta[64]
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;
  const int e = blockIdx.x / hkv;
  const int kvh = blockIdx.x - e * hkv;
  const KeyTile pe = plan[e];
  const __bf16* k = kv.k[pe.chunk];
  const __bf16* v = kv.v[pe.chunk];
  const int group = hq / hkv;
  const int key = 32 * wave + n;          // this lane's key within the tile
  const bool key_ok = key < pe.nrows;
  const int64_t krow = int64_t(pe.row0) + key;

  // B operands: this lane's key row of K and of V.
  bf16x8 kf[KS], vf[KS];
  {
    const __bf16* kp = k + (krow * hkv + kvh) * D + 8 * g;
    const __bf16* vp = v + (krow * hkv + kvh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(kp + 16 * ks) : bf16x8{};
      vf[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(vp + 16 * ks) : bf16x8{};
    }
  }
  f32x16 dkt[DT], dvt[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    dkt[i] = f32x16{};
    dvt[i] = f32x16{};
  }

  const int t_first = max(pe.delta, 0);       // first query (within the sequence) to visit
  const int nblk = pe.cost;                   // query blocks per head
  const int total = nblk * group;             // (head, block) steps, head-major
  auto issue = [&](int step, int stage) {
    const int hi = step / nblk, j = step - hi * nblk;
    const int h = kvh * group + hi;
    const int64_t first = int64_t(pe.q_start) + t_first + int64_t(j) * QB;
    const int64_t left = int64_t(pe.q_len) - t_first - int64_t(j) * QB;
    char* s = smem + stage * kStage;
    load_tile<D, true>(q, first, h, hq, left, s, wave, lane);
    load_tile<D, true>(dout, first, h, hq, left, s + T::kBytes, wave, lane);
    if (wave < 2) {  // lse2 (wave 0) and delta (wave 1) of the block's 64 rows, 4 bytes per lane
      const float* src = (wave == 0 ? lse2 : delta) + int64_t(h) * tq + first;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(s + 2 * T::kBytes + 256 * wave), 4,
                                               lane * 4, 0, 0, 0);
    }
  };

  // Query blocks that every query of the tile's 128 keys sees (all but the causal diagonal
  // and the ragged end): j in [j_full0, j_full1) of every head; the steps of a head run in
  // three loops (masked, unmasked, masked) so each loop body is one straight copy of the step.
  const bool tile_full = pe.nrows == kBwdKeysPerTile;
  // first block whose first query sees the tile's last key, and blocks wholly inside the sequence
  const int lead = pe.delta + kBwdKeysPerTile - 1 - t_first;
  const int j_full0 = tile_full ? min(nblk, max(0, (lead + QB - 1) / QB)) : nblk;
  const int j_full1 = tile_full ? max(j_full0, min(nblk, (pe.q_len - t_first) / QB)) : nblk;
  auto run_step = [&](int step, auto masked) {
    const int stage = step & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (step + 1 < total) issue(step + 1, stage ^ 1);
    const int j = step % nblk;
    const char* qt = smem + stage * kStage;
    const char* dt_ = qt + T::kBytes;
    const float* lse_s = reinterpret_cast<const float*>(qt + 2 * T::kBytes);
    const float* del_s = lse_s + 64;
    // Query (within the sequence) of register r of tile tt: t_first + 64 j + 32 tt + 8 (r / 4)
    // + 4 g + r % 4; visible iff it is < q_len and >= delta + key.
    const int tb = t_first + j * QB + 4 * g;
    const int lo = pe.delta + key, hi_excl = pe.q_len;
    f32x16 s0, s1, p0, p1;
    // S = Q K^T and dP = dO V^T (rows: tokens)
    rows_product2<D, true, true>(qt, kf, dt_, vf, n, g, s0, s1, p0, p1);
    bf16x8 pb[4], db[4];
    f32x16 ps0, ps1;
    // Registers 4 i .. 4 i + 3 of tile tt hold rows 32 tt + 8 i + 4 g .. + 3: their lse2 and
    // delta are one 16-byte LDS read each.  P = exp2(S c - lse2), dS = P (dP - delta).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 l0 = *reinterpret_cast<const float4*>(lse_s + 8 * i + 4 * g);
      const float4 l1 = *reinterpret_cast<const float4*>(lse_s + 32 + 8 * i + 4 * g);
      const float4 d0 = *reinterpret_cast<const float4*>(del_s + 8 * i + 4 * g);
      const float4 d1 = *reinterpret_cast<const float4*>(del_s + 32 + 8 * i + 4 * g);
      const float la[4] = {l0.x, l0.y, l0.z, l0.w}, lb[4] = {l1.x, l1.y, l1.z, l1.w};
      const float da[4] = {d0.x, d0.y, d0.z, d0.w}, dbv[4] = {d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int r = 4 * i + k4;
        float e0 = __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, -la[k4]));
        float e1 = __builtin_amdgcn_exp2f(fmaf(s1[r], scale_log2, -lb[k4]));
        if (decltype(masked)::value) {
          const int t0 = tb + 8 * i + k4, t1 = t0 + 32;
          e0 = key_ok && t0 >= lo && t0 < hi_excl ? e0 : 0.f;
          e1 = key_ok && t1 >= lo && t1 < hi_excl ? e1 : 0.f;
        }
        ps0[r] = e0;
        ps1[r] = e1;
        s0[r] = e0 * (p0[r] - da[k4]);                            // dS
        s1[r] = e1 * (p1[r] - dbv[k4]);
      }
    }
    pack_b(ps0, ps1, pb);
    pack_b(s0, s1, db);
    transposed_product<D>(dt_, pb, n, g, dvt);   // dV^T += dO^T P
    transposed_product<D>(qt, db, n, g, dkt);    // dK^T += Q^T dS
  };

  if (total > 0) issue(0, 0);
  for (int hi = 0; hi < group; ++hi) {
    const int base = hi * nblk;
    for (int j = 0; j < j_full0; ++j) run_step(base + j, std::true_type{});
    for (int j = j_full0; j < j_full1; ++j) run_step(base + j, std::false_type{});
    for (int j = j_full1; j < nblk; ++j) run_step(base + j, std::true_type{});
  }

  if (key_ok) {
    float* kp = const_cast<float*>(dkv.k[pe.chunk]) + (krow * hkv + kvh) * D + 4 * g;
    float* vp = const_cast<float*>(dkv.v[pe.chunk]) + (krow * hkv + kvh) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4* a = reinterpret_cast<float4*>(kp + 32 * dt + 8 * rq);
        float4* c = reinterpret_cast<float4*>(vp + 32 * dt + 8 * rq);
        const float4 ka = *a, va = *c;
        *a = make_float4(fmaf(dkt[dt][4 * rq], scale, ka.x), fmaf(dkt[dt][4 * rq + 1], scale, ka.y),
                         fmaf(dkt[dt][4 * rq + 2], scale, ka.z), fmaf(dkt[dt][4 * rq + 3], scale, ka.w));
        *c = make_float4(dvt[dt][4 * rq] + va.x, dvt[dt][4 * rq + 1] + va.y,
                         dvt[dt][4 * rq + 2] + va.z, dvt[dt][4 * rq + 3] + va.w);
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

hipError_t launch_bwd_delta(const void* do_, const float* o, const float* lse, int tq, int hq,
                            int d, float* delta, float* lse2, hipStream_t stream) {
  const int64_t rows = int64_t(tq) * hq;
  if (rows == 0) return hipSuccess;
  int64_t blocks = (rows * 16 + kThreads - 1) / kThreads;
  blocks = blocks < 8192 ? blocks : 8192;
  const auto* db = static_cast<const __bf16*>(do_);
  if (d == 128) {
    hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, db, o,
                       lse, tq, hq, delta, lse2);
  } else if (d == 64) {
    hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, db, o,
                       lse, tq, hq, delta, lse2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const ChunkPtrs<__bf16>& kv, int nchunks, const void* do_,
                         const float* lse, const float* delta, const cpattn_plan_entry* plan,
                         int n_tiles, int head_groups, int heads_per_tile, int hq, int hkv, int d,
                         int tq, float* dq, hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid(unsigned(n_tiles) * unsigned(head_groups));
  const float scale = 1.0f / sqrtf(float(d));
  const float scale_log2 = scale * 1.4426950408889634f;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, static_cast<const __bf16*>(q), kv,
                       nchunks, static_cast<const __bf16*>(do_), lse, delta, plan, head_groups,
                       heads_per_tile, hq, hkv, tq, scale, scale_log2, dq);
  };
  if (d == 128) launch(bwd_dq_kernel<128>);
  else if (d == 64) launch(bwd_dq_kernel<64>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const ChunkPtrs<__bf16>& kv, const void* do_,
                           const float* lse2, const float* delta, const KeyTile* plan, int n_tiles,
                           int hq, int hkv, int d, int tq, const ChunkPtrs<float>& dkv,
                           hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid(unsigned(n_tiles) * unsigned(hkv));
  const float scale = 1.0f / sqrtf(float(d));
  const float scale_log2 = scale * 1.4426950408889634f;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, static_cast<const __bf16*>(q), kv,
                       static_cast<const __bf16*>(do_), lse2, delta, plan, hq, hkv, tq, scale,
                       scale_log2, dkv);
  };
  if (d == 128) launch(bwd_dkdv_kernel<128>);
  else if (d == 64) launch(bwd_dkdv_kernel<64>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
