// Chunked causal attention backward, bf16 inputs, fp32 accumulation (gfx950).
//
// Gradients of O = softmax(Q K^T / sqrt(D) + mask) V for an upstream gradient dO,
// with the share's probabilities P = exp(S - LSE) rebuilt from the forward's final
// LSE (the online softmax of the "Megatron 6D parallelism guide", section 6, leaves
// exactly that LSE), dP = dO V^T and dS = P * (dP - delta), delta = rowsum(dO * O):
//   dQ += dS K / sqrt(D),   dK += dS^T Q / sqrt(D),   dV += P^T dO.
// Two launches, results deterministic (the only atomic is the arrival count of a split key
// tile, whose two partials are added commutatively):
//   bwd_delta   delta [hq, Tq] = rowsum(dO * O), HBM-bound, and the LSE in log2 units
//               (+inf for rows with no visible key) for the dK/dV work;
//   bwd_fused   the dQ and dK/dV work-groups in one grid, interleaved longest first by
//               the host, so each kind's last round is filled by the other kind:
//     dQ        query-stationary, the forward's tiling and its walk over the KV
//               chunks: per 64-key block S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, then
//               dQ^T += K^T dS^T; dQ is written once per launch;
//     dK/dV     key-stationary: a work-group owns 96 keys of one kv head in one
//               chunk and streams the query tokens that see them, 32 at a time, for
//               the query heads of the group (all, or half for a split tile).  Two
//               waves share 48 keys: one forms S = Q K^T, P and dV^T += dO^T P and
//               passes P through LDS, the other forms dP = dO V^T, dS and
//               dK^T += Q^T dS, so each holds one fragment set and one accumulator (two
//               work-groups per CU).  Query blocks that see every key of the tile (all
//               but the causal diagonal and the ragged end) skip the per-element mask.
// Matrix-core mapping (dQ; the dK/dV body describes its own 16x16 tiles below): every
// product is a v_mfma_f32_32x32x16_bf16 whose result
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kThreads = 256;              // 4 waves in every backward kernel
constexpr int BN = kBf16BlockN;            // keys per block of the dQ kernel
constexpr int QB = kBwdQueryBlock;         // query tokens per block of the dK/dV kernel
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
static_assert(QB == 32 && BN == 64, "the dQ kernel moves 64-row tiles, the dK/dV kernel 32-row tiles");

template <int D, int ROWS = 64>
struct Tile {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = ROWS * kRowBytes;       // one ROWS-row bf16 tile
  static constexpr int kRowsPerKB = 1024 / kRowBytes;   // rows one wave-wide load fills
  static constexpr int kLoadsPerWave = kBytes / 1024 / 4;
  static_assert(kLoadsPerWave >= 1, "the 4 waves share a tile's loads");
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
  // Swizzle of the dK/dV kernel's 32-row tiles, read by rows (16 consecutive rows, one chunk)
  // and by 16x16 transpose reads (8 consecutive rows, two adjacent chunks).  For D = 128 it is
  // a bijection over 16 rows that also puts each of 8 consecutive rows in its own chunk pair
  // (measured: half the bank-conflict cycles of swz_both on these reads).
  __device__ static __forceinline__ int swz_pair(int row) {
    return (D == 128) ? (2 * (row & 7) + ((row >> 3) & 1)) : ((row >> 1) & 7);
  }
  __device__ static __forceinline__ int off_pair(int row, int c) {
    return row * kRowBytes + ((c ^ swz_pair(row)) << 4);
  }
};

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // clamp to [0, 2^31 - 1] with 32-bit scalar operations (no 64-bit signed compare)
  const uint64_t u = uint64_t(bytes);
  const int n = (u >> 63) ? 0 : ((u >> 31) ? 0x7fffffff : int(u));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferWord3);
}

// Rows [first, first + ROWS) of a [T, H, D] bf16 tensor for head h, rows past `rows_left` reading
// as zero, into an LDS tile (this wave's quarter of it).
template <int D, bool BOTH, int ROWS = 64>
__device__ __forceinline__ void load_tile(const __bf16* base, int64_t first, int h, int nh,
                                          int64_t rows_left, char* lds, int wave, int lane) {
  using T = Tile<D, ROWS>;
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

// Transposed product: acc^T[d][col] += Tile^T[d][row] * B[row][col] over the tile's ROWS rows,
// the tile's columns gathered by transpose reads, B as bf16 fragments pb[ROWS / 16] (rows 16 kk ..).
template <int D, int ROWS = 64>
__device__ __forceinline__ void transposed_product(const char* tile, const bf16x8* pb, int n, int g,
                                                   f32x16* acc) {
  using T = Tile<D, ROWS>;
  constexpr int DT = D / 32;
  const int jr = (n & 15) >> 2, qq = n & 3, hh = n >> 4;
#pragma unroll
  for (int kk = 0; kk < ROWS / 16; ++kk) {
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

// Elements 4 h .. 4 h + 3 of a bf16 fragment from four floats, two per conversion.
__device__ __forceinline__ void set4(bf16x8& f, int h, const float* x) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_bit_cast(s16x8, f);
  const s16x2 a = __builtin_bit_cast(s16x2, bf16x2{(__bf16)x[0], (__bf16)x[1]});
  const s16x2 b = __builtin_bit_cast(s16x2, bf16x2{(__bf16)x[2], (__bf16)x[3]});
  v[4 * h] = a[0];
  v[4 * h + 1] = a[1];
  v[4 * h + 2] = b[0];
  v[4 * h + 3] = b[1];
  f = __builtin_bit_cast(bf16x8, v);
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
// LDS of a dQ work-group: two stages of a K tile (read by rows and transposed) and a V tile.
template <int D>
constexpr int dq_lds_bytes() { return 2 * 2 * Tile<D>::kBytes; }

// Work-group b of the dQ launch (tile b / head_groups of the query plan, head group
// b % head_groups), with `smem` its dq_lds_bytes<D>() of LDS.
template <int D>
__device__ __forceinline__ void dq_body(
    int b, char* smem, const __bf16* __restrict__ q, const ChunkPtrs<__bf16>& kv, int nchunks,
    const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, const cpattn_plan_entry* __restrict__ plan,
    int head_groups, int heads_per_tile, int hq, int hkv, int tq, float scale, float scale_log2,
    float* __restrict__ dq) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int kStage = 2 * T::kBytes;  // K tile (rows and transposed), then V tile (rows)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;
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

  // Block j of a chunk into LDS stage `stage`: K (read by rows and transposed), then V, through
  // buffer resources that end at the sequence's last key of the chunk (rows past it read as
  // zero).  The lane offsets within a tile are the same for every block; a chunk's K/V bases
  // and byte span are formed once per chunk, and a block only moves them.
  const int64_t kv_row_bytes = int64_t(hkv) * D * 2;
  const int64_t kv_blk_bytes = kv_row_bytes * BN;
  int voff_k[T::kLoadsPerWave], voff_v[T::kLoadsPerWave];
#pragma unroll
  for (int l = 0; l < T::kLoadsPerWave; ++l) {
    const int row = (wave * T::kLoadsPerWave + l) * T::kRowsPerKB + lane / T::kChunks;
    const int pc = lane % T::kChunks;
    voff_k[l] = row * int(kv_row_bytes) + ((pc ^ T::swz_both(row)) << 4);
    voff_v[l] = row * int(kv_row_bytes) + ((pc ^ T::swz_rows(row)) << 4);
  }
  struct ChunkSrc {
    const char* k;
    const char* v;
    int64_t span;   // bytes from the chunk's first key row of this kv head to its last one's end
  };
  auto chunk_src = [&](int c) {
    const int64_t base = (int64_t(tile[c].k_start) * hkv + kvh) * D;
    return ChunkSrc{reinterpret_cast<const char*>(kv.k[c] + base),
                    reinterpret_cast<const char*>(kv.v[c] + base),
                    int64_t(tile[c].k_len - 1) * kv_row_bytes + D * 2};
  };
  auto issue = [&](const ChunkSrc& cs, int j, int stage) __attribute__((always_inline)) {
    char* s = smem + stage * kStage;
    const int64_t off = int64_t(j) * kv_blk_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(cs.k + off, cs.span - off);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(cs.v + off, cs.span - off);
#pragma unroll
    for (int l = 0; l < T::kLoadsPerWave; ++l) {
      const int blk = wave * T::kLoadsPerWave + l;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(s + blk * 1024), 16, voff_k[l], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(s + T::kBytes + blk * 1024), 16,
                                               voff_v[l], 0, 0, 0);
    }
  };
  auto next_chunk = [&](int c) {
    ++c;
    while (c < nchunks && tile[c].cost == 0) ++c;
    return c;
  };

  int stage = 0;
  int c = next_chunk(-1);
  if (c < nchunks) issue(chunk_src(c), 0, 0);
  for (; c < nchunks;) {
    const cpattn_plan_entry pe = tile[c];
    const int cn = next_chunk(c);
    const ChunkSrc src_c = chunk_src(c);
    const ChunkSrc src_n = cn < nchunks ? chunk_src(cn) : src_c;
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
      if (j + 1 < nblk) issue(src_c, j + 1, stage ^ 1);
      else if (cn < nchunks) issue(src_n, 0, stage ^ 1);
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
// dK, dV: key-stationary.  Work-group = one tile of the key plan (96 keys of one kv head in
// one chunk), all query heads of the kv head's group.  The four waves form two pairs; pair p
// owns keys 48 p .. 48 p + 47 and splits the step's four products between its two waves:
//   wave A (even):  S = Q K^T, P = exp(S - LSE) (masked), P -> LDS, dV^T += dO^T P;
//   wave B (odd):   dP = dO V^T, P <- LDS, dS = P (dP - delta), dK^T += Q^T dS.
// Each wave thus holds one fragment set (K or V) and one accumulator (dV^T or dK^T), about
// 150 registers for D = 128, so two work-groups share a CU, and every Q or dO fragment read
// from LDS feeds three 16-key products.  Wave B works one step behind wave A (it needs A's P):
// the Q / dO / lse / delta tiles rotate through three LDS stages and P through two buffers,
// and one barrier per step orders everything.
// Products are v_mfma_f32_16x16x32_bf16 on 16-key tiles nt: a result tile keeps key 16 nt +
// (lane % 16) in every lane and rows 4 (lane / 16) + r in register r.  For the 32 queries of a
// step, rows 16 mt + 4 G + r (G = lane / 16) of the two 16-query tiles mt are the eight bf16
// values of one B operand in (mt, r) order; the matching A operands (dO^T, Q^T) are gathered
// in the same order by transpose reads.
// ---------------------------------------------------------------------------
// kSplit: the launch has split tiles (a build without the split epilogue otherwise, whose
// register allocation is the leaner one for the main loop).
// LDS of a dK/dV work-group: three stages of Q and dO tiles with their lse2 and delta, and
// two P buffers per wave pair.
template <int D>
constexpr int dkdv_lds_bytes() {
  return 3 * (2 * Tile<D, QB>::kBytes + 512) + 2 * 2 * (kPairKeys / 16) * 1024;
}

// Work-group wg of the dK/dV launch (part wg / hkv of the key plan, kv head wg % hkv), with
// `smem` its dkdv_lds_bytes<D>() of LDS and `arrivals` an LDS int.
template <int D, bool kSplit>
__device__ __forceinline__ void dkdv_body(
    int wg, char* smem, int& arrivals, const __bf16* __restrict__ q, const ChunkPtrs<__bf16>& kv,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ delta, const KeyPart* __restrict__ plan, int hq, int hkv, int tq,
    float scale, float scale_log2, const ChunkPtrs<float>& dkv, int* __restrict__ counters,
    float* __restrict__ scratch) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D, QB>;
  constexpr int KS = D / 32;                       // 32-wide k-steps over d
  constexpr int DT = D / 16;                       // 16-row tiles of d
  constexpr int NT = kPairKeys / 16;               // 16-key tiles of a pair
  constexpr int kStage = 2 * T::kBytes + 512;      // Q tile, dO tile, lse2[64], delta[64]
  constexpr int kPBytes = NT * 1024;               // P of one pair for one step, bf16

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i16 = lane & 15;                       // column (key) of a result tile
  const int G = lane >> 4;                         // 16-lane group
  const int e = wg / hkv;
  const int kvh = wg - e * hkv;
  const KeyPart pe = plan[e];
  const int group = hq / hkv;
  const int pair = wave >> 1;
  const bool role_a = (wave & 1) == 0;
  const int key0 = kPairKeys * pair;               // the pair's first key within the tile
  char* const pbuf = smem + 3 * kStage + pair * 2 * kPBytes;   // this pair's two P buffers

  const int t_first = max(pe.delta, 0);       // first query (within the sequence) to visit
  const int nblk = pe.cost;                   // query blocks per head
  const int h0 = pe.h_begin;                  // the part's query heads of the group: [h0, h1)
  const int total = nblk * (pe.h_end - h0);   // (head, block) steps, head-major
  // Loads of step (hi, j): rows t_first + 32 j .. + 31 of query head kvh * group + hi from Q and
  // dO, and their lse2 (wave 0) and delta (wave 1) values, each through a buffer resource that
  // ends at the sequence's last query (rows past it read as zero).  The lane offsets within a
  // tile are the same for every step; the step moves the resource bases.
  const int64_t row_bytes = int64_t(hq) * D * 2;
  const int64_t blk_bytes = row_bytes * QB;
  const int64_t q_first = int64_t(pe.q_start) + t_first;
  const char* const q0 = reinterpret_cast<const char*>(q + (q_first * hq + kvh * group) * D);
  const char* const o0 = reinterpret_cast<const char*>(dout + (q_first * hq + kvh * group) * D);
  const int64_t span0 = int64_t(pe.q_len - t_first - 1) * row_bytes + D * 2;   // bytes of block 0 on
  const float* const v0 = (wave == 0 ? lse2 : delta) + int64_t(kvh * group) * tq + q_first;
  const int rows0 = pe.q_len - t_first;
  int voff[T::kLoadsPerWave];
#pragma unroll
  for (int l = 0; l < T::kLoadsPerWave; ++l) {
    const int row = (wave * T::kLoadsPerWave + l) * T::kRowsPerKB + lane / T::kChunks;
    voff[l] = row * int(row_bytes) + (((lane % T::kChunks) ^ T::swz_pair(row)) << 4);
  }
  auto issue = [&](int hi, int j, int stage) __attribute__((always_inline)) {
    char* s = smem + stage * kStage;
    const int64_t off = int64_t(j) * blk_bytes + hi * (D * 2);
    const int64_t span = span0 - int64_t(j) * blk_bytes;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q0 + off, span);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o0 + off, span);
#pragma unroll
    for (int l = 0; l < T::kLoadsPerWave; ++l) {
      const int blk = wave * T::kLoadsPerWave + l;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(s + blk * 1024), 16, voff[l], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lds_void*)(s + T::kBytes + blk * 1024), 16, voff[l],
                                               0, 0, 0);
    }
    if (wave < 2) {
      const __amdgpu_buffer_rsrc_t r =
          make_rsrc(v0 + int64_t(hi) * tq + int64_t(j) * QB, int64_t(rows0 - j * QB) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(s + 2 * T::kBytes + 256 * wave), 4,
                                               lane * 4, 0, 0, 0);
    }
  };
  // Steps run head-major: (hi, j) of a step, advanced by one per step, and its LDS stage.
  struct Cursor {
    int hi, j = 0, stage = 0;
    __device__ explicit Cursor(int h) : hi(h) {}
    __device__ void next(int nb) {
      if (++j == nb) { j = 0; ++hi; }
      stage = stage == 2 ? 0 : stage + 1;
    }
  };
  // Lane-constant parts of the LDS reads.  Row reads (A operand of S and dP): query 16 mt +
  // i16, d-chunk 4 ks + G.  Transpose reads (A operand of dV^T and dK^T): the lane supplies
  // query 4 G + jr (+ 16 for elements 4..7) at d columns 16 dt + 4 qq .. + 3 and receives
  // d = 16 dt + i16 at queries 4 G .. 4 G + 3 (and 16 + 4 G ..).
  const int jr = i16 >> 2, qq = i16 & 3;
  auto tr_frag = [&](const char* tile, int dt) __attribute__((always_inline)) {
    const int c16 = 2 * dt + (qq >> 1);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(tile + T::off_pair(4 * G + jr, c16) + 8 * (qq & 1)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)(tile + T::off_pair(16 + 4 * G + jr, c16) + 8 * (qq & 1)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // This lane's row (key 16 nt + i16 of the pair) of a [T, hkv, D] tensor as B operands.
  auto key_frags = [&](const __bf16* base, bf16x8 (&f)[NT][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int key = key0 + 16 * nt + i16;
      const __bf16* p = base + ((int64_t(pe.row0) + key) * hkv + kvh) * D + 8 * G;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        f[nt][ks] = key < pe.nrows ? *reinterpret_cast<const bf16x8*>(p + 32 * ks) : bf16x8{};
    }
  };
  // acc^T tile (dt, nt) holds d = 16 dt + 4 G + r of key 16 nt + i16: fold it into the fp32
  // gradient rows (times `mul`).
  auto store_acc_rows = [&](float* base, const f32x4 (&acc)[NT][DT], float mul) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int key = key0 + 16 * nt + i16;
      if (key < pe.nrows) {
        float* p = base + ((int64_t(pe.row0) + key) * hkv + kvh) * D + 4 * G;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float4* c = reinterpret_cast<float4*>(p + 16 * dt);
          const float4 o = *c;
          *c = make_float4(fmaf(acc[nt][dt][0], mul, o.x), fmaf(acc[nt][dt][1], mul, o.y),
                           fmaf(acc[nt][dt][2], mul, o.z), fmaf(acc[nt][dt][3], mul, o.w));
        }
      }
    }
  };

  // The end of a part: an unsplit tile folds its accumulator into the gradient rows.  The two
  // halves of a split tile each store theirs to their slot of the unit's scratch, and then
  // count their arrival (device scope, after a release fence).  The second to arrive reads the
  // other's slot (after an acquire fence), adds it, and folds the sum. fp32 addition is
  // commutative, so the sum is the same whichever half arrives second.  Both roles call this
  // at the same point, so every wave meets the same barriers.
  auto finish = [&](float* base, f32x4 (&acc)[NT][DT], float mul) __attribute__((always_inline)) {
    if (!kSplit || pe.split < 0) {
      store_acc_rows(base, acc, mul);
      return;
    }
    const int64_t unit = int64_t(pe.split) * hkv + kvh;
    constexpr int kWaveFloats = NT * DT * 4 * 64;
    float* mine = scratch + (unit * 2 + pe.part) * bwd_part_floats(D) + wave * kWaveFloats;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(mine + ((nt * DT + dt) * 64 + lane) * 4) = acc[nt][dt];
    __threadfence();
    __syncthreads();
    if (tid == 0) arrivals = atomicAdd(counters + unit, 1);
    __syncthreads();
    if (arrivals == 0) return;   // the other half folds both
    __threadfence();
    const float* other = scratch + (unit * 2 + (pe.part ^ 1)) * bwd_part_floats(D) + wave * kWaveFloats;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[nt][dt] += *reinterpret_cast<const f32x4*>(other + ((nt * DT + dt) * 64 + lane) * 4);
    store_acc_rows(base, acc, mul);
  };

  if (total > 0) issue(h0, 0, 0);

  if (role_a) {
    bf16x8 kf[NT][KS];
    key_frags(kv.k[pe.chunk], kf);
    f32x4 dvt[NT][DT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dvt[nt][dt] = f32x4{};

    // Blocks that every query of the tile's keys sees in full (all but the causal diagonal and
    // the ragged end) skip the per-element mask.
    const bool tile_full = pe.nrows == kBwdKeysPerTile;
    const int lead = pe.delta + kBwdKeysPerTile - 1 - t_first;
    const int j_full0 = tile_full ? min(nblk, max(0, (lead + QB - 1) / QB)) : nblk;
    const int j_full1 = tile_full ? max(j_full0, min(nblk, (pe.q_len - t_first) / QB)) : nblk;

    auto a_step = [&](const Cursor& cur, int pb_sel, auto masked) __attribute__((always_inline)) {
      const char* qt = smem + cur.stage * kStage;
      const char* dt_ = qt + T::kBytes;
      const float* lse_s = reinterpret_cast<const float*>(qt + 2 * T::kBytes);
      bf16x8 pb[NT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 s[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {   // S = Q K^T, one Q fragment for the three key tiles
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(qt + T::off_pair(16 * mt + i16, 4 * ks + G));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[nt][ks], s[nt], 0, 0, 0);
        }
        // Register r holds query t_first + 32 j + 16 mt + 4 G + r of the sequence.
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + 16 * mt + 4 * G);
        const float la[4] = {l4.x, l4.y, l4.z, l4.w};
        int lo[NT], hi = 4;
        if (decltype(masked)::value) {   // visible registers r in [lo, hi) of each key tile
          const int tb = t_first + cur.j * QB + 16 * mt + 4 * G;
          hi = min(max(pe.q_len - tb, 0), 4);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int key = key0 + 16 * nt + i16;
            lo[nt] = key < pe.nrows ? min(max(pe.delta + key - tb, 0), 4) : 4;
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(fmaf(s[nt][r], scale_log2, -la[r]));
            if (decltype(masked)::value) p[r] = (r >= lo[nt] && r < hi) ? p[r] : 0.f;
          }
          set4(pb[nt], mt, p);
        }
      }
      char* pw = pbuf + pb_sel * kPBytes + lane * 16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<bf16x8*>(pw + nt * 1024) = pb[nt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {     // dV^T += dO^T P, one dO^T fragment for three tiles
        const bf16x8 a = tr_frag(dt_, dt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dvt[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt], dvt[nt][dt], 0, 0, 0);
      }
    };

    // One loop per run of masked or unmasked blocks, so that each loop body holds one copy of
    // the step.
    Cursor cur(h0);
    int s = 0;
    auto a_iter = [&](auto masked) __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      Cursor nx = cur;
      nx.next(nblk);
      if (s + 1 < total) issue(nx.hi, nx.j, nx.stage);
      a_step(cur, s & 1, masked);
      cur = nx;
      ++s;
    };
    for (int hi = h0; hi < pe.h_end; ++hi) {
      for (int j = 0; j < j_full0; ++j) a_iter(std::true_type{});
      for (int j = j_full0; j < j_full1; ++j) a_iter(std::false_type{});
      for (int j = j_full1; j < nblk; ++j) a_iter(std::true_type{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // wave B's last step

    finish(const_cast<float*>(dkv.v[pe.chunk]), dvt, 1.f);
  } else {
    bf16x8 vf[NT][KS];
    key_frags(kv.v[pe.chunk], vf);
    f32x4 dkt[NT][DT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dkt[nt][dt] = f32x4{};

    // wave A's step one earlier: its tiles are still in stage `cur.stage`, its P in pb_sel
    auto b_step = [&](const Cursor& cur, int pb_sel) __attribute__((always_inline)) {
      const char* qt = smem + cur.stage * kStage;
      const char* dt_ = qt + T::kBytes;
      const float* del_s = reinterpret_cast<const float*>(qt + 2 * T::kBytes + 256);
      const char* pr = pbuf + pb_sel * kPBytes + lane * 16;
      bf16x8 pf[NT], db[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pf[nt] = *reinterpret_cast<const bf16x8*>(pr + nt * 1024);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 p[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) p[nt] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {   // dP = dO V^T, one dO fragment for the three tiles
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(dt_ + T::off_pair(16 * mt + i16, 4 * ks + G));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            p[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vf[nt][ks], p[nt], 0, 0, 0);
        }
        const float4 d4 = *reinterpret_cast<const float4*>(del_s + 16 * mt + 4 * G);
        const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = float(pf[nt][4 * mt + r]) * (p[nt][r] - dl[r]);
          set4(db[nt], mt, x);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {     // dK^T += Q^T dS, one Q^T fragment for three tiles
        const bf16x8 a = tr_frag(qt, dt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dkt[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, db[nt], dkt[nt][dt], 0, 0, 0);
      }
    };

    Cursor cur(h0);   // the step wave B works on (one behind the loop counter)
    Cursor ld(h0);    // the step whose tiles the loop issues
    for (int s = 0; s <= total; ++s) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (s < total) {
        ld.next(nblk);
        if (s + 1 < total) issue(ld.hi, ld.j, ld.stage);
      }
      if (s >= 1) {
        b_step(cur, (s - 1) & 1);
        cur.next(nblk);
      }
    }

    finish(const_cast<float*>(dkv.k[pe.chunk]), dkt, scale);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// The gradient launch: the dQ work-groups and the dK/dV work-groups in one grid, in the
// longest-first order the host interleaves from both plans (order[b]: dQ work-group, or dK/dV
// work-group | kDkdvBit), so each kind's last, part-filled round is filled by the other kind.
// Both bodies run two work-groups per CU; the LDS buffer fits the larger of the two.
// ---------------------------------------------------------------------------
template <int D, bool kSplit>
__global__ __launch_bounds__(kThreads, 2) void bwd_fused_kernel(const BwdArgs a,
                                                                const uint32_t* __restrict__ order) {
  constexpr int kLds = dq_lds_bytes<D>() > dkdv_lds_bytes<D>() ? dq_lds_bytes<D>() : dkdv_lds_bytes<D>();
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  __shared__ int arrivals;
  const uint32_t w = order[blockIdx.x];
  const float scale = 1.0f / sqrtf(float(D));
  const float scale_log2 = scale * 1.4426950408889634f;
  const auto* q = static_cast<const __bf16*>(a.q);
  const auto* dout = static_cast<const __bf16*>(a.dout);
  if (w & kDkdvBit) {
    dkdv_body<D, kSplit>(int(w & ~kDkdvBit), smem, arrivals, q, a.kv, dout, a.lse2, a.delta,
                         a.kplan, a.hq, a.hkv, a.tq, scale, scale_log2, a.dkv, a.counters,
                         a.scratch);
  } else {
    dq_body<D>(int(w), smem, q, a.kv, a.nchunks, dout, a.lse, a.delta, a.qplan, a.head_groups,
               a.heads_per_tile, a.hq, a.hkv, a.tq, scale, scale_log2, a.dq);
  }
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

hipError_t launch_bwd_fused(const BwdArgs& a, const uint32_t* order, int n_wg, bool split, int d,
                            hipStream_t stream) {
  if (n_wg == 0) return hipSuccess;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(unsigned(n_wg)), dim3(kThreads), 0, stream, a, order);
  };
  if (d == 128) split ? launch(bwd_fused_kernel<128, true>) : launch(bwd_fused_kernel<128, false>);
  else if (d == 64) split ? launch(bwd_fused_kernel<64, true>) : launch(bwd_fused_kernel<64, false>);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
