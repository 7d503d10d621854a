// Chunked causal attention forward, bf16 inputs, fp32 accumulation (gfx950).
//
// One work-group = 4 waves = one tile of the host plan: up to 32 query tokens
// per wave, for heads_per_tile query heads of one GQA group (the waves of a
// tile share one kv head, so every K/V block staged in LDS serves all of them).
// The kernel walks the tile's key blocks (64 keys each) of ONE KV chunk, keeps a
// running max m and running sum l per query row (online softmax, the same
// update as the ring loop of the "Megatron 6D parallelism guide", section 6,
// applied across key blocks) and writes the normalised partial O = acc / l
// and LSE = m + ln l of that chunk.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64): the score tile is
// computed transposed, S^T[key][token] = K * Q^T, so the 32x32 accumulator puts
// one query token per lane column (lane % 32) and 16 of its keys per lane; lane
// l and lane l^32 together hold all 32 keys of that token.  Row statistics thus
// need one cross-half swap (v_permlane32_swap) per key block and no LDS.  The
// output is accumulated transposed too, O^T[d][token] = V^T * P^T: P comes
// straight from the score registers (bf16-rounded) as the B operand and V^T is
// the A operand read from LDS.  Both operands of each MFMA use the same
// (lane-group, element) -> k index mapping, so the contraction pairs the right
// keys whatever order the hardware sums them in.
//
// LDS per stage: K [64][D] bf16 (row-major, 16-byte chunks XOR-swizzled by row)
// and V^T [D][64] bf16 (keys permuted inside each group of 16 so that one lane's
// eight P keys are contiguous; chunks XOR-swizzled by row).  Two stages: block
// j+1 is fetched from HBM into registers while block j is computed, then stored
// to the other stage; one barrier per block.
//
// Masking: the host classifies blocks by global position, so only blocks on the
// causal diagonal or past the sequence end pay for per-element masking.  A row
// with no visible key keeps m = -inf and l = 0 and is written as (0, -inf).
#include "internal.h"

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = kBf16Waves * 64;
constexpr int BN = kBf16BlockN;  // keys per block

template <int D>
struct Layout {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per K row
  static constexpr int kKBytes = BN * D * 2;
  static constexpr int kVBytes = D * BN * 2;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kKLoads = BN * kChunks / kThreads;  // 16-byte K loads per thread
  static constexpr int kVTiles = (BN / 4) * kChunks;       // 4-key x 8-d tiles of V

  // byte offset of K (row r, chunk c) inside a stage
  __device__ static __forceinline__ int k_off(int r, int c) {
    const int sw = (D == 128) ? (r & 15) : ((r >> 1) & 7);
    return r * (D * 2) + ((c ^ sw) << 4);
  }
  // byte offset of V^T (row d, 16-byte chunk c of 8 key positions) inside a stage
  __device__ static __forceinline__ int vt_off(int d, int c) {
    return kKBytes + d * (BN * 2) + ((c ^ ((d >> 1) & 7)) << 4);
  }
};

// v_permlane32_swap with both operands = x leaves x of lanes 0..31 in the first
// result and x of lanes 32..63 in the second, each broadcast to both halves, so
// r[0] op r[1] combines lane l with lane l ^ 32 identically in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const cpattn_plan_entry* __restrict__ plan, int head_groups, int heads_per_tile, int hq,
    int hkv, int tq_total, float scale, float scale_log2, float* __restrict__ o,
    float* __restrict__ lse) {
  using L = Layout<D>;
  constexpr int KS = D / 16;  // k-steps of the score MFMA
  constexpr int DT = D / 32;  // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) char smem[2 * L::kStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // token column of the MFMA tiles
  const int g = lane >> 5;  // lane half

  const int b = blockIdx.x;
  const int e = b / head_groups;
  const int hg = b - e * head_groups;
  const cpattn_plan_entry pe = plan[e];
  const int head = hg * heads_per_tile + (wave % heads_per_tile);
  const int tok0 = (wave / heads_per_tile) * kBf16RowsPerWave;
  const int kvh = head / (hq / hkv);

  // Per-wave key range (rows tok0 .. tok0 + rows_w - 1 of the tile).
  const int rows_w = min(max(pe.nrows - tok0, 0), kBf16RowsPerWave);
  int nblk_w = 0, nfull_w = 0;
  if (rows_w > 0) {
    const int kend = max(0, min(pe.k_len, pe.delta + tok0 + rows_w));
    nblk_w = (kend + BN - 1) / BN;
    nfull_w = min(min(pe.k_len / BN, max(0, pe.delta + tok0 + 1) / BN), nblk_w);
  }
  const int nblk = pe.cost;  // blocks the whole tile visits (uniform)

  // Q fragment: B operand of S^T = K Q^T; lane holds Q[token n][16 ks + 8 g .. +7].
  bf16x8 qf[KS];
  {
    const bool ok = n < rows_w;
    const __bf16* qp = q + (int64_t(pe.row0 + tok0 + n) * hq + head) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ok) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      } else {
        qf[ks] = bf16x8{};
      }
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of raw scores (row n)
  float l_run = 0.f;        // running sum over this lane's keys

  // Global -> register staging of one K/V block.
  u32x4 kreg[L::kKLoads];
  u32x4 vreg[4];
  const int kc = tid % L::kChunks;
  const int kr = tid / L::kChunks;
  constexpr int kRowStep = kThreads / L::kChunks;
  const bool v_owner = tid < L::kVTiles;
  const int vdg = tid % L::kChunks;  // d chunk of the V tile
  const int vkg = tid / L::kChunks;  // 4-key group of the V tile
  const int64_t kv_stride = int64_t(hkv) * D;
  const __bf16* kbase = k + (int64_t(pe.k_start) * hkv + kvh) * D;
  const __bf16* vbase = v + (int64_t(pe.k_start) * hkv + kvh) * D;

  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < L::kKLoads; ++i) {
      const int key = j * BN + kr + i * kRowStep;
      if (key < pe.k_len) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + key * kv_stride + 8 * kc);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (v_owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = j * BN + 4 * vkg + i;
        if (key < pe.k_len) {
          vreg[i] = *reinterpret_cast<const u32x4*>(vbase + key * kv_stride + 8 * vdg);
        } else {
          vreg[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto stash = [&](int stage) {
    char* s = smem + stage * L::kStage;
#pragma unroll
    for (int i = 0; i < L::kKLoads; ++i)
      *reinterpret_cast<u32x4*>(s + L::k_off(kr + i * kRowStep, kc)) = kreg[i];
    if (v_owner) {
      // keys 4*vkg .. +3 land at positions swap(bits 2,3) inside their 16-group
      const int pos = 16 * (vkg >> 2) + 8 * (vkg & 1) + 4 * ((vkg >> 1) & 1);
      const int pc = pos >> 3, pb = (pos & 7) * 2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8 vdg + 2w (low halves) and 8 vdg + 2w + 1 (high halves)
        const unsigned a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xFFFFu) | (a1 << 16);
        lo[1] = (a2 & 0xFFFFu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
        const int d0 = 8 * vdg + 2 * w;
        *reinterpret_cast<u32x2*>(s + L::vt_off(d0, pc) + pb) = lo;
        *reinterpret_cast<u32x2*>(s + L::vt_off(d0 + 1, pc) + pb) = hi;
      }
    }
  };

  if (nblk > 0) fetch(0);

  for (int j = 0; j < nblk; ++j) {
    const int stage = j & 1;
    stash(stage);
    __syncthreads();
    if (j + 1 < nblk) fetch(j + 1);
    if (j < nblk_w) {
      const char* s = smem + stage * L::kStage;
      // ---- S^T = K Q^T for 64 keys (two 32-key tiles) ----
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(s + L::k_off(n, 2 * ks + g));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(s + L::k_off(32 + n, 2 * ks + g));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
      }
      // ---- mask (diagonal / ragged blocks only) ----
      if (j >= nfull_w) {
        // key (within block) of register r: 32 kt + 8 (r / 4) + 4 g + r % 4
        const int lim = min(pe.k_len - 1, pe.delta + tok0 + n) - j * BN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kin = 8 * (r >> 2) + 4 * g + (r & 3);
          if (kin > lim) s0[r] = -INFINITY;
          if (32 + kin > lim) s1[r] = -INFINITY;
        }
      }
      // ---- online softmax ----
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
      const float neg = -m_use * scale_log2;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, neg));
        s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], scale_log2, neg));
        psum += s0[r] + s1[r];
      }
      l_run = l_run * alpha + psum;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < DT; ++i) acc[i] *= alpha;
      }
      m_run = m_new;
      // P as bf16 B operands: key group kk takes registers 8 (kk % 2) .. +7 of tile kk / 2
      bf16x8 pf[4];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        pf[0][jj] = (__bf16)s0[jj];
        pf[1][jj] = (__bf16)s0[8 + jj];
        pf[2][jj] = (__bf16)s1[jj];
        pf[3][jj] = (__bf16)s1[8 + jj];
      }
      // ---- O^T += V^T P^T ----
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(s + L::vt_off(32 * dt + n, 2 * kk + g));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], acc[dt], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = m * scale + ln l ----
  const float l_tot = pair_sum(l_run);
  if (n < rows_w) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int64_t row = pe.row0 + tok0 + n;
    float* op = o + (row * hq + head) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4 val = make_float4(acc[dt][4 * rq] * inv, acc[dt][4 * rq + 1] * inv,
                                 acc[dt][4 * rq + 2] * inv, acc[dt][4 * rq + 3] * inv);
        *reinterpret_cast<float4*>(op + 32 * dt + 8 * rq) = val;
      }
    }
    if (g == 0) {
      lse[int64_t(head) * tq_total + row] = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v,
                                const cpattn_plan_entry* plan, int n_entries, int head_groups,
                                int heads_per_tile, int hq, int hkv, int d, int tq_total, float* o,
                                float* lse, hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  const dim3 grid(unsigned(n_entries) * unsigned(head_groups));
  const float scale = 1.0f / sqrtf(float(d));
  const float scale_log2 = scale * 1.4426950408889634f;
  const auto* qb = static_cast<const __bf16*>(q);
  const auto* kb = static_cast<const __bf16*>(k);
  const auto* vb = static_cast<const __bf16*>(v);
  if (d == 128) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, qb, kb, vb, plan,
                       head_groups, heads_per_tile, hq, hkv, tq_total, scale, scale_log2, o, lse);
  } else if (d == 64) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, qb, kb, vb, plan,
                       head_groups, heads_per_tile, hq, hkv, tq_total, scale, scale_log2, o, lse);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
