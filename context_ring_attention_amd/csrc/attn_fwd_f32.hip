// Chunked causal attention forward, fp32 inputs and arithmetic (gfx950 VALU).
//
// Same contract as the bf16 kernel (normalised O and LSE of a tile's rows over
// the keys of its KV chunks, written or merged into the running result), for
// callers that need fp32 accuracy.  One work-group handles 64 query tokens of
// one head; four lanes share a query row, each owning D/4 contiguous
// dimensions, and combine their partial dot products with two lane swaps.  Keys
// are staged through LDS in blocks of 32.  The softmax is an exact two-pass
// one: pass 1 finds each row's max m and sum l over every chunk, pass 2
// accumulates exp(s - m) / l * v.  Both passes evaluate every score with the
// same arithmetic, so pass 2 sees exactly the scores pass 1 reduced.
#include "internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
static_assert(kF32TokensPerTile * 4 == kThreads, "four lanes per query row");
constexpr int BN = kF32BlockN;         // 32 keys per block

template <int D, bool ACCUM>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const ChunkPtrs<float> kv, int nchunks,
    const cpattn_plan_entry* __restrict__ plan, int hq, int hkv, int tq_total, float scale,
    float* __restrict__ o, float* __restrict__ lse) {
  constexpr int DP = D / 4;  // dims per lane
  __shared__ float4 ks[BN * D / 4];
  __shared__ float4 vs[BN * D / 4];

  const int tid = threadIdx.x;
  const int r = tid >> 2;   // tile row
  const int p = tid & 3;    // dimension quarter
  const int e = blockIdx.x / hq;
  const int head = blockIdx.x - e * hq;
  const cpattn_plan_entry* tile = plan + int64_t(e) * nchunks;  // one entry per chunk
  const int row0 = tile[0].row0;
  const int kvh = head / (hq / hkv);
  const bool row_ok = r < tile[0].nrows;

  float qr[DP];
  {
    const float* qp = q + (int64_t(row0 + r) * hq + head) * D + p * DP;
#pragma unroll
    for (int i = 0; i < DP; i += 4) {
      float4 x = row_ok ? *reinterpret_cast<const float4*>(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      qr[i] = x.x; qr[i + 1] = x.y; qr[i + 2] = x.z; qr[i + 3] = x.w;
    }
  }
  const int64_t kv_stride = int64_t(hkv) * D;

  // Stage block j of chunk c (keys k_start + 32 j ..) into LDS.
  auto stage = [&](int c, int j, bool with_v) {
    const cpattn_plan_entry& pe = tile[c];
    const float* kbase = kv.k[c] + (int64_t(pe.k_start) * hkv + kvh) * D;
    const float* vbase = kv.v[c] + (int64_t(pe.k_start) * hkv + kvh) * D;
    for (int idx = tid; idx < BN * D / 4; idx += kThreads) {
      const int key = idx / (D / 4), cc = idx - key * (D / 4);
      const int gk = j * BN + key;
      const bool ok = gk < pe.k_len;
      ks[idx] = ok ? *reinterpret_cast<const float4*>(kbase + gk * kv_stride + 4 * cc)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
      if (with_v)
        vs[idx] = ok ? *reinterpret_cast<const float4*>(vbase + gk * kv_stride + 4 * cc)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto score = [&](int u) {
    const float* kr = reinterpret_cast<const float*>(ks) + u * D + p * DP;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < DP; ++i) part = fmaf(qr[i], kr[i], part);
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    return part * scale;
  };

  // pass 1: row max and row sum over every chunk
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const cpattn_plan_entry& pe = tile[c];
    const int lim_row = pe.delta + r;  // row sees keys u <= lim_row of this chunk
    for (int j = 0; j < pe.cost; ++j) {
      stage(c, j, false);
      __syncthreads();
      float sv[BN];
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < BN; ++u) {
        const int key = j * BN + u;
        const float sc = score(u);
        sv[u] = (key < pe.k_len && key <= lim_row) ? sc : -INFINITY;
        bm = fmaxf(bm, sv[u]);
      }
      const float m_new = fmaxf(m, bm);
      if (m_new != -INFINITY) {
        float bs = 0.f;
#pragma unroll
        for (int u = 0; u < BN; ++u) bs += expf(sv[u] - m_new);
        l = l * expf(m - m_new) + bs;
        m = m_new;
      }
      __syncthreads();
    }
  }
  // pass 2: output
  float acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) acc[i] = 0.f;
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const cpattn_plan_entry& pe = tile[c];
    const int lim_row = pe.delta + r;
    for (int j = 0; j < pe.cost; ++j) {
      stage(c, j, true);
      __syncthreads();
#pragma unroll 4
      for (int u = 0; u < BN; ++u) {
        const int key = j * BN + u;
        const float sc = score(u);
        const float w = (key < pe.k_len && key <= lim_row) ? expf(sc - m) * inv_l : 0.f;
        const float* vr = reinterpret_cast<const float*>(vs) + u * D + p * DP;
#pragma unroll
        for (int i = 0; i < DP; ++i) acc[i] = fmaf(w, vr[i], acc[i]);
      }
      __syncthreads();
    }
  }
  if (row_ok) {
    const int64_t row = row0 + r;
    float* op = o + (row * hq + head) * D + p * DP;
    float* lp = lse + int64_t(head) * tq_total + row;
    const float lse_new = l > 0.f ? m + logf(l) : -INFINITY;
    float wa = 0.f, wb = 1.f, lse_out = lse_new;
    bool write = true;
    if (ACCUM) {
      // (O, LSE) <- merge((O, LSE), (acc, lse_new)); an empty side leaves the other exact.
      const float lse_old = *lp;
      if (l == 0.f) {
        write = false;
      } else if (lse_old != -INFINITY) {
        const float mm = fmaxf(lse_old, lse_new);
        const float ea = expf(lse_old - mm), eb = expf(lse_new - mm);
        const float inv = 1.0f / (ea + eb);
        wa = ea * inv;
        wb = eb * inv;
        lse_out = mm + logf(ea + eb);
      }
    }
    if (write) {
#pragma unroll
      for (int i = 0; i < DP; i += 4) {
        float4 val = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
        if (ACCUM && wa != 0.f) {
          const float4 old = *reinterpret_cast<const float4*>(op + i);
          val = make_float4(wa * old.x + wb * val.x, wa * old.y + wb * val.y, wa * old.z + wb * val.z,
                            wa * old.w + wb * val.w);
        }
        *reinterpret_cast<float4*>(op + i) = val;
      }
      // every lane of the row has read lse_old above (same wave, program order)
      if (p == 0) *lp = lse_out;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const ChunkPtrs<float>& kv, int nchunks,
                               const cpattn_plan_entry* plan, int n_tiles, int hq, int hkv, int d,
                               int tq_total, bool accumulate, float* o, float* lse,
                               hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  const dim3 grid(unsigned(n_tiles) * unsigned(hq));
  const float scale = 1.0f / sqrtf(float(d));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, q, kv, nchunks, plan, hq, hkv,
                       tq_total, scale, o, lse);
  };
  if (d == 128) {
    if (accumulate) launch(attn_fwd_f32_kernel<128, true>);
    else launch(attn_fwd_f32_kernel<128, false>);
  } else if (d == 64) {
    if (accumulate) launch(attn_fwd_f32_kernel<64, true>);
    else launch(attn_fwd_f32_kernel<64, false>);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
