// Chunked causal attention forward, fp32 inputs and arithmetic (gfx950 VALU).
//
// Same contract as the bf16 kernel (normalised partial O and LSE of one KV
// chunk), for callers that need fp32 accuracy.  One work-group handles 64
// query tokens of one head; four lanes share a query row, each owning D/4
// contiguous dimensions, and combine their partial dot products with two lane
// swaps.  Keys are staged through LDS in blocks of 32.  The softmax is an exact
// two-pass one: pass 1 finds each row's max m and sum l, pass 2 accumulates
// exp(s - m) / l * v.  Both passes evaluate every score with the same
// arithmetic, so pass 2 sees exactly the scores pass 1 reduced.
#include "internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
static_assert(kF32TokensPerTile * 4 == kThreads, "four lanes per query row");
constexpr int BN = kF32BlockN;         // 32 keys per block

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
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
  const cpattn_plan_entry pe = plan[e];
  const int kvh = head / (hq / hkv);
  const bool row_ok = r < pe.nrows;
  const int nblk = pe.cost;
  const int lim_row = pe.delta + r;  // row sees keys u <= lim_row

  float qr[DP];
  {
    const float* qp = q + (int64_t(pe.row0 + r) * hq + head) * D + p * DP;
#pragma unroll
    for (int i = 0; i < DP; i += 4) {
      float4 x = row_ok ? *reinterpret_cast<const float4*>(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      qr[i] = x.x; qr[i + 1] = x.y; qr[i + 2] = x.z; qr[i + 3] = x.w;
    }
  }
  const int64_t kv_stride = int64_t(hkv) * D;
  const float* kbase = k + (int64_t(pe.k_start) * hkv + kvh) * D;
  const float* vbase = v + (int64_t(pe.k_start) * hkv + kvh) * D;

  auto stage = [&](int j, bool with_v) {
    for (int idx = tid; idx < BN * D / 4; idx += kThreads) {
      const int key = idx / (D / 4), c = idx - key * (D / 4);
      const int gk = j * BN + key;
      const bool ok = gk < pe.k_len;
      ks[idx] = ok ? *reinterpret_cast<const float4*>(kbase + gk * kv_stride + 4 * c)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
      if (with_v)
        vs[idx] = ok ? *reinterpret_cast<const float4*>(vbase + gk * kv_stride + 4 * c)
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

  // pass 1: row max and row sum
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < nblk; ++j) {
    stage(j, false);
    __syncthreads();
    float sv[BN];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < BN; ++u) {
      const int key = j * BN + u;
      const float s = score(u);
      sv[u] = (key < pe.k_len && key <= lim_row) ? s : -INFINITY;
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
  // pass 2: output
  float acc[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) acc[i] = 0.f;
  const float inv_l = l > 0.f ? 1.0f / l : 0.f;
  for (int j = 0; j < nblk; ++j) {
    stage(j, true);
    __syncthreads();
#pragma unroll 4
    for (int u = 0; u < BN; ++u) {
      const int key = j * BN + u;
      const float s = score(u);
      const float w = (key < pe.k_len && key <= lim_row) ? expf(s - m) * inv_l : 0.f;
      const float* vr = reinterpret_cast<const float*>(vs) + u * D + p * DP;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] = fmaf(w, vr[i], acc[i]);
    }
    __syncthreads();
  }
  if (row_ok) {
    const int64_t row = pe.row0 + r;
    float* op = o + (row * hq + head) * D + p * DP;
#pragma unroll
    for (int i = 0; i < DP; i += 4)
      *reinterpret_cast<float4*>(op + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    if (p == 0) lse[int64_t(head) * tq_total + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v,
                               const cpattn_plan_entry* plan, int n_entries, int hq, int hkv,
                               int d, int tq_total, float* o, float* lse, hipStream_t stream) {
  if (n_entries == 0) return hipSuccess;
  const dim3 grid(unsigned(n_entries) * unsigned(hq));
  const float scale = 1.0f / sqrtf(float(d));
  if (d == 128) {
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, plan, hq,
                       hkv, tq_total, scale, o, lse);
  } else if (d == 64) {
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, plan, hq,
                       hkv, tq_total, scale, o, lse);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
