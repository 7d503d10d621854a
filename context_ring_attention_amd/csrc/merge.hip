// LSE merge of two normalised partial attention results (HBM-bound).
//
// A normalised partial over a key set U is O = sum_u e^{s_u} v_u / sum_u e^{s_u} with
// LSE = ln sum_u e^{s_u}.  Two partials over disjoint key sets combine into the
// partial over their union: its LSE is ln(e^{lse_a} + e^{lse_b}), and its O mixes
// the two sides, each weighted by its share of the union's softmax mass,
// w_side = exp(lse_side - lse).  This is the combination step of the ring loop
// ("Megatron 6D parallelism guide", section 6) written for normalised partials.
// It is evaluated against mx = max(lse_a, lse_b): with ea = exp(lse_a - mx) and
// eb = exp(lse_b - mx) (one of them exactly 1), lse = mx + ln(ea + eb) and
// w_a = ea / (ea + eb), w_b = eb / (ea + eb).
//
// Layout: o [t, hq, d] fp32 (row (tok, h) is contiguous), lse [hq, t] fp32.
// Each thread owns one float4 of a row; a row's d/4 threads sit in one wave
// (d is a power of two <= 256, so d/4 divides 64), so every lane of a row
// reads lse_a before the same wave rewrites that row's lse_a.
#include "internal.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void merge_row_chunk(float4* __restrict__ oa, const float4* __restrict__ ob,
                                                float la, float lb, float4& out, float& lse_out,
                                                bool& write) {
  write = false;
  if (lb == -INFINITY) return;            // b empty: a unchanged exactly
  const float4 b = *ob;
  if (la == -INFINITY) {                  // a empty: take b exactly
    out = b;
    lse_out = lb;
    write = true;
    return;
  }
  const float4 a = *oa;
  const float mx = fmaxf(la, lb);
  const float ea = expf(la - mx);
  const float eb = expf(lb - mx);
  const float mass = ea + eb;
  const float inv = 1.0f / mass;
  const float wa = ea * inv, wb = eb * inv;
  out = make_float4(wa * a.x + wb * b.x, wa * a.y + wb * b.y, wa * a.z + wb * b.z,
                    wa * a.w + wb * b.w);
  lse_out = mx + logf(mass);
  write = true;
}

__global__ __launch_bounds__(kThreads) void merge_kernel(float* __restrict__ o_a,
                                                         float* __restrict__ lse_a,
                                                         const float* __restrict__ o_b,
                                                         const float* __restrict__ lse_b,
                                                         int64_t t, int hq, int vec_per_row,
                                                         int64_t total_vec) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total_vec; i += stride) {
    const int64_t row = i / vec_per_row;
    const int c = int(i - row * vec_per_row);
    const int64_t tok = row / hq;
    const int h = int(row - tok * hq);
    const int64_t li = int64_t(h) * t + tok;
    const float la = lse_a[li];
    const float lb = lse_b[li];
    float4 out;
    float lo;
    bool write;
    float4* pa = reinterpret_cast<float4*>(o_a) + i;
    merge_row_chunk(pa, reinterpret_cast<const float4*>(o_b) + i, la, lb, out, lo, write);
    if (write) {
      *pa = out;
      if (c == 0) lse_a[li] = lo;
    }
  }
}

}  // namespace

hipError_t launch_merge(float* o_a, float* lse_a, const float* o_b, const float* lse_b, int64_t t,
                        int hq, int d, hipStream_t stream) {
  const int vec_per_row = d / 4;
  const int64_t total_vec = t * hq * vec_per_row;
  // Rows must not straddle a wave: the grid-stride step is a multiple of 64
  // lanes, so that holds when vec_per_row divides 64.
  if (vec_per_row < 1 || 64 % vec_per_row != 0) return hipErrorInvalidValue;
  int64_t blocks = (total_vec + kThreads - 1) / kThreads;
  blocks = blocks < 8192 ? blocks : 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, o_a, lse_a,
                     o_b, lse_b, t, hq, vec_per_row, total_vec);
  return hipGetLastError();
}

}  // namespace cpattn
