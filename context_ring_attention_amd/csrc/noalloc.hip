// cpattn_fwd_chunks_noalloc: the streaming forward with its work plan in a static device array
// instead of a caller-supplied workspace, for callers that cannot allocate device memory.
//
// The forward's only device memory beyond its inputs and outputs is the work plan (32 bytes
// per token tile and chunk).  Here it lives in `scratch`, a file-scope device array of
// kScratchBytes that every GPU the library runs on holds until the process ends.  In host code
// the name `scratch` is only a stand-in for the symbol; its device address on each GPU comes
// from hipGetSymbolAddress, looked up once per device (with that device current) and kept, and
// that address is what the upload and the kernels use.  The host side of the plan is built in
// a static host array under a mutex, so a call allocates nothing, host or device.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on different
// streams, or from several threads without ordering their streams) race on it.  Nothing in it
// needs clearing: each call writes the whole plan its kernels read, ahead of them on its stream.
#include <mutex>

#include "internal.h"

namespace cpattn {
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;   // 131,072 plan records
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
DeviceScratch g_dev[kMaxDevices];

std::mutex g_host_mu;
alignas(256) char g_host[kScratchBytes];   // host image of the plan, rebuilt by every call

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" cpattn_status cpattn_fwd_chunks_noalloc(
    const void* q, const void* const* ks, const void* const* vs, int32_t nchunks,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* q_pos_offset,
    const int32_t* k_pos_offset, int32_t nseq, int32_t hq, int32_t hkv, int32_t d,
    cpattn_dtype dtype, int32_t causal, int32_t accumulate, float* o, float* lse,
    hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(CPATTN_ERR_HIP, "hipGetDevice failed (or device index >= %d)", kMaxDevices);
  DeviceScratch& ds = g_dev[dev];
  std::call_once(ds.once, [&] {
    ds.err = hipGetSymbolAddress(&ds.ptr, HIP_SYMBOL(scratch));
  });
  if (ds.err != hipSuccess || !ds.ptr)
    return set_error(CPATTN_ERR_HIP, "hipGetSymbolAddress of the static scratch failed: %s",
                     hipGetErrorString(ds.err));
  std::lock_guard<std::mutex> lock(g_host_mu);
  const cpattn_status st =
      fwd_impl(q, ks, vs, nchunks, cu_seqlens_q, cu_seqlens_k, q_pos_offset, k_pos_offset, nseq,
               hq, hkv, d, dtype, causal, accumulate, o, lse, ds.ptr, kScratchBytes, stream,
               g_host, kScratchBytes);
  if (st == CPATTN_ERR_WORKSPACE)
    return set_error(CPATTN_ERR_UNSUPPORTED,
                     "the work plan exceeds the %zu-byte static scratch of "
                     "cpattn_fwd_chunks_noalloc (use cpattn_fwd_chunks with a workspace)",
                     kScratchBytes);
  return st;
}
