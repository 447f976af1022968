// The sparse layer for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): hs2_sparse_attn with its
// workspace (the per-split partial results) taken from a fixed device array that the
// library holds on every GPU it runs on, instead of from the caller.
//
// Each GPU holds its own copy of `scratch`, at its own address. The host-side name of the
// array is only a stand-in: its device address is looked up once per device, with that
// device current, through hipGetSymbolAddress, and that address is what the kernels get.
// Every call on a GPU shares that GPU's array, so calls that overlap on one GPU (other
// streams, other threads) race on it; the array keeps the last call's contents, which no
// call relies on (every partial the combine reads is written first by the same call).
#include <mutex>

#include "hs2_launch.h"

namespace hs2 {
namespace {

static __device__ __align__(256) uint8_t scratch[HS2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call there).
hipError_t scratch_of_device(int dev, void** out) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  *out = g_scratch[dev];
  return g_lookup[dev];
}

}  // namespace
}  // namespace hs2

extern "C" hs2_status hs2_sparse_attn_noalloc(const hs2_seqs* batch, const void* q, const void* k, const void* v,
                                              const int32_t* sel_idx, int32_t n_heads, int32_t head_dim,
                                              int32_t window, int32_t top_k, float scale, void* out, float* lse,
                                              hs2_dtype dt, void* stream) {
  using namespace hs2;
  if (dt != HS2_BF16 && dt != HS2_F32)
    return set_error(HS2_ERR_UNSUPPORTED, "hs2_sparse_attn_noalloc takes bf16 or fp32 K/V");
  const hs2_status st = sparse_check(batch, q, k, v, sel_idx, n_heads, head_dim, window, top_k, scale, out, lse, dt);
  if (st != HS2_OK) return st;
  const size_t need = hs2_sparse_attn_workspace_size(batch, n_heads, head_dim, window, top_k, dt);
  if (need > (size_t)HS2_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "the batch needs %zu bytes of scratch, more than the %zu bytes of hs2_sparse_attn_noalloc "
             "(use hs2_sparse_attn with a workspace)", need, (size_t)HS2_NOALLOC_SCRATCH_BYTES);
    return set_error(HS2_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(HS2_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(HS2_ERR_UNSUPPORTED, "device index beyond 63");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s != nullptr && hipGetStreamDeviceId(s) != dev)
    return set_error(HS2_ERR_INVALID_ARG, "the stream belongs to another device than the current one");
  void* ws = nullptr;
  e = scratch_of_device(dev, &ws);
  if (e != hipSuccess) return set_error(HS2_ERR_HIP, hipGetErrorString(e));
  return hs2_sparse_attn(batch, q, k, v, sel_idx, n_heads, head_dim, window, top_k, scale, out, lse, ws,
                         (size_t)HS2_NOALLOC_SCRATCH_BYTES, dt, stream);
}
