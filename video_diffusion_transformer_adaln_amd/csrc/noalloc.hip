// The block forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): instead of a caller workspace, the block's intermediates (mod,
// h, q|k|V^T, o, x1, h2, u, and the scratch of split tails and of widened
// int8 weights where the config has them) live in a static device array of
// this library, `scratch`, of H3K_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs on holds
// its own copy of the array until the process ends.
//
// In host code `scratch` is only a host-side stand-in for the array: its
// device address on the current GPU comes from hipGetSymbolAddress, once per
// device, and only that address is handed to the kernels.  Calls on one GPU
// share the array (it keeps the last call's contents; no kernel of the block
// reads a workspace byte it has not written first, so nothing needs clearing),
// and calls that overlap in time on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "h3k.h"

namespace {

static __device__ __align__(256) char scratch[H3K_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
h3k_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return h3k::api_fail(H3K_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return h3k::api_fail(H3K_ERR_UNSUPPORTED, "device %d: at most %d devices hold a static scratch array", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s != hipSuccess || p == nullptr)
      return h3k::api_fail(H3K_ERR_HIP, "hipGetSymbolAddress of the static scratch array failed on device %d: %s",
                           dev, hipGetErrorString(s));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return H3K_OK;
}

}  // namespace

extern "C" h3k_status h3k_dit_block_forward_noalloc(const h3k_dit_config* cfg, const h3k_dit_block_weights* weights,
                                                    const void* x, const void* c, void* out, hipStream_t stream,
                                                    h3k_dit_stats* stats) {
  uint64_t need = 0;
  const h3k_status st = h3k_dit_workspace_size(cfg, 1, &need);   // validates the config
  if (st != H3K_OK) return st;
  if (need > H3K_NOALLOC_SCRATCH_BYTES)
    return h3k::api_fail(H3K_ERR_WORKSPACE,
                         "this block needs %llu bytes of workspace; the static scratch array holds %llu "
                         "(use h3k_dit_block_forward with a caller workspace)",
                         (unsigned long long)need, (unsigned long long)H3K_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const h3k_status sp = scratch_on_current_device(&ws);
  if (sp != H3K_OK) return sp;
  return h3k::api_forward(cfg, weights, 1, x, c, out, ws, H3K_NOALLOC_SCRATCH_BYTES, stream, stats);
}
