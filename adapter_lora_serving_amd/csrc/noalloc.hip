// lora_apply_linear_noalloc: lora_apply_linear with its workspace in a
// static device array instead of a caller buffer, for callers that cannot
// allocate (code under graph capture, serving loops that may not call the
// allocator, harnesses that forbid it).
//
// The array `scratch` below lives in device memory for as long as the
// library stays loaded; each GPU holds its own copy at its own address. Its
// name in host code is only a host-side stand-in: the device address is
// looked up once per device with hipGetSymbolAddress (on the first call made
// on that device) and only that address is ever passed to a kernel.
//
// Contents: the same regions as a lora_apply_linear workspace (the fused
// path's synchronisation counters, its partial tiles, h and the K parts of
// the segment tiles). The array starts zero-filled when the code object is
// loaded, which is the state the counters need; every completed call leaves
// them in a state the next call accepts, and nothing else needs clearing, so
// calls clear nothing. All calls on one GPU share the array: calls that
// overlap in time on one GPU (two streams, or graphs replayed concurrently)
// race on it and must not be issued.
#include "lora_mi355x.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "lora_kernels.h"

namespace {

constexpr size_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (looked up once per
// device, with that device current).
lora_status scratch_address(int dev, void** out) {
  void* p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev];
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LORA_ERR_HIP;
      __atomic_store_n(&g_scratch[dev], p, __ATOMIC_RELEASE);
    }
  }
  *out = p;
  return LORA_OK;
}

}  // namespace

extern "C" {

size_t lora_noalloc_scratch_bytes(void) { return kScratchBytes; }

lora_status lora_apply_linear_noalloc(int dtype, const void* x, void* y, int64_t T,
                                      int64_t in_features, const int64_t* out_slices,
                                      int32_t num_slices, const void* a, const void* b,
                                      int32_t slots, int32_t R, const int32_t* token_order,
                                      const int32_t* slot_indptr, const int32_t* ranks,
                                      const float* scalings, void* stream) {
  // sizes first (host arithmetic only): too large a call is refused before
  // any HIP call
  const size_t need = lora_apply_linear_workspace_bytes(T, in_features, slots, num_slices, R);
  if (need == 0) {
    // bad scalar arguments: lora_apply_linear names the error
    return lora_apply_linear(dtype, x, y, T, in_features, out_slices, num_slices, a, b, slots, R,
                             token_order, slot_indptr, ranks, scalings, nullptr, 0, stream);
  }
  if (need > kScratchBytes) return LORA_ERR_SCRATCH_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return LORA_ERR_INVALID_ARG;
    if (sdev != dev) return LORA_ERR_INVALID_ARG;   // the stream must be on the current device
  }
  void* ws = nullptr;
  const lora_status st = scratch_address(dev, &ws);
  if (st != LORA_OK) return st;
  return lora_apply_linear(dtype, x, y, T, in_features, out_slices, num_slices, a, b, slots, R,
                           token_order, slot_indptr, ranks, scalings, ws, kScratchBytes, stream);
}

}  // extern "C"
