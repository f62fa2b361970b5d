// ssm_selective_scan_fwd_noalloc: the forward scan with its scratch (the per-segment summaries
// of a sequence split along L, and the output pass's stored states where they fit) in a fixed
// device array of this library instead of a caller workspace, for callers that cannot allocate
// device memory.
//
// The array lives in every GPU the library runs on until the process ends. Host code never
// passes its name to a kernel (on the host it is only a stand-in for the device symbol): the
// device address is looked up once per device with hipGetSymbolAddress, with that device
// current, and that address is what the scan receives as its workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "scan_internal.h"
#include "ssm_scan.h"

static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, null until looked up

// The device address of `scratch` on `dev`, looked up on first use with `dev` current (the
// caller's current device is restored afterwards). Null on failure.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev]) return g_ptr[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !ptr) return nullptr;
  g_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" int ssm_selective_scan_fwd_noalloc(const ssm_scan_desc* desc, const void* x,
                                              const void* delta, const float* A, const void* B,
                                              const void* C, const float* D, const void* z,
                                              const float* delta_bias, int32_t delta_softplus,
                                              void* y, const ssm_scan_ext* ext, void* stream) {
  size_t need = 0;
  const int rc = ssm_selective_scan_workspace_size(desc, &need);
  if (rc != SSM_OK) return rc;
  // the stored states that let the correcting pass of a split sequence stop early are left out
  // when they do not fit (same results, that pass then runs every later segment to its end)
  const bool checks = need <= (size_t)SSM_NOALLOC_SCRATCH_BYTES;
  if (!checks && ssm::fwd_workspace_bytes(desc, false) > (size_t)SSM_NOALLOC_SCRATCH_BYTES)
    return SSM_ERR_SCRATCH_LIMIT;
  int dev = -1;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = hs ? hipStreamGetDevice(hs, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return SSM_ERR_HIP;
  void* ptr = scratch_on(dev);
  if (!ptr) return SSM_ERR_HIP;
  // nothing in the scratch needs to start at zero: the pass that writes a summary or a stored
  // state runs before the pass that reads it, on the same stream
  return ssm::fwd_ext(desc, x, delta, A, B, C, D, z, delta_bias, delta_softplus, y, ext, ptr,
                      (size_t)SSM_NOALLOC_SCRATCH_BYTES, stream, checks);
}
