// gb_noalloc.hip — gb_bucket_allreduce_local_noalloc: the bucket stream with
// its payload workspace in a static device array, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It allocates nothing per call: the
// array is part of the library's code object, one copy per GPU, held until
// the process ends.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "gb_internal.h"

namespace {

// The payloads of every rank (codes, then scales), at the layout
// gb_bucket_workspace_layout reports.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[GB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
gb_status scratch_address(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  char msg[256];
  if (e != hipSuccess) {
    std::snprintf(msg, sizeof msg, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return gb::fail_status(GB_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(msg, sizeof msg, "%s: device %d out of range", fn, dev);
    return gb::fail_status(GB_ERR_HIP, msg);
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      std::snprintf(msg, sizeof msg, "%s: hipGetSymbolAddress of the scratch array on device %d: %s", fn, dev,
                    hipGetErrorString(e));
      return gb::fail_status(GB_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GB_OK;
}

}  // namespace

extern "C" gb_status gb_bucket_allreduce_local_noalloc(float* out, const float* const* srcs, int k, size_t n,
                                                       size_t bucket_elems, int codec, int scale_mode,
                                                       void* stream) {
  return gb::traced_call("gb_bucket_allreduce_local_noalloc", stream, k, n, codec, [&](const char* fn) -> gb_status {
    // 0 for arguments the layout rejects: the shared validation reports those
    const size_t need = gb_bucket_workspace_bytes(codec, k, n, bucket_elems);
    if (need > GB_NOALLOC_SCRATCH_BYTES) {
      char msg[256];
      std::snprintf(msg, sizeof msg,
                    "%s: the payloads of k = %d ranks of n = %zu values need %zu bytes, more than the %zu-byte "
                    "static scratch; pass a workspace to gb_bucket_allreduce_local instead",
                    fn, k, n, need, (size_t)GB_NOALLOC_SCRATCH_BYTES);
      return gb::fail_status(GB_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
      gb_status s = scratch_address(fn, &ws);
      if (s != GB_OK) return s;
    }
    return gb::bucket_allreduce_local(fn, out, srcs, k, n, bucket_elems, codec, scale_mode, ws,
                                      need > 0 ? (size_t)GB_NOALLOC_SCRATCH_BYTES : 0, stream);
  });
}
