// gdn_noalloc.hip -- gdn_chunk_fwd for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace of these calls is a file-scope device array of GDN_NOALLOC_WORKSPACE_BYTES,
// one copy per device, held from the library's first use on that device until the process
// ends.  Its device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; host code uses only that address (the array's name denotes a
// host-side stand-in, not device memory).  Nothing here allocates: no hipMalloc, no
// hipFree, no allocating library routine.
//
// Every call on one device shares that device's array.  Nothing in it needs to start at
// zero (every kernel writes each workspace word it reads earlier in the same call), so the
// array is never cleared; but calls that overlap in time on one device (other streams,
// other threads) race on it and must be ordered by the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch` (looked up on first use there), or null.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" gdn_status gdn_chunk_fwd_noalloc(const gdn_problem* p, const void* q, const void* k,
                                            const void* v, const float* g, const float* beta,
                                            const float* h0, const int32_t* cu_seqlens, void* o,
                                            float* hT, uint32_t* status, void* stream) {
  if (!p) return GDN_E_NULL;
  // The composition the call runs decides how much workspace it needs (a pipelined call
  // keeps only two segments of tiles), so it is resolved first and then requested
  // explicitly: the same kernels and launches as the resolved choice of gdn_chunk_fwd.
  int32_t compose = GDN_COMPOSE_AUTO;
  gdn_status s = gdn_plan_compose(p, &compose);
  if (s != GDN_OK) return s;
  gdn_problem r = *p;
  r.compose = compose;
  size_t need = 0;
  s = gdn_workspace_bytes(&r, &need);
  if (s != GDN_OK) return s;
  if (need > (size_t)GDN_NOALLOC_WORKSPACE_BYTES) return GDN_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_on_current_device())) return GDN_E_LAUNCH;
  return gdn_chunk_fwd(&r, q, k, v, g, beta, h0, cu_seqlens, o, hT, status, ws,
                       need > 0 ? (size_t)GDN_NOALLOC_WORKSPACE_BYTES : 0, stream);
}
