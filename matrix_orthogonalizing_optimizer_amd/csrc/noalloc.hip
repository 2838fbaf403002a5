// ns_orthogonalize_noalloc: the Newton-Schulz orthogonalization of one
// matrix with its scratch memory in a file-scope device array instead of a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The array lives in the library's code object: every GPU the library is
// loaded on holds its own copy (MUON_NOALLOC_SCRATCH_BYTES) until the process
// ends.  In host code the array's name is not a device address; its address
// on a device comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in g_scratch_ptr.  Nothing in the array has to
// start at zero (every kernel of the chain writes what it later reads,
// padding included), so no clearing is needed between calls; calls that
// overlap in time on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "libmuon.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev (looked up once, with dev current).
muon_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return MUON_E_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MUON_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MUON_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MUON_E_HIP;
    if (e != hipSuccess || !p) return MUON_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace

extern "C" muon_status ns_orthogonalize_noalloc(void* X, int64_t rows, int64_t cols, int64_t ld,
                                                int32_t dtype, int32_t steps, const float* coeffs,
                                                int32_t method, void* stream) {
  size_t need = 0;
  const muon_status st = ns_orthogonalize_workspace_bytes(rows, cols, dtype, method, &need);
  if (st != MUON_OK) return st;
  if (need > (size_t)MUON_NOALLOC_SCRATCH_BYTES) return MUON_E_WORKSPACE;
  if (need == 0)  // empty matrix: argument checks only, nothing is launched
    return ns_orthogonalize(X, rows, cols, ld, dtype, steps, coeffs, method, nullptr, 0, stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if (s) {
    hipDevice_t d;
    if (hipStreamGetDevice(s, &d) != hipSuccess) return MUON_E_HIP;
    dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return MUON_E_HIP;
  }
  void* ws = nullptr;
  const muon_status sst = scratch_on(dev, &ws);
  if (sst != MUON_OK) return sst;
  return ns_orthogonalize(X, rows, cols, ld, dtype, steps, coeffs, method, ws,
                          (size_t)MUON_NOALLOC_SCRATCH_BYTES, stream);
}
