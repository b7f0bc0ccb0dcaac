// noalloc.hip -- engram_gate_forward_noalloc: the gate of engram_gate_forward without
// any allocation, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The bf16 gate needs scratch memory (the gain-folded key weights, the fp32 partial
// sums, the gates and the work-queue counters).  Here it lives in one file-scope device
// array of NOALLOC_SCRATCH_BYTES, which every device the library runs on holds from the
// moment the code object is loaded until the process ends.  Host code never uses the
// array's name as an address: the first call on a device (with that device current)
// looks up the device address with hipGetSymbolAddress, and every launch passes that
// address.  The kernels are those of engram_gate_forward; the counters that must start
// at zero are cleared by the gate's own preparation kernel on every call (a kernel, not
// hipMemsetAsync).  All calls on one device share the array: calls that overlap on a
// device race, so callers order them (one stream, or events).
#include <mutex>

#include "engram_internal.h"

namespace engram {
namespace {

__device__ __align__(256) char scratch[ENGRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDev = 64;
std::mutex g_mu;
void* g_ptr[kMaxDev];

// The device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

engram_status gate_forward_noalloc(const char* fn, GateArgs& a, hipStream_t stream) {
  const size_t bytes = gate_bf16_scratch_bytes(a, false);
  if (bytes > (size_t)ENGRAM_NOALLOC_SCRATCH_BYTES)
    return fail(ENGRAM_ERR_UNSUPPORTED, "%s: these shapes need %zu bytes of scratch, above the fixed %zu", fn, bytes,
                (size_t)ENGRAM_NOALLOC_SCRATCH_BYTES);
  void* p = nullptr;
  const hipError_t e = scratch_address(&p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return hip_fail(e, "engram_gate_forward_noalloc: hipGetSymbolAddress(scratch)");
  }
  a.part_dot = (float*)p;
  launch_gate_bf16(a, false, stream);
  return check_launch(fn);
}

}  // namespace engram
