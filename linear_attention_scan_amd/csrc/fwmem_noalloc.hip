// fwmem_scan_fwd_noalloc: the whole-sequence scan for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). It is fwmem_scan_fwd with its workspace taken from `scratch`, a
// fixed file-scope device array, instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` (at its own address)
// until the process ends. Host code never uses the array's name as a device address:
// on a device's first call the address is looked up with hipGetSymbolAddress, with that
// device current, and kept per device; every later call on that device passes the kept
// pointer to the scan's kernels, exactly as fwmem_scan_fwd passes a caller workspace.
//
// The workspace needs no initialisation (the prep phase writes every record before the
// propagate phase reads it), so nothing is cleared between calls; the array keeps the
// last call's contents. All calls on one GPU share the array: calls that overlap in time
// on one GPU (two streams, two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fwmem.h"

namespace {

constexpr size_t kScratchBytes = (size_t)FWMEM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_dev[kMaxDevices];

// The device address of `scratch` on the current device (null on failure).
void* scratch_ptr(int dev) {
  DeviceScratch& d = g_dev[dev];
  std::call_once(d.once, [&d]() {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    d.ptr = d.err == hipSuccess ? p : nullptr;
  });
  return d.ptr;
}

}  // namespace

extern "C" fwmem_status fwmem_scan_fwd_noalloc(const fwmem_shape* shape, const void* q,
                                               const void* k, const void* v,
                                               const float* beta, const float* lambda,
                                               const fwmem_mode* mode, const void* S_in,
                                               void* out, void* S_out, fwmem_stream stream) {
  size_t need = 0;
  const fwmem_status st = fwmem_scan_workspace_bytes(shape, mode, &need);
  if (st != FWMEM_OK) return st;
  if (need > kScratchBytes) return FWMEM_ESCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FWMEM_ELAUNCH;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return FWMEM_ELAUNCH;
  return fwmem_scan_fwd(shape, q, k, v, beta, lambda, mode, S_in, out, S_out, ws, kScratchBytes,
                        stream);
}
