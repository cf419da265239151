// muon_step_noalloc: muon_step with its workspace in a static device array,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable, so every device the library
// is loaded on holds its own copy, at its own address, until the process
// ends.  On the host the array's name is only a stand-in for the symbol, not
// a device address: the address a kernel may use comes from
// hipGetSymbolAddress, asked once per device with that device current, and
// that pointer is the only one this file hands to muon_step.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/muon.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;              // device address of this device's copy of scratch
  hipError_t err = hipErrorNotReady;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

extern "C" muon_status muon_step_noalloc(const muon_plan* plan, int32_t batch, const muon_batch_buffers* bufs,
                                         const muon_hparams* hp, void* stream) {
  if (!plan || !bufs || !hp) return MUON_ERR_INVALID_ARG;
  size_t need = 0;
  muon_status st = muon_workspace_bytes(plan, batch, hp->precision, &need);
  if (st != MUON_OK) return st;
  // a batch whose workspace exceeds the static array is refused before
  // anything touches the device
  if (need > (size_t)MUON_NOALLOC_SCRATCH_BYTES) return MUON_ERR_WORKSPACE_TOO_SMALL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MUON_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MUON_ERR_UNSUPPORTED;
  DeviceScratch& d = g_scratch[dev];
  // first call on this device (it is current): look up its copy's address
  std::call_once(d.once, [&d]() { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
  if (d.err != hipSuccess || d.ptr == nullptr) return MUON_ERR_HIP;
  // The kernels write every workspace byte they later read, so nothing needs
  // clearing between calls.
  return muon_step(plan, batch, bufs, hp, d.ptr, (size_t)MUON_NOALLOC_SCRATCH_BYTES, stream);
}
