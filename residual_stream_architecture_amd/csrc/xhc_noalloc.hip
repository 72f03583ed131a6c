// xhc_forward_noalloc: the forward update with its scratch memory in a
// static device array of the library instead of a caller's workspace, for
// callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy from the moment the code object is loaded until the
// process ends.  Its name is a host-side stand-in in host code: the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device (with that device current) on the first call there and kept in a
// per-device table.  Only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "xhc_launch.h"
#include "xhc_plan.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[XHC_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (NULL: not taken yet)

// The device address of the current device's copy of `scratch`, or NULL.
void* scratch_of_current_device() {
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

extern "C" int xhc_forward_noalloc(const xhc_desc* desc, const xhc_fwd_args* args, xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::prepare_forward(desc, args, &p);
  if (rc) return rc;
  // the timer creates HIP events: not for callers that cannot allocate
  if (args->timer) return XHC_ERR_UNSUPPORTED;
  if (p.fwd_bytes > (size_t)XHC_NOALLOC_SCRATCH_BYTES) return XHC_ERR_SCRATCH;
  (void)hipGetLastError();   // report only this call's own launch errors
  void* ws = scratch_of_current_device();
  if (!ws) return XHC_ERR_HIP;
  return xhc::launch_forward(p, args, ws, reinterpret_cast<hipStream_t>(stream));
}
