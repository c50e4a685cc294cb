// pkv_noalloc.hip -- the static split workspace of pkv_paged_decode_noalloc.
//
// One file-scope device array per GPU that the library runs on, sized
// PKV_NOALLOC_SCRATCH_BYTES, holding the split partials (and the arrival
// counters of the in-kernel merge) for callers that cannot allocate.  In host
// code `scratch` names a host-side stand-in, not a device address: the device
// address of each GPU's copy is looked up once per device, with that device
// current, and only that address is handed to kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;

struct DeviceScratch {
  void *ptr = nullptr;   // device address of this device's copy of `scratch`
  bool cleared = false;  // its counter head has been zeroed once
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxScratchDevices];

}  // namespace

int noalloc_scratch(void **ptr, bool *cleared) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return PKV_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceScratch &d = g_dev[dev];
  if (!d.ptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_DEVICE;
    d.ptr = p;
  }
  *ptr = d.ptr;
  *cleared = d.cleared;
  return PKV_OK;
}

void noalloc_mark_cleared() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_dev[dev].cleared = true;
}

}  // namespace pkv
