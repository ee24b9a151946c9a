// hla2_noalloc.hip -- hla2_forward_noalloc: the forward pass with its workspace in a
// fixed device array the library holds, for callers that cannot allocate device memory.
//
// The array lives in this translation unit only, so its code object (and with it the
// array's device memory) is loaded on a device the first time this entry point runs there.
// Host code never passes the array's name to a kernel or a copy: on the host that name is
// a stand-in, not a device address.  Its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current, and is kept.
#include <mutex>

#include "hla2.h"
#include "hla2_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[HLA2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not taken yet)

// The current device's address of the array, or null on a runtime error.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int hla2_forward_noalloc(const void *q, const void *k, const void *v, void *out, int B, int H, int n,
                                    int d, int dv, float decay, int normalize, int chunk, hla2_dtype_t dtype,
                                    float *den_out, hipStream_t stream) {
  // everything is validated on the host before the first runtime call
  size_t need = 0;
  int rc = hla2::forward_check(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, (int)dtype, den_out, nullptr,
                               0, &need);
  if (rc != HLA2_OK) return rc;
  if (need > (size_t)HLA2_NOALLOC_SCRATCH_BYTES) return HLA2_ERR_UNSUPPORTED;
  void *ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return HLA2_ERR_LAUNCH;
  }
  return hla2::forward_run(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, (int)dtype, den_out, nullptr, ws,
                           need > 0 ? (size_t)HLA2_NOALLOC_SCRATCH_BYTES : 0, 0, nullptr, stream);
}
