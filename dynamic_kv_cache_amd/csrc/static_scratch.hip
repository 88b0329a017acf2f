// Handles that allocate nothing: fastocr_create_static places a handle's
// scratch (split states, logits, scores, kept set, warm-up statistics,
// arrival counters) in a file-scope device array instead of device memory
// from hipMalloc.  The array exists once per GPU the library runs on and is
// held until the process ends; every static handle on a GPU uses that GPU's
// copy, so at most one static handle per GPU is live at a time.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fastocr.h"
#include "internal.h"

namespace {

constexpr size_t kStaticScratchBytes = (size_t)FASTOCR_STATIC_SCRATCH_MIB << 20;
constexpr int kMaxDevices = 64;

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress (below)
// and is the only way host code refers to it.
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)
bool g_in_use[kMaxDevices];        // a live static handle holds that device's scratch

void release_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (device >= 0 && device < kMaxDevices) g_in_use[device] = false;
}

}  // namespace

extern "C" int fastocr_create_static(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out) {
  if (!cfg || !out) return FASTOCR_ERR_INVALID_ARG;
  *out = nullptr;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) return FASTOCR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_in_use[device]) return FASTOCR_ERR_STATE;
  if (!g_scratch_ptr[device]) {
    // first use on this device (it is current): this device's copy of the array
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return FASTOCR_ERR_HIP;
    g_scratch_ptr[device] = ptr;
  }
  const int rc = fastocr::create_handle(cfg, hip_stream, out, g_scratch_ptr[device], kStaticScratchBytes,
                                        &release_scratch);
  if (rc == FASTOCR_OK) g_in_use[device] = true;
  return rc;
}
