// kvsel_compress without a caller workspace: for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The workspace is a file-scope device
// array of kNoAllocScratchBytes, one copy per GPU, which the runtime sets up
// when it loads this library's code on that GPU and which lives until the
// process ends.  Its device address comes from hipGetSymbolAddress, once per
// device with that device current; host code never passes the array's own
// name to a kernel (on the host that name is only a stand-in, not a device
// address).
//
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// (other streams, other host threads) race.  The workspace needs no
// clearing between calls (kvsel_compress accepts arbitrary initial bytes),
// so nothing is zeroed here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "kvsel.h"
#include "kvsel_internal.h"

#define KVSEL_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 256;

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::atomic<void *> g_scratch[kMaxDevices];  // device address of `scratch` per device, once set up
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (its device address), set up on
// the first call on that device.
kvsel_status scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return kvsel::set_error(KVSEL_EHIP, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
  if (dev < 0 || dev >= kMaxDevices) return kvsel::set_error(KVSEL_EUNSUPPORTED, "device ordinal out of range");
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return kvsel::set_error(KVSEL_EHIP,
                                (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e)).c_str());
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return KVSEL_OK;
}

}  // namespace

KVSEL_API kvsel_status kvsel_compress_noalloc(const kvsel_problem *p, const void *Q, const void *K, const void *V,
                                              int32_t *idx, void *K_out, void *V_out, float *pooled,
                                              kvsel_stream_t stream) {
  size_t need = 0;
  kvsel_status s = kvsel_plan(p, &need, nullptr);
  if (s != KVSEL_OK) return s;
  if (need > kNoAllocScratchBytes)
    return kvsel::set_error(KVSEL_EUNSUPPORTED,
                            ("the problem needs " + std::to_string(need) + " bytes of workspace, more than the " +
                             std::to_string(kNoAllocScratchBytes) +
                             " of kvsel_compress_noalloc's scratch: use kvsel_compress with a workspace")
                                .c_str());
  void *ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != KVSEL_OK) return s;
  return kvsel_compress(p, Q, K, V, idx, K_out, V_out, pooled, ws, kNoAllocScratchBytes, stream);
}
