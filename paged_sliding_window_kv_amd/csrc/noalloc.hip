// kvc_attend_noalloc (declared in include/kvc.h): kvc_attend for callers that
// cannot allocate, with its split partials in a file-scope device array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "handle.hpp"
#include "kvc.h"

using kvc::fail;
using kvc::guarded;

static constexpr size_t kScratchBytes = size_t(32) << 20;  // KVC_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == KVC_NOALLOC_SCRATCH_BYTES, "scratch size and its public constant must agree");

// The split partials of kvc_attend_noalloc.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code this name is only
// a stand-in for the symbol: its device address, one per device, comes from
// hipGetSymbolAddress and is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
int scratch_address(kvc_stream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVC_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(KVC_ERR_INVALID_ARGUMENT, "the stream belongs to device %d; make it the current device (now %d)",
                  static_cast<int>(sdev), dev);
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVC_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVC_OK;
}

}  // namespace

extern "C" int kvc_attend_noalloc(const kvc_t* cache, const void* q, int32_t num_q, float sm_scale, void* o,
                                  float* lse, kvc_stream_t stream) {
  return guarded("kvc_attend_noalloc", [&] {
    if (!cache) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    void* ws = nullptr;
    if (int s = scratch_address(stream, &ws)) return s;
    return kvc::attend_fixed_workspace(cache, q, num_q, sm_scale, o, lse, ws, kScratchBytes, stream);
  });
}
