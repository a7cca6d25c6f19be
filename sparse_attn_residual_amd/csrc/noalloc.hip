// fl_loop_attn_noalloc: fl_loop_attn with its workspace (the dequantized
// 64-column tile images of the attended columns) in a device array the
// library owns, for callers that cannot allocate device memory.
//
// `scratch` is one file-scope device array per GPU (each device that loads
// the library holds its own copy until the process ends).  Its device
// address is looked up once per device, with that device current, on the
// entry point's first call there; host code only ever passes that address,
// never the array's name (which names a host-side shadow).  Every call on a
// GPU shares its array: calls that overlap on one GPU race.  The tile images
// are written in full before they are read, so nothing needs clearing.
#include <cstdio>
#include <mutex>

#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = FL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

}  // namespace

extern "C" fl_status fl_loop_attn_noalloc(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_r,
                                          const int32_t* sel, const fl_state* state, fl_stream stream) {
  char msg[256];
  // the size check first: it needs no device
  const size_t need = (r >= 2 && K_r < 1) ? 0 : fl::attn_workspace_need(cache, r, K_r, dtype);
  if (need > kScratchBytes) {
    std::snprintf(msg, sizeof msg,
                  "fl_loop_attn_noalloc: this call needs %zu bytes of scratch; the library's array holds %zu "
                  "(FL_NOALLOC_SCRATCH_BYTES): use fl_loop_attn with a workspace",
                  need, kScratchBytes);
    return fl::report(FL_EUNSUPPORTED, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    std::snprintf(msg, sizeof msg, "fl_loop_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return fl::report(FL_EHIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(msg, sizeof msg, "fl_loop_attn_noalloc: device %d beyond the %d this entry point serves", dev,
                  kMaxDevices);
    return fl::report(FL_EUNSUPPORTED, msg);
  }
  // once per device, with that device current (it is: hipGetDevice above)
  std::call_once(g_once[dev], [dev] { g_lookup[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch)); });
  if (g_lookup[dev] != hipSuccess) {
    std::snprintf(msg, sizeof msg, "fl_loop_attn_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(g_lookup[dev]));
    return fl::report(FL_EHIP, msg);
  }
  return fl_loop_attn(cache, r, q, dtype, K_r, sel, state, g_ptr[dev], kScratchBytes, stream);
}
