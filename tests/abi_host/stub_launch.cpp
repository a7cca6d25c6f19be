// Host stand-ins for the launch layer (launch.hpp), so that the C ABI's
// validation code (abi.cpp) can run on the CPU under AddressSanitizer.
// Every launcher only counts the call; the validator's "device" copies are
// plain memcpy, so the tests hand it host arrays as device pointers.
#include <cstring>

#include "launch.hpp"

int g_launches = 0;

namespace fl {

static hipError_t counted() {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_quant_base(const CacheGeo&, const void*, const void*, fl_dtype, uint8_t*, hipStream_t) {
  return counted();
}
hipError_t launch_build_slot(const CacheGeo&, int, int32_t*, hipStream_t) { return counted(); }
hipError_t launch_paper_quant(const CacheGeo&, int, const void*, const void*, fl_dtype, uint8_t*, hipStream_t) {
  return counted();
}
hipError_t launch_append(const CacheGeo&, int, int, const void*, const void*, fl_dtype, uint8_t*, uint8_t*, int32_t*,
                         int32_t*, int32_t*, hipStream_t) {
  return counted();
}
hipError_t launch_quant_res(const CacheGeo&, int, const void*, const void*, fl_dtype, uint8_t*, hipStream_t) {
  return counted();
}
hipError_t launch_topk(const float*, long long, const int32_t*, long long, int, int, int, int32_t*, long long, float*,
                       long long, hipStream_t, const int32_t*, long long) {
  return counted();
}
hipError_t launch_copy_sel(const int32_t*, int, int, int32_t*, hipStream_t, long long) { return counted(); }
hipError_t launch_attn(const AttnArgs&, uint8_t*, hipStream_t) { return counted(); }
hipError_t launch_um(const AttnArgs&, uint8_t*, hipStream_t) { return counted(); }
hipError_t launch_mass(const AttnArgs&, const int32_t*, int, float*, uint8_t*, hipStream_t, uint32_t*, bool* built) {
  if (built) *built = false;
  return counted();
}
hipError_t launch_active(int, int, int, const void*, const void*, fl_dtype, const int32_t*, int, int, int32_t*, float*,
                         hipStream_t) {
  return counted();
}
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return counted(); }

hipError_t copy_to_host(void* dst, const void* src, size_t bytes, hipStream_t) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t copy_rows_to_host(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width, size_t rows,
                             hipStream_t) {
  for (size_t i = 0; i < rows; ++i)
    std::memcpy((char*)dst + i * dst_pitch, (const char*)src + i * src_pitch, width);
  return hipSuccess;
}
hipError_t copy_d2d_async(void* dst, const void* src, size_t bytes, hipStream_t) {
  std::memcpy(dst, src, bytes);
  return counted();
}

}  // namespace fl
