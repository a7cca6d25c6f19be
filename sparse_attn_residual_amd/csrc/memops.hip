// Memory operations of the C ABI layer outside the kernels: the synchronous
// host copies of the FL_CHECK validator and a device-to-device copy on the
// caller's stream.  Kept behind the launch layer so that the validation code
// can be exercised on the CPU against host arrays.
#include "launch.hpp"

namespace fl {

hipError_t copy_to_host(void* dst, const void* src, size_t bytes, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  return hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
}

hipError_t copy_rows_to_host(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width,
                             size_t rows, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  return hipMemcpy2D(dst, dst_pitch, src, src_pitch, width, rows, hipMemcpyDeviceToHost);
}

hipError_t copy_d2d_async(void* dst, const void* src, size_t bytes, hipStream_t st) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
}

}  // namespace fl
