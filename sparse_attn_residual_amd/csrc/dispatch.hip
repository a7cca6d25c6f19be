// Dispatch of the prefill attention family between the vector-ALU kernels
// (fp32 inputs, head dim 64) and the matrix-core kernels (bf16, head dim 128).
#include "launch.hpp"

namespace fl {

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t st);
hipError_t launch_um_valu(const AttnArgs& a, hipStream_t st);
hipError_t launch_mass_valu(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, hipStream_t st);
hipError_t launch_attn_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st);
hipError_t launch_um_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st);
hipError_t launch_mass_mfma(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                            hipStream_t st, uint32_t* hist, bool* hist_built);

bool use_mfma(const AttnArgs& a) { return a.dt == FL_BF16 && a.c.d == 128; }

hipError_t launch_attn(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  return use_mfma(a) ? launch_attn_mfma(a, ws, st) : launch_attn_valu(a, st);
}
hipError_t launch_um(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  return use_mfma(a) ? launch_um_mfma(a, ws, st) : launch_um_valu(a, st);
}
hipError_t launch_mass(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                       hipStream_t st, uint32_t* hist, bool* hist_built) {
  if (use_mfma(a)) return launch_mass_mfma(a, cand, K_prev, mass, ws, st, hist, hist_built);
  if (hist_built) *hist_built = false;
  return launch_mass_valu(a, cand, K_prev, mass, st);
}

}  // namespace fl
