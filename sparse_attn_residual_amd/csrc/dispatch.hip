// Dispatch of the prefill attention family between the vector-ALU kernels
// (fp32 inputs, head dim 64) and the bf16 matrix-core kernels (head dim 128).
#include "launch.hpp"

namespace fl {

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t st);
hipError_t launch_um_valu(const AttnArgs& a, hipStream_t st);
hipError_t launch_mass_valu(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, hipStream_t st);

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) { return launch_attn_valu(a, st); }
hipError_t launch_um(const AttnArgs& a, hipStream_t st) { return launch_um_valu(a, st); }
hipError_t launch_mass(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, hipStream_t st) {
  return launch_mass_valu(a, cand, K_prev, mass, st);
}

}  // namespace fl
