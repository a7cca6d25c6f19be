// fl_select_active: the next loop's active-token set (p1 §4.1 and §D.1:
// later loops recompute only nested active sets of budget k(r); the guide's
// §3 summary: tokens ranked by their normalized hidden-state change, top-k
// kept).  The score of a candidate token is the relative L2 change of its
// hidden state across the loop just run, ||h_cur - h_prev|| / ||h_prev||,
// accumulated in fp32; the selection reuses the top-K kernel (ties to the
// lower position, ascending output).
#include "launch.hpp"

namespace fl {

constexpr int kActThreads = 256;  // four wavefronts, one candidate token each

template <typename T>
__device__ inline void load8(const T* p, float* x);
template <>
__device__ inline void load8<float>(const float* p, float* x) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <>
__device__ inline void load8<uint16_t>(const uint16_t* p, float* x) {
  const uint4 w = *(const uint4*)p;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(ws[k] << 16);
    x[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
  }
}

// One wavefront per candidate (b, t): lanes stride over the D dims, eight
// at a time (16- or 32-byte loads), then a wave reduction.
template <typename T>
__global__ __launch_bounds__(kActThreads) void k_active_score(const T* __restrict__ h_prev,
                                                              const T* __restrict__ h_cur, int S, int D, int B,
                                                              const int32_t* __restrict__ rows_prev, int n_prev,
                                                              float* __restrict__ score) {
  const long long w = (long long)blockIdx.x * (kActThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (w >= (long long)B * n_prev) return;  // whole wavefronts leave together
  const int b = (int)(w / n_prev), t = (int)(w - (long long)b * n_prev);
  const int j = rows_prev ? rows_prev[w] : t;
  const long long off = ((long long)b * S + j) * D;
  float num = 0.0f, den = 0.0f;
  for (int e = lane * 8; e < D; e += kWave * 8) {
    float p[8], c[8];
    load8<T>(h_prev + off + e, p);
    load8<T>(h_cur + off + e, c);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dlt = c[k] - p[k];
      num = __builtin_fmaf(dlt, dlt, num);
      den = __builtin_fmaf(p[k], p[k], den);
    }
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if (lane == 0) score[w] = den > 0.0f ? __builtin_sqrtf(num) / __builtin_sqrtf(den) : (num > 0.0f ? INFINITY : 0.0f);
}

hipError_t launch_active(int B, int S, int D, const void* h_prev, const void* h_cur, fl_dtype dt,
                         const int32_t* rows_prev, int n_prev, int k, int32_t* rows_out, float* score,
                         hipStream_t st) {
  const long long waves = (long long)B * n_prev;
  const dim3 grid((unsigned)((waves + kActThreads / kWave - 1) / (kActThreads / kWave)));
  if (dt == FL_BF16)
    FL_LAUNCH(k_active_score<uint16_t>, grid, dim3(kActThreads), 0, st, (const uint16_t*)h_prev,
                       (const uint16_t*)h_cur, S, D, B, rows_prev, n_prev, score);
  else
    FL_LAUNCH(k_active_score<float>, grid, dim3(kActThreads), 0, st, (const float*)h_prev,
                       (const float*)h_cur, S, D, B, rows_prev, n_prev, score);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (k == n_prev) return launch_copy_sel(rows_prev, B, n_prev, rows_out, st);
  return launch_topk(score, n_prev, rows_prev, n_prev, B, n_prev, k, rows_out, k, nullptr, 0, st);
}

}  // namespace fl
