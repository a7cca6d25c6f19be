// Vector-ALU kernels of the prefill loop attention: one wavefront per query
// row (or per candidate column for the mass pass), lanes split the head
// dimension, columns are visited in ascending order.  These serve the fp32
// inputs and head dim 64 (any dtype); bf16 inputs at head dim 128 go to the
// matrix-core kernels of attn_mfma.hip.
//
// Each quantity follows its definition on the FlashLoop pages:
//   loop 1 dense attention (the workload's dense first loop; p1 §D.1),
//   cached mass M and reused part U (p1 §4.2 and §D.2; guide §3, eq. 3),
//   sparse loop-r update of the active rows (p1 §4.1, §4.2),
//   column mass of the candidates over the rows loop r recomputes (p1 §4.2:
//   the previous loop's attention decides which columns matter).
#include "launch.hpp"

namespace fl {

template <typename T, int E>
__device__ inline void load_row(const T* row, int lane, float* x) {
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = load_elem<T>(row + lane * E + e);
}

template <int E>
__device__ inline void load_kv(const CacheGeo& c, int r, int b, int h, int j, int lane, bool bf16, float* k, float* v) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool paper = c.fmt == kFmtPaper;
    float kk = paper ? paper_elem(c, r, 0, b, kv_head(c, h), j, 0, lane * E + e)
                     : chain_elem(c, r, 0, b, kv_head(c, h), j, 0, lane * E + e);
    float vv = paper ? paper_elem(c, r, 0, b, kv_head(c, h), j, 1, lane * E + e)
                     : chain_elem(c, r, 0, b, kv_head(c, h), j, 1, lane * E + e);
    k[e] = bf16 ? round_bf16(kk) : kk;
    v[e] = bf16 ? round_bf16(vv) : vv;
  }
}

template <int E>
__device__ inline float dot_lanes(const float* q, const float* k) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) s = __builtin_fmaf(q[e], k[e], s);
  return wave_sum(s);
}

// Loop-r attention, one wave per row of loop r.
template <typename T, int E>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a, float tau) {
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & (kWave - 1);
  const long long w = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int r = a.r;
  const int nq = r == 1 ? c.S : c.n[r];
  if (w >= (long long)c.B * c.H * nq) return;
  const int t = (int)(w % nq);
  const int h = (int)((w / nq) % c.H);
  const int b = (int)(w / ((long long)nq * c.H));
  if (t >= count_of(c, r, b)) return;  // past this sequence's rows (ragged counts)
  const int d = c.d;
  const bool bf16 = a.dt == FL_BF16;
  const int i = r == 1 ? t : c.rows[r][(long long)b * nq + t];
  float q[E];
  load_row<T, E>((const T*)a.q + w * d, lane, q);
  float m = -INFINITY, l = 0.0f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  const int ncol = r == 1 ? i + 1 : a.K;
  const int32_t* sel = r == 1 ? nullptr : a.sel + ((long long)b * c.H + h) * a.K;
  for (int tt = 0; tt < ncol; ++tt) {
    const int j = sel ? sel[tt] : tt;
    if (j > i) break;  // columns ascending: the rest are in the causal future
    float kk[E], vv[E];
    load_kv<E>(c, r, b, h, j, lane, bf16, kk, vv);
    const float s = tau * dot_lanes<E>(q, kk);
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);
    const float p = expf(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + p * vv[e];
    m = mn;
  }
  const long long pos = ((long long)b * c.H + h) * c.S + i;
  if (r == 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a.O[pos * d + lane * E + e] = acc[e] / l;
      a.U[pos * d + lane * E + e] = 0.0f;
    }
    if (lane == 0) {
      a.lse[pos] = m + logf(l);
      a.M[pos] = 1.0f;
    }
  } else if (l > 0.0f && a.lsel) {
    const float b2 = m + logf(l);
    float cu, ca;
    mixed_coeffs(a.M[pos], b2, a.lsel[pos], cu, ca);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const long long o = pos * d + lane * E + e;
      const float u = cu * a.U[o];
      a.O[o] = u + ca * (acc[e] / l);
      a.U[o] = u;
    }
    if (lane == 0) {
      a.lse[pos] = b2;
      a.M[pos] = ca;
    }
  } else if (l > 0.0f) {
    const float Mi = a.M[pos];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const long long o = pos * d + lane * E + e;
      a.O[o] = a.U[o] + Mi * (acc[e] / l);
    }
    if (lane == 0) a.lse[pos] = m + logf(l);
  } else if (lane == 0) {
    a.lse[pos] = -INFINITY;
  }
}

// Compact index of row i in loop rr's query tensor.
__device__ inline int q_index(const CacheGeo& c, int rr, int b, int i) {
  return rr == 1 ? i : c.slot[rr][(long long)b * c.S + i];
}

// Cached mass and reused part of loop r, one wave per row of A_r.
template <typename T, int E>
__global__ __launch_bounds__(256) void k_um_valu(AttnArgs a, float tau) {
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & (kWave - 1);
  const long long w = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int r = a.r;
  const int nr = c.n[r];
  if (w >= (long long)c.B * c.H * nr) return;
  const int t = (int)(w % nr);
  const int h = (int)((w / nr) % c.H);
  const int b = (int)(w / ((long long)nr * c.H));
  if (t >= count_of(c, r, b)) return;  // past this sequence's rows (ragged counts)
  const int d = c.d;
  const bool bf16 = a.dt == FL_BF16;
  const int i = c.rows[r][(long long)b * nr + t];
  const int nprev = r - 1 == 1 ? c.S : c.n[r - 1];
  const int qi = q_index(c, r - 1, b, i);
  if (qi < 0) return;  // row not active at loop r-1: sets not nested (precondition)
  float q[E];
  load_row<T, E>((const T*)a.q + (((long long)b * c.H + h) * nprev + qi) * d, lane, q);
  const long long pos = ((long long)b * c.H + h) * c.S + i;
  const float Mp = a.M[pos], lp = a.lse[pos];
  float sum = 0.0f, ez = 0.0f, C[E];
#pragma unroll
  for (int e = 0; e < E; ++e) C[e] = 0.0f;
  if (Mp > 0.0f) {
    const int32_t* sel = a.sel + ((long long)b * c.H + h) * a.K;
    for (int tt = 0; tt < a.K; ++tt) {
      const int j = sel[tt];
      if (j > i) break;
      float kk[E], vv[E];
      load_kv<E>(c, r - 1, b, h, j, lane, bf16, kk, vv);
      const float s = tau * dot_lanes<E>(q, kk);
      const float x = expf(s - lp);
      const float P = Mp * x;
      sum += P;
      ez += x;
#pragma unroll
      for (int e = 0; e < E; ++e) C[e] = __builtin_fmaf(P, vv[e], C[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const long long o = pos * d + lane * E + e;
    a.U[o] = a.O[o] - C[e];
  }
  if (lane == 0) {
    a.M[pos] = sum;
    // loop r-1 log-sum-exp over J_i (the mixed-logit combine reads it)
    if (a.lsel) a.lsel[pos] = ez > 0.0f ? lp + logf(ez) : -INFINITY;
  }
}

// Column mass of the candidates, one wave per candidate column.
template <typename T, int E>
__global__ __launch_bounds__(256) void k_mass_valu(AttnArgs a, const int32_t* cand, int K_prev, float* mass,
                                                   float tau) {
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & (kWave - 1);
  const long long w = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int r = a.r;
  if (w >= (long long)c.B * c.H * K_prev) return;
  const int tt = (int)(w % K_prev);
  const int h = (int)((w / K_prev) % c.H);
  const int b = (int)(w / ((long long)K_prev * c.H));
  const int d = c.d;
  const bool bf16 = a.dt == FL_BF16;
  const int j = cand ? cand[w] : tt;
  float kk[E], vv[E];
  load_kv<E>(c, r - 1, b, h, j, lane, bf16, kk, vv);
  const int nr = count_of(c, r, b);
  const int nprev = r - 1 == 1 ? c.S : c.n[r - 1];
  const int32_t* rows = c.rows[r] + (long long)b * c.n[r];
  int lo = 0, hi = nr;  // first row >= j
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (rows[mid] < j) lo = mid + 1; else hi = mid;
  }
  float acc = 0.0f;
  for (int t = lo; t < nr; ++t) {
    const int i = rows[t];
    const long long pos = ((long long)b * c.H + h) * c.S + i;
    const float Mp = a.M[pos];
    if (!(Mp > 0.0f)) continue;
    const int qi = q_index(c, r - 1, b, i);
    if (qi < 0) continue;  // not active at loop r-1 (precondition)
    float q[E];
    load_row<T, E>((const T*)a.q + (((long long)b * c.H + h) * nprev + qi) * d, lane, q);
    const float s = tau * dot_lanes<E>(q, kk);
    acc += Mp * expf(s - a.lse[pos]);
  }
  if (lane == 0) mass[w] = acc;
}

static float softmax_scale(int d) { return (float)(1.0 / __builtin_sqrt((double)d)); }

#define FL_DISPATCH_VALU(KERNEL, GRID, ...)                                                     \
  do {                                                                                          \
    const bool bf = a.dt == FL_BF16;                                                            \
    if (a.c.d == 64) {                                                                          \
      if (bf) FL_LAUNCH((KERNEL<uint16_t, 1>), GRID, dim3(256), 0, st, __VA_ARGS__);   \
      else FL_LAUNCH((KERNEL<float, 1>), GRID, dim3(256), 0, st, __VA_ARGS__);         \
    } else {                                                                                    \
      if (bf) FL_LAUNCH((KERNEL<uint16_t, 2>), GRID, dim3(256), 0, st, __VA_ARGS__);   \
      else FL_LAUNCH((KERNEL<float, 2>), GRID, dim3(256), 0, st, __VA_ARGS__);         \
    }                                                                                           \
  } while (0)

static dim3 wave_grid(long long waves) { return dim3((unsigned)((waves + 3) / 4)); }

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t st) {
  const int nq = a.r == 1 ? a.c.S : a.c.n[a.r];
  FL_DISPATCH_VALU(k_attn_valu, wave_grid((long long)a.c.B * a.c.H * nq), a, softmax_scale(a.c.d));
  return hipGetLastError();
}

hipError_t launch_um_valu(const AttnArgs& a, hipStream_t st) {
  FL_DISPATCH_VALU(k_um_valu, wave_grid((long long)a.c.B * a.c.H * a.c.n[a.r]), a, softmax_scale(a.c.d));
  return hipGetLastError();
}

hipError_t launch_mass_valu(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, hipStream_t st) {
  FL_DISPATCH_VALU(k_mass_valu, wave_grid((long long)a.c.B * a.c.H * K_prev), a, cand, K_prev, mass,
                   softmax_scale(a.c.d));
  return hipGetLastError();
}

}  // namespace fl
