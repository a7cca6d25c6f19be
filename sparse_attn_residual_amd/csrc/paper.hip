// fl_kv_resq for the paper's own cache format (p1 App. E: INT4 asymmetric
// group-wise quantization with group size 64 for the base and every
// residual; post-RoPE keys per channel, values per token; the 64 most recent
// tokens kept in BF16).  The stream layout is described next to
// paper_stream_bytes in common.hpp.
//
// One group's arithmetic is that of the workload format's residuals with 15
// levels: z = fp16 rounded down of the minimum, s = fp16 rounded up of
// ((max - z) / 15), c = clamp(rint((x - z) / s), 0, 15) (0 when s == 0), and
// x_hat = fma(c, s, z); the base quantizes x itself, loop r >= 2 the residual
// x^(r) - x_hat^(r-1) of its active tokens.  A key group is one channel over
// 64 consecutive entries of the stream, a value group 64 dims of one token.
// The file is compiled with floating-point contraction off.
#include "launch.hpp"

namespace fl {

struct GroupQ {
  uint16_t s16, z16;
  float s, z;
};

__device__ __forceinline__ GroupQ group_q4(float lo, float hi) {
  GroupQ q;
  q.z16 = f2h_down(lo);
  q.z = h2f(q.z16);
  q.s16 = f2h_up((hi - q.z) / 15.0f);
  q.s = h2f(q.s16);
  return q;
}
__device__ __forceinline__ uint32_t code_q4(float x, const GroupQ& q) {
  if (q.s == 0.0f) return 0;
  float c = rintf((x - q.z) / q.s);
  c = fminf(fmaxf(c, 0.0f), 15.0f);
  return (uint32_t)c;
}

// Keys: one block per (l, b, hk, group of 64 entries).  Each thread forms
// 32 dims of one entry (the residual against the previous loop's values,
// rebuilt with 16-byte loads) into an LDS block [64][128]; then two threads
// per channel reduce its 64 entries, quantize, and the codes are packed per
// entry from LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_pq_keys(CacheGeo c, int r, const T* __restrict__ k, uint8_t* __restrict__ out) {
  __shared__ float xs[kPGroup][128 + 1];
  __shared__ float smin[2][128], smax[2][128];
  __shared__ uint8_t codes[kPGroup][128];
  const int m = paper_entries(c, r);
  const int nblk = (m + kPGroup - 1) / kPGroup;
  const int blk = (int)(blockIdx.x % nblk);
  const long long lbh = blockIdx.x / nblk;
  const int hk = (int)(lbh % c.Hkv);
  const int b = (int)((lbh / c.Hkv) % c.B);
  const int l = (int)(lbh / ((long long)c.Hkv * c.B));
  const int t0 = blk * kPGroup;
  const int t1 = min(t0 + kPGroup, paper_body(c, r, b));
  if (t0 >= t1) return;  // the whole block: no quantized entry here
  const int stride = c.n[r];   // input rows per (l, b, hk) (n[1] == S)
  {
    const int e = threadIdx.x >> 2, qd = threadIdx.x & 3;   // entry, 32 dims
    const int t = t0 + e;
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    if (t < t1) {
      load_group16<T>(k + (lbh * stride + t) * 128 + qd * 32, x);
      if (r > 1) {
        const int j = c.rows[r][(long long)b * c.n[r] + t];
        float p[16];
        paper_chain16(c, r - 1, l, b, hk, j, 0, qd * 32, p);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = x[i] - p[i];
        paper_chain16(c, r - 1, l, b, hk, j, 0, qd * 32 + 16, p);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[16 + i] = x[16 + i] - p[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) xs[e][qd * 32 + i] = x[i];
  }
  __syncthreads();
  const int ch = threadIdx.x & 127, half = threadIdx.x >> 7;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (t0 + half * 32 + i < t1) {
      const float v = xs[half * 32 + i][ch];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
  }
  smin[half][ch] = lo;
  smax[half][ch] = hi;
  __syncthreads();
  const GroupQ q = group_q4(fminf(smin[0][ch], smin[1][ch]), fmaxf(smax[0][ch], smax[1][ch]));
  uint8_t* st = out + lbh * c.pbytes[r];
#pragma unroll
  for (int i = 0; i < 32; ++i) codes[half * 32 + i][ch] = (uint8_t)code_q4(xs[half * 32 + i][ch], q);
  if (half == 0) {
    uint16_t* meta = (uint16_t*)(st + (long long)m * kPRec + (long long)blk * kPKMeta);
    meta[ch] = q.s16;
    meta[128 + ch] = q.z16;
  }
  __syncthreads();
  const int e = threadIdx.x >> 2, qd = threadIdx.x & 3;   // entry, 32 channels
  const int t = t0 + e;
  if (t < t1) {
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= (uint32_t)codes[e][qd * 32 + u * 8 + n] << (4 * n);
      w[u] = word;
    }
    *(uint4*)(st + (long long)t * kPRec + qd * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Values: one thread per (l, b, hk, entry, 64-dim group).
template <typename T>
__global__ __launch_bounds__(256) void k_pq_values(CacheGeo c, int r, const T* __restrict__ v,
                                                   uint8_t* __restrict__ out) {
  const int m = paper_entries(c, r);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int g = (int)(gid & 1);
  const long long et = gid >> 1;
  const int t = (int)(et % m);
  const long long lbh = et / m;
  if (lbh >= (long long)c.L * c.B * c.Hkv) return;
  const int hk = (int)(lbh % c.Hkv);
  const int b = (int)((lbh / c.Hkv) % c.B);
  const int l = (int)(lbh / ((long long)c.Hkv * c.B));
  if (t >= paper_body(c, r, b)) return;
  const int stride = c.n[r];
  const T* src = v + (lbh * stride + t) * 128 + g * 64;
  float x[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) x[e] = load_elem<T>(src + e);
  if (r > 1) {
    const int j = c.rows[r][(long long)b * c.n[r] + t];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float p[16];
      paper_chain16(c, r - 1, l, b, hk, j, 1, g * 64 + q4 * 16, p);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[q4 * 16 + e] = x[q4 * 16 + e] - p[e];
    }
  }
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int e = 1; e < 64; ++e) {
    lo = fminf(lo, x[e]);
    hi = fmaxf(hi, x[e]);
  }
  const GroupQ q = group_q4(lo, hi);
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) word |= code_q4(x[u * 8 + n], q) << (4 * n);
    w[u] = word;
  }
  uint8_t* rec = out + lbh * c.pbytes[r] + (long long)t * kPRec;
  *(uint4*)(rec + 64 + g * 32) = make_uint4(w[0], w[1], w[2], w[3]);
  *(uint4*)(rec + 64 + g * 32 + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  uint16_t* vm = (uint16_t*)(rec + 128 + g * 4);
  vm[0] = q.s16;
  vm[1] = q.z16;
  if (g == 0) *(uint2*)(rec + 136) = make_uint2(0, 0);  // deterministic padding
}

// Tail: the loop's own K and V of the tail tokens as bf16, one thread per
// (l, b, hk, tail token, K|V, 16 dims).
template <typename T>
__global__ __launch_bounds__(256) void k_pq_tail(CacheGeo c, int r, const T* __restrict__ k,
                                                 const T* __restrict__ v, uint8_t* __restrict__ out) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int q16 = (int)(gid & 7), kv = (int)((gid >> 3) & 1);
  const long long rest = gid >> 4;
  const int tt = (int)(rest % kPTailN);
  const long long lbh = rest / kPTailN;
  if (lbh >= (long long)c.L * c.B * c.Hkv) return;
  const int b = (int)((lbh / c.Hkv) % c.B);
  int t, j;   // input row and position
  if (r == 1) {
    j = c.Sq + tt;
    t = j;
    if (j >= c.S) return;
  } else {
    t = paper_body(c, r, b) + tt;
    if (t >= count_of(c, r, b)) return;
    j = c.rows[r][(long long)b * c.n[r] + t];
  }
  const int stride = c.n[r];
  const int m = paper_entries(c, r);
  const T* src = (kv ? v : k) + (lbh * stride + t) * 128 + q16 * 16;
  uint16_t* dst = (uint16_t*)(out + lbh * c.pbytes[r] + (long long)m * kPRec +
                              (long long)((m + kPGroup - 1) / kPGroup) * kPKMeta + (long long)(j - c.Sq) * kPTail +
                              kv * 256) + q16 * 16;
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    w[u] = (uint32_t)f32_to_bf16(load_elem<T>(src + 2 * u)) | ((uint32_t)f32_to_bf16(load_elem<T>(src + 2 * u + 1)) << 16);
  *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
  *(uint4*)(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
}

hipError_t launch_paper_quant(const CacheGeo& c, int r, const void* k, const void* v, fl_dtype dt, uint8_t* out,
                              hipStream_t st) {
  const int m = paper_entries(c, r);
  const long long lbh = (long long)c.L * c.B * c.Hkv;
  const bool bf = dt == FL_BF16;
  if (m > 0) {
    const unsigned nk = (unsigned)(lbh * ((m + kPGroup - 1) / kPGroup));
    const unsigned nv = (unsigned)((lbh * m * 2 + 255) / 256);
    if (bf) {
      FL_LAUNCH(k_pq_keys<uint16_t>, dim3(nk), dim3(256), 0, st, c, r, (const uint16_t*)k, out);
      FL_LAUNCH(k_pq_values<uint16_t>, dim3(nv), dim3(256), 0, st, c, r, (const uint16_t*)v, out);
    } else {
      FL_LAUNCH(k_pq_keys<float>, dim3(nk), dim3(256), 0, st, c, r, (const float*)k, out);
      FL_LAUNCH(k_pq_values<float>, dim3(nv), dim3(256), 0, st, c, r, (const float*)v, out);
    }
  }
  const unsigned nt = (unsigned)((lbh * kPTailN * 16 + 255) / 256);
  if (bf)
    FL_LAUNCH(k_pq_tail<uint16_t>, dim3(nt), dim3(256), 0, st, c, r, (const uint16_t*)k, (const uint16_t*)v,
                       out);
  else
    FL_LAUNCH(k_pq_tail<float>, dim3(nt), dim3(256), 0, st, c, r, (const float*)k, (const float*)v, out);
  return hipGetLastError();
}

}  // namespace fl
