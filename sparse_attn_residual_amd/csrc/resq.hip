// fl_kv_resq kernels: the quantized loop-1 base and the low-bit residuals of
// the active tokens against the reconstructed previous loop (p1 §4.3, §D.3;
// guide §3).  HBM-bound: every thread owns one 32-dim group of one token's K
// or V row, so a token's 2*G threads read its K and V rows contiguously.
//
// The operation sequence is fixed so that codes are bit-exact: fp32 max/min
// and subtraction, IEEE fp32 division, round-half-even, clamp, directed fp16
// rounding of scale (up) and zero (down); no fused multiply-add except the
// single-rounding residual dequantization fma(code, scale, zero).  The file is
// compiled with floating-point contraction off.
#include "launch.hpp"

namespace fl {

// Base codes of one 32-dim group of K (kv = 0) or V (kv = 1) into record rec
// (thread sub == 0 also zeroes the record's padding).
__device__ inline void base_group(const float* x, uint8_t* rec, int d, int rb, int kv, int g, int sub) {
  const int G = d / kGroup;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) a = fmaxf(a, fabsf(x[i]));
  const uint16_t sh = f2h_up(a / 127.0f);
  const float s = h2f(sh);
  uint32_t packed[kGroup / 4];
#pragma unroll
  for (int w = 0; w < kGroup / 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      int c = 0;
      if (s != 0.0f) {
        float q = rintf(x[4 * w + t] / s);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        c = (int)q;
      }
      word |= ((uint32_t)(uint8_t)(int8_t)c) << (8 * t);
    }
    packed[w] = word;
  }
  uint4* dst = (uint4*)(rec + kv * d + g * kGroup);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  ((uint16_t*)(rec + 2 * d))[kv * G + g] = sh;
  if (sub == 0) {
    for (int p = 2 * d + 4 * G; p < rb; ++p) rec[p] = 0;  // deterministic padding
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_quant_base(const T* __restrict__ k, const T* __restrict__ v,
                                                    uint8_t* __restrict__ base, long long ntok, int d, int rb) {
  const int G = d / kGroup;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long tok = gid / (2 * G);
  int sub = (int)(gid - tok * (2 * G));
  if (tok >= ntok) return;
  const int kv = sub >= G;
  const int g = sub - kv * G;
  float x[kGroup];
  load_group16<T>((kv ? v : k) + tok * d + g * kGroup, x);
  base_group(x, base + tok * rb, d, rb, kv, g, sub);
}

// Residual codes of one group: delta = x - prev against the reconstruction
// of the previous loop, into record rec of a b-bit stream.
__device__ inline void res_group(const float* x, const float* prev, uint8_t* rec, int d, int bits, int rb, int kv,
                                 int g, int sub) {
  const int G = d / kGroup;
  float delta[kGroup];
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    delta[i] = x[i] - prev[i];
    lo = i == 0 ? delta[i] : fminf(lo, delta[i]);
    hi = i == 0 ? delta[i] : fmaxf(hi, delta[i]);
  }
  const float levels = (float)((1 << bits) - 1);
  const uint16_t zh = f2h_down(lo);
  const float z = h2f(zh);
  const float w = hi - z;
  const uint16_t sh = f2h_up(w / levels);
  const float s = h2f(sh);
  int code[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    int cc = 0;
    if (s != 0.0f) {
      float q = rintf((delta[i] - z) / s);
      q = fminf(fmaxf(q, 0.0f), levels);
      cc = (int)q;
    }
    code[i] = cc;
  }
  const int C = d * bits / 8;
  if (bits == 4) {
    uint32_t wds[4];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      uint32_t word = 0;
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) word |= (uint32_t)code[8 * w4 + t8] << (4 * t8);
      wds[w4] = word;
    }
    *(uint4*)(rec + kv * C + g * 16) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  } else {
    uint32_t wds[2];
#pragma unroll
    for (int w2 = 0; w2 < 2; ++w2) {
      uint32_t word = 0;
#pragma unroll
      for (int t16 = 0; t16 < 16; ++t16) word |= (uint32_t)code[16 * w2 + t16] << (2 * t16);
      wds[w2] = word;
    }
    *(uint2*)(rec + kv * C + g * 8) = make_uint2(wds[0], wds[1]);
  }
  uint16_t* meta = (uint16_t*)(rec + 2 * C);
  meta[(2 * kv) * G + g] = sh;
  meta[(2 * kv + 1) * G + g] = zh;
  if (sub == 0) {
    for (int p = 2 * C + 8 * G; p < rb; ++p) rec[p] = 0;
  }
}

// One thread per (active row, group, K|V) of loop r >= 2.
template <typename T>
__global__ __launch_bounds__(256) void k_quant_res(CacheGeo c, int r, const T* __restrict__ k,
                                                   const T* __restrict__ v, uint8_t* __restrict__ res) {
  const int d = c.d, G = d / kGroup, nr = c.n[r], bits = c.bits[r];
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long row = gid / (2 * G);  // over [L][B][H][n_r]
  int sub = (int)(gid - row * (2 * G));
  long long total = (long long)c.L * c.B * c.Hkv * nr;  // rows of every KV head
  if (row >= total) return;
  const int kv = sub >= G;
  const int g = sub - kv * G;
  const int t = (int)(row % nr);
  long long lbh = row / nr;
  const int hk = (int)(lbh % c.Hkv);
  const int b = (int)((lbh / c.Hkv) % c.B);
  const int l = (int)(lbh / ((long long)c.Hkv * c.B));
  if (t >= count_of(c, r, b)) return;  // past this sequence's rows (ragged counts)
  const int j = c.rows[r][(long long)b * nr + t];

  float x[kGroup], prev[kGroup];
  load_group16<T>((kv ? v : k) + row * d + g * kGroup, x);
  chain_group(c, r - 1, l, b, hk, j, kv, g, prev);
  res_group(x, prev, res + row * c.res_rb[r], d, bits, c.res_rb[r], kv, g, sub);
}

// Decode append, loop 1: the base records of position pos of every (l, b, hk)
// from k, v [L][B][Hkv][d].
template <typename T>
__global__ __launch_bounds__(256) void k_append_base(CacheGeo c, int pos, const T* __restrict__ k,
                                                     const T* __restrict__ v, uint8_t* __restrict__ base) {
  const int d = c.d, G = d / kGroup;
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long lbh = gid / (2 * G);
  int sub = (int)(gid - lbh * (2 * G));
  if (lbh >= (long long)c.L * c.B * c.Hkv) return;
  const int kv = sub >= G;
  const int g = sub - kv * G;
  float x[kGroup];
  load_group16<T>((kv ? v : k) + lbh * d + g * kGroup, x);
  base_group(x, base + (lbh * c.S + pos) * c.base_rb, d, c.base_rb, kv, g, sub);
}

// Decode append, loop r >= 2: position pos becomes row t = cnt[r][b] of every
// sequence (rows[r], slot[r]) and its residual against x_hat^(r-1) is record t.
// A sequence at capacity (t == n[r]) is left alone.
template <typename T>
__global__ __launch_bounds__(256) void k_append_res(CacheGeo c, int r, int pos, const T* __restrict__ k,
                                                    const T* __restrict__ v, uint8_t* __restrict__ res,
                                                    int32_t* __restrict__ rows, int32_t* __restrict__ slot) {
  const int d = c.d, G = d / kGroup, nr = c.n[r];
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long lbh = gid / (2 * G);
  int sub = (int)(gid - lbh * (2 * G));
  if (lbh >= (long long)c.L * c.B * c.Hkv) return;
  const int kv = sub >= G;
  const int g = sub - kv * G;
  const int hk = (int)(lbh % c.Hkv);
  const int b = (int)((lbh / c.Hkv) % c.B);
  const int l = (int)(lbh / ((long long)c.Hkv * c.B));
  const int t = c.cnt[r][b];
  if (t < 0 || t >= nr) return;
  float x[kGroup], prev[kGroup];
  load_group16<T>((kv ? v : k) + lbh * d + g * kGroup, x);
  chain_group(c, r - 1, l, b, hk, pos, kv, g, prev);
  res_group(x, prev, res + (lbh * nr + t) * c.res_rb[r], d, c.bits[r], c.res_rb[r], kv, g, sub);
  if (l == 0 && hk == 0 && sub == 0) {
    rows[(long long)b * nr + t] = pos;
    slot[(long long)b * c.S + pos] = t;
  }
}

// The counts follow once every record of the append is written.
__global__ void k_count_up(int32_t* cnt, int n, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B && cnt[b] < n) cnt[b] += 1;
}

// slot[b][j] = index of j in rows[b][0..cnt_b) or -1 (binary search; rows
// ascending; rows of sequence b start at b * n; cnt NULL: cnt_b = n).
__global__ void k_build_slot(const int32_t* __restrict__ rows, int n, const int32_t* __restrict__ cnt, int S, int B,
                             int32_t* __restrict__ slot) {
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)B * S) return;
  int b = (int)(gid / S), j = (int)(gid % S);
  const int32_t* rb = rows + (long long)b * n;
  const int cb = cnt ? cnt[b] : n;
  int lo = 0, hi = cb;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (rb[mid] < j) lo = mid + 1; else hi = mid;
  }
  slot[gid] = (lo < cb && rb[lo] == j) ? lo : -1;
}

hipError_t launch_quant_base(const CacheGeo& c, const void* k, const void* v, fl_dtype dt, uint8_t* base,
                             hipStream_t st) {
  long long ntok = (long long)c.L * c.B * c.Hkv * c.S;
  long long threads = ntok * 2 * (c.d / kGroup);
  dim3 grid((unsigned)((threads + 255) / 256));
  if (dt == FL_BF16)
    FL_LAUNCH(k_quant_base<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v,
                       base, ntok, c.d, c.base_rb);
  else
    FL_LAUNCH(k_quant_base<float>, grid, dim3(256), 0, st, (const float*)k, (const float*)v, base, ntok,
                       c.d, c.base_rb);
  return hipGetLastError();
}

hipError_t launch_build_slot(const CacheGeo& c, int r, int32_t* slot, hipStream_t st) {
  long long n = (long long)c.B * c.S;
  FL_LAUNCH(k_build_slot, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, c.rows[r], c.n[r], c.cnt[r],
                     c.S, c.B, slot);
  return hipGetLastError();
}

hipError_t launch_append(const CacheGeo& c, int r, int pos, const void* k, const void* v, fl_dtype dt,
                         uint8_t* base, uint8_t* res, int32_t* rows, int32_t* slot, int32_t* cnt, hipStream_t st) {
  const long long threads = (long long)c.L * c.B * c.Hkv * 2 * (c.d / kGroup);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const bool bf = dt == FL_BF16;
  if (r == 1) {
    if (bf)
      FL_LAUNCH(k_append_base<uint16_t>, grid, dim3(256), 0, st, c, pos, (const uint16_t*)k,
                         (const uint16_t*)v, base);
    else
      FL_LAUNCH(k_append_base<float>, grid, dim3(256), 0, st, c, pos, (const float*)k, (const float*)v,
                         base);
    return hipGetLastError();
  }
  if (bf)
    FL_LAUNCH(k_append_res<uint16_t>, grid, dim3(256), 0, st, c, r, pos, (const uint16_t*)k,
                       (const uint16_t*)v, res, rows, slot);
  else
    FL_LAUNCH(k_append_res<float>, grid, dim3(256), 0, st, c, r, pos, (const float*)k, (const float*)v, res,
                       rows, slot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FL_LAUNCH(k_count_up, dim3((unsigned)((c.B + 255) / 256)), dim3(256), 0, st, cnt, c.n[r], c.B);
  return hipGetLastError();
}

hipError_t launch_quant_res(const CacheGeo& c, int r, const void* k, const void* v, fl_dtype dt, uint8_t* res,
                            hipStream_t st) {
  long long rowsn = (long long)c.L * c.B * c.Hkv * c.n[r];
  long long threads = rowsn * 2 * (c.d / kGroup);
  dim3 grid((unsigned)((threads + 255) / 256));
  if (dt == FL_BF16)
    FL_LAUNCH(k_quant_res<uint16_t>, grid, dim3(256), 0, st, c, r, (const uint16_t*)k, (const uint16_t*)v,
                       res);
  else
    FL_LAUNCH(k_quant_res<float>, grid, dim3(256), 0, st, c, r, (const float*)k, (const float*)v, res);
  return hipGetLastError();
}

}  // namespace fl
