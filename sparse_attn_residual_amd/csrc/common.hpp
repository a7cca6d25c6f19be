// Device-side helpers shared by the FlashLoop kernels (gfx950, wave64).
//
// Record geometry and dequantization follow the packed cache layout declared
// in include/flashloop.h (p1 §4.3 and App. G: a quantized anchor plus packed
// low-bit residual streams read directly by the attention kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "flashloop.h"

namespace fl {

constexpr int kWave = 64;
constexpr int kGroup = 32;  // quantization group (dims)

// ---------------------------------------------------------------- geometry
// Kernel-side copy of the cache description (passed by value).
struct CacheGeo {
  int L, B, H, S, d, R;
  int Hkv;                       // key/value heads (the streams are per KV head)
  int T;                         // tokens a decode step attends: positions [0, T)
  int fmt;                       // FL_FMT_WORKLOAD or FL_FMT_PAPER (record layout below)
  int Sq;                        // paper format: quantized positions [0, Sq), the tail [Sq, S)
  // paper format, per loop: entries of a stream (loop 1: Sq) and its bytes;
  // res[1] points at the base.  Kept as arrays so that a loop index selects
  // them without choosing between fields.
  int pm[FL_MAX_LOOPS + 1];
  long long pbytes[FL_MAX_LOOPS + 1];
  int G;                         // query heads per KV head, H / Hkv
  int n[FL_MAX_LOOPS + 1];
  int bits[FL_MAX_LOOPS + 1];
  int res_rb[FL_MAX_LOOPS + 1];  // residual record bytes per loop
  int base_rb;                   // base record bytes
  const int32_t* rows[FL_MAX_LOOPS + 1];
  const int32_t* slot[FL_MAX_LOOPS + 1];
  const int32_t* cnt[FL_MAX_LOOPS + 1];  // per-sequence |A_r| (NULL: n[r] for every sequence)
  const uint8_t* base;
  const uint8_t* res[FL_MAX_LOOPS + 1];
};

__host__ __device__ inline int pad16(int n) { return (n + 15) & ~15; }
__host__ __device__ inline int base_record_bytes(int d) { return pad16(2 * d + 4 * (d / kGroup)); }
__host__ __device__ inline int residual_record_bytes(int d, int bits) {
  return pad16(2 * (d * bits / 8) + 8 * (d / kGroup));
}

// Rows of A_r in sequence b: n[r] is the capacity and stride of rows[r] and
// of the loop-r streams, cnt[r][b] the count when sequences differ.
__device__ __forceinline__ int count_of(const CacheGeo& c, int r, int b) {
  // n[1] == S and cnt[1] == NULL.  The capacity is taken as a wave-uniform
  // value first, so the compiler does not turn the choice into one load
  // through a pointer into the by-value geometry argument (which would copy
  // the whole argument to scratch).
  const int n = __builtin_amdgcn_readfirstlane(c.n[r]);
  const int32_t* cnt = c.cnt[r];
  return cnt ? cnt[b] : n;
}
// KV head that query head h reads (grouped-query attention; G = 1: h).
__device__ __forceinline__ int kv_head(const CacheGeo& c, int h) { return h / c.G; }
// Address of the base record of token j of (layer l, seq b, KV head hk).
__device__ __forceinline__ const uint8_t* base_rec(const CacheGeo& c, int l, int b, int hk, int j) {
  long long idx = (((long long)l * c.B + b) * c.Hkv + hk) * c.S + j;
  return c.base + idx * c.base_rb;
}
// Address of the loop-r residual record number t (t = slot) of (l, b, hk).
__device__ __forceinline__ const uint8_t* res_rec(const CacheGeo& c, int r, int l, int b, int hk, int t) {
  long long idx = (((long long)l * c.B + b) * c.Hkv + hk) * c.n[r] + t;
  return c.res[r] + idx * c.res_rb[r];
}

// ---------------------------------------------------------------- numbers
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// float -> bf16 bits, round to nearest even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32), which rounds in the default mode.
typedef __bf16 fl_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float fl_f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint16_t f32_to_bf16(float x) {
  const fl_bf16x2_t v = __builtin_convertvector(fl_f32x2_t{x, 0.0f}, fl_bf16x2_t);
  return (uint16_t)__builtin_bit_cast(uint32_t, v);
}
__device__ inline float round_bf16(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Workgroup barrier for data exchanged through LDS only: the wave's LDS
// operations have completed (lgkmcnt 0) and the compiler may not move memory
// operations across it, but unlike __syncthreads (whose release fence waits
// for every outstanding memory operation) it leaves the wave's global loads
// and global->LDS copies in flight.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}
// Order-preserving uint32 key of a float (larger float, larger key; -0 ranks
// as +0; no float maps to 0).
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Histogram of a decode head's loop-1 logits by the top kHistBits bits of
// their order keys: loop 1 leaves it in the first kHistBins entries of the
// head's selection row, loop 2's selection starts from it.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ inline uint16_t f2h_rn(float x) { return __half_as_ushort(__float2half_rn(x)); }

// fp16 rounded toward +inf of a finite float within the fp16 range.
__device__ inline uint16_t f2h_up(float y) {
  uint16_t h = f2h_rn(y);
  if (h2f(h) < y) {
    if (h == 0x8000u) h = 0x0001u;           // -0 -> smallest positive subnormal
    else if (h & 0x8000u) h = (uint16_t)(h - 1u);  // negative: magnitude shrinks
    else h = (uint16_t)(h + 1u);
  }
  return h;
}
// fp16 rounded toward -inf of a finite float within the fp16 range.
__device__ inline uint16_t f2h_down(float y) {
  uint16_t h = f2h_rn(y);
  if (h2f(h) > y) {
    if (h == 0x0000u) h = 0x8001u;           // +0 -> smallest negative subnormal
    else if (h & 0x8000u) h = (uint16_t)(h + 1u);  // negative: magnitude grows
    else h = (uint16_t)(h - 1u);
  }
  return h;
}

// Loads of one input element (float or bf16 bits) as float.
template <typename T> __device__ inline float load_elem(const T* p);
template <> __device__ inline float load_elem<float>(const float* p) { return *p; }
template <> __device__ inline float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// ---------------------------------------------------------------- dequant
// Element e (0 <= e < d) of K (kv = 0) or V (kv = 1) of a base record.
__device__ inline float base_elem(const uint8_t* rec, int d, int kv, int e) {
  int8_t c = (int8_t)rec[kv * d + e];
  const uint16_t* sc = (const uint16_t*)(rec + 2 * d) + kv * (d / kGroup);
  return (float)c * h2f(sc[e / kGroup]);
}
// Dequantized residual element: fma(code, scale, zero), one rounding.
__device__ inline float res_elem(const uint8_t* rec, int d, int bits, int kv, int e) {
  int C = d * bits / 8;
  int per = 8 / bits;
  uint8_t byte = rec[kv * C + e / per];
  int code = (byte >> (bits * (e % per))) & ((1 << bits) - 1);
  const uint16_t* meta = (const uint16_t*)(rec + 2 * C);
  int G = d / kGroup;
  float s = h2f(meta[(2 * kv) * G + e / kGroup]);
  float z = h2f(meta[(2 * kv + 1) * G + e / kGroup]);
  return __builtin_fmaf((float)code, s, z);
}

// Reconstruction x_hat^(r) of element e of token j: the base plus the
// residuals of loops 2..r in which j was active (sets are nested, so the
// chain stops at the first loop where j is inactive).
__device__ __forceinline__ float chain_elem(const CacheGeo& c, int r, int l, int b, int hk, int j, int kv, int e) {
  float x = base_elem(base_rec(c, l, b, hk, j), c.d, kv, e);
  for (int rr = 2; rr <= r; ++rr) {
    int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    x = x + res_elem(res_rec(c, rr, l, b, hk, t), c.d, c.bits[rr], kv, e);
  }
  return x;
}

// The same reconstruction for the 32 dims [32g, 32g+32) of one group, with
// the records read by vector loads: the operations and their order are those
// of chain_elem, so the values are the same.
__device__ __forceinline__ void chain_group(const CacheGeo& c, int r, int l, int b, int hk, int j, int kv, int g, float* x) {
  const int d = c.d, G = d / kGroup;
  const uint8_t* rec = base_rec(c, l, b, hk, j);
  const uint4 w0 = *(const uint4*)(rec + kv * d + g * kGroup);
  const uint4 w1 = *(const uint4*)(rec + kv * d + g * kGroup + 16);
  const float s = h2f(((const uint16_t*)(rec + 2 * d))[kv * G + g]);
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int e = 0; e < kGroup; ++e) x[e] = (float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) * s;
  for (int rr = 2; rr <= r; ++rr) {
    const int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    const uint8_t* q = res_rec(c, rr, l, b, hk, t);
    const int bits = c.bits[rr];
    const int C = d * bits / 8;
    const uint16_t* meta = (const uint16_t*)(q + 2 * C);
    const float rs = h2f(meta[(2 * kv) * G + g]);
    const float rz = h2f(meta[(2 * kv + 1) * G + g]);
    if (bits == 4) {
      const uint4 pw = *(const uint4*)(q + kv * C + g * 16);
      const uint32_t ws[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
      for (int e = 0; e < kGroup; ++e)
        x[e] = x[e] + __builtin_fmaf((float)((ws[e >> 3] >> (4 * (e & 7))) & 15), rs, rz);
    } else {
      const uint2 pw = *(const uint2*)(q + kv * C + g * 8);
      const uint32_t ws[2] = {pw.x, pw.y};
#pragma unroll
      for (int e = 0; e < kGroup; ++e)
        x[e] = x[e] + __builtin_fmaf((float)((ws[e >> 4] >> (2 * (e & 15))) & 3), rs, rz);
    }
  }
}

// chain_group for a chain of exactly NR residual loops (r = NR + 1): every
// slot lookup is issued first, then every record of a loop where j is
// active, so the loads of one token are two round trips rather than two per
// loop.  The sets nest, so "active at loop rr" (slot >= 0) holds for a
// prefix of the loops, and the sum runs over the same terms in the same
// order as chain_group's: the values are the same.
template <int NR>
__device__ __forceinline__ void chain_group_n(const CacheGeo& c, int l, int b, int hk, int j, int kv, int g, float* x) {
  const int d = c.d, G = d / kGroup;
  int t[NR > 0 ? NR : 1];
#pragma unroll
  for (int k = 0; k < NR; ++k) t[k] = c.slot[k + 2][(long long)b * c.S + j];
  const uint8_t* rec = base_rec(c, l, b, hk, j);
  const uint4 w0 = *(const uint4*)(rec + kv * d + g * kGroup);
  const uint4 w1 = *(const uint4*)(rec + kv * d + g * kGroup + 16);
  const float s = h2f(((const uint16_t*)(rec + 2 * d))[kv * G + g]);
  uint4 cw[NR > 0 ? NR : 1];
  uint32_t sz[NR > 0 ? NR : 1];  // scale | zero << 16
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    cw[k] = make_uint4(0, 0, 0, 0);
    sz[k] = 0;
    if (t[k] >= 0) {
      const uint8_t* q = res_rec(c, k + 2, l, b, hk, t[k]);
      const int C = d * c.bits[k + 2] / 8;
      const uint16_t* meta = (const uint16_t*)(q + 2 * C);
      if (c.bits[k + 2] == 4) {
        cw[k] = *(const uint4*)(q + kv * C + g * 16);
      } else {
        const uint2 pw = *(const uint2*)(q + kv * C + g * 8);
        cw[k].x = pw.x;
        cw[k].y = pw.y;
      }
      sz[k] = (uint32_t)meta[(2 * kv) * G + g] | ((uint32_t)meta[(2 * kv + 1) * G + g] << 16);
    }
  }
  const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int e = 0; e < kGroup; ++e) x[e] = (float)(int8_t)(w[e >> 2] >> (8 * (e & 3))) * s;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (t[k] < 0) break;
    const float rs = h2f((uint16_t)sz[k]), rz = h2f((uint16_t)(sz[k] >> 16));
    if (c.bits[k + 2] == 4) {
      const uint32_t ws[4] = {cw[k].x, cw[k].y, cw[k].z, cw[k].w};
#pragma unroll
      for (int e = 0; e < kGroup; ++e)
        x[e] = x[e] + __builtin_fmaf((float)((ws[e >> 3] >> (4 * (e & 7))) & 15), rs, rz);
    } else {
      const uint32_t ws[2] = {cw[k].x, cw[k].y};
#pragma unroll
      for (int e = 0; e < kGroup; ++e)
        x[e] = x[e] + __builtin_fmaf((float)((ws[e >> 4] >> (2 * (e & 15))) & 3), rs, rz);
    }
  }
}

// ---------------------------------------------------------------- the paper's format
// (FL_FMT_PAPER, head dim 128).  Every (layer, sequence, KV head) owns one
// stream per loop: m entries (loop 1: the positions [0, Sq); loop r: the
// capacity n[r] of its compact rows) of kPRec bytes
//   K codes 64 B | V codes 64 B (4-bit, dim 2i in the low nibble of byte i) |
//   V scale, zero (fp16) of dims 0-63, then of dims 64-127 | zero padding,
// then ceil(m / 64) key blocks of kPKMeta bytes (fp16 scale of channels
// 0..127, then their fp16 zeros) for entries [64 blk, 64 blk + 64), then 64
// tail slots of kPTail bytes (K then V, bf16) for positions Sq + slot.
constexpr int kFmtPaper = FL_FMT_PAPER;
constexpr int kPRec = 144, kPKMeta = 512, kPTail = 512, kPGroup = 64, kPTailN = 64;
__host__ __device__ inline long long paper_stream_bytes(int m) {
  return (long long)m * kPRec + (long long)((m + kPGroup - 1) / kPGroup) * kPKMeta + (long long)kPTailN * kPTail;
}
__device__ __forceinline__ const uint8_t* paper_stream(const CacheGeo& c, int r, int l, int b, int hk) {
  const long long lbh = ((long long)l * c.B + b) * c.Hkv + hk;
  return c.res[r] + lbh * c.pbytes[r];
}
__host__ __device__ __forceinline__ int paper_entries(const CacheGeo& c, int r) { return c.pm[r]; }

// Dequantized dims [e0, e0 + 16) (e0 a multiple of 16) of K (kv = 0) or V of
// entry t of a paper-format stream with m entries: fma(code, scale, zero).
// Codes, key scales and zeros come in with 8- and 16-byte loads.
__device__ __forceinline__ void paper_deq16(const uint8_t* st, int m, int t, int kv, int e0, float* x) {
  const uint8_t* rec = st + (long long)t * kPRec;
  const uint2 w = *(const uint2*)(rec + kv * 64 + e0 / 2);
  const uint32_t ws[2] = {w.x, w.y};
  if (kv == 0) {
    const uint8_t* meta = st + (long long)m * kPRec + (long long)(t / kPGroup) * kPKMeta;
    const uint4 s0 = *(const uint4*)(meta + e0 * 2), s1 = *(const uint4*)(meta + e0 * 2 + 16);
    const uint4 z0 = *(const uint4*)(meta + 256 + e0 * 2), z1 = *(const uint4*)(meta + 256 + e0 * 2 + 16);
    const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint32_t zw[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float code = (float)((ws[e >> 3] >> (4 * (e & 7))) & 15);
      const float s = h2f((uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
      const float z = h2f((uint16_t)(zw[e >> 1] >> (16 * (e & 1))));
      x[e] = __builtin_fmaf(code, s, z);
    }
  } else {
    const uint32_t vm = *(const uint32_t*)(rec + 128 + (e0 / 64) * 4);
    const float s = h2f((uint16_t)vm), z = h2f((uint16_t)(vm >> 16));
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = __builtin_fmaf((float)((ws[e >> 3] >> (4 * (e & 7))) & 15), s, z);
  }
}

// One element of paper_chain16 (the quantizers' previous-loop values).
__device__ __forceinline__ float paper_deq1(const uint8_t* st, int m, int t, int kv, int e) {
  const uint8_t* rec = st + (long long)t * kPRec;
  const float code = (float)((rec[kv * 64 + e / 2] >> (4 * (e & 1))) & 15);
  if (kv == 0) {
    const uint16_t* meta = (const uint16_t*)(st + (long long)m * kPRec + (long long)(t / kPGroup) * kPKMeta);
    return __builtin_fmaf(code, h2f(meta[e]), h2f(meta[128 + e]));
  }
  const uint16_t* vm = (const uint16_t*)(rec + 128 + (e / 64) * 4);
  return __builtin_fmaf(code, h2f(vm[0]), h2f(vm[1]));
}
__device__ __forceinline__ const uint16_t* paper_tail(const CacheGeo& c, int r, int l, int b, int hk, int j, int kv) {
  const int m = paper_entries(c, r);
  return (const uint16_t*)(paper_stream(c, r, l, b, hk) + (long long)m * kPRec +
                           (long long)((m + kPGroup - 1) / kPGroup) * kPKMeta + (long long)(j - c.Sq) * kPTail +
                           kv * 256);
}
__device__ __forceinline__ float paper_elem(const CacheGeo& c, int r, int l, int b, int hk, int j, int kv, int e) {
  if (j >= c.Sq) {
    int rr = 1;
    for (int q = 2; q <= r; ++q) {
      if (c.slot[q][(long long)b * c.S + j] < 0) break;
      rr = q;
    }
    return bf16_to_f32(paper_tail(c, rr, l, b, hk, j, kv)[e]);
  }
  float x = paper_deq1(paper_stream(c, 1, l, b, hk), c.pm[1], j, kv, e);
  for (int rr = 2; rr <= r; ++rr) {
    const int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    x = x + paper_deq1(paper_stream(c, rr, l, b, hk), c.pm[rr], t, kv, e);
  }
  return x;
}
// Entries of sequence b's loop-r stream that are quantized: positions [0, Sq)
// at loop 1; at loop r the active rows below Sq (rows ascend).
__device__ __forceinline__ int paper_body(const CacheGeo& c, int r, int b) {
  if (r == 1) return c.Sq;
  const int cnt = count_of(c, r, b);
  const int32_t* rows = c.rows[r] + (long long)b * c.n[r];
  int lo = 0, hi = cnt;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rows[mid] < c.Sq) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// x_hat^(r) of dims [e0, e0 + 16) of K or V of token j (KV head hk): a tail
// token reads the bf16 slot of the last loop <= r in which it is active; any
// other token adds, in fp32 and loop order, the base and the residuals of
// the loops in which it is active (sets are nested).
__device__ __forceinline__ void paper_chain16(const CacheGeo& c, int r, int l, int b, int hk, int j, int kv, int e0,
                                     float* x) {
  if (j >= c.Sq) {
    int rr = 1;
    for (int q = 2; q <= r; ++q) {
      if (c.slot[q][(long long)b * c.S + j] < 0) break;
      rr = q;
    }
    const uint4* tv = (const uint4*)(paper_tail(c, rr, l, b, hk, j, kv) + e0);
    const uint4 a0 = tv[0], a1 = tv[1];
    const uint32_t aw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = __uint_as_float((e & 1) ? (aw[e >> 1] & 0xffff0000u) : (aw[e >> 1] << 16));
    return;
  }
  paper_deq16(paper_stream(c, 1, l, b, hk), c.pm[1], j, kv, e0, x);
  for (int rr = 2; rr <= r; ++rr) {
    const int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    float y[16];
    paper_deq16(paper_stream(c, rr, l, b, hk), c.pm[rr], t, kv, e0, y);
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = x[e] + y[e];
  }
}

// K and V of token j at loop r, dims [e0, e0 + 16), in one pass over its
// chain (each loop's slot and records read once), and, when PREV is set,
// V at loop r-1: the values paper_chain16 gives for (r, K), (r, V), (r-1, V).
template <bool PREV>
__device__ __forceinline__ void paper_token16(const CacheGeo& c, int r, int l, int b, int hk, int j, int e0,
                                              float* kx, float* vx, float* vprev) {
  if (j >= c.Sq) {
    int rr = 1;
    for (int q = 2; q <= r; ++q) {
      if (c.slot[q][(long long)b * c.S + j] < 0) break;
      rr = q;
    }
    // the slot of loop r-1 when the token is active at loop r, else the same one
    const int rp = rr == r && r >= 2 ? r - 1 : rr;
    const uint4* tk = (const uint4*)(paper_tail(c, rr, l, b, hk, j, 0) + e0);
    const uint4* tv = (const uint4*)(paper_tail(c, rr, l, b, hk, j, 1) + e0);
    const uint4 k0 = tk[0], k1 = tk[1], v0 = tv[0], v1 = tv[1];
    const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      kx[e] = __uint_as_float((e & 1) ? (kw[e >> 1] & 0xffff0000u) : (kw[e >> 1] << 16));
      vx[e] = __uint_as_float((e & 1) ? (vw[e >> 1] & 0xffff0000u) : (vw[e >> 1] << 16));
    }
    if (PREV) {
      if (rp == rr) {
#pragma unroll
        for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
      } else {
        const uint4* tp = (const uint4*)(paper_tail(c, rp, l, b, hk, j, 1) + e0);
        const uint4 p0 = tp[0], p1 = tp[1];
        const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int e = 0; e < 16; ++e)
          vprev[e] = __uint_as_float((e & 1) ? (pw[e >> 1] & 0xffff0000u) : (pw[e >> 1] << 16));
      }
    }
    return;
  }
  const uint8_t* st = paper_stream(c, 1, l, b, hk);
  paper_deq16(st, c.pm[1], j, 0, e0, kx);
  paper_deq16(st, c.pm[1], j, 1, e0, vx);
  if (PREV) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
  }
  for (int rr = 2; rr <= r; ++rr) {
    const int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    if (PREV && rr == r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
    }
    const uint8_t* sr = paper_stream(c, rr, l, b, hk);
    float y[16];
    paper_deq16(sr, c.pm[rr], t, 0, e0, y);
#pragma unroll
    for (int e = 0; e < 16; ++e) kx[e] = kx[e] + y[e];
    paper_deq16(sr, c.pm[rr], t, 1, e0, y);
#pragma unroll
    for (int e = 0; e < 16; ++e) vx[e] = vx[e] + y[e];
  }
}

// The 32 input elements [src, src + 32) of one group as floats, read with
// 16-byte loads (src 16-byte aligned).
template <typename T> __device__ inline void load_group16(const T* src, float* x);
template <> __device__ inline void load_group16<uint16_t>(const uint16_t* src, float* x) {
  const uint4* p = (const uint4*)src;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = p[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[8 * i + 2 * k] = __uint_as_float(ws[k] << 16);
      x[8 * i + 2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
    }
  }
}
template <> __device__ inline void load_group16<float>(const float* src, float* x) {
  const float4* p = (const float4*)src;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 w = p[i];
    x[4 * i] = w.x;
    x[4 * i + 1] = w.y;
    x[4 * i + 2] = w.z;
    x[4 * i + 3] = w.w;
  }
}

// Coefficients of the mixed-logit row update O = cu U + ca A (A the softmax
// of loop r over J_i, b its log-sum-exp, M the cached mass, L the loop r-1
// log-sum-exp over J_i): one softmax over the new logits on J_i and the old
// ones elsewhere, cu = 1 / D, ca = M rho / D with rho = e^{b - L} and
// D = 1 - M + M rho, formed without overflow.  Rows with M = 0 or L = -inf
// keep the mass-rescaled coefficients (cu = 1, ca = M).
__device__ inline void mixed_coeffs(float M, float b, float L, float& cu, float& ca) {
  cu = 1.0f;
  ca = M;
  if (!(M > 0.0f) || !(L > -INFINITY)) return;
  const float g = logf(M) + (b - L);  // log(M rho)
  if (g > 0.0f) {
    const float e = expf(-g);
    const float D = (1.0f - M) * e + 1.0f;
    cu = e / D;
    ca = 1.0f / D;
  } else {
    const float e = expf(g);
    const float D = (1.0f - M) + e;
    cu = 1.0f / D;
    ca = e / D;
  }
}

// ---------------------------------------------------------------- reductions
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64).
// Returns the exclusive prefix of `v`; *total receives the block sum.
template <int NT>
__device__ inline int block_exclusive_scan(int v, int* smem /* >= NT/64 + 1 ints */, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) smem[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      int t = smem[w];
      smem[w] = acc;
      acc += t;
    }
    smem[NT / kWave] = acc;
  }
  __syncthreads();
  int res = smem[wid] + x - v;
  *total = smem[NT / kWave];
  __syncthreads();
  return res;
}

}  // namespace fl
