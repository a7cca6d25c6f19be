// Exact top-K selection per problem (p1 §4.2 and §D.2: the top-K key columns
// ranked by the preceding loop's statistics; ties go to the lower position).
//
// One 1024-thread block per problem.  Keys are mapped to order-preserving
// uint32 values and held in registers (ITEMS consecutive candidates per
// thread, so register order is candidate order).  Four 8-bit radix passes
// find the K-th largest key T and how many keys equal to T are needed; the
// selection is then every key above T plus the first `need` keys equal to T
// in candidate order.  Two block scans give each selected entry its output
// position, so the output is ascending and the result is unique.  No
// floating-point atomics; the result is deterministic.
#include "launch.hpp"

namespace fl {

constexpr int kTopkThreads = 1024;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ keys, long long key_stride,
                                                       const int32_t* cand, long long cand_stride, int n, int K,
                                                       int32_t* sel_out, long long sel_stride, float* keys_out,
                                                       long long keys_out_stride) {
  __shared__ uint32_t hist[256];
  __shared__ int scan_smem[kTopkThreads / kWave + 1];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_rem;
  const int p = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int t0 = tid * ITEMS;
  const float* kp = keys + (long long)p * key_stride;
  const int32_t* cp = cand ? cand + (long long)p * cand_stride : nullptr;

  uint32_t u[ITEMS];
  int32_t idx[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int t = t0 + i;
    u[i] = t < n ? order_key(kp[t]) : 0u;
    idx[i] = t < n ? (cp ? cp[t] : t) : 0;
  }
  __syncthreads();  // every read of keys/cand precedes any write (in-place use)

  uint32_t prefix = 0, mask = 0;
  int rem = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int t = t0 + i;
      bool part = t < n && (u[i] & mask) == prefix;
      const uint32_t dg = (u[i] >> shift) & 255u;
      if (pass == 0) {
        // keys of one problem share their leading digit: aggregate per wave
        for (int it = 0; it < 4; ++it) {
          uint64_t pm = __ballot(part);
          if (pm == 0) break;
          const int leader = __ffsll((long long)pm) - 1;
          const uint32_t ld = __shfl(dg, leader, kWave);
          const uint64_t same = __ballot(part && dg == ld);
          if (lane == leader) atomicAdd(&hist[ld], (uint32_t)__popcll(same));
          if (dg == ld) part = false;
        }
      }
      if (part) atomicAdd(&hist[dg], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      uint32_t dsel = 0;
      int r2 = rem;
      for (int dd = 255; dd >= 0; --dd) {
        const int hcount = (int)hist[dd];
        if (acc + hcount >= rem) {
          dsel = (uint32_t)dd;
          r2 = rem - acc;
          break;
        }
        acc += hcount;
      }
      sh_digit = dsel;
      sh_rem = r2;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  // rank of keys equal to T in candidate order
  int eq = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) eq += (t0 + i < n && u[i] == T);
  int tot;
  int eq_before = block_exclusive_scan<kTopkThreads>(eq, scan_smem, &tot);
  int take = 0;
  {
    int e = eq_before;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const bool valid = t0 + i < n;
      if (valid && u[i] > T) ++take;
      else if (valid && u[i] == T) {
        if (e < rem) ++take;
        ++e;
      }
    }
  }
  int pos = block_exclusive_scan<kTopkThreads>(take, scan_smem, &tot);
  int32_t* so = sel_out + (long long)p * sel_stride;
  float* ko = keys_out ? keys_out + (long long)p * keys_out_stride : nullptr;
  int e = eq_before;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool valid = t0 + i < n;
    bool tk = false;
    if (valid && u[i] > T) tk = true;
    else if (valid && u[i] == T) {
      tk = e < rem;
      ++e;
    }
    if (tk && pos < K) {
      so[pos] = idx[i];
      if (ko) ko[pos] = key_value(u[i]);
      ++pos;
    }
  }
}

__global__ void k_copy_sel(const int32_t* __restrict__ cand, int P, int K, int32_t* __restrict__ sel) {
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)P * K) return;
  sel[gid] = cand ? cand[gid] : (int32_t)(gid % K);
}

hipError_t launch_copy_sel(const int32_t* cand, int P, int K, int32_t* sel, hipStream_t st) {
  long long n = (long long)P * K;
  hipLaunchKernelGGL(k_copy_sel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cand, P, K, sel);
  return hipGetLastError();
}

hipError_t launch_topk(const float* keys, long long key_stride, const int32_t* cand, long long cand_stride, int P,
                       int n, int K, int32_t* sel_out, long long sel_stride, float* keys_out,
                       long long keys_out_stride, hipStream_t st) {
  const int items = (n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(P), block(kTopkThreads);
#define FL_TOPK(IT)                                                                                             \
  hipLaunchKernelGGL(k_topk<IT>, grid, block, 0, st, keys, key_stride, cand, cand_stride, n, K, sel_out,       \
                     sel_stride, keys_out, keys_out_stride)
  if (items <= 1) FL_TOPK(1);
  else if (items <= 4) FL_TOPK(4);
  else if (items <= 8) FL_TOPK(8);
  else if (items <= 16) FL_TOPK(16);
  else if (items <= 32) FL_TOPK(32);
  else if (items <= 64) FL_TOPK(64);
  else return hipErrorInvalidValue;
#undef FL_TOPK
  return hipGetLastError();
}

}  // namespace fl
