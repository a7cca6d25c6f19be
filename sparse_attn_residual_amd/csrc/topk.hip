// Exact top-K selection per problem (p1 §4.2 and §D.2: the top-K key columns
// ranked by the preceding loop's statistics; ties go to the lower position).
//
// One 1024-thread block per problem.  Keys are mapped to order-preserving
// uint32 values and held in registers, loaded coalesced: thread t holds the
// candidates i*1024 + t.  Four 8-bit radix passes (LDS histogram, parallel
// digit search) find the K-th largest key T and how many keys equal to T are
// needed; the selection is every key above T plus the first `need` keys equal
// to T in candidate order.  Ranks in candidate order come from wave ballots
// and a small per-row table, so the output is ascending and the result is
// unique.  No floating-point atomics; deterministic.
#include "launch.hpp"

namespace fl {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// Per-row counts of a flag bitmask (bit i = candidate i*1024 + tid): fills
// wtab[w][i] with the flagged count of the waves before w in row i and
// rowoff[i] with the flagged count of the rows before i.  The rank of a
// flagged candidate in candidate order is then
//   rowoff[i] + wtab[w][i] + popcount(ballot_i & lanes below).
template <int ITEMS>
__device__ inline void row_counts(uint64_t bits, int (*wtab)[ITEMS], int* rowoff) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = __ballot((bits >> i) & 1);
    if (lane == 0) wtab[wv][i] = __popcll(m);
  }
  __syncthreads();
  if (threadIdx.x < ITEMS) {
    const int i = threadIdx.x;
    int acc = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int t = wtab[w][i];
      wtab[w][i] = acc;
      acc += t;
    }
    rowoff[i] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < ITEMS; ++i) {
      const int t = rowoff[i];
      rowoff[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
}

template <int ITEMS, bool CAND>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ keys, long long key_stride,
                                                       const int32_t* cand, long long cand_stride, int n, int K,
                                                       int32_t* sel_out, long long sel_stride, float* keys_out,
                                                       long long keys_out_stride) {
  static_assert(ITEMS <= 64, "bitmasks hold 64 rows");
  __shared__ uint32_t hist[256];
  __shared__ int wtab[kTopkWaves][ITEMS];
  __shared__ int rowoff[ITEMS];
  __shared__ int wsum[4];
  __shared__ uint32_t sh_digit;
  __shared__ int sh_rem;
  const int p = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const float* kp = keys + (long long)p * key_stride;

  // Loads are unconditional (clamped index) so that all of them are issued
  // before the first is waited for; out-of-range items are masked after.
  uint32_t u[ITEMS];
  int32_t idx[CAND ? ITEMS : 1];
  float raw[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int e = min(i * kTopkThreads + tid, n - 1);
    raw[i] = kp[e];
    if (CAND) idx[i] = cand[(long long)p * cand_stride + e];
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) u[i] = i * kTopkThreads + tid < n ? order_key(raw[i]) : 0u;
  __syncthreads();  // every read of keys/cand precedes any write (in-place use)

  uint32_t prefix = 0, mask = 0;
  int rem = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int e = i * kTopkThreads + tid;
      bool part = e < n && (u[i] & mask) == prefix;
      const uint32_t dg = (u[i] >> shift) & 255u;
      if (pass == 0) {
        // keys of one problem share their leading digit: aggregate per wave
        for (int it = 0; it < 4; ++it) {
          const uint64_t pm = __ballot(part);
          if (pm == 0) break;
          const int leader = __ffsll((long long)pm) - 1;
          const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)dg, leader);
          const uint64_t same = __ballot(part && dg == ld);
          if (lane == leader) atomicAdd(&hist[ld], (uint32_t)__popcll(same));
          if (dg == ld) part = false;
        }
      }
      if (part) atomicAdd(&hist[dg], 1u);
    }
    __syncthreads();
    // digit of the rem-th largest: inclusive scan of the histogram from the
    // top by the first four waves (tid < 256 covers whole waves)
    int v = 0, x = 0;
    if (tid < 256) {
      v = (int)hist[255 - tid];
      x = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      if (lane == kWave - 1) wsum[wv] = x;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wv; ++w) x += wsum[w];
      const int excl = x - v;
      if (excl < rem && x >= rem) {
        sh_digit = (uint32_t)(255 - tid);
        sh_rem = rem - excl;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;
  // keys equal to T: the first `rem` of them in candidate order are taken
  uint64_t eq = 0, take = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const bool valid = i * kTopkThreads + tid < n;
    if (valid && u[i] == T) eq |= 1ull << i;
    if (valid && u[i] > T) take |= 1ull << i;
  }
  row_counts<ITEMS>(eq, wtab, rowoff);
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = __ballot((eq >> i) & 1);
    const int rk = rowoff[i] + wtab[wv][i] + __popcll(m & below);
    if (((eq >> i) & 1) && rk < rem) take |= 1ull << i;
  }
  __syncthreads();
  row_counts<ITEMS>(take, wtab, rowoff);
  int32_t* so = sel_out + (long long)p * sel_stride;
  float* ko = keys_out ? keys_out + (long long)p * keys_out_stride : nullptr;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = __ballot((take >> i) & 1);
    const int rk = rowoff[i] + wtab[wv][i] + __popcll(m & below);
    if (((take >> i) & 1) && rk < K) {
      so[rk] = CAND ? idx[i] : i * kTopkThreads + tid;
      if (ko) ko[rk] = key_value(u[i]);
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
  if (n < 1 || K < 1 || K > n) return hipErrorInvalidValue;
  const int items = (n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(P), block(kTopkThreads);
#define FL_TOPK(IT)                                                                                             \
  do {                                                                                                          \
    if (cand)                                                                                                   \
      hipLaunchKernelGGL((k_topk<IT, true>), grid, block, 0, st, keys, key_stride, cand, cand_stride, n, K,     \
                         sel_out, sel_stride, keys_out, keys_out_stride);                                       \
    else                                                                                                        \
      hipLaunchKernelGGL((k_topk<IT, false>), grid, block, 0, st, keys, key_stride, cand, cand_stride, n, K,    \
                         sel_out, sel_stride, keys_out, keys_out_stride);                                       \
  } while (0)
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
