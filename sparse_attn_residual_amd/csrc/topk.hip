// Exact top-K selection per problem (p1 §4.2 and §D.2: the top-K key columns
// ranked by the preceding loop's statistics; ties go to the lower position).
//
// One 1024-thread block per problem.  Keys are mapped to order-preserving
// uint32 values and held in registers, loaded coalesced: thread t holds the
// candidates i*1024 + t.  The K-th largest key T, and how many keys equal
// to T are needed, come from histogram levels over a shrinking key range
// (2048 bins, one LDS atomic per key) that end in an exact radix select
// among the at most 2048 keys of one bin.  The selection is every key above
// T plus the first `need` keys equal to T in candidate order.  Ranks in
// candidate order come from wave ballots and a small per-row table, so the
// output is ascending and the result is unique.  No floating-point atomics;
// deterministic.
#include "launch.hpp"

namespace fl {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

__device__ inline float key_value(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

// Per-row counts of a flag bitmask (bit i = candidate i*1024 + tid): fills
// wtab[w][i] with the flagged count of the waves before w in row i and
// rowoff[i] with the flagged count of the rows before i.  The rank of a
// flagged candidate in candidate order is then
//   rowoff[i] + wtab[w][i] + popcount(ballot_i & lanes below).
// Both prefix sums are parallel: thread (i, w) scans row i over the waves in
// a group of kTopkWaves lanes, then one wave scans the row totals.
template <int ITEMS>
__device__ inline void row_counts(uint64_t bits, int (*wtab)[64], int* rowoff) {
  static_assert(ITEMS * kTopkWaves <= kTopkThreads && kTopkWaves == 16 && ITEMS <= kWave, "scan shape");
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = __ballot((bits >> i) & 1);
    if (lane == 0) wtab[wv][i] = __popcll(m);
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < ITEMS * kTopkWaves) {
    const int i = t / kTopkWaves, w = t % kTopkWaves;
    const int c = wtab[w][i];
    int x = c;
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const int y = __shfl_up(x, o, kTopkWaves);
      if (w >= o) x += y;
    }
    wtab[w][i] = x - c;
    if (w == kTopkWaves - 1) rowoff[i] = x;
  }
  __syncthreads();
  if (t < kWave) {
    const int c = t < ITEMS ? rowoff[t] : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (t >= o) x += y;
    }
    if (t < ITEMS) rowoff[t] = x - c;
  }
  __syncthreads();
}

constexpr int kBins = 2048;     // value bins of the first stage
constexpr int kCandCap = 2048;  // keys of the threshold bin resolved exactly (2 per thread)

struct TopkShared {
  uint32_t hist[kBins];         // value bins; the first 256 also serve as digit histogram
  uint32_t cu[kCandCap];        // keys of the threshold bin
  int wtab[kTopkWaves][64];
  int rowoff[64];
  int wsum[kTopkWaves];
  uint32_t wmin[kTopkWaves], wmax[kTopkWaves];
  uint32_t digit;
  int rem, bstar, cnt, ncand, bad, eqc;
};

// Block-wide inclusive prefix sum of one value per thread.
__device__ inline int block_incl_scan(int x, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[wv] = x;
  __syncthreads();
  for (int w = 0; w < wv; ++w) x += wsum[w];
  __syncthreads();
  return x;
}

// Radix select over NI keys per thread (bit i of vmask: key i valid): the
// K-th largest key T, how many keys equal to T are among the K largest (rem)
// and how many keys equal T (eqc).  8-bit passes with an LDS digit histogram
// and a parallel digit search; the first p0 digits are known to be those of
// prefix0 (shared by every key), so the passes start at digit p0.
template <int NI>
__device__ inline void radix_find(const uint32_t* v, uint64_t vmask, int K, int p0, uint32_t prefix0,
                                  TopkShared& sh, uint32_t& T, int& rem, int& eqc) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  uint32_t mask = p0 > 0 ? 0xFFFFFFFFu << (32 - 8 * p0) : 0u;
  uint32_t prefix = prefix0 & mask;
  rem = K;
  for (int pass = p0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      bool part = ((vmask >> i) & 1) && (v[i] & mask) == prefix;
      const uint32_t dg = (v[i] >> shift) & 255u;
      if (pass == p0) {
        // keys of one problem share their leading digit: aggregate per wave
        for (int it = 0; it < 4; ++it) {
          const uint64_t pm = __ballot(part);
          if (pm == 0) break;
          const int leader = __ffsll((long long)pm) - 1;
          const uint32_t ld = (uint32_t)__builtin_amdgcn_readlane((int)dg, leader);
          const uint64_t same = __ballot(part && dg == ld);
          if (lane == leader) atomicAdd(&sh.hist[ld], (uint32_t)__popcll(same));
          if (dg == ld) part = false;
        }
      }
      if (part) atomicAdd(&sh.hist[dg], 1u);
    }
    __syncthreads();
    // digit of the rem-th largest: inclusive scan of the histogram from the
    // top by the first four waves (tid < 256 covers whole waves)
    int c = 0, x = 0;
    if (tid < 256) {
      c = (int)sh.hist[255 - tid];
      x = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      if (lane == kWave - 1) sh.wsum[wv] = x;
    }
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wv; ++w) x += sh.wsum[w];
      const int excl = x - c;
      if (excl < rem && x >= rem) {
        sh.digit = (uint32_t)(255 - tid);
        sh.rem = rem - excl;
        sh.eqc = c;
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= 255u << shift;
    rem = sh.rem;
    eqc = sh.eqc;
    __syncthreads();
  }
  T = prefix;
}

// Block-wide min and max of one pair per thread.
__device__ inline void block_minmax(uint32_t& mn, uint32_t& mx, TopkShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
  }
  if (lane == 0) {
    sh.wmin[wv] = mn;
    sh.wmax[wv] = mx;
  }
  __syncthreads();
  mn = sh.wmin[0];
  mx = sh.wmax[0];
  for (int w = 1; w < kTopkWaves; ++w) {
    mn = min(mn, sh.wmin[w]);
    mx = max(mx, sh.wmax[w]);
  }
  __syncthreads();
}

// Bin of key u at one level of the search over the key range [lo, hi]
// (order-preserving keys).  The first level uses kBins equal-width value
// bins of the float keys (flo, fscale) when the range is finite; later
// levels take the next 11 bits of u - lo below its leading bit (shift).
// Both are monotone non-decreasing in the key: a key in a higher bin is
// larger than every key in a lower one.
__device__ inline int level_bin(uint32_t u, uint32_t lo, bool by_value, float flo, float fscale, int shift) {
  if (by_value) {
    const int bn = (int)((key_value(u) - flo) * fscale);
    return bn < kBins - 1 ? bn : kBins - 1;
  }
  return (int)((u - lo) >> shift);
}

// One 1024-thread block per problem.  The threshold (the K-th largest key T
// and how many keys equal to T are among the K largest) is found by
// histogram levels over a shrinking key range: each level bins the keys in
// the range into kBins bins (one LDS atomic per key) and finds the bin
// holding the rank sought.  If that bin holds at most kCandCap keys they are
// gathered into LDS and a radix select among them gives T exactly;
// otherwise the range shrinks to that bin's keys (at most four levels: the
// first by value, then 11 bits of the order-preserving key at a time), and
// a range of one value is T itself.  The output stage takes every key above
// T and the first keys equal to T in candidate order, ranked with wave
// ballots: ascending, unique.  Keys must not be NaN.
template <int ITEMS, bool CAND>
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float* __restrict__ keys, long long key_stride,
                                                       const int32_t* cand, long long cand_stride, int n, int K,
                                                       int32_t* sel_out, long long sel_stride, float* keys_out,
                                                       long long keys_out_stride) {
  static_assert(ITEMS <= 32, "at most 32768 keys per problem");
  __shared__ TopkShared sh;
  const int p = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const float* kp = keys + (long long)p * key_stride;

  // Loads are unconditional (clamped index) so that all of them are issued
  // before the first is waited for; out-of-range items are masked after.
  // u = 0 marks an item past n (no finite or infinite key maps to 0).
  // Candidate positions wait in LDS (dynamic, ITEMS * 1024 ints) for the
  // output stage, which keeps them out of registers.
  extern __shared__ int32_t sh_idx[];
  uint32_t u[ITEMS];
  {
    float raw[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int e = min(i * kTopkThreads + tid, n - 1);
      raw[i] = kp[e];
      if (CAND) sh_idx[i * kTopkThreads + tid] = cand[(long long)p * cand_stride + e];
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) u[i] = i * kTopkThreads + tid < n ? order_key(raw[i]) : 0u;
  }
  __syncthreads();  // every read of keys/cand precedes any write (in-place use)

  // ---- range of the keys
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    lo = min(lo, u[i] ? u[i] : 0xFFFFFFFFu);
    hi = max(hi, u[i]);
  }
  block_minmax(lo, hi, sh);

  uint32_t T = lo;
  int rem = K;       // rank sought among the keys in [lo, hi]
  int eqc = -1;      // keys equal to T once known (-1: rank them)
  int nrange = n;    // keys in [lo, hi]
  for (int level = 0; level < 5; ++level) {
    if (lo == hi) {  // every key left is T
      T = lo;
      eqc = nrange;
      break;
    }
    const float flo = key_value(lo), fhi = key_value(hi);
    const float fscale = (float)kBins / (fhi - flo);
    const bool by_value = level == 0 && fscale < INFINITY && fscale > 0.0f;
    const int shift = max(0, 32 - __clz((int)(hi - lo)) - 11);
    if (tid == 0) sh.ncand = 0;
    // keys in range: u - lo <= span (lo >= 1 excludes u = 0)
    const uint32_t span = hi - lo;
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
      if (u[i] - lo <= span) atomicAdd(&sh.hist[level_bin(u[i], lo, by_value, flo, fscale, shift)], 1u);
    __syncthreads();
    // bins from the top: thread t covers bins kBins-1-2t and kBins-2-2t
    const int b0 = kBins - 1 - 2 * tid, b1 = b0 - 1;
    const int c0 = (int)sh.hist[b0], c1 = (int)sh.hist[b1];
    const int incl = block_incl_scan(c0 + c1, sh.wsum);
    const int excl = incl - c0 - c1;  // keys in bins above b0
    if (excl < rem && excl + c0 >= rem) {
      sh.bstar = b0;
      sh.rem = rem - excl;
      sh.cnt = c0;
    } else if (excl + c0 < rem && incl >= rem) {
      sh.bstar = b1;
      sh.rem = rem - excl - c0;
      sh.cnt = c1;
    }
    __syncthreads();
    const int bs = sh.bstar, cnt = sh.cnt;
    rem = sh.rem;
    // recompute the bins below rather than keep all of them live across the
    // scan (the copies hide the equality from the compiler)
    uint32_t lo2 = lo;
    float flo2 = flo, fscale2 = fscale;
    asm volatile("" : "+v"(lo2), "+v"(flo2), "+v"(fscale2));
    if (cnt <= kCandCap) {
      // ---- the bin's keys into LDS, exact select among them
#pragma unroll
      for (int i = 0; i < ITEMS; ++i)
        if (u[i] - lo2 <= span && level_bin(u[i], lo2, by_value, flo2, fscale2, shift) == bs)
          sh.cu[atomicAdd(&sh.ncand, 1)] = u[i];
      __syncthreads();
      const int nc = sh.ncand;
      const uint32_t cv[2] = {tid < nc ? sh.cu[tid] : 0u, tid + kTopkThreads < nc ? sh.cu[tid + kTopkThreads] : 0u};
      const uint64_t cm = (tid < nc ? 1ull : 0ull) | (tid + kTopkThreads < nc ? 2ull : 0ull);
      const int rb = rem;
      __syncthreads();
      radix_find<2>(cv, cm, rb, 0, 0u, sh, T, rem, eqc);
      break;
    }
    nrange = cnt;
    // ---- narrow the range to the bin's keys
    uint32_t nlo = 0xFFFFFFFFu, nhi = 0u;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      if (u[i] - lo2 <= span && level_bin(u[i], lo2, by_value, flo2, fscale2, shift) == bs) {
        nlo = min(nlo, u[i]);
        nhi = max(nhi, u[i]);
      }
    }
    block_minmax(nlo, nhi, sh);
    lo = nlo;
    hi = nhi;
  }

  // keys equal to T: the first `rem` of them in candidate order are taken
  uint64_t eq = 0, take = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {  // T >= 1: items past n never match
    if (u[i] == T) eq |= 1ull << i;
    if (u[i] > T) take |= 1ull << i;
  }
  if (eqc == rem) {
    take |= eq;  // every key equal to T is taken: no ranking among them
  } else {
    row_counts<ITEMS>(eq, sh.wtab, sh.rowoff);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const uint64_t m = __ballot((eq >> i) & 1);
      const int rk = sh.rowoff[i] + sh.wtab[wv][i] + __popcll(m & below);
      if (((eq >> i) & 1) && rk < rem) take |= 1ull << i;
    }
    __syncthreads();
  }
  row_counts<ITEMS>(take, sh.wtab, sh.rowoff);
  int32_t* so = sel_out + (long long)p * sel_stride;
  float* ko = keys_out ? keys_out + (long long)p * keys_out_stride : nullptr;
  // candidate positions are recomputed here from a copy of tid: otherwise the
  // compiler keeps all ITEMS of them from the loads and spills them
  int tid2 = tid;
  asm volatile("" : "+v"(tid2));
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const uint64_t m = __ballot((take >> i) & 1);
    const int rk = sh.rowoff[i] + sh.wtab[wv][i] + __popcll(m & below);
    if (((take >> i) & 1) && rk < K) {
      so[rk] = CAND ? sh_idx[i * kTopkThreads + tid2] : i * kTopkThreads + tid2;
      if (ko) ko[rk] = key_value(u[i]);
    }
  }
}

// Top-K given the first histogram level (a decode step's loop 2: loop 1
// leaves each head's histogram of its logits by the top 11 order-key bits in
// the first kBins entries of the head's selection row).  Thread t holds the
// keys of positions 32t .. 32t+31, so positions ascend with (thread, item)
// and every rank in position order is one block-wide prefix sum plus a
// popcount inside the thread.  The histogram gives the threshold bin b*;
// keys above it are taken, and the keys in it (their number is the bin's
// count, at most kCandCap here) are compacted into LDS in position order,
// where a radix select over their low 21 bits finds T and how many keys equal
// to T are needed; equal keys are taken in position order.  A bin of more than
// kCandCap keys takes a radix select over all the keys instead.  Output:
// the selected positions ascending and, if keys_out is set, their keys in the
// same order (keys and keys_out, histogram and sel_out may be the same rows:
// every read precedes the first barrier, every write follows it).
__global__ __launch_bounds__(kTopkThreads) void k_topk_hist(const float* keys, long long key_stride, int n, int K,
                                                          int32_t* sel_out, long long sel_stride, float* keys_out,
                                                          long long keys_out_stride) {
  constexpr int NI = 32;
  static_assert(kBins == kHistBins && NI * kTopkThreads == 32768, "one problem of at most 32768 keys");
  __shared__ TopkShared sh;
  __shared__ uint8_t ctake[kCandCap];
  const int p = blockIdx.x;
  const int tid = threadIdx.x;
  const float* kp = keys + (long long)p * key_stride;
  const int32_t* hrow = sel_out + (long long)p * sel_stride;
  const int pos0 = tid * NI;
  if (tid == 0) {  // (a histogram without the K-th key leaves these: every key is then a candidate)
    sh.bstar = 0;
    sh.rem = K;
    sh.cnt = n;
  }
  // the given bins, from the top: thread t has kBins-1-2t and kBins-2-2t
  const int c0 = hrow[kBins - 1 - 2 * tid], c1 = hrow[kBins - 2 - 2 * tid];
  uint32_t u[NI];  // order keys; 0 past n (no key maps to 0)
  if (((key_stride & 3) == 0) && ((reinterpret_cast<uintptr_t>(keys) & 15) == 0) && pos0 + NI <= n) {
    const float4* k4 = (const float4*)(kp + pos0);
#pragma unroll
    for (int k = 0; k < NI / 4; ++k) {
      const float4 v = k4[k];
      u[4 * k] = order_key(v.x);
      u[4 * k + 1] = order_key(v.y);
      u[4 * k + 2] = order_key(v.z);
      u[4 * k + 3] = order_key(v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float v = kp[min(pos0 + i, n - 1)];
      u[i] = pos0 + i < n ? order_key(v) : 0u;
    }
  }
  // threshold bin: the scan's first barrier follows every read of the rows
  const int incl = block_incl_scan(c0 + c1, sh.wsum);
  const int excl = incl - c0 - c1;
  if (excl < K && excl + c0 >= K) {
    sh.bstar = kBins - 1 - 2 * tid;
    sh.rem = K - excl;
    sh.cnt = c0;
  } else if (excl + c0 < K && incl >= K) {
    sh.bstar = kBins - 2 - 2 * tid;
    sh.rem = K - excl - c0;
    sh.cnt = c1;
  }
  __syncthreads();
  const uint32_t bs = (uint32_t)sh.bstar;
  int rem = sh.rem;
  uint32_t above = 0, cand = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t bn = u[i] >> (32 - kHistBits);
    if (u[i] != 0u && bn > bs) above |= 1u << i;
    if (u[i] != 0u && bn == bs) cand |= 1u << i;
  }
  const int nct = __popc(cand);
  const int cincl = block_incl_scan(nct, sh.wsum);
  if (tid == kTopkThreads - 1) sh.ncand = cincl;
  __syncthreads();
  const int ncand = sh.ncand;
  uint32_t T;
  int eqc;
  uint32_t take = above;
  if (ncand <= kCandCap) {
    // ---- the bin's keys into LDS in position order, exact select among them
    int slot = cincl - nct;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if ((cand >> i) & 1) sh.cu[slot++] = u[i];
    __syncthreads();
    const uint32_t cv[2] = {tid < ncand ? sh.cu[tid] : 0u, tid + kTopkThreads < ncand ? sh.cu[tid + kTopkThreads] : 0u};
    const uint64_t cm = (tid < ncand ? 1ull : 0ull) | (tid + kTopkThreads < ncand ? 2ull : 0ull);
    const int rb = rem;
    // the bin's keys share their top kHistBits bits: the passes start at the second digit
    radix_find<2>(cv, cm, rb, 1, bs << (32 - kHistBits), sh, T, rem, eqc);
    // which slots are taken: keys above T, and the first rem keys equal to T
    const int s0 = 2 * tid, s1 = 2 * tid + 1;
    const uint32_t k0 = s0 < ncand ? sh.cu[s0] : 0u, k1 = s1 < ncand ? sh.cu[s1] : 0u;
    const int e0 = k0 == T, e1 = k1 == T;   // k = 0 (no slot) never equals T >= 1
    int ee = 0;
    if (eqc != rem) ee = block_incl_scan(e0 + e1, sh.wsum) - e0 - e1;
    if (s0 < ncand) ctake[s0] = k0 > T || (e0 && (eqc == rem || ee < rem));
    if (s1 < ncand) ctake[s1] = k1 > T || (e1 && (eqc == rem || ee + e0 < rem));
    __syncthreads();
    slot = cincl - nct;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if ((cand >> i) & 1) {
        if (ctake[slot]) take |= 1u << i;
        ++slot;
      }
  } else {
    // ---- a crowded bin: radix select over every key
    uint64_t vm = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (u[i] != 0u) vm |= 1ull << i;
    radix_find<NI>(u, vm, K, 0, 0u, sh, T, rem, eqc);
    uint32_t eq = 0;
    take = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (u[i] > T) take |= 1u << i;
      if (u[i] == T) eq |= 1u << i;
    }
    if (eqc == rem) {
      take |= eq;
    } else {
      const int ne = __popc(eq);
      int rk = block_incl_scan(ne, sh.wsum) - ne;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if ((eq >> i) & 1) {
          if (rk < rem) take |= 1u << i;
          ++rk;
        }
    }
  }
  // ---- output in position order
  const int ntk = __popc(take);
  int rk = block_incl_scan(ntk, sh.wsum) - ntk;
  int32_t* so = sel_out + (long long)p * sel_stride;
  float* ko = keys_out ? keys_out + (long long)p * keys_out_stride : nullptr;
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if ((take >> i) & 1) {
      if (rk < K) {
        so[rk] = pos0 + i;
        if (ko) ko[rk] = key_value(u[i]);
      }
      ++rk;
    }
}

__global__ void k_copy_sel(const int32_t* __restrict__ cand, int P, int K, int32_t* __restrict__ sel,
                           long long sel_stride) {
  long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)P * K) return;
  const long long p = gid / K, i = gid - p * K;
  sel[p * sel_stride + i] = cand ? cand[gid] : (int32_t)i;
}

hipError_t launch_copy_sel(const int32_t* cand, int P, int K, int32_t* sel, hipStream_t st, long long sel_stride) {
  long long n = (long long)P * K;
  FL_LAUNCH(k_copy_sel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cand, P, K, sel,
                     sel_stride > 0 ? sel_stride : K);
  return hipGetLastError();
}

hipError_t launch_topk(const float* keys, long long key_stride, const int32_t* cand, long long cand_stride, int P,
                       int n, int K, int32_t* sel_out, long long sel_stride, float* keys_out,
                       long long keys_out_stride, hipStream_t st, bool given_hist) {
  if (n < 1 || K < 1 || K > n) return hipErrorInvalidValue;
  if (given_hist && (cand || n > 32768 || sel_stride < kHistBins)) return hipErrorInvalidValue;
  const int items = (n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(P), block(kTopkThreads);
  if (given_hist) {
    FL_LAUNCH(k_topk_hist, grid, block, 0, st, keys, key_stride, n, K, sel_out, sel_stride, keys_out,
              keys_out_stride);
    return hipGetLastError();
  }
#define FL_TOPK(IT)                                                                                             \
  do {                                                                                                          \
    if (cand) {                                                                                                 \
      const int lds = (IT) * kTopkThreads * (int)sizeof(int32_t);                                               \
      static const hipError_t attr = hipFuncSetAttribute((const void*)k_topk<IT, true>,                  \
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);      \
      if (attr != hipSuccess) return attr;                                                                      \
      FL_LAUNCH((k_topk<IT, true>), grid, block, lds, st, keys, key_stride, cand, cand_stride, n, K,     \
                sel_out, sel_stride, keys_out, keys_out_stride);                                                \
    } else {                                                                                                    \
      FL_LAUNCH((k_topk<IT, false>), grid, block, 0, st, keys, key_stride, cand, cand_stride, n, K,      \
                sel_out, sel_stride, keys_out, keys_out_stride);                                                \
    }                                                                                                           \
  } while (0)
  if (items <= 1) FL_TOPK(1);
  else if (items <= 4) FL_TOPK(4);
  else if (items <= 8) FL_TOPK(8);
  else if (items <= 16) FL_TOPK(16);
  else if (items <= 32) FL_TOPK(32);
  else return hipErrorInvalidValue;
#undef FL_TOPK
  return hipGetLastError();
}

}  // namespace fl
