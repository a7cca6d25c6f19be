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

// Inclusive prefix sum inside each 16-lane row of a wavefront by DPP moves:
// shifts by 1, 2, 4 and 8 lanes.  Every lane of the row must be active.
__device__ inline int row_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  return x;
}

// Inclusive prefix sum over a wavefront by DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane
// of rows 0 and 2 added into rows 1 and 3, and the last lane of row 1 into
// rows 2 and 3.  Every lane of the wave must be active.
__device__ inline int wave_incl_scan(int x) {
  x = row_incl_scan(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// Per-row counts of a flag bitmask (bit i = candidate i*1024 + tid): fills
// wtab[w][i] with the flagged count of the waves before w in row i and
// rowoff[i] with the flagged count of the rows before i.  The rank of a
// flagged candidate in candidate order is then
//   rowoff[i] + wtab[w][i] + popcount(ballot_i & lanes below).
// Both prefix sums are parallel: thread (i, w) scans row i over the waves in
// one 16-lane row of a wavefront, then one wave scans the row totals.
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
    const int x = row_incl_scan(c);  // the 16 waves' counts of item i: one 16-lane row
    wtab[w][i] = x - c;
    if (w == kTopkWaves - 1) rowoff[i] = x;
  }
  __syncthreads();
  if (t < kWave) {
    const int c = t < ITEMS ? rowoff[t] : 0;
    const int x = wave_incl_scan(c);
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

// Block-wide inclusive prefix sum of one value per thread.  CLOSE = false
// leaves out the closing barrier: the caller has another barrier between
// this scan's reads of wsum and the next scan's write.
template <bool CLOSE = true>
__device__ inline int block_incl_scan(int x, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  x = wave_incl_scan(x);
  if (lane == kWave - 1) wsum[wv] = x;
  lds_barrier();
  for (int w = 0; w < wv; ++w) x += wsum[w];
  if (CLOSE) lds_barrier();
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
      x = wave_incl_scan(c);
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
    if (((take >> i) & 1) && rk >= 0 && rk < K) {
      so[rk] = CAND ? sh_idx[i * kTopkThreads + tid2] : i * kTopkThreads + tid2;
      if (ko) ko[rk] = key_value(u[i]);
    }
  }
}

// Top-K given the first histogram level: each problem's histogram of its
// keys by the top 11 order-key bits (a decode step's loop 2: loop 1 leaves it
// in the first kBins entries of the head's selection row; a prefill
// selection: the column-mass pass counts each mass it writes).  Thread t
// holds the keys of positions 32t .. 32t+31, so positions ascend with
// (thread, item) and every rank in position order is one block-wide prefix
// sum plus a popcount inside the thread.  The histogram gives the bin of the
// K-th largest key and its rank there; two more histogram levels over the
// next 11 and 10 bits of the keys still in the bin (LDS atomics of those keys
// only, re-read from the stage; the second level is skipped when the first
// leaves a single key) give the K-th largest key T itself and how many keys
// equal to T are needed.  FULL: n == 32768, every thread's 32 positions lie
// inside the problem (no per-key range masks).
// Every key above T is taken, and the keys equal to T in position order.
// Output: the selected positions ascending and, if keys_out is set, their
// keys in the same order (keys and keys_out, histogram and sel_out may be the
// same rows: a problem's reads all precede the barrier after which its
// writes begin).
// Persistent: one block per CU walks problems blockIdx.x, + gridDim.x, ...;
// the next problem's keys are copied into LDS (direct global->LDS loads, 256
// keys per load instruction: the fewer copy instructions, the sooner the
// output stores behind them leave) while this one is worked on from
// registers (from after this problem's histogram levels on).  Each thread
// reads its 32-key run in 16-byte groups starting at group t mod 8, so the
// eight runs of a 1 KB chunk are read from distinct banks (and, with 16
// bytes of padding after every chunk, those of two neighbouring chunks); its
// registers keep that order and masks rotate between register and position
// order.
// Barriers inside a problem exchange LDS data only and leave that copy in
// flight; the wait for it comes at the top of the next problem.
constexpr int kTkRun = 32;                       // keys per thread
constexpr int kTkKeys = kTkRun * kTopkThreads;   // 32768
constexpr int kTkChunk = 256 + 4;                // staged words per 256 keys (16 bytes of padding)
constexpr int kTkStage = kTkKeys / 256 * kTkChunk;  // staged words
constexpr int kTopkHistBlocks = 256;             // MI355X: one per CU

template <bool FULL>
__global__ __launch_bounds__(kTopkThreads) void k_topk_hist(const float* keys, long long key_stride, int P, int n,
                                                          int K, const int32_t* hist, long long hist_stride,
                                                          int32_t* sel_out, long long sel_stride, float* keys_out,
                                                          long long keys_out_stride) {
  constexpr int NI = kTkRun;
  static_assert(kBins == kHistBins, "the given histogram is the first level");
  __shared__ TopkShared sh;
  __shared__ __align__(16) float stage[kTkStage];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int pos0 = tid * NI;

  // copy of problem q's keys into the stage (positions in order): FULL, 16
  // bytes per lane, wave w moving the 256-key chunks w, w + 16, ...;
  // otherwise 4 bytes per lane (64-key chunks), so that every key past n
  // reads as 0 (the resource ends at n)
  auto stage_keys = [&](int q) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(keys + (long long)q * key_stride), (short)0, n * 4, 0x00020000);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // offsets made here, not kept across problems
    if (FULL) {
      for (int ch = wv; ch < kTkKeys / 256; ch += kTopkWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(stage + ch * kTkChunk), 16, ch * 1024 + ln * 16, 0, 0, 0);
    } else {
      for (int ch = wv; ch < kTkKeys / 64; ch += kTopkWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(stage + (ch >> 2) * kTkChunk + (ch & 3) * 64), 4,
            ch * 256 + ln * 4, 0, 0, 0);
    }
  };
  // Thread t reads its 32 keys as eight 16-byte groups starting at group
  // t mod 8 (so the eight threads of one 1 KB chunk hit distinct banks) and
  // keeps them in that order: register j holds position pos0 + nat(j), with
  // nat(j) = (j + 4 (t mod 8)) mod 32.  Bit j of a register-order mask is
  // bit nat(j) of the position-order mask: rotl by rot, and back by rotr.
  const int rot = 4 * (tid & 7);
  auto to_pos = [&](uint32_t m) { return rot ? (m << rot) | (m >> (32 - rot)) : m; };
  auto to_reg = [&](uint32_t m) { return rot ? (m >> rot) | (m << (32 - rot)) : m; };
  int p = blockIdx.x;
  if (p >= P) return;
  stage_keys(p);
  int c0, c1;  // the given bins, from the top: thread t has kBins-1-2t and kBins-2-2t
  {
    const int32_t* hrow = hist + (long long)p * hist_stride;
    c0 = hrow[kBins - 1 - 2 * tid];
    c1 = hrow[kBins - 2 - 2 * tid];
  }
  for (; p < P; p += gridDim.x) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies and loads have landed
    __syncthreads();
    // the thread's keys (register order) and which of them lie inside the
    // problem
    const float* run = stage + (pos0 >> 8) * kTkChunk + (pos0 & 255);
    const int lim = n - pos0;
    const uint32_t valid =
        FULL || lim >= NI ? 0xffffffffu : to_reg(lim <= 0 ? 0u : (1u << lim) - 1u);
    uint32_t u[NI];  // order keys; 0 past n (no key maps to 0)
#pragma unroll
    for (int i = 0; i < NI / 4; ++i) {
      const float4 kv = *(const float4*)(run + ((4 * i + rot) & (NI - 1)));
      const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = order_key(kk[e]);  // the stage holds 0.0f past n: read, then dropped
        u[4 * i + e] = FULL || ((valid >> (4 * i + e)) & 1u) ? k : 0u;
      }
    }
    if (tid == 0) {  // (a histogram without the K-th key leaves these: every key is then in the bin)
      sh.bstar = 0;
      sh.rem = K;
      sh.cnt = n;
    }
    // threshold bin (the scan's barrier also ends every read of the stage;
    // the barrier below closes the scan)
    {
      const int incl = block_incl_scan<false>(c0 + c1, sh.wsum);
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
      lds_barrier();
    }
    // the threshold's leading bits: the keys with u >> shift == prefix hold it
    uint32_t prefix = (uint32_t)sh.bstar;
    int shift = 32 - kHistBits;
    int rem = sh.rem, cnt = sh.cnt;
    // The bin is split by the next 11, then 10 bits of its keys (marked in
    // the registers, counted by LDS atomics of the keys still in the bin
    // only), down to one value: the threshold T, with cnt keys equal to it.
    // A sub-bin left with a single key ends the search there.
    auto level = [&](const int nb) {
      for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
      // the thread's keys still in the bin (few: most threads have none),
      // marked without branches, then counted one set bit at a time with the
      // key read again from the stage (it holds this problem's keys until
      // the levels are done; register j is position nat(j)); each key is
      // also left in its sub-bin's slot of cu, which keeps the key itself
      // when the sub-bin has only that one
      uint32_t mm = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) mm |= (u[i] >> shift) == prefix ? 1u << i : 0u;
      if (!FULL) mm &= valid;
      lds_barrier();
      while (mm) {
        const int i = __builtin_ctz(mm);
        mm &= mm - 1u;
        const uint32_t k = order_key(run[(i + rot) & (NI - 1)]);
        const uint32_t sb = (k >> (shift - nb)) & ((1u << nb) - 1u);
        atomicAdd(&sh.hist[sb], 1u);
        sh.cu[sb] = k;
      }
      lds_barrier();
      const int b0 = kBins - 1 - 2 * tid, b1 = b0 - 1;
      const int h0 = (int)sh.hist[b0], h1 = (int)sh.hist[b1];
      const int incl = block_incl_scan<false>(h0 + h1, sh.wsum);  // closed by the barrier below
      const int excl = incl - h0 - h1;
      if (excl < rem && excl + h0 >= rem) {
        sh.bstar = b0;
        sh.rem = rem - excl;
        sh.cnt = h0;
      } else if (excl + h0 < rem && incl >= rem) {
        sh.bstar = b1;
        sh.rem = rem - excl - h0;
        sh.cnt = h1;
      }
      lds_barrier();
      // (the next writes of these come after the next level's barriers)
      prefix = (prefix << nb) | (uint32_t)sh.bstar;
      shift -= nb;
      rem = sh.rem;
      cnt = sh.cnt;
    };
    level(11);
    if (cnt == 1) {
      // one key left with these leading bits: it is the threshold
      prefix = sh.cu[sh.bstar];
      shift = 0;
    } else {
      level(10);
    }
    const uint32_t T = prefix;
    const int eqc = cnt;
    // The next problem's keys into the stage and its bins into registers.
    // Issued after the histogram levels: the compiler cannot tell their LDS
    // atomics from the copy's destination and would wait for the copy before
    // each of them.
    // (the bins first: loads complete in order, so a wait for them does not
    // wait for the copy)
    const int pn = p + gridDim.x;
    if (pn < P) {
      const int32_t* hrow = hist + (long long)pn * hist_stride;
      c0 = hrow[kBins - 1 - 2 * tid];
      c1 = hrow[kBins - 2 - 2 * tid];
      stage_keys(pn);
    }
    // take every key above T and the first rem keys equal to T
    uint32_t take = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {  // T >= 1: items past n never match
      if (u[i] > T) take |= 1u << i;
      if (u[i] == T) eq |= 1u << i;
    }
    if (eqc == rem) {
      take |= eq;
    } else {
      // the first rem keys equal to T in position order (ranks as in the
      // output below)
      const int ne = __popc(eq);
      const int rk = block_incl_scan(ne, sh.wsum) - ne;
      const uint32_t eqp = to_pos(eq);
      int rotq = rot;
      asm volatile("" : "+v"(rotq));  // rank masks made here, not kept across problems
#pragma unroll
      for (int g = 0; g < NI / 4; ++g) {
        const int np0 = (4 * g + rotq) & (NI - 1);
        int re = rk + __popc(eqp & ((1u << np0) - 1u));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          const int t = (eq >> i) & 1;
          if (t && re < rem) take |= 1u << i;
          re += t;
        }
      }
    }
    // ---- output in position order: register j goes to rank rk plus the
    // taken keys at positions before nat(j); the 4-key groups of registers
    // are consecutive positions, so the rank steps by one inside a group
    const int ntk = __popc(take);
    // (closed by the barrier at the top of the next problem)
    const int rk = block_incl_scan<false>(ntk, sh.wsum) - ntk;
    const uint32_t takep = to_pos(take);
    int32_t* so = sel_out + (long long)p * sel_stride;
    float* ko = keys_out ? keys_out + (long long)p * keys_out_stride : nullptr;
    const bool safe = !__builtin_amdgcn_ballot_w64(rk < 0 || rk + ntk > K);
    int roto = rot;
    asm volatile("" : "+v"(roto));  // rank masks made here, not kept across problems
#pragma unroll
    for (int g = 0; g < NI / 4; ++g) {
      const int np0 = (4 * g + roto) & (NI - 1);  // position of register 4g
      unsigned ro = (unsigned)(rk + __popc(takep & ((1u << np0) - 1u)));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        const unsigned t = (take >> i) & 1u;
        // outputs only at ranks 0 .. K-1 (only a histogram that disagreed
        // with the keys could ask for more)
        if (t && (safe || ro < (unsigned)K)) {
          so[ro] = pos0 + np0 + e;
          if (ko) ko[ro] = key_value(u[i]);
        }
        ro += t;
      }
    }
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
                       long long keys_out_stride, hipStream_t st, const int32_t* given_hist,
                       long long hist_stride) {
  if (n < 1 || K < 1 || K > n) return hipErrorInvalidValue;
  if (given_hist && (cand || n > 32768 || hist_stride < kHistBins)) return hipErrorInvalidValue;
  const int items = (n + kTopkThreads - 1) / kTopkThreads;
  dim3 grid(P), block(kTopkThreads);
  if (given_hist) {
    // persistent blocks, one per CU (the key stage takes most of the LDS)
    const int nb = P < kTopkHistBlocks ? P : kTopkHistBlocks;
    // every thread's 32 positions inside the problem: no per-key range masks
    if (n == kTkKeys)
      FL_LAUNCH(k_topk_hist<true>, dim3(nb), block, 0, st, keys, key_stride, P, n, K, given_hist, hist_stride,
                sel_out, sel_stride, keys_out, keys_out_stride);
    else
      FL_LAUNCH(k_topk_hist<false>, dim3(nb), block, 0, st, keys, key_stride, P, n, K, given_hist, hist_stride,
                sel_out, sel_stride, keys_out, keys_out_stride);
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
