// Matrix-core kernels of the prefill loop attention (bf16 inputs, head dim 128).
//
// What is computed follows the FlashLoop pages: loop 1 is dense causal
// attention over the reconstructed base (p1 §D.1 and the workload's dense
// first loop); loop r >= 2 recomputes the active rows only against the
// selected columns and rescales by the cached mass (p1 §4.1, §4.2, §D.2;
// guide §3); the cached mass M and reused part U come from loop r-1's
// probabilities over the selected columns (p1 §D.2: the selection keeps the
// chosen key positions together with their share of the full distribution).
//
// Design (gfx950, wave64):
//  * a block of NW waves owns 32 * NW query rows (twelve waves, three per
//    SIMD, when the launch is large; else four, two blocks per CU); a wave
//    keeps its 32 rows' queries in registers as the B operand of S^T = K Q^T
//    (v_mfma_f32_32x32x16_bf16), so each lane holds one query row's scores
//    and the row softmax needs one cross-half exchange per tile;
//  * key tiles of 64 columns: K stored row-major (bf16) and V transposed
//    (fp16) in LDS; the K and V fragments are read a few MFMAs ahead of use;
//  * P is rounded to fp16 (not bf16) for O^T += V^T P^T on
//    v_mfma_f32_32x32x16_f16: P in [0, 1] needs significand, not range, and
//    bf16 rounding alone would spend the whole error budget; the bf16 value
//    v~ converts to fp16 exactly;
//  * every record a loop attends is dequantized once per loop by
//    k_build_tiles into 64-column tile images laid out exactly like the LDS
//    tiles (p1 §4.4: the engine gathers the chosen tokens and keys into
//    dense buffers); the attention kernel copies them into a two-image LDS
//    ring by direct buffer->LDS loads, the next tile's copy in flight while
//    the current one is used.  Dequantizing inside the attention kernel
//    instead would repeat the work for every row block and the vector ALUs
//    are already the busier unit on gfx950.
#include <cstdlib>
#include <cstring>

#include "launch.hpp"

namespace fl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kBN = 64;             // key columns per tile
constexpr int kNoPos = 0x7fffffff;  // padding column: masked for every row
// Lazy rescale: the weights P = 2^(x*c2 - mref) of a tile are formed against
// the current reference mref (log2 units) and used as they are while every one
// of them fits fp16 (up to 65504; fp16 rounds them with the same relative
// error at any size and keeps them normal down to 2^-14, i.e. scores up to ~30
// below the largest weight).  Only when one does not (a lane's fp32 sum of its
// 32 rounded weights is then not finite, above 32 * 65504) does the reference
// move: to the tile maximum, for the rows whose maximum exceeds it by more
// than kRescale.
constexpr float kRescale = 15.0f;
constexpr float kRescaleP = 32.0f * 65504.0f;  // largest sum of 32 finite fp16 weights

// Tile image: the exact LDS layout of one 64-column tile, built once per loop
// in HBM and copied into LDS by direct global->LDS loads.
//   K   [64][kKP]  bf16  (row = column of the tile, 272-byte rows)
//   V^T [128][kVP] fp16  (row = head dim, 144-byte rows; within each 16
//                        columns, the 8 a lane multiplies are stored
//                        contiguously: see vt_col)
//   pos [64]       int32 (position of each column, kNoPos for padding)
//   vsh            int32: the tile's V^T holds v~ * 2^-vsh, vsh >= 0 the
//                  smallest shift that brings the tile's largest |v~| below
//                  2^15 (fp16's range ends at 65504; bf16 values reach 3.4e38)
constexpr int kKP = kD + 8;
constexpr int kVP = kBN + 8;
constexpr int kImgV = kBN * kKP * 2;          // 17408
constexpr int kImgPos = kImgV + kD * kVP * 2;  // 35840
constexpr int kImgShift = kImgPos + kBN * 4;   // 36096
constexpr int kImgBytes = 36 * 1024;           // 36864: 36 chunks of 1 KB (36100 used)
static_assert(kImgShift + 4 <= kImgBytes, "tile image layout");
constexpr int kImgChunks = kImgBytes / 1024;
// Tile ring of the attention kernel: two images resident, the next one
// copied while this one is used (72 KB of LDS).

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------- tile images
// Column slot of tile column x in the V^T image.  In the S^T = K Q^T
// accumulator a lane of half hf holds, per 16 columns, columns 4hf..4hf+3
// and 8+4hf..8+4hf+3; storing those eight next to each other lets the PV
// product read its B fragment with one 16-byte LDS load.
__host__ __device__ constexpr int vt_col(int x) {
  return (x & ~15) + ((x >> 2) & 1) * 8 + ((x >> 3) & 1) * 4 + (x & 3);
}
static_assert(vt_col(0) == 0 && vt_col(4) == 8 && vt_col(8) == 4 && vt_col(12) == 12 && vt_col(21) == 25,
              "V^T column slots");
// The same for the 16x16x32 products of the 48-row dense kernel: there a lane
// of group g (lane / 16) holds, per 32 columns, columns 4g..4g+3 and
// 16+4g..16+4g+3 of its row, stored as slots 8g..8g+7.
__host__ __device__ constexpr int vt_col16(int x) {
  return (x & ~31) + ((x >> 2) & 3) * 8 + ((x >> 4) & 1) * 4 + (x & 3);
}
static_assert(vt_col16(0) == 0 && vt_col16(4) == 8 && vt_col16(16) == 4 && vt_col16(21) == 13 &&
                  vt_col16(31) == 31 && vt_col16(44) == 56,
              "V^T column slots (16x16 products)");

// One tile image in LDS (img, kImgBytes) from 256 threads of a block: the
// columns tile*64 .. +64 of a selection row (sel NULL: those positions
// themselves; past K: padding), reconstructed at loop rc for KV head hk of
// sequence b.  NR >= 0: the workload format with a chain of exactly NR
// residual loops (rc = NR + 1), its loads batched (chain_group_n); NR < 0:
// any chain.  Ends with a block barrier: the image is complete.
// V16: V^T columns in the slots of the 16x16x32 products (vt_col16).
template <int NR, bool V16 = false>
__device__ inline void build_tile(uint8_t* img, float* wmax, const CacheGeo& c, int rc, const int32_t* selrow, int K,
                                  int tile, int b, int hk) {
  const int t = threadIdx.x;
  const int col = t >> 2, g = t & 3;
  const int idx = tile * kBN + col;
  const int j = idx < K ? (selrow ? selrow[idx] : idx) : -1;
  float x[32];
  // K rows (bf16)
  if (j >= 0) {
    if (c.fmt == kFmtPaper) {
      paper_chain16(c, rc, 0, b, hk, j, 0, g * 32, x);
      paper_chain16(c, rc, 0, b, hk, j, 0, g * 32 + 16, x + 16);
    } else if (NR >= 0) {
      chain_group_n<NR < 0 ? 0 : NR>(c, 0, b, hk, j, 0, g, x);
    } else {
      chain_group(c, rc, 0, b, hk, j, 0, g, x);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.0f;
  }
  {
    uint4* dst = (uint4*)(img + (col * kKP + g * 32) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_uint4(pack_bf16x2(x[8 * i], x[8 * i + 1]), pack_bf16x2(x[8 * i + 2], x[8 * i + 3]),
                          pack_bf16x2(x[8 * i + 4], x[8 * i + 5]), pack_bf16x2(x[8 * i + 6], x[8 * i + 7]));
  }
  // V^T rows: v~ = bf16(x) scaled by the tile's power-of-two shift, in fp16
  // (exact for magnitudes above 2^-14 after the shift; smaller ones round to
  // fp16's subnormal grid, at most 2^-25 off, and the shift only appears for
  // tiles whose largest magnitude is at least 2^15)
  if (j >= 0) {
    if (c.fmt == kFmtPaper) {
      paper_chain16(c, rc, 0, b, hk, j, 1, g * 32, x);
      paper_chain16(c, rc, 0, b, hk, j, 1, g * 32 + 16, x + 16);
    } else if (NR >= 0) {
      chain_group_n<NR < 0 ? 0 : NR>(c, 0, b, hk, j, 1, g, x);
    } else {
      chain_group(c, rc, 0, b, hk, j, 1, g, x);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.0f;
  }
  // the tile's largest |v~| decides its shift (almost always 0)
  {
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      x[e] = round_bf16(x[e]);
      mx = fmaxf(mx, fabsf(x[e]));
    }
    mx = wave_max(mx);
    if ((t & 63) == 0) wmax[t >> 6] = mx;
  }
  __syncthreads();
  const float tmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // 2^e <= tmax < 2^(e+1); the shift brings tmax below 2^15
  const int vsh = tmax >= 32768.0f ? ((__float_as_int(tmax) >> 23) & 255) - 127 - 14 : 0;
  {
    _Float16* vt = (_Float16*)(img + kImgV);
    const int vc = V16 ? vt_col16(col) : vt_col(col);
#pragma unroll
    for (int e = 0; e < 32; ++e) vt[(g * 32 + e) * kVP + vc] = (_Float16)__builtin_ldexpf(x[e], -vsh);
  }
  if (g == 0) ((int*)(img + kImgPos))[col] = j >= 0 ? j : kNoPos;
  if (t == 0) *(int*)(img + kImgShift) = vsh;
  __syncthreads();
}

// One block of 256 threads per tile: the image built in LDS (build_tile),
// then written out with 16-byte stores.  Every packed record a loop attends
// is dequantized exactly once here (p1 §4.4: chosen keys gathered into dense
// buffers; p1 App. G: attention works from the packed streams).
template <int NR, bool V16 = false>
__global__ __launch_bounds__(256) void k_build_tiles(CacheGeo c, int rc, const int32_t* __restrict__ sel, int K,
                                                     int ntiles, uint8_t* __restrict__ out) {
  __shared__ __align__(16) uint8_t img[kImgBytes];
  __shared__ float wmax[4];
  // sel NULL: the tiles of positions 0..K-1 are the same for every query
  // head of a KV head, so they are built once per (b, KV head)
  const int bh = blockIdx.x / ntiles;
  const int tile = blockIdx.x - bh * ntiles;
  const int nh = sel ? c.H : c.Hkv;
  const int b = bh / nh;
  const int hk = sel ? kv_head(c, bh - b * nh) : bh - b * nh;
  build_tile<NR, V16>(img, wmax, c, rc, sel ? sel + (long long)bh * K : nullptr, K, tile, b, hk);
  uint4* dst = (uint4*)(out + ((long long)bh * ntiles + tile) * kImgBytes);
  const uint4* src = (const uint4*)img;
  for (int i = threadIdx.x; i < kImgBytes / 16; i += 256) dst[i] = src[i];
}

// ------------------------------------------------------------- main kernel
enum { kModeAttn = 0, kModeUM = 1 };

struct MfmaArgs {
  AttnArgs a;
  const uint8_t* tiles;   // tile images [B][H][ntiles_total] (not read when the block builds its own)
  int ntiles_total;       // tiles per (b, h)
  int nblk;               // row blocks per (b, h)
  int rc;                 // loop whose reconstructions the tiles hold
  float c2;               // tau * log2(e)
};

// Direct global->LDS copy of one image of CH 1 KB chunks, the chunks spread
// over the block's NW waves (16 bytes per lane and chunk).  The copies use the
// buffer form (buffer_load_dwordx4 ... lds) on a resource that spans the
// images one block reads: while a copy of the global-segment form is in
// flight the compiler drains every LDS read (lgkmcnt(0)) before each use,
// which serializes the matrix-operand reads; the buffer form counts on vmcnt
// only, so the reads ahead of an MFMA overlap.  Offsets past the resource's
// size read zeros.
__device__ inline __amdgpu_buffer_rsrc_t img_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}
template <int NW, int CH>
__device__ inline void dma_img(__amdgpu_buffer_rsrc_t rs, int off, uint8_t* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int ch = wv; ch < CH; ch += NW)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + ch * 1024), 16, off + ch * 1024 + lane * 16, 0,
                                             0, 0);
}
template <int NW>
__device__ inline void dma_tile(__amdgpu_buffer_rsrc_t rs, int off, uint8_t* lds) {
  dma_img<NW, kImgChunks>(rs, off, lds);
}


// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Wait until the wave's copies of every image but the last `keep` issued
// have landed (in-order completion): the wave issues ceil or floor of
// CH / NW chunk loads per image and no other vector-memory operation in the
// loops that use these waits.
template <int NW, int CH, int K>
__device__ inline void wait_keep() {
  constexpr int hi = (CH + NW - 1) / NW, lo = CH / NW;
  const int wv = threadIdx.x >> 6;
  if (wv < CH - lo * NW || hi == lo)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(K * hi));
  else
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(K * lo));
}
template <int NW, int CH>
__device__ inline void wait_imgs_but(int keep) {
  if (keep >= 2) wait_keep<NW, CH, 2>();
  else if (keep == 1) wait_keep<NW, CH, 1>();
  else __builtin_amdgcn_s_waitcnt(0);
}
template <int NW>
__device__ inline void wait_tiles_but(int keep) {
  wait_imgs_but<NW, kImgChunks>(keep);
}

// sched_group_barrier masks: MFMA and LDS-read instruction classes.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// S^T = K Q^T for one tile: the lane's row against the tile's 64 columns.
// The K fragments of the next two k-steps are read while the current ones
// are multiplied (the registers of the loop allow two steps ahead).
__device__ inline void qk_tile(const uint8_t* T, const bf16x8_t* qf, int l32, int hf, f32x16_t& s0, f32x16_t& s1) {
  constexpr int A = 2;
  const __bf16* kt = (const __bf16*)T;
  s0 = f32x16_t{};
  s1 = f32x16_t{};
  bf16x8_t ka[A], kb[A];
#pragma unroll
  for (int i = 0; i < A; ++i) {
    ka[i] = *(const bf16x8_t*)&kt[l32 * kKP + i * 16 + hf * 8];
    kb[i] = *(const bf16x8_t*)&kt[(32 + l32) * kKP + i * 16 + hf * 8];
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % A], qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[ks % A], qf[ks], s1, 0, 0, 0);
    if (ks + A < 8) {
      ka[ks % A] = *(const bf16x8_t*)&kt[l32 * kKP + (ks + A) * 16 + hf * 8];
      kb[ks % A] = *(const bf16x8_t*)&kt[(32 + l32) * kKP + (ks + A) * 16 + hf * 8];
    }
  }
  // keep that order: the first 2A reads, then one MFMA per read, then the rest
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * A, 0);
#pragma unroll
  for (int i = 0; i < 16 - 2 * A; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * A, 0);
}

// Softmax of one tile for the lane's row, first part: the causal mask.
// Copies the scores into x with -inf where the column lies after the row.
__device__ inline void softmax_mask(const uint8_t* T, f32x16_t s0, f32x16_t s1, int ipos, int blk_min, int hf,
                                    float* x) {
  const int* tpos = (const int*)(T + kImgPos);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    x[v] = s0[v];
    x[16 + v] = s1[v];
  }
  if (tpos[kBN - 1] > blk_min || ipos < 0) {
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      const int col = (v >> 4) * 32 + 8 * ((v & 15) >> 2) + 4 * hf + (v & 3);
      if (tpos[col] > ipos) x[v] = -INFINITY;
    }
  }
}

// Lazy rescale: the reference max mref (log2 units) moves to the row max of
// the tile only when that max exceeds it by more than kRescale (or it is
// unset); the row sum and accumulators are rescaled then.
__device__ inline void softmax_rescale(const float* x, float c2, float& mref, float& lsum, f32x16_t* o) {
  float mt = x[0];
#pragma unroll
  for (int v = 1; v < 32; ++v) mt = fmaxf(mt, x[v]);
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * c2;
  const bool need = mt > mref + kRescale;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float mn = need ? mt : mref;
    const float alpha = need ? __builtin_amdgcn_exp2f(mref - mn) : 1.0f;
    mref = mn;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
  }
}

// Second part: P = 2^(x*c2 - base) rounded to fp16; returns the lane's sum
// of exactly those fp16 weights (pairs summed into fp32 by v_dot2 with 1s,
// in two chains).
__device__ inline float softmax_probs(const float* x, float base, float c2, f16x8_t* pf) {
  const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k2 * 8 + e], c2, -base));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k2 * 8 + e + 1], c2, -base));
      const f16x2_t h = {(_Float16)p0, (_Float16)p1};
      pf[k2][e] = h[0];
      pf[k2][e + 1] = h[1];
      if (e & 2)
        ls1 = __builtin_amdgcn_fdot2(h, one2, ls1, false);
      else
        ls0 = __builtin_amdgcn_fdot2(h, one2, ls0, false);
    }
  }
  return ls0 + ls1;
}

// O^T += V^T P^T for one tile ("GEMM phase", second half).
__device__ inline void pv_tile(const uint8_t* T, const f16x8_t* pf, int l32, int hf, f32x16_t* o) {
  const _Float16* vt = (const _Float16*)(T + kImgV);
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f16x8_t vf = *(const f16x8_t*)&vt[(db * 32 + l32) * kVP + k2 * 16 + hf * 8];
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[k2], o[db], 0, 0, 0);
    }
  }
  // eight V fragment reads in flight ahead of the MFMAs that use them
  constexpr int A = 8;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A, 0);
#pragma unroll
  for (int i = 0; i < 16 - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, A, 0);
}

// Output of one row (64 of its 128 dims per lane): loop 1 writes O, U = 0,
// M = 1 and lse; a sparse loop patches O = U + M * acc / l and lse (or
// lse = -inf when no column was left); the cached-mass pass writes
// U = O - M_prev * acc and M = M_prev * l.
// The accumulators hold 2^-osh times the products (V shifts); osc = 2^osh.
template <int MODE>
__device__ inline void write_row(const AttnArgs& a, int r, long long bhS, int i, int hf, float mref, float lt,
                                 const f32x16_t* o, float osc, float um_off = 0.0f) {
  if (i < 0) return;
  const long long rowp = (bhS + i) * kD;
  if (MODE == kModeAttn) {
    if (r == 1) {
      const float inv = (1.0f / lt) * osc;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int dcol = db * 32 + qq * 8 + hf * 4;
          f32x4_t ov = {o[db][qq * 4] * inv, o[db][qq * 4 + 1] * inv, o[db][qq * 4 + 2] * inv,
                        o[db][qq * 4 + 3] * inv};
          *(f32x4_t*)&a.O[rowp + dcol] = ov;
          *(f32x4_t*)&a.U[rowp + dcol] = f32x4_t{};
        }
      }
      if (hf == 0) {
        a.lse[bhS + i] = (mref + __log2f(lt)) * 0.6931471805599453f;
        a.M[bhS + i] = 1.0f;
      }
    } else if (lt > 0.0f && a.lsel) {
      const float b2 = (mref + __log2f(lt)) * 0.6931471805599453f;
      float cu, ca;
      mixed_coeffs(a.M[bhS + i], b2, a.lsel[bhS + i], cu, ca);
      const float sc = (ca / lt) * osc;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int dcol = db * 32 + qq * 8 + hf * 4;
          const f32x4_t uv = *(const f32x4_t*)&a.U[rowp + dcol];
          f32x4_t ov, un;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            un[e] = cu * uv[e];
            ov[e] = un[e] + sc * o[db][qq * 4 + e];
          }
          *(f32x4_t*)&a.O[rowp + dcol] = ov;
          *(f32x4_t*)&a.U[rowp + dcol] = un;
        }
      }
      if (hf == 0) {
        a.lse[bhS + i] = b2;
        a.M[bhS + i] = ca;
      }
    } else if (lt > 0.0f) {
      const float Mi = a.M[bhS + i];
      const float sc = (Mi / lt) * osc;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int dcol = db * 32 + qq * 8 + hf * 4;
          const f32x4_t uv = *(const f32x4_t*)&a.U[rowp + dcol];
          f32x4_t ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = uv[e] + sc * o[db][qq * 4 + e];
          *(f32x4_t*)&a.O[rowp + dcol] = ov;
        }
      }
      if (hf == 0) a.lse[bhS + i] = (mref + __log2f(lt)) * 0.6931471805599453f;
    } else if (hf == 0) {
      a.lse[bhS + i] = -INFINITY;
    }
  } else {
    // The sums are against the reference mref; the loop r-1 probabilities
    // are P = 2^(x - um_off) with um_off = lse_prev log2 e - log2 M_prev (+inf
    // when M_prev = 0), so both take Mu = 2^(mref - um_off) (none if the row
    // saw no selected column: lt = 0).
    const float Mu = (lt > 0.0f && um_off != INFINITY) ? __builtin_amdgcn_exp2f(mref - um_off) : 0.0f;
    const float Mo = Mu * osc;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int dcol = db * 32 + qq * 8 + hf * 4;
        const f32x4_t ov = *(const f32x4_t*)&a.O[rowp + dcol];
        f32x4_t uv;
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[e] = ov[e] - Mo * o[db][qq * 4 + e];
        *(f32x4_t*)&a.U[rowp + dcol] = uv;
      }
    }
    if (hf == 0) {
      a.M[bhS + i] = Mu * lt;
      // loop r-1 log-sum-exp over J_i (the mixed-logit combine reads it)
      if (a.lsel) a.lsel[bhS + i] = lt > 0.0f ? (mref + __log2f(lt)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// NW waves of 32 query rows each (BM = 32 * NW).  Per 64-column tile:
// S^T = K Q^T on the matrix cores, the probabilities on the vector ALUs,
// then O^T += V^T P^T.  Several waves per SIMD (twelve waves per block, or
// two blocks of four) let one wave's vector work run under another's matrix
// work.  Tile images arrive by direct global->LDS loads issued one tile
// ahead into a two-image ring, so the loop itself writes no LDS.
// RING: tile images resident in LDS.  Two: the next tile is copied while this
// one is used; one: the copy waits for the block's waves to finish the tile
// (three blocks per CU then cover each other's copies).
// SRC 0: the tiles are images built beforehand (k_build_tiles) and copied
// in; SRC 1 (four waves, one-image ring, the sparse loops' attention): the
// block's 256 threads build each tile from the packed records in LDS
// themselves (build_tile) - no image round trip and no extra launch, but
// every row block of a head repeats the dequantization, and the builder's
// registers next to the attention state leave two blocks per CU.
// SPLIT > 1 (one-image ring of prebuilt tiles): the waves form NW / SPLIT
// row groups of 32 rows times SPLIT column splits.  Each step copies SPLIT
// consecutive tiles and split s takes the s-th of them; at the end splits
// 1.. hand their (reference, sum, accumulators) to split 0 through LDS, which
// merges them in split order (fixed: deterministic).  Fewer rows per block
// and a shorter tile chain per wave: for launches too small to fill the chip.
template <int NW, int MODE, int RING, int SRC, int SPLIT = 1>
__global__ __launch_bounds__(64 * NW, NW == 4 ? (SRC == 0 && RING == 1 ? 3 : 2) : 1) void k_attn_mfma(MfmaArgs m) {
  static_assert(SRC == 0 || (NW == 4 && RING == 1), "blocks build their tiles with 256 threads into one image");
  static_assert(SPLIT == 1 || (SRC == 0 && RING == 1 && NW % SPLIT == 0), "column splits: prebuilt tiles, one step");
  constexpr int G = NW / SPLIT;   // row groups
  constexpr int BM = 32 * G;
  constexpr int AHEAD = RING - 1;
  extern __shared__ __align__(16) uint8_t lds[];   // RING steps of SPLIT tile images
  __shared__ int sh_ntiles;
  __shared__ float sh_wmax[4];
  const AttnArgs& a = m.a;
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hf = lane >> 5;       // half of the wave
  const int l32 = lane & 31;
  const int rg = SPLIT == 1 ? wv : wv % G;  // row group
  const int sp = SPLIT == 1 ? 0 : wv / G;   // column split

  // block -> (b, h, row block); every XCD gets whole heads, heavy blocks first
  const int nunits = c.B * c.H * m.nblk;
  int u = blockIdx.x;
  if ((nunits & 7) == 0) u = (u & 7) * (nunits >> 3) + (u >> 3);
  const int bh = u / m.nblk;
  const int blk = m.nblk - 1 - (u - bh * m.nblk);
  const int b = bh / c.H;

  const int r = a.r;
  const bool dense = r == 1 && MODE == kModeAttn;
  const int nrows = dense ? c.S : count_of(c, r, b);
  const int row0 = blk * BM;
  if (row0 >= nrows) return;  // past this sequence's rows (ragged counts): the whole block
  const long long bhS = (long long)bh * c.S;
  // loop 1 reads the tiles of its KV head (built once per KV head)
  const long long tbh = dense ? (long long)b * c.Hkv + kv_head(c, bh - b * c.H) : bh;
  const uint8_t* imgs = SRC ? nullptr : m.tiles + tbh * m.ntiles_total * kImgBytes;
  const int32_t* selrow = SRC ? a.sel + (long long)bh * a.K : nullptr;
  const int hk = kv_head(c, bh - b * c.H);
  const __amdgpu_buffer_rsrc_t rs = img_rsrc(imgs, SRC ? 0 : m.ntiles_total * kImgBytes);
  // Tile 0 is needed by every block that has a column at all: its copy is
  // issued first, under the query loads and the tile count below.
  if (!SRC && m.ntiles_total > 0) dma_img<NW, kImgChunks * SPLIT>(rs, 0, lds);

  // ---- the lane's row and its queries (B operand of S^T = K Q^T)
  int ipos = -1;
  bf16x8_t qf[8];
  {
    const int t = row0 + rg * 32 + l32;
    long long qrow = 0;
    if (t < nrows) {
      if (dense) {
        ipos = t;
        qrow = bhS + t;
      } else {
        ipos = c.rows[r][(long long)b * c.n[r] + t];
        if (MODE == kModeAttn) {
          qrow = (long long)bh * c.n[r] + t;
        } else {
          const int rp = r - 1;
          const int qi = rp == 1 ? ipos : c.slot[rp][(long long)b * c.S + ipos];
          const int np = rp == 1 ? c.S : c.n[rp];
          if (qi < 0) ipos = -1;  // not nested (precondition): leave the row alone
          qrow = (long long)bh * np + (qi < 0 ? 0 : qi);
        }
      }
    }
    const bf16x8_t* qp = (const bf16x8_t*)((const uint16_t*)a.q + qrow * kD);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = ipos >= 0 ? qp[ks * 2 + hf] : bf16x8_t{};
  }
  int blk_min, blk_max;
  {
    const int t0 = row0, t1 = min(row0 + BM, nrows) - 1;
    if (dense) {
      blk_min = t0;
      blk_max = t1;
    } else {
      blk_min = c.rows[r][(long long)b * c.n[r] + t0];
      blk_max = c.rows[r][(long long)b * c.n[r] + t1];
    }
  }
  // Tiles the block reads: those whose first column is <= blk_max (first
  // columns ascend).  Loop 1's tiles are the positions in order; otherwise
  // wave 0 probes up to 64 tiles at once and keeps the segment the answer
  // lies in (one round up to 64 tiles, two up to 4096).
  if (wv == 0) {
    int base = 0;
    if (dense) {
      base = min(m.ntiles_total, blk_max / kBN + 1);
    } else {
      int end = m.ntiles_total;  // answer in [base, end]; tiles [base, end) unprobed
      while (end > base) {
        const int len = end - base;
        const int step = (len + 63) >> 6;
        bool le = false;
        if (lane * step < len) {
          const int t = base + lane * step;
          const int p0 = SRC ? selrow[t * kBN] : *(const int*)(imgs + (long long)t * kImgBytes + kImgPos);
          le = p0 <= blk_max;
        }
        const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
        if (cnt == 0) break;
        const int nb = base + (cnt - 1) * step + 1;
        end = min(base + cnt * step, end);
        base = nb;
      }
    }
    if (lane == 0) sh_ntiles = base;
  }

  // row state: mref = reference max (log2 units), lsum = partial row sum
  float mref = -INFINITY, lsum = 0.0f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};
  // cached-mass pass: the row's loop r-1 statistics as one exponent offset,
  // P = M 2^(x - lse log2 e) = 2^(x - um_off)
  float um_off = INFINITY;
  if (MODE == kModeUM && ipos >= 0) {
    const float Mp = a.M[bhS + ipos];
    if (Mp > 0.0f) um_off = a.lse[bhS + ipos] * 1.4426950408889634f - __log2f(Mp);
  }
  __syncthreads();
  const int nt = sh_ntiles;

  // ---- prologue: the first max(AHEAD, 1) tiles into the ring (tile 0 issued above)
  if (SRC) {
    if (nt > 0) build_tile<-1>(lds, sh_wmax, c, m.rc, selrow, a.K, 0, b, hk);
  } else {
    for (int k = 1; k < AHEAD && k < nt; ++k) dma_tile<NW>(rs, k * kImgBytes, lds + k * kImgBytes);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // V shift of the accumulators: o holds 2^-osh times the products, osh the
  // largest tile shift seen so far (wave-uniform; 0 unless some |v~| >= 2^15).
  // A tile of smaller shift d below osh enters with its weights scaled by
  // 2^-d (folded into the exponent); the row sum always adds the unscaled ones.
  int osh = 0;
  const int nsteps = SPLIT == 1 ? nt : (nt + SPLIT - 1) / SPLIT;
  for (int ks = 0; ks < nsteps; ++ks) {
    const int tt = ks * SPLIT + sp;  // this wave's tile
    const uint8_t* T = lds + (SPLIT == 1 ? tt % RING : sp) * kImgBytes;
    // tile tt+AHEAD goes into the slot tile tt-1 left (all waves passed it)
    if (AHEAD > 0 && tt + AHEAD < nt)
      dma_tile<NW>(rs, (tt + AHEAD) * kImgBytes, lds + ((tt + AHEAD) % RING) * kImgBytes);
    if (SPLIT == 1 || tt < nt) {
      f32x16_t s0, s1;
      qk_tile(T, qf, l32, hf, s0, s1);
      float x[32];
      softmax_mask(T, s0, s1, ipos, blk_min, hf, x);
      const int tsh = __builtin_amdgcn_readfirstlane(*(const int*)(T + kImgShift));
      if (tsh > osh) {
        const float f = __builtin_ldexpf(1.0f, osh - tsh);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= f;
        osh = tsh;
      }
      const int dsh = osh - tsh;
      // Weights against the current reference: only if a lane's weights
      // overflowed fp16 (its sum is not finite) or a valid row has no
      // reference yet is the tile max taken, the lazy rescale applied and the
      // weights formed again.  The cached-mass pass does the same and brings
      // its sums to the loop r-1 statistics at the end (write_row): weights
      // formed against the loop r-1 log-sum-exp itself would fall into fp16's
      // subnormal range for a row whose selected columns carry little of its
      // mass, and lose their relative precision there.
      f16x8_t pf[4];
      float ls = softmax_probs(x, (mref == -INFINITY ? 0.0f : mref) + (float)dsh, m.c2, pf);
      {
        const bool bad = (ipos >= 0 && mref == -INFINITY) || !(ls <= kRescaleP);
        if (__builtin_amdgcn_ballot_w64(bad)) {
          softmax_rescale(x, m.c2, mref, lsum, o);
          ls = softmax_probs(x, (mref == -INFINITY ? 0.0f : mref) + (float)dsh, m.c2, pf);
        }
      }
      lsum += dsh == 0 ? ls : __builtin_ldexpf(ls, dsh);
      pv_tile(T, pf, l32, hf, o);
    }
    if (SRC) {
      // every wave is done with the slot: build the next tile in it
      if (tt + 1 < nt) {
        lds_barrier();
        build_tile<-1>(lds, sh_wmax, c, m.rc, selrow, a.K, tt + 1, b, hk);
      }
      continue;
    }
    if (AHEAD == 0) {
      // every wave is done with the slot: copy the next step's tiles into it
      if (ks + 1 < nsteps) {
        lds_barrier();
        dma_img<NW, kImgChunks * SPLIT>(rs, (ks + 1) * SPLIT * kImgBytes, lds);
        __builtin_amdgcn_s_waitcnt(0);
      }
    } else {
      // tile tt+1 must be in LDS for every wave
      wait_tiles_but<NW>(min(tt + AHEAD, nt - 1) - (tt + 1));
    }
    lds_barrier();
  }

  // ---- epilogue: each lane writes 64 of its row's 128 dims
  float lt = lsum + __shfl_xor(lsum, 32, 64);
  if constexpr (SPLIT > 1) {
    // Splits 1.. leave their state in LDS (the images are no longer read:
    // every wave passed the loop's last barrier), lane-major 16-byte slots.
    constexpr int kPart = 17 * 1024;
    static_assert((SPLIT - 1) * G * kPart <= SPLIT * kImgBytes, "merge buffers fit the images");
    if (sp > 0) {
      f32x4_t* po = (f32x4_t*)(lds + ((sp - 1) * G + rg) * kPart);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          po[(db * 4 + qq) * 64 + lane] = f32x4_t{o[db][qq * 4], o[db][qq * 4 + 1], o[db][qq * 4 + 2], o[db][qq * 4 + 3]};
      po[16 * 64 + lane] = f32x4_t{mref, lt, (float)osh, 0.0f};
    }
    lds_barrier();
    if (sp > 0) return;
    // Split 0 merges in split order: the common reference M = max of the
    // references and shift OSH = max of the shifts; split s enters with
    // weight 2^(mref_s - M)
    // (0 for a split that saw no column of the row) and its accumulators
    // with 2^(osh_s - OSH) more.
    float ms[SPLIT], ls[SPLIT];
    int os[SPLIT];
    ms[0] = mref;
    ls[0] = lt;
    os[0] = osh;
#pragma unroll
    for (int s = 1; s < SPLIT; ++s) {
      const f32x4_t st4 = ((const f32x4_t*)(lds + ((s - 1) * G + rg) * kPart))[16 * 64 + lane];
      ms[s] = st4[0];
      ls[s] = st4[1];
      os[s] = (int)st4[2];
    }
    float M = ms[0];
    int OSH = os[0];
#pragma unroll
    for (int s = 1; s < SPLIT; ++s) {
      M = fmaxf(M, ms[s]);
      OSH = max(OSH, os[s]);
    }
    float f[SPLIT];
    lt = 0.0f;
#pragma unroll
    for (int s = 0; s < SPLIT; ++s) {
      const float w = ms[s] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms[s] - M);
      lt += w * ls[s];
      f[s] = w * __builtin_ldexpf(1.0f, os[s] - OSH);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= f[0];
#pragma unroll
    for (int s = 1; s < SPLIT; ++s) {
      const f32x4_t* po = (const f32x4_t*)(lds + ((s - 1) * G + rg) * kPart);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x4_t v = po[(db * 4 + qq) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[db][qq * 4 + e] = __builtin_fmaf(f[s], v[e], o[db][qq * 4 + e]);
        }
    }
    mref = M;
    osh = OSH;
  }
  write_row<MODE>(a, r, bhS, ipos, hf, mref, lt, o, __builtin_ldexpf(1.0f, osh), um_off);
}

// ------------------------------------------------------------- dense loop 1, 48 rows per wave
// Loop-1 attention over every position on 16x16x32 products: each wave owns
// RB 16-row blocks of queries (RB = 3: 48 rows, two waves per SIMD), so every
// K or V^T fragment a lane reads from LDS feeds RB products (three: 1.5x the
// matrix work per LDS byte of the 32-row kernel).  In S^T = K Q^T a lane of group
// g = lane / 16 holds, for row l16 = lane % 16 of each row block, columns
// 16kb + 4g .. +3 of the tile (kb = 0..3): a row's 64 columns lie in four
// lanes, which reduce a row's maximum or sum with two exchanges.  The
// weights of columns 32j + {4g..4g+3, 16+4g..16+4g+3} form the lane's B
// fragment of O^T += V^T P^T for k-step j, matched by the tile image's V^T
// column slots (vt_col16).  Lazy rescale, V shifts and outputs as in the
// 32-row kernel.

template <int RB>
__device__ inline void qk_tile48(const uint8_t* T, const bf16x8_t (*qf)[4], int l16, int g, f32x4_t (*s)[RB]) {
  constexpr int A = RB == 3 ? 3 : 2;  // fragments read ahead
  const __bf16* kt = (const __bf16*)T;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4_t{};
  // fragment f = ks * 4 + kb: key row 16kb + l16, dims 32ks + 8g .. +7
  bf16x8_t kf[A];
#pragma unroll
  for (int f = 0; f < A; ++f) kf[f] = *(const bf16x8_t*)&kt[((f & 3) * 16 + l16) * kKP + (f >> 2) * 32 + g * 8];
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    const int kb = f & 3, ks = f >> 2;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[f % A], qf[rb][ks], s[kb][rb], 0, 0, 0);
    if (f + A < 16) {
      const int fn = f + A;
      kf[f % A] = *(const bf16x8_t*)&kt[((fn & 3) * 16 + l16) * kKP + (fn >> 2) * 32 + g * 8];
    }
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A, 0);
#pragma unroll
  for (int i = 0; i < 16 - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, RB, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, RB * A, 0);
}

template <int RB>
__device__ inline void pv_tile48(const uint8_t* T, const f16x8_t (*pf)[2], int l16, int g, f32x4_t (*o)[RB]) {
  constexpr int A = RB == 3 ? 3 : 2;  // fragments read ahead
  const _Float16* vt = (const _Float16*)(T + kImgV);
  // fragment f = j * 8 + db: V^T rows 16db + l16, column slots 32j + 8g .. +7
  f16x8_t vf[A];
#pragma unroll
  for (int f = 0; f < A; ++f) vf[f] = *(const f16x8_t*)&vt[((f & 7) * 16 + l16) * kVP + (f >> 3) * 32 + g * 8];
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    const int db = f & 7, j = f >> 3;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[f % A], pf[rb][j], o[db][rb], 0, 0, 0);
    if (f + A < 16) {
      const int fn = f + A;
      vf[f % A] = *(const f16x8_t*)&vt[((fn & 7) * 16 + l16) * kVP + (fn >> 3) * 32 + g * 8];
    }
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, A, 0);
#pragma unroll
  for (int i = 0; i < 16 - A; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, RB, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, RB * A, 0);
}

// Weights of one row block: P = 2^(x*c2 - base) in fp16 for the lane's 16
// columns (x[8j + e]: k-step j, slot e); returns the lane's sum of exactly
// those fp16 weights.
__device__ inline float probs48(const float* x, float base, float c2, f16x8_t* pf) {
  const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
  float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * j + e], c2, -base));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * j + e + 1], c2, -base));
      const f16x2_t h = {(_Float16)p0, (_Float16)p1};
      pf[j][e] = h[0];
      pf[j][e + 1] = h[1];
      if (e & 2)
        ls1 = __builtin_amdgcn_fdot2(h, one2, ls1, false);
      else
        ls0 = __builtin_amdgcn_fdot2(h, one2, ls0, false);
    }
  }
  return ls0 + ls1;
}

// Rescale of one row block: the row's tile maximum over its four lanes.
template <int RB>
__device__ inline void rescale48(const float* x, float c2, float& mref, float& lsum, f32x4_t (*o)[RB], int rb) {
  float mt = x[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mt = fmaxf(mt, x[v]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * c2;
  const bool need = mt > mref + kRescale;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float mn = need ? mt : mref;
    const float alpha = need ? __builtin_amdgcn_exp2f(mref - mn) : 1.0f;
    mref = mn;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
  }
}

template <int NW, int RB>
__global__ __launch_bounds__(64 * NW, 1) void k_attn_dense48(MfmaArgs m) {
  constexpr int WR = 16 * RB;  // rows per wave
  constexpr int BM = WR * NW;
  constexpr int RING = 2;
  extern __shared__ __align__(16) uint8_t lds[];   // two tile images
  const AttnArgs& a = m.a;
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;
  const int l16 = lane & 15;

  // block -> (b, h, row block); every XCD gets whole heads, heavy blocks first
  const int nunits = c.B * c.H * m.nblk;
  int u = blockIdx.x;
  if ((nunits & 7) == 0) u = (u & 7) * (nunits >> 3) + (u >> 3);
  const int bh = u / m.nblk;
  const int blk = m.nblk - 1 - (u - bh * m.nblk);
  const int b = bh / c.H;
  const int nrows = c.S;
  const int row0 = blk * BM;
  if (row0 >= nrows) return;
  const long long bhS = (long long)bh * c.S;
  const long long tbh = (long long)b * c.Hkv + kv_head(c, bh - b * c.H);
  const uint8_t* imgs = m.tiles + tbh * m.ntiles_total * kImgBytes;
  const __amdgpu_buffer_rsrc_t rs = img_rsrc(imgs, m.ntiles_total * kImgBytes);
  if (m.ntiles_total > 0) dma_img<NW, kImgChunks>(rs, 0, lds);

  // the lane's rows (one per row block) and their queries
  const int w0 = row0 + wv * WR;
  int ipos[RB];
  bf16x8_t qf[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = w0 + rb * 16 + l16;
    ipos[rb] = t < nrows ? t : -1;
    const bf16x8_t* qp = (const bf16x8_t*)((const uint16_t*)a.q + (bhS + (t < nrows ? t : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[rb][ks] = ipos[rb] >= 0 ? qp[ks * 4 + g] : bf16x8_t{};
  }
  // tiles of the block: up to its last row; the wave computes those up to
  // its own last row (none if it has no row)
  const int nt = min(m.ntiles_total, (min(row0 + BM, nrows) - 1) / kBN + 1);
  const int wmax = w0 < nrows ? min(w0 + WR, nrows) - 1 : -1;

  float mref[RB], lsum[RB];
  f32x4_t o[8][RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mref[rb] = -INFINITY;
    lsum[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][rb] = f32x4_t{};
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // V shift of the accumulators (as in the 32-row kernel)
  int osh = 0;
  f32x4_t s[4][RB];
  f16x8_t pf[RB][2];
  // The weights pf of tile t from its scores s: mask, V shift, lazy rescale.
  auto weights = [&](int t) {
    const uint8_t* T = lds + (t % RING) * kImgBytes;
    // x[rb][8j + e]: column 32j + 16(e / 4) + 4g + e % 4
    float x[RB][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[rb][kb * 4 + i] = s[kb][rb][i];
    // causal mask (positions are the columns themselves; padding columns
    // lie past every row), only on tiles that reach past the wave's first row
    if (t * kBN + kBN - 1 > w0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int col = t * kBN + (v >> 2) * 16 + 4 * g + (v & 3);
          if (col > ipos[rb]) x[rb][v] = -INFINITY;
        }
    }
    const int tsh = __builtin_amdgcn_readfirstlane(*(const int*)(T + kImgShift));
    if (tsh > osh) {
      const float f = __builtin_ldexpf(1.0f, osh - tsh);
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[db][rb] *= f;
      osh = tsh;
    }
    const int dsh = osh - tsh;
    // lazy rescale as in the 32-row kernel; a lane holds 16 weights of each
    // of its rows, so a sum above 16 * 65504 means one overflowed fp16
    float ls[RB];
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ls[rb] = probs48(x[rb], (mref[rb] == -INFINITY ? 0.0f : mref[rb]) + (float)dsh, m.c2, pf[rb]);
      bad |= (ipos[rb] >= 0 && mref[rb] == -INFINITY) || !(ls[rb] <= 16.0f * 65504.0f);
    }
    if (__builtin_amdgcn_ballot_w64(bad)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        rescale48<RB>(x[rb], m.c2, mref[rb], lsum[rb], o, rb);
        ls[rb] = probs48(x[rb], (mref[rb] == -INFINITY ? 0.0f : mref[rb]) + (float)dsh, m.c2, pf[rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lsum[rb] += dsh == 0 ? ls[rb] : __builtin_ldexpf(ls[rb], dsh);
  };
  for (int tt = 0; tt < nt; ++tt) {
    const uint8_t* T = lds + (tt % RING) * kImgBytes;
    // tile tt+1 goes into the slot tile tt-1 left (all waves passed it)
    if (tt + 1 < nt) dma_tile<NW>(rs, (tt + 1) * kImgBytes, lds + ((tt + 1) % RING) * kImgBytes);
    if (tt * kBN <= wmax) {
      qk_tile48<RB>(T, qf, l16, g, s);
      weights(tt);
      pv_tile48<RB>(T, pf, l16, g, o);
    }
    // tile tt+1 must be in LDS for every wave
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }

  // ---- epilogue: a lane writes dims 16db + 4g .. +3 of each of its rows
  const float osc = __builtin_ldexpf(1.0f, osh);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = lsum[rb];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int i = ipos[rb];
    if (i < 0) continue;
    const long long rowp = (bhS + i) * kD;
    const float inv = (1.0f / lt) * osc;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int dcol = db * 16 + 4 * g;
      f32x4_t ov = o[db][rb] * inv;
      *(f32x4_t*)&a.O[rowp + dcol] = ov;
      *(f32x4_t*)&a.U[rowp + dcol] = f32x4_t{};
    }
    if (g == 0) {
      a.lse[bhS + i] = (mref[rb] + __log2f(lt)) * 0.6931471805599453f;
      a.M[bhS + i] = 1.0f;
    }
  }
}

// ------------------------------------------------------------- column mass
// c_j = sum_{i in A_r, i >= j} P^(r-1)_ij for the candidate columns (p1 §4.2
// and §D.2: columns ranked by the preceding loop's attention statistics over
// the rows loop r recomputes), with P^(r-1)_ij = M_i 2^(x_ij - lse_i log2 e),
// evaluated as 2^(x_ij - (lse_i log2 e - log2 M_i)).
// Column-stationary: a block of NW waves owns 32 * NW candidate columns (a
// lane owns one column; its K fragments stay in registers as the B operand of
// S = Q K^T).  The rows of A_r are first laid out once per call as 64-row
// images (k_build_rows: queries of loop r-1, the exponent offset and the
// position of each row) that every column block then streams through an LDS
// ring by direct global->LDS loads, as the attention kernel streams its
// column tiles.  Column sums accumulate in a fixed order: deterministic.
constexpr int kMassRows = 64;
// Row image: q [64][kKP] bf16 | off [64] f32 | pos [64] int32, 18 KB.
//   off = lse * log2(e) - log2(M), P = 2^(x - off); +inf: the row adds nothing
//   pos = row position, -1 past the last active row
constexpr int kRowOffAt = kMassRows * kKP * 2;         // 17408
constexpr int kRowPosAt = kRowOffAt + kMassRows * 4;   // 17664
constexpr int kRowBytes = 18 * 1024;
constexpr int kRowChunks = kRowBytes / 1024;
constexpr int kMassNW = 8;      // waves per block: 256 columns
constexpr int kMassRing = 3;    // row images resident in LDS (54 KB)
constexpr int kMassAhead = kMassRing - 1;

static_assert(kRowBytes == kRowImgBytes && kMassRows == 64, "row image size (launch.hpp)");

// One block of 256 threads per row image: four threads per row, 32 dims each.
__global__ __launch_bounds__(256) void k_build_rows(AttnArgs a, int ntr, uint8_t* __restrict__ out,
                                                   uint32_t* __restrict__ hist, int nhist) {
  const CacheGeo& c = a.c;
  // the mass histogram the column-mass pass fills starts at zero
  for (int i = blockIdx.x * 256 + threadIdx.x; hist && i < nhist; i += gridDim.x * 256) hist[i] = 0u;
  const int bh = blockIdx.x / ntr;
  const int tile = blockIdx.x - bh * ntr;
  const int b = bh / c.H;
  const int t = threadIdx.x;
  const int row = t >> 2, qd = t & 3;
  const int r = a.r, rp = r - 1;
  const int nr = c.n[r];  // stride of rows[r]
  const int np = rp == 1 ? c.S : c.n[rp];
  const int tr = tile * kMassRows + row;
  int i = -1, qi = -1;
  if (tr < count_of(c, r, b)) {
    i = c.rows[r][(long long)b * nr + tr];
    qi = rp == 1 ? i : c.slot[rp][(long long)b * c.S + i];
  }
  uint4 q4[4];
  if (qi >= 0) {
    const uint4* src = (const uint4*)((const uint16_t*)a.q + ((long long)bh * np + qi) * kD + qd * 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) q4[k] = src[k];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) q4[k] = make_uint4(0, 0, 0, 0);
  }
  uint8_t* img = out + ((long long)bh * ntr + tile) * kRowBytes;
  uint4* dst = (uint4*)(img + (row * kKP + qd * 32) * 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[k] = q4[k];
  if (qd == 0) {
    float off = INFINITY;
    if (qi >= 0) {
      const long long p = (long long)bh * c.S + i;
      const float Mp = a.M[p];
      if (Mp > 0.0f) off = a.lse[p] * 1.4426950408889634f - __log2f(Mp);
    }
    ((float*)(img + kRowOffAt))[row] = off;
    ((int*)(img + kRowPosAt))[row] = i;
  }
}

struct MassArgs {
  AttnArgs a;
  int K_prev;
  float* mass;
  const uint8_t* tiles;   // compact tiles of the candidates (not read when BASE)
  int ntiles_total;
  int tiles_kv;           // tiles built per (b, KV head): no candidate list
  const uint8_t* rows;    // row images [B*H][ntr]
  int ntr;
  int ncb;                // column blocks per (b, h)
  float c2;
  uint32_t* hist;         // [B*H][kHistBins] counts of the masses by order-key bin, or NULL
};

template <bool BASE, int NW>
__global__ __launch_bounds__(64 * NW) void k_mass_mfma(MassArgs m) {
  constexpr int W = 32 * NW;
  extern __shared__ __align__(16) uint8_t lds[];  // kMassRing row images
  __shared__ int sh_t0, sh_jmax;
  const AttnArgs& a = m.a;
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  const int nunits = c.B * c.H * m.ncb;
  int u = blockIdx.x;
  if ((nunits & 7) == 0) u = (u & 7) * (nunits >> 3) + (u >> 3);
  const int bh = u / m.ncb;
  const int cb = u - bh * m.ncb;
  const int b = bh / c.H, h = bh - b * c.H;
  // candidate tiles built without a candidate list are per (b, KV head)
  const long long tbh = m.tiles_kv ? (long long)b * c.Hkv + kv_head(c, h) : bh;

  // ---- this lane's candidate column: position jpos, candidate index cidx
  const int cidx = cb * W + wv * 32 + l32;
  int jpos = kNoPos;
  bf16x8_t kf[8];
  if (BASE) {
    if (cidx < c.S) {
      jpos = cidx;
      const uint8_t* rec = base_rec(c, 0, b, kv_head(c, h), cidx);
      const uint16_t* sc = (const uint16_t*)(rec + 2 * kD);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint2 w = *(const uint2*)(rec + ks * 16 + hf * 8);
        const float s = h2f(sc[ks >> 1]);
        const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (float)(int8_t)(ws[e >> 2] >> (8 * (e & 3))) * s;
          kf[ks][e] = __builtin_bit_cast(__bf16, f32_to_bf16(v));
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = bf16x8_t{};
    }
  } else {
    const int tile = cidx / kBN, col = cidx - tile * kBN;
    if (cidx < m.K_prev) {
      const uint8_t* tp = m.tiles + ((long long)tbh * m.ntiles_total + tile) * kImgBytes;
      jpos = ((const int*)(tp + kImgPos))[col];
      const bf16x8_t* kr = (const bf16x8_t*)(tp + col * kKP * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = kr[ks * 2 + hf];
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = bf16x8_t{};
    }
  }
  // smallest and largest column position of the block (columns ascend): rows
  // below the smallest see none of them, rows at or past the largest all
  const int nr = count_of(c, a.r, b);
  if (threadIdx.x == 0) {
    int jmin;
    if (BASE) {
      jmin = cb * W;
      sh_jmax = min(cb * W + W - 1, c.S - 1);
    } else {
      const int ci = cb * W, cl = min(cb * W + W - 1, m.K_prev - 1);
      const uint8_t* t0p = m.tiles + ((long long)tbh * m.ntiles_total + ci / kBN) * kImgBytes;
      const uint8_t* t1p = m.tiles + ((long long)tbh * m.ntiles_total + cl / kBN) * kImgBytes;
      jmin = ((const int*)(t0p + kImgPos))[ci % kBN];
      sh_jmax = ((const int*)(t1p + kImgPos))[cl % kBN];
    }
    const int32_t* rows = c.rows[a.r] + (long long)b * c.n[a.r];
    int lo = 0, hi = nr;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rows[mid] < jmin) lo = mid + 1; else hi = mid;
    }
    sh_t0 = lo;
  }
  __syncthreads();
  const int tile0 = sh_t0 / kMassRows;
  const int ntl = sh_t0 < nr ? (nr + kMassRows - 1) / kMassRows - tile0 : 0;
  const int jmax = sh_jmax;
  const uint8_t* rimg = m.rows + ((long long)bh * m.ntr + tile0) * kRowBytes;

  const __amdgpu_buffer_rsrc_t rs = img_rsrc(rimg, ntl * kRowBytes);
  for (int k = 0; k < kMassAhead && k < ntl; ++k) dma_img<NW, kRowChunks>(rs, k * kRowBytes, lds + k * kRowBytes);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  float acc = 0.0f;
  for (int tt = 0; tt < ntl; ++tt) {
    const uint8_t* T = lds + (tt % kMassRing) * kRowBytes;
    // image tt+kMassAhead goes into the slot image tt-1 left (all waves passed it)
    if (tt + kMassAhead < ntl)
      dma_img<NW, kRowChunks>(rs, (tt + kMassAhead) * kRowBytes, lds + ((tt + kMassAhead) % kMassRing) * kRowBytes);
    const __bf16* tq = (const __bf16*)T;
    const float* toff = (const float*)(T + kRowOffAt);
    const int* tpos = (const int*)(T + kRowPosAt);
    f32x16_t s[2];
    s[0] = s[1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const bf16x8_t qf = *(const bf16x8_t*)&tq[(ib * 32 + l32) * kKP + ks * 16 + hf * 8];
        s[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[ks], s[ib], 0, 0, 0);
      }
    }
    // rows ascend: once the image's first row lies at or after the block's
    // last column, every row of it sees every column (no mask)
    if (tpos[0] >= jmax) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 offv = *(const float4*)&toff[ib * 32 + 8 * g + 4 * hf];
          const float offs[4] = {offv.x, offv.y, offv.z, offv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc += __builtin_amdgcn_exp2f(__builtin_fmaf(s[ib][4 * g + e], m.c2, -offs[e]));
        }
      }
    } else {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rbase = ib * 32 + 8 * g + 4 * hf;
          const float4 offv = *(const float4*)&toff[rbase];
          const int4 pv = *(const int4*)&tpos[rbase];
          const float offs[4] = {offv.x, offv.y, offv.z, offv.w};
          const int ps[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ib][4 * g + e], m.c2, -offs[e]));
            acc += (ps[e] >= jpos) ? p : 0.0f;
          }
        }
      }
    }
    // image tt+1 must be in LDS for every wave
    wait_imgs_but<NW, kRowChunks>(min(tt + kMassAhead, ntl - 1) - (tt + 1));
    lds_barrier();
  }
  acc += __shfl_xor(acc, 32, 64);
  const bool mine = hf == 0 && jpos != kNoPos;
  if (mine) m.mass[(long long)bh * m.K_prev + cidx] = acc;
  if (m.hist) {
    // each column's mass counted once into its head's histogram by the top
    // kHistBits bits of its order key (the first level of the selection);
    // lanes with the same bin add together
    const uint32_t bin = order_key(acc) >> (32 - kHistBits);
    bool part = mine;
    while (__builtin_amdgcn_ballot_w64(part)) {
      const uint64_t pm = __builtin_amdgcn_ballot_w64(part);
      const int leader = __ffsll((long long)pm) - 1;
      const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
      const uint64_t same = __builtin_amdgcn_ballot_w64(part && bin == lb);
      if (lane == leader) atomicAdd(&m.hist[(long long)bh * kHistBins + lb], (uint32_t)__popcll(same));
      if (bin == lb) part = false;
    }
  }
}

// ------------------------------------------------------------- host side
static_assert(kImgBytes == kTileImgBytes && kBN == 64, "tile image size (launch.hpp)");

// Tile images of K columns (sel NULL: positions 0..K-1) at loop rc.
// V16: V^T in the column slots of the 48-row dense kernel.
static hipError_t launch_gather(const CacheGeo& c, int rc, const int32_t* sel, int K, uint8_t* out, hipStream_t st,
                                bool v16 = false) {
  const int nt = (K + kBN - 1) / kBN;
  const int nh = sel ? c.H : c.Hkv;
  const dim3 grid((unsigned)(c.B * nh * nt));
  if (v16) {
    if (c.fmt != kFmtPaper && rc == 1)
      FL_LAUNCH((k_build_tiles<0, true>), grid, dim3(256), 0, st, c, rc, sel, K, nt, out);
    else
      FL_LAUNCH((k_build_tiles<-1, true>), grid, dim3(256), 0, st, c, rc, sel, K, nt, out);
    return hipGetLastError();
  }
  switch (c.fmt == kFmtPaper ? -1 : rc - 1) {
    case 0: FL_LAUNCH(k_build_tiles<0>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 1: FL_LAUNCH(k_build_tiles<1>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 2: FL_LAUNCH(k_build_tiles<2>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 3: FL_LAUNCH(k_build_tiles<3>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 4: FL_LAUNCH(k_build_tiles<4>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 5: FL_LAUNCH(k_build_tiles<5>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 6: FL_LAUNCH(k_build_tiles<6>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    case 7: FL_LAUNCH(k_build_tiles<7>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
    default: FL_LAUNCH(k_build_tiles<-1>, grid, dim3(256), 0, st, c, rc, sel, K, nt, out); break;
  }
  return hipGetLastError();
}

template <int NW, int MODE, int RING, int SRC = 0, int SPLIT = 1>
static hipError_t launch_one(const MfmaArgs& m, hipStream_t st) {
  constexpr size_t lds = (size_t)RING * SPLIT * kImgBytes;
  // once per kernel and process (static initialisation is thread-safe)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_attn_mfma<NW, MODE, RING, SRC, SPLIT>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int nunits = m.a.c.B * m.a.c.H * m.nblk;
  FL_LAUNCH((k_attn_mfma<NW, MODE, RING, SRC, SPLIT>), dim3(nunits), dim3(64 * NW), lds, st, m);
  return hipGetLastError();
}

constexpr int kWideBlocks = 1024;
// Sparse launches take the most column splits whose blocks all fit on the
// chip at once: four splits (32-row blocks, four images: one block per CU),
// else two (64-row blocks, two per CU), else none (128-row blocks, three per
// CU).  Measured on the deep 16K R = 8 workload, loops 4-8: 39/36/35/34/34 us
// unsplit, 37/31/26/25/23 us split; a split launch that needs a second round
// of blocks is slower than the unsplit one (8K workload, loop 2: 45 vs 58 us).
constexpr int kCUs = 256;

static float c2_of(int d) { return (float)(1.4426950408889634 / __builtin_sqrt((double)d)); }

// 384-row blocks of twelve waves (three per SIMD, one block per CU) when
// 256-row blocks would fill the chip four times over; otherwise 128-row
// blocks of four waves: a dense loop 1 with a two-image ring (two blocks per
// CU), the sparse loops and the cached-mass pass with one image (three
// blocks per CU: measured faster there, slower for the dense loop; six-wave
// blocks, two per CU, were slower everywhere).
template <int MODE>
static hipError_t launch_rows(MfmaArgs& m, int n, hipStream_t st, bool own_tiles = false) {
  if constexpr (MODE == kModeAttn) {
    if (own_tiles) {
      m.nblk = (n + 127) / 128;
      return launch_one<4, MODE, 1, 1>(m, st);
    }
  }
  if ((long long)m.a.c.B * m.a.c.H * ((n + 255) / 256) >= kWideBlocks) {
    m.nblk = (n + 383) / 384;
    return launch_one<12, MODE, 2>(m, st);
  }
  m.nblk = (n + 127) / 128;
  if (MODE == kModeAttn && m.a.r == 1) return launch_one<4, MODE, 2>(m, st);
  const long long bh = (long long)m.a.c.B * m.a.c.H;
  if (bh * ((n + 31) / 32) <= kCUs) {
    m.nblk = (n + 31) / 32;
    return launch_one<4, MODE, 1, 0, 4>(m, st);
  }
  if (bh * ((n + 63) / 64) <= 2 * kCUs) {
    m.nblk = (n + 63) / 64;
    return launch_one<4, MODE, 1, 0, 2>(m, st);
  }
  return launch_one<4, MODE, 1>(m, st);
}

// Whether a sparse loop's row blocks build their tiles in LDS themselves
// (FL_TILES=lds, a measurement aid) instead of reading the images built once
// per loop (the default).  Measured slower at every size: 7.6 vs 6.2 ms for
// the 32K step, and even for heads of one or two row blocks (loops 7 and 8
// of the deep 16K workload, 0.17 vs 0.05 ms), where a few dozen blocks each
// build all their tiles in turn while the image builder spreads the same
// work over hundreds of blocks.
static bool own_tiles(int) {
  const char* e = std::getenv("FL_TILES");
  return e && std::strcmp(e, "lds") == 0;
}

// Dense loop 1 on the 48-row kernel (384-row blocks of eight waves, two per
// SIMD, one block per CU) when 256-row blocks would fill the chip four times
// over; smaller launches keep the 32-row kernel's 128-row blocks (two per
// CU), which measured 3 % faster there than 192-row blocks of the 48-row one
// (8K workload, loop 1: 0.32 vs 0.33 ms).
static bool dense48(const CacheGeo& c) {
  return (long long)c.B * c.H * ((c.S + 255) / 256) >= kWideBlocks;
}
template <int NW, int RB>
static hipError_t launch_dense48(MfmaArgs& m, hipStream_t st) {
  constexpr size_t lds = 2 * (size_t)kImgBytes;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_attn_dense48<NW, RB>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  constexpr int BM = 16 * RB * NW;
  m.nblk = (m.a.c.S + BM - 1) / BM;
  FL_LAUNCH((k_attn_dense48<NW, RB>), dim3((unsigned)(m.a.c.B * m.a.c.H * m.nblk)), dim3(64 * NW), lds, st, m);
  return hipGetLastError();
}

// Loop-r attention: r == 1 dense over every position, r >= 2 over S_r.
// ws: gather_bytes(c, K) bytes (K = S at r == 1).
hipError_t launch_attn_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  MfmaArgs m{};
  m.a = a;
  m.c2 = c2_of(a.c.d);
  m.rc = a.r;
  const int K = a.r == 1 ? a.c.S : a.K;
  m.ntiles_total = (K + kBN - 1) / kBN;
  if (a.r >= 2 && own_tiles(a.c.n[a.r])) return launch_rows<kModeAttn>(m, a.c.n[a.r], st, true);
  const bool d48 = a.r == 1 && dense48(a.c);
  hipError_t e = launch_gather(a.c, a.r, a.r == 1 ? nullptr : a.sel, K, ws, st, d48);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  if (d48) return launch_dense48<8, 3>(m, st);
  return launch_rows<kModeAttn>(m, a.r == 1 ? a.c.S : a.c.n[a.r], st);
}

// Cached mass and reused part of loop r over S_r = a.sel (chain r-1).
hipError_t launch_um_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  MfmaArgs m{};
  m.a = a;
  m.c2 = c2_of(a.c.d);
  m.rc = a.r - 1;
  m.ntiles_total = (a.K + kBN - 1) / kBN;
  hipError_t e = launch_gather(a.c, a.r - 1, a.sel, a.K, ws, st);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  return launch_rows<kModeUM>(m, a.c.n[a.r], st);
}

// Column mass of the candidates (r == 2 with cand == NULL reads the base
// directly; otherwise the candidates' chains r-1 are gathered into ws first).
// ws: [candidate tiles: gather_bytes(c, K_prev), only when gathered]
//     [row images: row_img_bytes(B, H, n_r)]
template <bool BASE>
static hipError_t launch_mass_one(const MassArgs& m, hipStream_t st) {
  constexpr size_t lds = (size_t)kMassRing * kRowBytes;
  static const hipError_t attr = hipFuncSetAttribute((const void*)k_mass_mfma<BASE, kMassNW>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int nunits = m.a.c.B * m.a.c.H * m.ncb;
  FL_LAUNCH((k_mass_mfma<BASE, kMassNW>), dim3(nunits), dim3(64 * kMassNW), lds, st, m);
  return hipGetLastError();
}

hipError_t launch_mass_mfma(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                            hipStream_t st, uint32_t* hist, bool* hist_built) {
  MassArgs m{};
  m.a = a;
  m.K_prev = K_prev;
  m.mass = mass;
  m.c2 = c2_of(a.c.d);
  m.ncb = (K_prev + 32 * kMassNW - 1) / (32 * kMassNW);
  // loop-1 chain = the base records themselves (workload format)
  const bool base = !cand && a.r == 2 && a.c.fmt != kFmtPaper;
  uint8_t* rows = ws;
  if (!base) {
    hipError_t e = launch_gather(a.c, a.r - 1, cand, K_prev, ws, st);
    if (e != hipSuccess) return e;
    m.tiles = ws;
    m.ntiles_total = (K_prev + kBN - 1) / kBN;
    m.tiles_kv = cand == nullptr;
    rows = ws + gather_bytes(a.c, K_prev);
  }
  m.ntr = (a.c.n[a.r] + kMassRows - 1) / kMassRows;
  m.rows = rows;
  // the histogram is zeroed by the row-image builder, so it is built only
  // when that runs (no active rows: every mass is 0, nothing to rank by it)
  m.hist = m.ntr > 0 ? hist : nullptr;
  if (hist_built) *hist_built = m.hist != nullptr;
  if (m.ntr > 0) {
    FL_LAUNCH(k_build_rows, dim3((unsigned)(a.c.B * a.c.H * m.ntr)), dim3(256), 0, st, a, m.ntr, rows, m.hist,
              a.c.B * a.c.H * kHistBins);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return base ? launch_mass_one<true>(m, st) : launch_mass_one<false>(m, st);
}

}  // namespace fl
