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
// Lazy rescale threshold (log2 units): a weight P = 2^(x*c2 - mref) may reach
// 2^15 before the reference moves.  fp16 holds it (max 65504), rounds it with
// the same relative error at any size, and keeps weights normal down to 2^-14,
// i.e. scores up to 29 below the row maximum; a lower threshold would only
// rescale more often.
constexpr float kRescale = 15.0f;
constexpr float kRescaleP = 32768.0f;  // 2^kRescale

// Tile image: the exact LDS layout of one 64-column tile, built once per loop
// in HBM and copied into LDS by direct global->LDS loads.
//   K   [64][kKP]  bf16  (row = column of the tile, 272-byte rows)
//   V^T [128][kVP] fp16  (row = head dim, 144-byte rows; within each 16
//                        columns, the 8 a lane multiplies are stored
//                        contiguously: see vt_col)
//   pos [64]       int32 (position of each column, kNoPos for padding)
constexpr int kKP = kD + 8;
constexpr int kVP = kBN + 8;
constexpr int kImgV = kBN * kKP * 2;          // 17408
constexpr int kImgPos = kImgV + kD * kVP * 2;  // 35840
constexpr int kImgBytes = 36 * 1024;           // 36864: 36 chunks of 1 KB (36096 used)
constexpr int kImgChunks = kImgBytes / 1024;
// Tile ring of the attention kernel: two images resident, the next one
// copied while this one is used (72 KB of LDS).
constexpr int kRing = 2;
constexpr int kAhead = kRing - 1;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
// v~ = bf16(x), stored as fp16 (exact for every bf16 value above 2^-17 in
// magnitude; smaller ones round to the fp16 subnormal grid).
__device__ inline _Float16 bf16_as_f16(float x) { return (_Float16)round_bf16(x); }

// ------------------------------------------------------------- tile images
// One block of 256 threads per tile: columns sel[tile*64 .. +64) (sel NULL:
// positions tile*64 ..), reconstructed at loop rc, staged in LDS in the image
// layout and written out with 16-byte stores.  Every packed record a loop
// attends is dequantized exactly once here (p1 §4.4: chosen keys gathered into
// dense buffers; p1 App. G: attention works from the packed streams).
// Column slot of tile column x in the V^T image.  In the S^T = K Q^T
// accumulator a lane of half hf holds, per 16 columns, columns 4hf..4hf+3
// and 8+4hf..8+4hf+3; storing those eight next to each other lets the PV
// product read its B fragment with one 16-byte LDS load.
__host__ __device__ constexpr int vt_col(int x) {
  return (x & ~15) + ((x >> 2) & 1) * 8 + ((x >> 3) & 1) * 4 + (x & 3);
}
static_assert(vt_col(0) == 0 && vt_col(4) == 8 && vt_col(8) == 4 && vt_col(12) == 12 && vt_col(21) == 25,
              "V^T column slots");

__global__ __launch_bounds__(256) void k_build_tiles(CacheGeo c, int rc, const int32_t* __restrict__ sel, int K,
                                                     int ntiles, uint8_t* __restrict__ out) {
  __shared__ __align__(16) uint8_t img[kImgBytes];
  // sel NULL: the tiles of positions 0..K-1 are the same for every query
  // head of a KV head, so they are built once per (b, KV head)
  const int bh = blockIdx.x / ntiles;
  const int tile = blockIdx.x - bh * ntiles;
  const int nh = sel ? c.H : c.Hkv;
  const int b = bh / nh;
  const int hk = sel ? kv_head(c, bh - b * nh) : bh - b * nh;
  const int t = threadIdx.x;
  const int col = t >> 2, g = t & 3;
  const int idx = tile * kBN + col;
  const int j = idx < K ? (sel ? sel[(long long)bh * K + idx] : idx) : -1;
  float x[32];
  // K rows (bf16)
  if (j >= 0) {
    if (c.fmt == kFmtPaper) {
      paper_chain16(c, rc, 0, b, hk, j, 0, g * 32, x);
      paper_chain16(c, rc, 0, b, hk, j, 0, g * 32 + 16, x + 16);
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
  // V^T rows (bf16 value in fp16)
  if (j >= 0) {
    if (c.fmt == kFmtPaper) {
      paper_chain16(c, rc, 0, b, hk, j, 1, g * 32, x);
      paper_chain16(c, rc, 0, b, hk, j, 1, g * 32 + 16, x + 16);
    } else {
      chain_group(c, rc, 0, b, hk, j, 1, g, x);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.0f;
  }
  {
    _Float16* vt = (_Float16*)(img + kImgV);
    const int vc = vt_col(col);
#pragma unroll
    for (int e = 0; e < 32; ++e) vt[(g * 32 + e) * kVP + vc] = bf16_as_f16(x[e]);
  }
  if (g == 0) ((int*)(img + kImgPos))[col] = j >= 0 ? j : kNoPos;
  __syncthreads();
  uint4* dst = (uint4*)(out + ((long long)bh * ntiles + tile) * kImgBytes);
  const uint4* src = (const uint4*)img;
  for (int i = t; i < kImgBytes / 16; i += 256) dst[i] = src[i];
}

// ------------------------------------------------------------- main kernel
enum { kModeAttn = 0, kModeUM = 1 };

struct MfmaArgs {
  AttnArgs a;
  const uint8_t* tiles;   // tile images [B][H][ntiles_total]
  int ntiles_total;       // tiles per (b, h)
  int nblk;               // row blocks per (b, h)
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

// Workgroup barrier for the tile ring: the wave's LDS reads have returned
// (lgkmcnt 0) and the compiler may not move memory operations across it, but
// unlike __syncthreads it does not drain the wave's in-flight tile copies.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
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
// unset); the row sum and accumulators are rescaled then.  Otherwise every
// weight 2^(x*c2 - mref) stays below 2^kRescale and fp16 holds it.
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
template <int MODE>
__device__ inline void write_row(const AttnArgs& a, int r, long long bhS, int i, int hf, float mref, float lt,
                                 const f32x16_t* o) {
  if (i < 0) return;
  const long long rowp = (bhS + i) * kD;
  if (MODE == kModeAttn) {
    if (r == 1) {
      const float inv = 1.0f / lt;
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
      const float sc = ca / lt;
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
      const float sc = Mi / lt;
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
    const float Mp = a.M[bhS + i];
    const float Mu = Mp > 0.0f ? Mp : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int dcol = db * 32 + qq * 8 + hf * 4;
        const f32x4_t ov = *(const f32x4_t*)&a.O[rowp + dcol];
        f32x4_t uv;
#pragma unroll
        for (int e = 0; e < 4; ++e) uv[e] = ov[e] - Mu * o[db][qq * 4 + e];
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
template <int NW, int MODE>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void k_attn_mfma(MfmaArgs m) {
  constexpr int BM = 32 * NW;
  extern __shared__ __align__(16) uint8_t lds[];   // kRing tile images
  __shared__ int sh_ntiles;
  const AttnArgs& a = m.a;
  const CacheGeo& c = a.c;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hf = lane >> 5;       // half of the wave
  const int l32 = lane & 31;

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
  const uint8_t* imgs = m.tiles + tbh * m.ntiles_total * kImgBytes;

  // ---- the lane's row and its queries (B operand of S^T = K Q^T)
  int ipos = -1;
  bf16x8_t qf[8];
  {
    const int t = row0 + wv * 32 + l32;
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
  if (threadIdx.x == 0) {
    int lo = 0, hi = m.ntiles_total;  // first tile whose first column lies beyond blk_max
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int p0 = *(const int*)(imgs + (long long)mid * kImgBytes + kImgPos);
      if (p0 <= blk_max) lo = mid + 1; else hi = mid;
    }
    sh_ntiles = lo;
  }

  // row state: mref = reference max (log2 units), lsum = partial row sum
  float mref = -INFINITY, lsum = 0.0f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};
  if (MODE == kModeUM) {
    // loop r-1 statistics of the row: P = M * 2^(x - lse*log2e)
    float Mp = 0.0f, lp = 0.0f;
    if (ipos >= 0) {
      Mp = a.M[bhS + ipos];
      lp = a.lse[bhS + ipos];
    }
    mref = (Mp > 0.0f) ? lp * 1.4426950408889634f : INFINITY;
  }
  __syncthreads();
  const int nt = sh_ntiles;

  // ---- prologue: the first kAhead tiles into the ring
  const __amdgpu_buffer_rsrc_t rs = img_rsrc(imgs, m.ntiles_total * kImgBytes);
  for (int k = 0; k < kAhead && k < nt; ++k) dma_tile<NW>(rs, k * kImgBytes, lds + k * kImgBytes);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int tt = 0; tt < nt; ++tt) {
    const uint8_t* T = lds + (tt % kRing) * kImgBytes;
    // tile tt+kAhead goes into the slot tile tt-1 left (all waves passed it)
    if (tt + kAhead < nt)
      dma_tile<NW>(rs, (tt + kAhead) * kImgBytes, lds + ((tt + kAhead) % kRing) * kImgBytes);
    f32x16_t s0, s1;
    qk_tile(T, qf, l32, hf, s0, s1);
    float x[32];
    softmax_mask(T, s0, s1, ipos, blk_min, hf, x);
    // Weights against the current reference (UM: the fixed loop r-1
    // statistics).  ATTN: only if a lane's sum exceeds 2^kRescale (so some
    // weight might) or a valid row has no reference yet is the tile max
    // taken, the lazy rescale applied and the weights formed again.
    f16x8_t pf[4];
    float ls = softmax_probs(x, (MODE == kModeAttn && mref == -INFINITY) ? 0.0f : mref, m.c2, pf);
    if (MODE == kModeAttn) {
      const bool bad = (ipos >= 0 && mref == -INFINITY) || !(ls <= kRescaleP);
      if (__builtin_amdgcn_ballot_w64(bad)) {
        softmax_rescale(x, m.c2, mref, lsum, o);
        ls = softmax_probs(x, mref == -INFINITY ? 0.0f : mref, m.c2, pf);
      }
    }
    lsum += ls;
    pv_tile(T, pf, l32, hf, o);
    // tile tt+1 must be in LDS for every wave
    wait_tiles_but<NW>(min(tt + kAhead, nt - 1) - (tt + 1));
    lds_barrier();
  }

  // ---- epilogue: each lane writes 64 of its row's 128 dims
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  write_row<MODE>(a, r, bhS, ipos, hf, mref, lt, o);
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

size_t row_img_bytes(int B, int H, int n) {
  return (size_t)B * H * ((n + kMassRows - 1) / kMassRows) * kRowBytes;
}

// One block of 256 threads per row image: four threads per row, 32 dims each.
__global__ __launch_bounds__(256) void k_build_rows(AttnArgs a, int ntr, uint8_t* __restrict__ out) {
  const CacheGeo& c = a.c;
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
  if (hf == 0 && jpos != kNoPos) m.mass[(long long)bh * m.K_prev + cidx] = acc;
}

// ------------------------------------------------------------- host side
size_t gather_bytes(const CacheGeo& c, int K) {
  const int nt = (K + kBN - 1) / kBN;
  return (size_t)c.B * c.H * nt * kImgBytes;
}

// Tile images of K columns (sel NULL: positions 0..K-1) at loop rc.
hipError_t launch_gather(const CacheGeo& c, int rc, const int32_t* sel, int K, uint8_t* out, hipStream_t st) {
  const int nt = (K + kBN - 1) / kBN;
  const int nh = sel ? c.H : c.Hkv;
  hipLaunchKernelGGL(k_build_tiles, dim3((unsigned)(c.B * nh * nt)), dim3(256), 0, st, c, rc, sel, K, nt, out);
  return hipGetLastError();
}

template <int NW, int MODE>
static hipError_t launch_one(const MfmaArgs& m, hipStream_t st) {
  constexpr size_t lds = (size_t)kRing * kImgBytes;
  // once per kernel and process (static initialisation is thread-safe)
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)k_attn_mfma<NW, MODE>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int nunits = m.a.c.B * m.a.c.H * m.nblk;
  hipLaunchKernelGGL((k_attn_mfma<NW, MODE>), dim3(nunits), dim3(64 * NW), lds, st, m);
  return hipGetLastError();
}

constexpr int kWideBlocks = 1024;

static float c2_of(int d) { return (float)(1.4426950408889634 / __builtin_sqrt((double)d)); }

// 384-row blocks of twelve waves (three per SIMD, one block per CU) when
// 256-row blocks would fill the chip four times over; otherwise 128-row
// blocks of four waves, two blocks per CU.
template <int MODE>
static hipError_t launch_rows(MfmaArgs& m, int n, hipStream_t st) {
  if ((long long)m.a.c.B * m.a.c.H * ((n + 255) / 256) >= kWideBlocks) {
    m.nblk = (n + 383) / 384;
    return launch_one<12, MODE>(m, st);
  }
  m.nblk = (n + 127) / 128;
  return launch_one<4, MODE>(m, st);
}

// Loop-r attention: r == 1 dense over every position, r >= 2 over S_r.
// ws: gather_bytes(c, K) bytes (K = S at r == 1).
hipError_t launch_attn_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  MfmaArgs m{};
  m.a = a;
  m.c2 = c2_of(a.c.d);
  const int K = a.r == 1 ? a.c.S : a.K;
  hipError_t e = launch_gather(a.c, a.r, a.r == 1 ? nullptr : a.sel, K, ws, st);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  m.ntiles_total = (K + kBN - 1) / kBN;
  return launch_rows<kModeAttn>(m, a.r == 1 ? a.c.S : a.c.n[a.r], st);
}

// Cached mass and reused part of loop r over S_r = a.sel (chain r-1).
hipError_t launch_um_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  MfmaArgs m{};
  m.a = a;
  m.c2 = c2_of(a.c.d);
  hipError_t e = launch_gather(a.c, a.r - 1, a.sel, a.K, ws, st);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  m.ntiles_total = (a.K + kBN - 1) / kBN;
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
  hipLaunchKernelGGL((k_mass_mfma<BASE, kMassNW>), dim3(nunits), dim3(64 * kMassNW), lds, st, m);
  return hipGetLastError();
}

hipError_t launch_mass_mfma(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                            hipStream_t st) {
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
  if (m.ntr > 0) {
    hipLaunchKernelGGL(k_build_rows, dim3((unsigned)(a.c.B * a.c.H * m.ntr)), dim3(256), 0, st, a, m.ntr, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return base ? launch_mass_one<true>(m, st) : launch_mass_one<false>(m, st);
}

}  // namespace fl
