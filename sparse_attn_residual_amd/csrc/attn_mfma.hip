// Matrix-core kernels of the prefill loop attention (bf16 inputs, head dim 128).
//
// What is computed follows the FlashLoop pages: loop 1 is dense causal
// attention over the reconstructed base (p1 §D.1 and the workload's dense
// first loop); loop r >= 2 recomputes the active rows only against the
// selected columns and rescales by the cached mass (p1 §4.1, §4.2, §D.2;
// guide §3); the cached mass M and reused part U come from loop r-1's
// probabilities over the selected columns (p1 §D.2: cached key indices and
// their global mass).
//
// Design (gfx950, wave64):
//  * a 256-thread block owns BM = 4 waves x 32*RB query rows; a wave keeps
//    its queries in registers as the B operand of S^T = K Q^T
//    (v_mfma_f32_32x32x16_bf16), so each lane holds one query row's scores
//    and the row softmax needs one cross-half exchange per tile;
//  * key tiles of 64 columns: K stored row-major (bf16) and V transposed
//    (fp16) in LDS, double buffered, the next tile's global loads in flight
//    while the current one is multiplied;
//  * P is rounded to fp16 (not bf16) for O^T += V^T P^T on
//    v_mfma_f32_32x32x16_f16: P in [0, 1] needs significand, not range, and
//    bf16 rounding alone would spend the whole error budget; the bf16 value
//    v~ converts to fp16 exactly;
//  * loop 1 dequantizes the int8 base records into the LDS tiles inside the
//    kernel; sparse loops read the compact tiles gathered by k_gather_cols
//    (p1 §4.4: selected tokens and keys gathered into compact buffers).
#include "launch.hpp"

namespace fl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kBN = 64;        // key columns per tile
constexpr int kKP = kD + 8;    // LDS pitch of the K tile (bf16 elements): 272 B
constexpr int kVP = kBN + 4;   // LDS pitch of the V^T tile (fp16 elements): 136 B
constexpr int kNoPos = 0x7fffffff;  // padding column: masked for every row
constexpr float kRescale = 8.0f;    // lazy rescale threshold (log2 units): P <= 2^8

struct __align__(16) Tile {
  __bf16 k[kBN * kKP];
  _Float16 vt[kD * kVP];
  int pos[kBN];
};

// Compact gathered tiles (k_gather_cols): per (b, h, tile): K [64][128] bf16,
// then V^T [128][64] fp16, then positions [64] int32.
constexpr int kTileKBytes = kBN * kD * 2;
constexpr int kTileVBytes = kD * kBN * 2;
constexpr int kTileBytes = kTileKBytes + kTileVBytes + kBN * 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}
// v~ = bf16(x) converted to fp16 (exact for every bf16 value above 2^-17 in
// magnitude; smaller values round to the fp16 subnormal grid).
__device__ inline _Float16 bf16_as_f16(float x) { return (_Float16)round_bf16(x); }
__device__ inline void bf16x2_as_f16(float a, float b, _Float16& ha, _Float16& hb) {
  const uint32_t w = pack_bf16x2(a, b);
  ha = (_Float16)__uint_as_float(w << 16);
  hb = (_Float16)__uint_as_float(w & 0xFFFF0000u);
}

// ------------------------------------------------------------- tile loaders
// Loop-1 loader: columns j0..j0+63 of the int8 base of (b, h), NT threads.
template <int NT>
struct BaseRegs {
  static constexpr int KCH = kBN * kD / NT;        // K codes per thread (16 or 32)
  static constexpr int VCOL = kBN * 32 / NT;       // V columns per thread (4 or 8)
  uint32_t kc[KCH / 4];
  uint16_t ks;
  uint32_t vc[VCOL];
  uint16_t vs[VCOL];
};

template <int NT>
__device__ inline void fetch_base(const uint8_t* recs, int rb, int S, int j0, BaseRegs<NT>& R) {
  using BR = BaseRegs<NT>;
  const int t = threadIdx.x;
  constexpr int PER = kD / BR::KCH;  // threads per column for K
  const int col = t / PER, part = t % PER;
  const int j = j0 + col;
  if (j < S) {
    const uint8_t* rec = recs + (uint32_t)j * rb;
#pragma unroll
    for (int w = 0; w < BR::KCH / 16; ++w) {
      const uint4 v = *(const uint4*)(rec + part * BR::KCH + w * 16);
      R.kc[4 * w] = v.x; R.kc[4 * w + 1] = v.y; R.kc[4 * w + 2] = v.z; R.kc[4 * w + 3] = v.w;
    }
    R.ks = ((const uint16_t*)(rec + 2 * kD))[part * BR::KCH / 32];
  } else {
#pragma unroll
    for (int w = 0; w < BR::KCH / 4; ++w) R.kc[w] = 0;
    R.ks = 0;
  }
  const int d4 = t & 31, jg = t >> 5;
#pragma unroll
  for (int e = 0; e < BR::VCOL; ++e) {
    const int jj = j0 + jg * BR::VCOL + e;
    if (jj < S) {
      const uint8_t* rec = recs + (uint32_t)jj * rb;
      R.vc[e] = *(const uint32_t*)(rec + kD + d4 * 4);
      R.vs[e] = ((const uint16_t*)(rec + 2 * kD))[4 + (d4 >> 3)];
    } else {
      R.vc[e] = 0;
      R.vs[e] = 0;
    }
  }
}

template <int NT>
__device__ inline void store_base(int S, int j0, const BaseRegs<NT>& R, Tile& T) {
  using BR = BaseRegs<NT>;
  const int t = threadIdx.x;
  constexpr int PER = kD / BR::KCH;
  const int col = t / PER, part = t % PER;
  {
    const float s = h2f(R.ks);
    uint32_t o[BR::KCH / 2];
#pragma unroll
    for (int i = 0; i < BR::KCH / 4; ++i) {
      const uint32_t w = R.kc[i];
      o[2 * i] = pack_bf16x2((float)(int8_t)(w) * s, (float)(int8_t)(w >> 8) * s);
      o[2 * i + 1] = pack_bf16x2((float)(int8_t)(w >> 16) * s, (float)(int8_t)(w >> 24) * s);
    }
    uint4* dst = (uint4*)&T.k[col * kKP + part * BR::KCH];
#pragma unroll
    for (int i = 0; i < BR::KCH / 8; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
  {
    const int d4 = t & 31, jg = t >> 5;
    _Float16 out[4][BR::VCOL];
#pragma unroll
    for (int e = 0; e < BR::VCOL; ++e) {
      const float s = h2f(R.vs[e]);
      const uint32_t w = R.vc[e];
      bf16x2_as_f16((float)(int8_t)(w) * s, (float)(int8_t)(w >> 8) * s, out[0][e], out[1][e]);
      bf16x2_as_f16((float)(int8_t)(w >> 16) * s, (float)(int8_t)(w >> 24) * s, out[2][e], out[3][e]);
    }
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      _Float16* dst = &T.vt[(d4 * 4 + dd) * kVP + jg * BR::VCOL];
      if constexpr (BR::VCOL == 4) {
        *(f16x4_t*)dst = f16x4_t{out[dd][0], out[dd][1], out[dd][2], out[dd][3]};
      } else {
        *(f16x4_t*)dst = f16x4_t{out[dd][0], out[dd][1], out[dd][2], out[dd][3]};
        *(f16x4_t*)(dst + 4) = f16x4_t{out[dd][4], out[dd][5], out[dd][6], out[dd][7]};
      }
    }
  }
  if (t < kBN) T.pos[t] = (j0 + t < S) ? j0 + t : kNoPos;
}

// Compact-tile loader (sparse loops), NT threads.
template <int NT>
struct CompactRegs {
  static constexpr int N16 = kTileKBytes / 16 / NT;  // uint4 per thread per half (4 or 2)
  uint4 k[N16];
  uint4 v[N16];
  int pos;
};

template <int NT>
__device__ inline void fetch_compact(const uint8_t* tile, CompactRegs<NT>& R) {
  using CR = CompactRegs<NT>;
  const int t = threadIdx.x;
  const uint4* ks = (const uint4*)(tile + t * CR::N16 * 16);
  const uint4* vs = (const uint4*)(tile + kTileKBytes + t * CR::N16 * 16);
#pragma unroll
  for (int i = 0; i < CR::N16; ++i) {
    R.k[i] = ks[i];
    R.v[i] = vs[i];
  }
  R.pos = t < kBN ? ((const int*)(tile + kTileKBytes + kTileVBytes))[t] : 0;
}

template <int NT>
__device__ inline void store_compact(const CompactRegs<NT>& R, Tile& T) {
  using CR = CompactRegs<NT>;
  const int t = threadIdx.x;
  // K: byte offset t*N16*16 in a [64][128] bf16 tile
  const int kb = t * CR::N16 * 8;  // element offset
  uint4* kd = (uint4*)&T.k[(kb / kD) * kKP + kb % kD];
  // V^T: element offset in a [128][64] fp16 tile
  const int vb = t * CR::N16 * 8;
  _Float16* vd = &T.vt[(vb / kBN) * kVP + vb % kBN];
#pragma unroll
  for (int i = 0; i < CR::N16; ++i) {
    kd[i] = R.k[i];
    // rows of V^T are 136 B apart in LDS: store in 8-byte halves
    const uint4 w = R.v[i];
    *(uint2*)(vd + 8 * i) = make_uint2(w.x, w.y);
    *(uint2*)(vd + 8 * i + 4) = make_uint2(w.z, w.w);
  }
  if (t < kBN) T.pos[t] = R.pos;
}

// ------------------------------------------------------------- main kernel
enum { kModeAttn = 0, kModeUM = 1 };

struct MfmaArgs {
  AttnArgs a;
  const uint8_t* tiles;   // compact tiles [B][H][ntiles] (sparse loaders)
  int ntiles_total;       // tiles per (b, h) in `tiles`
  int nblk;               // row blocks per (b, h)
  float c2;               // tau * log2(e)
};

// NW waves of 32 query rows each; BM = 32 * NW rows per block.
template <int NW, int MODE, bool BASE>
__global__ __launch_bounds__(64 * NW) void k_attn_mfma(MfmaArgs m) {
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NW;
  __shared__ Tile tiles[2];
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
  const int b = bh / c.H, h = bh - b * c.H;

  const int r = a.r;
  const bool dense = r == 1 && MODE == kModeAttn;
  const int nrows = dense ? c.S : c.n[r];
  const int row0 = blk * BM;
  const long long bhS = (long long)bh * c.S;

  // ---- the lane's row, its queries (B operand of S^T = K Q^T)
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
  const uint8_t* ctiles = BASE ? nullptr : m.tiles + (long long)bh * m.ntiles_total * kTileBytes;
  const uint8_t* recs = BASE ? base_rec(c, 0, b, h, 0) : nullptr;
  if (threadIdx.x == 0) {
    int nt;
    if (BASE) {
      nt = (min(blk_max, c.S - 1) + kBN) / kBN;
    } else {
      int lo = 0, hi = m.ntiles_total;  // first tile whose first column lies beyond blk_max
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int p0 = ((const int*)(ctiles + (long long)mid * kTileBytes + kTileKBytes + kTileVBytes))[0];
        if (p0 <= blk_max) lo = mid + 1; else hi = mid;
      }
      nt = lo;
    }
    sh_ntiles = nt;
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
  const int ntiles = sh_ntiles;

  BaseRegs<NT> breg;
  CompactRegs<NT> creg;
  if (ntiles > 0) {
    if (BASE) {
      fetch_base<NT>(recs, c.base_rb, c.S, 0, breg);
      store_base<NT>(c.S, 0, breg, tiles[0]);
    } else {
      fetch_compact<NT>(ctiles, creg);
      store_compact<NT>(creg, tiles[0]);
    }
  }
  __syncthreads();

  for (int tt = 0; tt < ntiles; ++tt) {
    const Tile& T = tiles[tt & 1];
    const bool more = tt + 1 < ntiles;
    if (more) {
      if (BASE) fetch_base<NT>(recs, c.base_rb, c.S, (tt + 1) * kBN, breg);
      else fetch_compact<NT>(ctiles + (long long)(tt + 1) * kTileBytes, creg);
    }
    // ---- S^T = K Q^T for the 64 columns of the tile
    f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t k0 = *(const bf16x8_t*)&T.k[l32 * kKP + ks * 16 + hf * 8];
      const bf16x8_t k1 = *(const bf16x8_t*)&T.k[(32 + l32) * kKP + ks * 16 + hf * 8];
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[ks], s1, 0, 0, 0);
    }
    // ---- softmax of the lane's row over the tile's columns
    float x[32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = s0[v];
      x[16 + v] = s1[v];
    }
    if (T.pos[kBN - 1] > blk_min || ipos < 0) {
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int col = (v >> 4) * 32 + 8 * ((v & 15) >> 2) + 4 * hf + (v & 3);
        if (T.pos[col] > ipos) x[v] = -INFINITY;
      }
    }
    if (MODE == kModeAttn) {
      float mt = x[0];
#pragma unroll
      for (int v = 1; v < 32; ++v) mt = fmaxf(mt, x[v]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * m.c2;
      // rescale only when the row max outgrows the reference by 2^8 (or the
      // reference is unset); otherwise P stays below 2^8 and fp16 holds it
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
    const float base = (MODE == kModeAttn && mref == -INFINITY) ? 0.0f : mref;
    f16x8_t pf[4];
    float ls = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[k2 * 8 + e], m.c2, -base));
        ls += p;
        pf[k2][e] = (_Float16)p;
      }
    }
    lsum += ls;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int c0 = k2 * 16 + hf * 4;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const _Float16* vp = &T.vt[(db * 32 + l32) * kVP + c0];
        const f16x4_t lo4 = *(const f16x4_t*)vp;
        const f16x4_t hi4 = *(const f16x4_t*)(vp + 8);
        const f16x8_t vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[k2], o[db], 0, 0, 0);
      }
    }
    if (more) {
      if (BASE) store_base<NT>(c.S, (tt + 1) * kBN, breg, tiles[(tt + 1) & 1]);
      else store_compact<NT>(creg, tiles[(tt + 1) & 1]);
    }
    __syncthreads();
  }

  // ---- epilogue: each lane writes 64 of its row's 128 dims
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  if (ipos < 0) return;
  const int i = ipos;
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
    if (hf == 0) a.M[bhS + i] = Mu * lt;
  }
}

// ------------------------------------------------------------- gather
// Compact tiles of the selected columns' reconstructions at loop `rc`:
// K~ (bf16, row-major) and V~ (bf16 value stored as fp16, transposed).
// One thread per (column, 32-dim group, K|V).
__global__ __launch_bounds__(256) void k_gather_cols(CacheGeo c, int rc, const int32_t* __restrict__ sel, int K,
                                                     int ntiles, uint8_t* __restrict__ out) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_bh = ntiles * kBN * 8;
  if (gid >= (long long)c.B * c.H * per_bh) return;
  const int bh = (int)(gid / per_bh);
  const int rem = (int)(gid - (long long)bh * per_bh);
  const int colg = rem >> 3;  // column slot in [0, ntiles*64)
  const int sub = rem & 7;
  const int kv = sub >> 2, g = sub & 3;
  const int b = bh / c.H, h = bh - b * c.H;
  const int tile = colg / kBN, col = colg - tile * kBN;
  uint8_t* tp = out + ((long long)bh * ntiles + tile) * kTileBytes;
  const int j = colg < K ? (sel ? sel[(long long)bh * K + colg] : colg) : -1;  // sel NULL: every position
  if (sub == 0) ((int*)(tp + kTileKBytes + kTileVBytes))[col] = j >= 0 ? j : kNoPos;
  float x[32];
  if (j >= 0) {
#pragma unroll 4
    for (int e = 0; e < 32; ++e) x[e] = chain_elem(c, rc, 0, b, h, j, kv, g * 32 + e);
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.0f;
  }
  if (kv == 0) {
    uint32_t w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    uint4* dst = (uint4*)(tp + (col * kD + g * 32) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else {
    _Float16* vt = (_Float16*)(tp + kTileKBytes);
#pragma unroll
    for (int e = 0; e < 32; ++e) vt[(g * 32 + e) * kBN + col] = bf16_as_f16(x[e]);
  }
}

// ------------------------------------------------------------- column mass
// c_j = sum_{i in A_r, i >= j} P^(r-1)_ij for the candidate columns (p1 §4.2
// and §D.2: columns ranked by the preceding loop's attention statistics over
// the rows loop r recomputes), with P^(r-1)_ij = M_i 2^(x_ij - lse_i log2 e).
// A block owns 128 candidate columns (32 per wave, their K fragments held in
// registers as the B operand of S = Q K^T, so each lane owns one column) and
// streams the active rows' loop r-1 queries through LDS in tiles of 64 rows,
// double buffered.  Column sums accumulate in a fixed order: deterministic.
constexpr int kMassRows = 64;
constexpr int kThreads = 256;

struct __align__(16) RowTile {
  __bf16 q[kMassRows * kKP];
  float off[kMassRows];   // lse * log2(e), +inf when the row had no column left
  float M[kMassRows];
  int pos[kMassRows];
};

struct MassArgs {
  AttnArgs a;
  const int32_t* cand;    // NULL: every position (r == 2 over the base)
  int K_prev;
  float* mass;
  const uint8_t* tiles;   // compact tiles of the candidates (cand != NULL)
  int ntiles_total;
  int ncb;                // column blocks per (b, h)
  float c2;
};

struct RowRegs {
  uint4 q[4];
  float off, M;
  int pos;
};

__device__ inline void fetch_rows(const CacheGeo& c, const AttnArgs& a, int b, int bh, int t0, RowRegs& R) {
  const int t = threadIdx.x;
  const int row = t >> 2, qd = t & 3;
  const int r = a.r, rp = r - 1;
  const int nr = c.n[r];
  const int np = rp == 1 ? c.S : c.n[rp];
  int tr = t0 + row;
  int qi = -1, i = -1;
  if (tr < nr) {
    i = c.rows[r][(long long)b * nr + tr];
    qi = rp == 1 ? i : c.slot[rp][(long long)b * c.S + i];
  }
  if (qi >= 0) {
    const uint4* src = (const uint4*)((const uint16_t*)a.q + ((long long)bh * np + qi) * kD + qd * 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) R.q[k] = src[k];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) R.q[k] = make_uint4(0, 0, 0, 0);
  }
  R.pos = -1;
  R.off = INFINITY;
  R.M = 0.0f;
  if (t < kMassRows) {
    const int tr2 = t0 + t;
    if (tr2 < nr) {
      const int i2 = c.rows[r][(long long)b * nr + tr2];
      const int q2 = rp == 1 ? i2 : c.slot[rp][(long long)b * c.S + i2];
      const long long p = (long long)bh * c.S + i2;
      const float Mp = a.M[p];
      if (q2 >= 0 && Mp > 0.0f) {
        R.pos = i2;
        R.M = Mp;
        R.off = a.lse[p] * 1.4426950408889634f;
      }
    }
  }
}

__device__ inline void store_rows(const RowRegs& R, RowTile& T) {
  const int t = threadIdx.x;
  const int row = t >> 2, qd = t & 3;
  uint4* dst = (uint4*)&T.q[row * kKP + qd * 32];
#pragma unroll
  for (int k = 0; k < 4; ++k) dst[k] = R.q[k];
  if (t < kMassRows) {
    T.pos[t] = R.pos;
    T.off[t] = R.off;
    T.M[t] = R.M;
  }
}

template <bool BASE>
__global__ __launch_bounds__(kThreads) void k_mass_mfma(MassArgs m) {
  __shared__ RowTile rt[2];
  __shared__ int sh_t0;
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

  // ---- this lane's candidate column: position jpos, candidate index cidx
  const int cidx = cb * 128 + wv * 32 + l32;
  int jpos = kNoPos;
  bf16x8_t kf[8];
  if (BASE) {
    if (cidx < c.S) {
      jpos = cidx;
      const uint8_t* rec = base_rec(c, 0, b, h, cidx);
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
      const uint8_t* tp = m.tiles + ((long long)bh * m.ntiles_total + tile) * kTileBytes;
      jpos = ((const int*)(tp + kTileKBytes + kTileVBytes))[col];
      const bf16x8_t* kr = (const bf16x8_t*)(tp + col * kD * 2);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = kr[ks * 2 + hf];
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = bf16x8_t{};
    }
  }
  // smallest column position of the block: rows below it see none of them
  const int nr = c.n[a.r];
  if (threadIdx.x == 0) {
    int jmin;
    if (BASE) {
      jmin = cb * 128;
    } else {
      const int ci = cb * 128;
      const int tile = ci / kBN;
      const uint8_t* tp = m.tiles + ((long long)bh * m.ntiles_total + tile) * kTileBytes;
      jmin = ((const int*)(tp + kTileKBytes + kTileVBytes))[ci - tile * kBN];
    }
    const int32_t* rows = c.rows[a.r] + (long long)b * nr;
    int lo = 0, hi = nr;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rows[mid] < jmin) lo = mid + 1; else hi = mid;
    }
    sh_t0 = lo;
  }
  __syncthreads();
  const int t0 = sh_t0;
  const int ntl = (nr - t0 + kMassRows - 1) / kMassRows;
  // the block's largest column position (tiles beyond it need no mask)
  int jmax_l = jpos == kNoPos ? -1 : jpos;
  float acc = 0.0f;
  RowRegs rr;
  if (ntl > 0) {
    fetch_rows(c, a, b, bh, t0, rr);
    store_rows(rr, rt[0]);
  }
  __syncthreads();
  for (int tt = 0; tt < ntl; ++tt) {
    const RowTile& T = rt[tt & 1];
    const bool more = tt + 1 < ntl;
    if (more) fetch_rows(c, a, b, bh, t0 + (tt + 1) * kMassRows, rr);
    f32x16_t s[2];
    s[0] = s[1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const bf16x8_t qf = *(const bf16x8_t*)&T.q[(ib * 32 + l32) * kKP + ks * 16 + hf * 8];
        s[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[ks], s[ib], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rbase = ib * 32 + 8 * g + 4 * hf;
        const float4 offv = *(const float4*)&T.off[rbase];
        const float4 Mv = *(const float4*)&T.M[rbase];
        const int4 pv = *(const int4*)&T.pos[rbase];
        const float offs[4] = {offv.x, offv.y, offv.z, offv.w};
        const float Ms[4] = {Mv.x, Mv.y, Mv.z, Mv.w};
        const int ps[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = Ms[e] * __builtin_amdgcn_exp2f(__builtin_fmaf(s[ib][4 * g + e], m.c2, -offs[e]));
          acc += (ps[e] >= jpos) ? p : 0.0f;
        }
      }
    }
    if (more) store_rows(rr, rt[(tt + 1) & 1]);
    __syncthreads();
  }
  (void)jmax_l;
  acc += __shfl_xor(acc, 32, 64);
  if (hf == 0 && jpos != kNoPos) m.mass[(long long)bh * m.K_prev + cidx] = acc;
}

// ------------------------------------------------------------- host side
size_t gather_bytes(const CacheGeo& c, int K) {
  const int nt = (K + kBN - 1) / kBN;
  return (size_t)c.B * c.H * nt * kTileBytes;
}

hipError_t launch_gather(const CacheGeo& c, int rc, const int32_t* sel, int K, uint8_t* out, hipStream_t st) {
  const int nt = (K + kBN - 1) / kBN;
  const long long threads = (long long)c.B * c.H * nt * kBN * 8;
  hipLaunchKernelGGL(k_gather_cols, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, c, rc, sel, K, nt,
                     out);
  return hipGetLastError();
}

template <int NW, int MODE, bool BASE>
static hipError_t launch_one(const MfmaArgs& m, hipStream_t st) {
  const int nunits = m.a.c.B * m.a.c.H * m.nblk;
  hipLaunchKernelGGL((k_attn_mfma<NW, MODE, BASE>), dim3(nunits), dim3(64 * NW), 0, st, m);
  return hipGetLastError();
}

static float c2_of(int d) { return (float)(1.4426950408889634 / __builtin_sqrt((double)d)); }

// Sparse-row launch: 8-wave blocks when they still fill the chip twice.
template <int MODE>
static hipError_t launch_rows(MfmaArgs& m, int n, hipStream_t st) {
  if ((long long)m.a.c.B * m.a.c.H * ((n + 255) / 256) >= 512) {
    m.nblk = (n + 255) / 256;
    return launch_one<8, MODE, false>(m, st);
  }
  m.nblk = (n + 127) / 128;
  return launch_one<4, MODE, false>(m, st);
}

// Loop-r attention: r == 1 dense over the base; r >= 2 over gathered tiles
// (ws: gather_bytes(c, K) bytes).
hipError_t launch_attn_mfma(const AttnArgs& a, uint8_t* ws, hipStream_t st) {
  MfmaArgs m{};
  m.a = a;
  m.c2 = c2_of(a.c.d);
  if (a.r == 1) {
    m.nblk = (a.c.S + 255) / 256;
    return launch_one<8, kModeAttn, true>(m, st);
  }
  hipError_t e = launch_gather(a.c, a.r, a.sel, a.K, ws, st);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  m.ntiles_total = (a.K + kBN - 1) / kBN;
  return launch_rows<kModeAttn>(m, a.c.n[a.r], st);
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
hipError_t launch_mass_mfma(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                            hipStream_t st) {
  MassArgs m{};
  m.a = a;
  m.cand = cand;
  m.K_prev = K_prev;
  m.mass = mass;
  m.c2 = c2_of(a.c.d);
  m.ncb = (K_prev + 127) / 128;
  const int nunits = a.c.B * a.c.H * m.ncb;
  if (!cand && a.r == 2) {  // loop-1 chain = the base records themselves
    hipLaunchKernelGGL(k_mass_mfma<true>, dim3(nunits), dim3(kThreads), 0, st, m);
    return hipGetLastError();
  }
  hipError_t e = launch_gather(a.c, a.r - 1, cand, K_prev, ws, st);
  if (e != hipSuccess) return e;
  m.tiles = ws;
  m.ntiles_total = (K_prev + kBN - 1) / kBN;
  hipLaunchKernelGGL(k_mass_mfma<false>, dim3(nunits), dim3(kThreads), 0, st, m);
  return hipGetLastError();
}

}  // namespace fl
