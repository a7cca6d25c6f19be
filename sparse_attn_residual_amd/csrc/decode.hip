// fl_loop_decode kernels: one new token per (layer, sequence, head) attends
// its whole cached context at every loop (guide §1 and Cell 1: decode is
// bound by the bytes of the cache it reads; p1 App. G: attention works from
// the packed base and residual streams, with the selection fused in).
//
// Work split: one 256-thread block per (layer, b, h).  Eight lanes share one
// token record (16 dims each), so a wavefront streams eight consecutive
// 272-byte base records per step with 16-byte loads; every 8-lane group keeps
// its own online-softmax state, merged through LDS at the end.
#include "launch.hpp"

namespace fl {

constexpr int kDecThreads = 256;
constexpr int kDecGroups = kDecThreads / 8;  // 8 lanes per token

template <typename T>
__device__ inline void load_q16(const T* q, int sub, float* x) {
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = load_elem<T>(q + sub * 16 + e);
}

__device__ inline void unpack_i8x16(const uint4& w, float* c) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int t = 0; t < 4; ++t) c[4 * k + t] = (float)(int8_t)(ws[k] >> (8 * t));
  }
}

// Merge the per-group (m, l, acc[d]) states held in LDS; writes O and lse for
// dims handled by threads < d.  Returns nothing; final values are in out_O.
struct GroupState {
  float m[kDecGroups];
  float l[kDecGroups];
  float acc[kDecGroups][128];
};

// Sum over the 8 lanes of a group with DPP moves (no LDS round trip):
// xor 1 and xor 2 within quads, then the mirrored half-row pairs quad 0 of
// the group with quad 1.
__device__ inline float group8_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

constexpr float kDecRescale = 16.0f;  // lazy rescale threshold (natural log units)

// Online-softmax state of one 8-lane group (per lane: 16 dims of acc)
// merged with the group whose lanes are `o` apart (o = 8, 16, 32: the groups
// of one wavefront, lane by lane over the same dims).
__device__ inline void merge_groups(float& m, float& l, float* acc, int o) {
  const float m2 = __shfl_xor(m, o, kWave);
  const float l2 = __shfl_xor(l, o, kWave);
  const float mx = fmaxf(m, m2);
  const float f1 = m == -INFINITY ? 0.0f : __expf(m - mx);
  const float f2 = m2 == -INFINITY ? 0.0f : __expf(m2 - mx);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = acc[e] * f1 + __shfl_xor(acc[e], o, kWave) * f2;
  m = mx;
}

constexpr int kDenseThreads = 512;  // one block per (layer, sequence, query-head group)

// Loop 1: dense over all S cached tokens, d == 128.  A block of NT threads
// (NT/8 groups of 8 lanes, one token per group per step) walks the slab of S
// records of one KV head for GQ of the query heads that read it (grouped-query
// attention: each record is fetched once for all GQ heads; GQ = 1 otherwise).
// The block's waves cover consecutive tokens, so few slabs (and pages) are
// read at once on the chip.  Each group's softmax keeps a reference maximum
// per head that only moves when a score exceeds it by more than kDecRescale,
// so the accumulators are rescaled rarely.  Group states merge within each
// wavefront by lane shuffles, then across wavefronts in LDS.  Every head's
// arithmetic is the same whatever GQ is.
template <typename T, int NT, int GQ, bool PAPER>
__global__ __launch_bounds__(NT) void k_decode_dense(DecodeArgs a, float tau) {
  constexpr int NG = NT / 8, NW = NT / kWave;
  static_assert(GQ * 128 <= NT, "one thread per output dim of every head");
  __shared__ float wm[GQ][NW], wl[GQ][NW], wacc[GQ][NW][128];
  __shared__ uint32_t hist[GQ][kHistBins];  // each head's logits by key (loop 2's selection)
  __shared__ float lgs[GQ][NW][64];          // a wave's logits of a step, stored as whole lines
  const CacheGeo& c = a.c;
  const int HB = c.H / GQ;                 // query-head groups per sequence
  const long long blk = blockIdx.x;        // over [L][B][HB]
  const int hb = (int)(blk % HB);
  const int b = (int)((blk / HB) % c.B);
  const int l = (int)(blk / ((long long)HB * c.B));
  const int h0 = hb * GQ;                  // GQ divides H / Hkv: one KV head
  const long long lbh0 = ((long long)l * c.B + b) * c.H + h0;
  const int d = 128;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane & 7;        // 16-dim slice of the record
  const int grp = lane >> 3;       // token within the wave's step
  const int gid = wv * 8 + grp;    // group id in the block
  const int g = sub >> 1;          // quantization group of the slice
  for (int i = threadIdx.x; i < GQ * kHistBins; i += NT) (&hist[0][0])[i] = 0u;
  __syncthreads();
  float q[GQ][16], m[GQ], lsum[GQ], acc[GQ][16];
#pragma unroll
  for (int u = 0; u < GQ; ++u) {
    load_q16<T>((const T*)a.q + (lbh0 + u) * d, sub, q[u]);
    m[u] = -INFINITY;
    lsum[u] = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
  }
  const uint8_t* recs = base_rec(c, l, b, kv_head(c, h0), 0);
  float* logit = a.logits + lbh0 * c.S;
  const uint16_t* scl = (const uint16_t*)(recs + 2 * d);
  if (PAPER) {
    // The paper's format.  Each 8-lane group takes 8 consecutive tokens of
    // one 64-token key block, so the block's per-channel key scales and zeros
    // are folded into the query once: q.k = sum (q s) c + sum q z.  A value
    // group's zero is carried as one running sum per lane (its 16 dims share
    // it) and added before the merge.  Tail tokens (bf16) come last.
    const uint8_t* st = paper_stream(c, 1, l, b, kv_head(c, h0));
    const int body = min(c.Sq, c.T);
    const int nb = (body + kPGroup - 1) / kPGroup;
    float zacc[GQ];
#pragma unroll
    for (int u = 0; u < GQ; ++u) zacc[u] = 0.0f;
    for (int blk = gid / 8; blk < nb; blk += NG / 8) {
      const uint8_t* meta = st + (long long)c.Sq * kPRec + (long long)blk * kPKMeta;
      const uint4 s0 = *(const uint4*)(meta + sub * 32), s1 = *(const uint4*)(meta + sub * 32 + 16);
      const uint4 z0 = *(const uint4*)(meta + 256 + sub * 32), z1 = *(const uint4*)(meta + 256 + sub * 32 + 16);
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const uint32_t zw[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      float qs[GQ][16], qz[GQ];
#pragma unroll
      for (int u = 0; u < GQ; ++u) {
        qz[u] = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          qs[u][e] = q[u][e] * h2f((uint16_t)(sw[e >> 1] >> (16 * (e & 1))));
          qz[u] = __builtin_fmaf(q[u][e], h2f((uint16_t)(zw[e >> 1] >> (16 * (e & 1)))), qz[u]);
        }
      }
      const int t0 = blk * kPGroup + (gid & 7) * 8;
      // the group's 8 records are all requested before the first is used
      uint2 kwa[8], vwa[8];
      uint32_t vma[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint8_t* rec = st + (long long)min(t0 + i, body - 1) * kPRec;
        kwa[i] = *(const uint2*)(rec + sub * 8);
        vwa[i] = *(const uint2*)(rec + 64 + sub * 8);
        vma[i] = *(const uint32_t*)(rec + 128 + (sub >> 2) * 4);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = t0 + i;
        if (j >= body) break;  // the same for the group's 8 lanes
        const float vs = h2f((uint16_t)vma[i]), vz = h2f((uint16_t)(vma[i] >> 16));
        const uint32_t kws[2] = {kwa[i].x, kwa[i].y}, vws[2] = {vwa[i].x, vwa[i].y};
#pragma unroll
        for (int u = 0; u < GQ; ++u) {
          float part = qz[u];
#pragma unroll
          for (int e = 0; e < 16; ++e) part = __builtin_fmaf(qs[u][e], (float)((kws[e >> 3] >> (4 * (e & 7))) & 15), part);
          const float sc = tau * group8_sum_dpp(part);
          if (sub == 0) {
            lgs[u][wv][(gid & 7) * 8 + i] = sc;
            atomicAdd(&hist[u][order_key(sc) >> (32 - kHistBits)], 1u);
          }
          if (sc > m[u] + kDecRescale) {
            const float alpha = __expf(m[u] - sc);
            lsum[u] *= alpha;
            zacc[u] *= alpha;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[u][e] *= alpha;
            m[u] = sc;
          }
          const float pr = __expf(sc - m[u]);
          lsum[u] += pr;
          const float pv = pr * vs;
          zacc[u] = __builtin_fmaf(pr, vz, zacc[u]);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[u][e] = __builtin_fmaf(pv, (float)((vws[e >> 3] >> (4 * (e & 7))) & 15), acc[u][e]);
        }
      }
      // the key block's 64 logits (the wave's eight groups), two whole lines
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      if (blk * kPGroup + lane < body) {
#pragma unroll
        for (int u = 0; u < GQ; ++u) logit[(long long)u * c.S + blk * kPGroup + lane] = lgs[u][wv][lane];
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int u = 0; u < GQ; ++u) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] += zacc[u];
    }
    for (int j = body + gid; j < c.T; j += NG) {  // the bf16 tail
      float kx[16], vx[16];
      paper_chain16(c, 1, l, b, kv_head(c, h0), j, 0, sub * 16, kx);
      paper_chain16(c, 1, l, b, kv_head(c, h0), j, 1, sub * 16, vx);
#pragma unroll
      for (int u = 0; u < GQ; ++u) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) part = __builtin_fmaf(q[u][e], kx[e], part);
        const float sc = tau * group8_sum_dpp(part);
        if (sub == 0) {
          logit[(long long)u * c.S + j] = sc;
          atomicAdd(&hist[u][order_key(sc) >> (32 - kHistBits)], 1u);
        }
        if (sc > m[u] + kDecRescale) {
          const float alpha = __expf(m[u] - sc);
          lsum[u] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[u][e] *= alpha;
          m[u] = sc;
        }
        const float pr = __expf(sc - m[u]);
        lsum[u] += pr;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[u][e] = __builtin_fmaf(pr, vx[e], acc[u][e]);
      }
    }
  }
  // The block takes 256 positions per step, each wave 32 consecutive ones in
  // four rounds of 8 (one per 8-lane group): its 32 logits then fill one
  // 128-byte line, staged in LDS and stored by one instruction.  Stored by
  // each token's group as it went (32 bytes per wave and round: partial lines
  // among the record reads), they made the 48-layer loop at 32K positions
  // ~2 ms slower (21.3 against 19.3 ms), and slower still in some physical
  // placements of the cache.
  // round it: step it / 4, round it % 4; position w0 + 8 (it % 4) + grp
  for (int it = 0; !PAPER && (it >> 2) * (32 * NW) < c.T; ++it) {
    const int w0 = (it >> 2) * (32 * NW) + wv * 32;
    const int j = w0 + (it & 3) * 8 + grp;
    if (j < c.T) {  // the same for the group's 8 lanes
      const uint8_t* rec = recs + (long long)j * c.base_rb;
      const uint4 kw = *(const uint4*)(rec + sub * 16);
      const uint4 vw = *(const uint4*)(rec + d + sub * 16);
      const uint16_t* sc = (const uint16_t*)((const uint8_t*)scl + (long long)j * c.base_rb);
      const float ks = h2f(sc[g]);
      const float vs = h2f(sc[4 + g]);
      float cv[16];
      unpack_i8x16(kw, cv);
      float p[GQ];
#pragma unroll
      for (int u = 0; u < GQ; ++u) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) part = __builtin_fmaf(q[u][e], cv[e], part);
        const float s = tau * group8_sum_dpp(part * ks);
        if (sub == 0) {
          lgs[u][wv][(it & 3) * 8 + grp] = s;
          atomicAdd(&hist[u][order_key(s) >> (32 - kHistBits)], 1u);
        }
        if (s > m[u] + kDecRescale) {
          const float alpha = __expf(m[u] - s);  // 0 on the group's first token
          lsum[u] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[u][e] *= alpha;
          m[u] = s;
        }
        p[u] = __expf(s - m[u]);
        lsum[u] += p[u];
      }
      unpack_i8x16(vw, cv);
#pragma unroll
      for (int u = 0; u < GQ; ++u) {
        const float pv = p[u] * vs;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[u][e] = __builtin_fmaf(pv, cv[e], acc[u][e]);
      }
    }
    // after the fourth round, the wave's logits of this step (LDS operations of
    // one wave complete in order: its stores are visible to its reads once
    // they have completed)
    if ((it & 3) == 3) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      if (lane < 32 && w0 + lane < c.T) {
#pragma unroll
        for (int u = 0; u < GQ; ++u) logit[(long long)u * c.S + w0 + lane] = lgs[u][wv][lane];
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    }
  }
#pragma unroll
  for (int u = 0; u < GQ; ++u) {
    merge_groups(m[u], lsum[u], acc[u], 8);
    merge_groups(m[u], lsum[u], acc[u], 16);
    merge_groups(m[u], lsum[u], acc[u], 32);
    if (grp == 0) {
      if (sub == 0) {
        wm[u][wv] = m[u];
        wl[u][wv] = lsum[u];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) wacc[u][wv][sub * 16 + e] = acc[u][e];
    }
  }
  __syncthreads();
  if (threadIdx.x < GQ * d) {
    const int u = threadIdx.x / d, t = threadIdx.x - u * d;
    float mx = -INFINITY;
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, wm[u][w]);
    float L = 0.0f, A = 0.0f;
    for (int w = 0; w < NW; ++w) {
      const float f = wm[u][w] == -INFINITY ? 0.0f : __expf(wm[u][w] - mx);
      L += wl[u][w] * f;
      A += wacc[u][w][t] * f;
    }
    const long long lbh = lbh0 + u;
    a.O[lbh * d + t] = A / L;
    a.U[lbh * d + t] = 0.0f;
    if (t == 0) {
      a.lse[lbh] = mx + __logf(L);
      a.M[lbh] = 1.0f;
    }
  }
  // the histograms go to the front of each head's selection row (which loop
  // 1 does not otherwise use) when the row holds them
  if (c.S >= kHistBins) {
    for (int i = threadIdx.x; i < GQ * kHistBins; i += NT) {
      const int u = i / kHistBins, bin = i - u * kHistBins;
      a.sel[(lbh0 + u) * c.S + bin] = (int32_t)hist[u][bin];
    }
  }
}

template <typename T>
static void launch_dense(const DecodeArgs& a, float tau, hipStream_t st) {
  // query heads per block: two when the group size is even.  Four heads per
  // block read each record once but need 176 VGPRs (one 512-thread block per
  // CU); two heads need 112 (two blocks per CU) and ran the 4-head groups'
  // loop 7-8 % faster despite reading each record twice.
  const int gq = a.c.G % 2 == 0 ? 2 : 1;
  const unsigned nblk = (unsigned)((long long)a.c.L * a.c.B * (a.c.H / gq));
  if (a.c.fmt == kFmtPaper)  // one query head per block: the reads are reconstructions, not raw records
    FL_LAUNCH((k_decode_dense<T, kDenseThreads, 1, true>), dim3((unsigned)((long long)a.c.L * a.c.B * a.c.H)),
                       dim3(kDenseThreads), 0, st, a, tau);
  else if (gq == 2)
    FL_LAUNCH((k_decode_dense<T, kDenseThreads, 2, false>), dim3(nblk), dim3(kDenseThreads), 0, st, a, tau);
  else
    FL_LAUNCH((k_decode_dense<T, kDenseThreads, 1, false>), dim3(nblk), dim3(kDenseThreads), 0, st, a, tau);
}

constexpr int kMaxFastLoops = 5;  // loops whose slot lookups are batched
constexpr int kNF = kMaxFastLoops - 1;

// Raw loads of the 16 dims [sub*16, sub*16+16) of one token: base codes and
// scales, and for loops 2..kMaxFastLoops the residual codes and meta of the
// loops the token was active in (slot >= 0).  Split from the decoding so
// that the loads of several tokens can be in flight together.
template <int NR>
struct TokLoads {
  uint4 kw, vw;
  uint32_t sc;                 // K scale | V scale << 16
  uint2 kr[NR], vr[NR];
  uint32_t meta[NR][2];        // K scale | zero << 16, V scale | zero << 16
};

// NR: residual loops 2..NR+1 whose loads are batched (NR = min(r, 5) - 1).
template <int NR>
__device__ inline void tok_load(const CacheGeo& c, int l, int b, int h, int j, const int* slot, int sub,
                                TokLoads<NR>& t) {
  constexpr int d = 128, G = 4;
  const uint8_t* rec = base_rec(c, l, b, kv_head(c, h), j);
  t.kw = *(const uint4*)(rec + sub * 16);
  t.vw = *(const uint4*)(rec + d + sub * 16);
  const uint16_t* sc = (const uint16_t*)(rec + 2 * d);
  t.sc = (uint32_t)sc[sub >> 1] | ((uint32_t)sc[G + (sub >> 1)] << 16);
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    t.kr[k] = t.vr[k] = make_uint2(0, 0);
    t.meta[k][0] = t.meta[k][1] = 0;
    if (slot[k] >= 0) {
      const int rr = k + 2, bits = c.bits[rr], C = d * bits / 8;
      const uint8_t* rrec = res_rec(c, rr, l, b, kv_head(c, h), slot[k]);
      if (bits == 4) {
        t.kr[k] = *(const uint2*)(rrec + sub * 8);
        t.vr[k] = *(const uint2*)(rrec + C + sub * 8);
      } else {
        t.kr[k].x = *(const uint32_t*)(rrec + sub * 4);
        t.vr[k].x = *(const uint32_t*)(rrec + C + sub * 4);
      }
      const uint16_t* mt = (const uint16_t*)(rrec + 2 * C);
      const int g = sub >> 1;
      t.meta[k][0] = (uint32_t)mt[g] | ((uint32_t)mt[G + g] << 16);
      t.meta[k][1] = (uint32_t)mt[2 * G + g] | ((uint32_t)mt[3 * G + g] << 16);
    }
  }
}

// The token's K and V reconstructed at loop r from its loads: base, plus the
// residuals of loops 2..r in which it was active; loops beyond kMaxFastLoops
// are looked up here one at a time.  K and V are rebuilt in two passes (K
// before the score, V after it) so that only one 16-element array is live
// next to the loads; every element sees the same operations in the same order
// either way.
template <int NR>
__device__ __forceinline__ void tok_key(const CacheGeo& c, int r, int l, int b, int h, int j, const int* slot, int sub,
                                        const TokLoads<NR>& t, float* kx) {
  constexpr int d = 128, G = 4;
  {
    const float ks = h2f((uint16_t)t.sc);
    const uint32_t kws[4] = {t.kw.x, t.kw.y, t.kw.z, t.kw.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) kx[e] = (float)(int8_t)(kws[e >> 2] >> (8 * (e & 3))) * ks;
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (slot[k] < 0) continue;
    const int bits = c.bits[k + 2];
    const float krs = h2f((uint16_t)t.meta[k][0]), krz = h2f((uint16_t)(t.meta[k][0] >> 16));
    if (bits == 4) {
      const uint32_t kq[2] = {t.kr[k].x, t.kr[k].y};
#pragma unroll
      for (int e = 0; e < 16; ++e) kx[e] = kx[e] + __builtin_fmaf((float)((kq[e >> 3] >> (4 * (e & 7))) & 15), krs, krz);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) kx[e] = kx[e] + __builtin_fmaf((float)((t.kr[k].x >> (2 * e)) & 3), krs, krz);
    }
  }
  for (int rr = kMaxFastLoops + 1; NR == kNF && rr <= r && slot[kNF - 1] >= 0; ++rr) {
    const int ts = c.slot[rr][(long long)b * c.S + j];
    if (ts < 0) break;
    const int bits = c.bits[rr], g = sub >> 1;
    const uint8_t* rrec = res_rec(c, rr, l, b, kv_head(c, h), ts);
    const uint16_t* mt = (const uint16_t*)(rrec + 2 * (d * bits / 8));
    const float krs = h2f(mt[g]), krz = h2f(mt[G + g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kc = bits == 4 ? (rrec[sub * 8 + (e >> 1)] >> (4 * (e & 1))) & 15
                               : (rrec[sub * 4 + (e >> 2)] >> (2 * (e & 3))) & 3;
      kx[e] = kx[e] + __builtin_fmaf((float)kc, krs, krz);
    }
  }
}

// V at loop r, and at loop r-1 when PREV is set.
template <bool PREV, int NR>
__device__ __forceinline__ void tok_value(const CacheGeo& c, int r, int l, int b, int h, int j, const int* slot,
                                          int sub, const TokLoads<NR>& t, float* vx, float* vprev) {
  constexpr int d = 128, G = 4;
  {
    const float vs = h2f((uint16_t)(t.sc >> 16));
    const uint32_t vws[4] = {t.vw.x, t.vw.y, t.vw.z, t.vw.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) vx[e] = (float)(int8_t)(vws[e >> 2] >> (8 * (e & 3))) * vs;
  }
  if (PREV) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if (slot[k] < 0) continue;
    const int bits = c.bits[k + 2];
    const float vrs = h2f((uint16_t)t.meta[k][1]), vrz = h2f((uint16_t)(t.meta[k][1] >> 16));
    if (PREV && k + 2 == r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
    }
    if (bits == 4) {
      const uint32_t vq[2] = {t.vr[k].x, t.vr[k].y};
#pragma unroll
      for (int e = 0; e < 16; ++e) vx[e] = vx[e] + __builtin_fmaf((float)((vq[e >> 3] >> (4 * (e & 7))) & 15), vrs, vrz);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) vx[e] = vx[e] + __builtin_fmaf((float)((t.vr[k].x >> (2 * e)) & 3), vrs, vrz);
    }
  }
  bool active_r = r >= 2 && r <= NR + 1 && slot[r - 2] >= 0;
  for (int rr = kMaxFastLoops + 1; NR == kNF && rr <= r && slot[kNF - 1] >= 0; ++rr) {
    const int ts = c.slot[rr][(long long)b * c.S + j];
    if (ts < 0) break;
    if (PREV && rr == r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
      active_r = true;
    }
    const int bits = c.bits[rr], C = d * bits / 8, g = sub >> 1;
    const uint8_t* rrec = res_rec(c, rr, l, b, kv_head(c, h), ts);
    const uint16_t* mt = (const uint16_t*)(rrec + 2 * C);
    const float vrs = h2f(mt[2 * G + g]), vrz = h2f(mt[3 * G + g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int vc = bits == 4 ? (rrec[C + sub * 8 + (e >> 1)] >> (4 * (e & 1))) & 15
                               : (rrec[C + sub * 4 + (e >> 2)] >> (2 * (e & 3))) & 3;
      vx[e] = vx[e] + __builtin_fmaf((float)vc, vrs, vrz);
    }
  }
  // a token inactive at loop r has x_hat^(r-1) == x_hat^(r)
  if (PREV && !active_r) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
  }
}

// Index stage of a chunk of 64 selected tokens: lane L takes token
// t = t0 + L and loads its position, its slot in loops 2..kMaxFastLoops and
// (pruned loops) its previous logit.
template <bool PRUNED, int NR>
__device__ inline void chunk_index(const DecodeArgs& a, int b, int t0, int lane, const int32_t* sel,
                                   const float* logit, int& j, int* slot, float& old) {
  const CacheGeo& c = a.c;
  const int t = t0 + lane;
  j = t < a.K ? sel[t] : -1;
  old = (PRUNED && t < a.K) ? logit[t] : 0.0f;
#pragma unroll
  for (int k = 0; k < NR; ++k) slot[k] = j >= 0 ? c.slot[k + 2][(long long)b * c.S + j] : -1;
}

// One token's score and the group's online-softmax update up to its weight:
// returns p = exp(s - m) for a valid token (the caller adds p * v) and, pruned,
// pj = the previous loop's weight of the token (added to P here; the caller
// adds pj * v^(r-1) to C).
template <bool PRUNED>
__device__ __forceinline__ float tok_weight(const float* q, const float* kx, float tau, float old, float Mprev,
                                            float lprev, bool valid, int sub, float* lg, float& m, float& lsum,
                                            float* acc, float& P, float& pj) {
  float part = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) part = __builtin_fmaf(q[e], kx[e], part);
  const float s = tau * group8_sum_dpp(part);
  pj = 0.0f;
  if (!valid) return 0.0f;
  if (sub == 0) *lg = s;
  if (PRUNED) {
    pj = Mprev * __expf(old - lprev);
    P += pj;
  }
  if (s > m + kDecRescale) {  // lazy rescale, as in the dense loop
    const float alpha = __expf(m - s);
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= alpha;
    m = s;
  }
  const float p = __expf(s - m);
  lsum += p;
  return p;
}

// The valid token's value terms: acc += p * v and, pruned, C += pj * v^(r-1).
template <bool PRUNED>
__device__ __forceinline__ void tok_add(float p, float pj, const float* vx, const float* vp, float* acc, float* C) {
  if (PRUNED) {
#pragma unroll
    for (int e = 0; e < 16; ++e) C[e] = __builtin_fmaf(pj, vp[e], C[e]);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(p, vx[e], acc[e]);
}

// Loop r >= 2 over the K selected tokens (sel/logits compacted at the front).
// Each wave walks chunks of 64 selected tokens: the index stage of the next
// chunk (positions, slots, old logits; one token per lane) is in flight while
// the current chunk's records are read, two tokens per 8-lane group at a time.
// Blocks per CU the sparse kernel is built for: three (at most 168 VGPRs, a
// third wave per SIMD for more loads in flight) where that fits without
// spilling; otherwise what the code needs.
constexpr int dec_sparse_blocks(bool pruned, int NR) { return (NR <= 2 || (NR == 3 && !pruned)) ? 3 : 1; }

template <typename T, bool PRUNED, int NR, bool PAPER>
__global__ __launch_bounds__(kDecThreads, dec_sparse_blocks(PRUNED, NR))
void k_decode_sparse(DecodeArgs a, float tau) {
  __shared__ GroupState gs;
  __shared__ float csum[PRUNED ? kDecGroups : 1][128];
  __shared__ float psum[kDecGroups];
  // a chunk's 64 logits, stored in two whole lines at the end of the chunk
  // (stored token by token they are partial-line writes among the gathers)
  __shared__ float lgst[kDecThreads / kWave][64];
  const CacheGeo& c = a.c;
  const long long lbh = blockIdx.x;
  const int h = (int)(lbh % c.H);
  const int b = (int)((lbh / c.H) % c.B);
  const int l = (int)(lbh / ((long long)c.H * c.B));
  const int d = 128;
  const int r = a.r;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane & 7;
  const int grp = lane >> 3;
  const int gid = wv * 8 + grp;
  constexpr int kWaves = kDecThreads / kWave;
  float q[16];
  load_q16<T>((const T*)a.q + lbh * d, sub, q);
  const float Mprev = a.M[lbh];
  const float lprev = a.lse[lbh];
  float m = -INFINITY, lsum = 0.0f, acc[16], C[16], P = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = C[e] = 0.0f;
  const int32_t* sel = a.sel + lbh * c.S;
  float* logit = a.logits + lbh * c.S;
  const int nch = (a.K + 63) / 64;

  int jn = -1, sn[NR];
  float on = 0.0f;
  if (wv < nch) chunk_index<PRUNED, NR>(a, b, wv * 64, lane, sel, logit, jn, sn, on);
  for (int ch = wv; ch < nch; ch += kWaves) {
    const int jc = jn;
    int sc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) sc[k] = sn[k];
    const float oc = on;
    if (ch + kWaves < nch) chunk_index<PRUNED, NR>(a, b, (ch + kWaves) * 64, lane, sel, logit, jn, sn, on);
    const int t0 = ch * 64;
    const int nv = min(64, a.K - t0);  // valid tokens of the chunk (a prefix)
    // Order the chunk's tokens by how many residual loops they carry (slots
    // are nested: active at loop k+2 implies active at every earlier loop),
    // most first, invalid tokens last, so that the eight tokens a wave step
    // reads share their residual work and the wave skips loops none of them
    // has.  src: lane (= token of the chunk) taken at sorted position L.
    int src_of_pos;
    {
      int nres = jc >= 0 ? 0 : -1;
#pragma unroll
      for (int k = 0; k < NR; ++k) nres += (sc[k] >= 0) ? 1 : 0;
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int pos = 0, base = 0;
#pragma unroll
      for (int v = NR; v >= -1; --v) {
        const uint64_t mv = __ballot(nres == v);
        if (nres == v) pos = base + __popcll(mv & below);
        base += __popcll(mv);
      }
      src_of_pos = __builtin_amdgcn_ds_permute(pos * 4, lane);
    }
#pragma unroll 1
    for (int it = 0; it * 8 < nv; it += 2) {  // wave-uniform trip count
      // sorted positions it*8+grp and (it+1)*8+grp; invalid ones read token 0
      int j2[2], s2[2][NR], tt[2];
      float o2[2];
      bool v2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int src = __shfl(src_of_pos, (it + u) * 8 + grp, kWave);
        tt[u] = t0 + src;
        j2[u] = __shfl(jc, src, kWave);
#pragma unroll
        for (int k = 0; k < NR; ++k) s2[u][k] = __shfl(sc[k], src, kWave);
        o2[u] = __shfl(oc, src, kWave);
        v2[u] = j2[u] >= 0;
        if (!v2[u]) {
          j2[u] = 0;
#pragma unroll
          for (int k = 0; k < NR; ++k) s2[u][k] = -1;
        }
      }
      TokLoads<NR> t2[2];
      if (!PAPER) {
        tok_load(c, l, b, h, j2[0], s2[0], sub, t2[0]);
        tok_load(c, l, b, h, j2[1], s2[1], sub, t2[1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (PAPER) {
          // the paper's format: K, V at loop r (and V at loop r-1) rebuilt here
          float kx[16], vx[16], vp[16], pj;
          paper_token16<PRUNED>(c, r, l, b, kv_head(c, h), j2[u], sub * 16, kx, vx, vp);
          const float p = tok_weight<PRUNED>(q, kx, tau, o2[u], Mprev, lprev, v2[u], sub, &lgst[wv][tt[u] - t0], m,
                                             lsum, acc, P, pj);
          if (v2[u]) tok_add<PRUNED>(p, pj, vx, vp, acc, C);
        } else {
          float p, pj;
          {
            float kx[16];
            tok_key<NR>(c, r, l, b, h, j2[u], s2[u], sub, t2[u], kx);
            p = tok_weight<PRUNED>(q, kx, tau, o2[u], Mprev, lprev, v2[u], sub, &lgst[wv][tt[u] - t0], m, lsum, acc,
                                   P, pj);
          }
          if (v2[u]) {
            float vx[16], vp[16];
            tok_value<PRUNED, NR>(c, r, l, b, h, j2[u], s2[u], sub, t2[u], vx, vp);
            tok_add<PRUNED>(p, pj, vx, vp, acc, C);
          }
        }
      }
    }
    // the chunk's logits (each valid token's, written above by its group;
    // LDS operations of one wave complete in order)
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    if (lane < nv) logit[t0 + lane] = lgst[wv][lane];
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
  if (sub == 0) {
    gs.m[gid] = m;
    gs.l[gid] = lsum;
    psum[gid] = P;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    gs.acc[gid][sub * 16 + e] = acc[e];
    if (PRUNED) csum[gid][sub * 16 + e] = C[e];
  }
  __syncthreads();
  if (threadIdx.x < d) {
    float Mr = Mprev, Ud = a.U[lbh * d + threadIdx.x];
    if (PRUNED) {
      float ps = 0.0f, cs = 0.0f;
      for (int g = 0; g < kDecGroups; ++g) {
        ps += psum[g];
        cs += csum[g][threadIdx.x];
      }
      Mr = ps;
      Ud = a.O[lbh * d + threadIdx.x] - cs;
    }
    float mx = -INFINITY;
    for (int g = 0; g < kDecGroups; ++g) mx = fmaxf(mx, gs.m[g]);
    float L = 0.0f, A = 0.0f;
    for (int g = 0; g < kDecGroups; ++g) {
      const float f = gs.m[g] == -INFINITY ? 0.0f : __expf(gs.m[g] - mx);
      L += gs.l[g] * f;
      A += gs.acc[g][threadIdx.x] * f;
    }
    a.O[lbh * d + threadIdx.x] = Ud + Mr * (A / L);
    a.U[lbh * d + threadIdx.x] = Ud;
    if (threadIdx.x == 0) {
      a.lse[lbh] = mx + __logf(L);
      a.M[lbh] = Mr;
    }
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const float tau = (float)(1.0 / __builtin_sqrt((double)a.c.d));
  const long long P = (long long)a.c.L * a.c.B * a.c.H;
  const bool bf = a.dt == FL_BF16;
  if (a.r == 1) {
    if (bf)
      launch_dense<uint16_t>(a, tau, st);
    else
      launch_dense<float>(a, tau, st);
    return hipGetLastError();
  }
  const int pruned = a.K < a.K_prev;
  hipError_t e;
  if (pruned) {
    const int32_t* cand = (a.r == 2 && a.K_prev == a.c.T) ? nullptr : a.sel;
    // loop 1 left each head's logit histogram at the front of its selection row
    const bool given = !cand && a.c.S >= kHistBins;
    e = launch_topk(a.logits, a.c.S, cand, a.c.S, (int)P, a.K_prev, a.K, a.sel, a.c.S, a.logits, a.c.S, st,
                    given ? a.sel : nullptr, a.c.S);
    if (e != hipSuccess) return e;
  } else if (a.r == 2) {
    // every position stays selected: sel = 0..T-1 (rows of stride S); the
    // loop-1 logits are already in place
    e = launch_copy_sel(nullptr, (int)P, a.c.T, a.sel, st, a.c.S);
    if (e != hipSuccess) return e;
  }
  if (a.c.fmt == kFmtPaper) {  // tokens rebuilt one at a time: no batched residual loads
    switch (pruned * 2 + (bf ? 1 : 0)) {
      case 0: FL_LAUNCH((k_decode_sparse<float, false, 1, true>), dim3((unsigned)P), dim3(kDecThreads), 0,
                                 st, a, tau); break;
      case 1: FL_LAUNCH((k_decode_sparse<uint16_t, false, 1, true>), dim3((unsigned)P), dim3(kDecThreads),
                                 0, st, a, tau); break;
      case 2: FL_LAUNCH((k_decode_sparse<float, true, 1, true>), dim3((unsigned)P), dim3(kDecThreads), 0,
                                 st, a, tau); break;
      default: FL_LAUNCH((k_decode_sparse<uint16_t, true, 1, true>), dim3((unsigned)P), dim3(kDecThreads),
                                  0, st, a, tau); break;
    }
    return hipGetLastError();
  }
  const int nr = (a.r < kMaxFastLoops ? a.r : kMaxFastLoops) - 1;
  switch (nr * 4 + pruned * 2 + (bf ? 1 : 0)) {
#define FL_DEC_CASE(NR, PR, BF, T)                                                                                 \
  case NR * 4 + PR * 2 + BF:                                                                                       \
    FL_LAUNCH((k_decode_sparse<T, PR, NR, false>), dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau); \
    break;
#define FL_DEC_NR(NR)                 \
  FL_DEC_CASE(NR, 0, 0, float)        \
  FL_DEC_CASE(NR, 0, 1, uint16_t)     \
  FL_DEC_CASE(NR, 1, 0, float)        \
  FL_DEC_CASE(NR, 1, 1, uint16_t)
    FL_DEC_NR(1)
    FL_DEC_NR(2)
    FL_DEC_NR(3)
    FL_DEC_NR(4)
#undef FL_DEC_NR
#undef FL_DEC_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fl
