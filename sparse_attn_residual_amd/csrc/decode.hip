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

__device__ inline float group8_sum(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  return v;
}

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

// Loop 1: dense over all S cached tokens, d == 128.
template <typename T>
__global__ __launch_bounds__(kDecThreads) void k_decode_dense(DecodeArgs a, float tau) {
  __shared__ GroupState gs;
  const CacheGeo& c = a.c;
  const long long lbh = blockIdx.x;
  const int h = (int)(lbh % c.H);
  const int b = (int)((lbh / c.H) % c.B);
  const int l = (int)(lbh / ((long long)c.H * c.B));
  const int d = 128;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int sub = lane & 7;        // 16-dim slice of the record
  const int grp = lane >> 3;       // token within the wave's step
  const int gid = wv * 8 + grp;    // group id in the block
  float q[16];
  load_q16<T>((const T*)a.q + lbh * d, sub, q);
  float m = -INFINITY, lsum = 0.0f, acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  const uint8_t* recs = base_rec(c, l, b, h, 0);
  float* logit = a.logits + lbh * c.S;
  const int G = d / kGroup;
  for (int j = wv * 8 + grp; j < c.S; j += kDecThreads / 8) {
    const uint8_t* rec = recs + (long long)j * c.base_rb;
    const uint4 kw = *(const uint4*)(rec + sub * 16);
    const uint4 vw = *(const uint4*)(rec + d + sub * 16);
    const uint16_t* sc = (const uint16_t*)(rec + 2 * d);
    const float ks = h2f(sc[sub >> 1]);
    const float vs = h2f(sc[G + (sub >> 1)]);
    float cv[16];
    unpack_i8x16(kw, cv);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) part = __builtin_fmaf(q[e], cv[e], part);
    const float s = tau * group8_sum(part * ks);
    if (sub == 0) logit[j] = s;
    const float mn = fmaxf(m, s);
    const float alpha = __expf(m - mn);
    const float p = __expf(s - mn);
    lsum = lsum * alpha + p;
    const float pv = p * vs;
    unpack_i8x16(vw, cv);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(pv, cv[e], acc[e] * alpha);
    m = mn;
  }
  if (sub == 0) {
    gs.m[gid] = m;
    gs.l[gid] = lsum;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) gs.acc[gid][sub * 16 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < d) {
    float mx = -INFINITY;
    for (int g = 0; g < kDecGroups; ++g) mx = fmaxf(mx, gs.m[g]);
    float L = 0.0f, A = 0.0f;
    for (int g = 0; g < kDecGroups; ++g) {
      const float f = gs.m[g] == -INFINITY ? 0.0f : __expf(gs.m[g] - mx);
      L += gs.l[g] * f;
      A += gs.acc[g][threadIdx.x] * f;
    }
    a.O[lbh * d + threadIdx.x] = A / L;
    a.U[lbh * d + threadIdx.x] = 0.0f;
    if (threadIdx.x == 0) {
      a.lse[lbh] = mx + __logf(L);
      a.M[lbh] = 1.0f;
    }
  }
}

constexpr int kMaxFastLoops = 5;  // loops whose slot lookups are issued together

// The 16 dims [sub*16, sub*16+16) of K and V of token j reconstructed at
// loop r (and V at loop r-1 when vprev is set): the base plus the residuals
// of loops 2..r in which j was active.  Every slot lookup and record load of
// the token is issued before any of them is used.
template <bool PREV>
__device__ inline void token16(const CacheGeo& c, int r, int l, int b, int h, int j, int sub, float* kx, float* vx,
                               float* vprev) {
  constexpr int d = 128, G = 4;
  const uint8_t* rec = base_rec(c, l, b, h, j);
  const uint4 kw = *(const uint4*)(rec + sub * 16);
  const uint4 vw = *(const uint4*)(rec + d + sub * 16);
  const uint16_t* sc = (const uint16_t*)(rec + 2 * d);
  const uint16_t ksh = sc[sub >> 1], vsh = sc[G + (sub >> 1)];
  int slot[kMaxFastLoops - 1];
#pragma unroll
  for (int k = 0; k < kMaxFastLoops - 1; ++k) slot[k] = (k + 2 <= r) ? c.slot[k + 2][(long long)b * c.S + j] : -1;
  uint2 kr[kMaxFastLoops - 1], vr[kMaxFastLoops - 1];
  uint32_t meta[kMaxFastLoops - 1][2];
#pragma unroll
  for (int k = 0; k < kMaxFastLoops - 1; ++k) {
    kr[k] = vr[k] = make_uint2(0, 0);
    meta[k][0] = meta[k][1] = 0;
    if (slot[k] >= 0) {
      const int rr = k + 2, bits = c.bits[rr], C = d * bits / 8;
      const uint8_t* rrec = res_rec(c, rr, l, b, h, slot[k]);
      if (bits == 4) {
        kr[k] = *(const uint2*)(rrec + sub * 8);
        vr[k] = *(const uint2*)(rrec + C + sub * 8);
      } else {
        kr[k].x = *(const uint32_t*)(rrec + sub * 4);
        vr[k].x = *(const uint32_t*)(rrec + C + sub * 4);
      }
      const uint16_t* mt = (const uint16_t*)(rrec + 2 * C);
      const int g = sub >> 1;
      meta[k][0] = (uint32_t)mt[g] | ((uint32_t)mt[G + g] << 16);          // K scale, zero
      meta[k][1] = (uint32_t)mt[2 * G + g] | ((uint32_t)mt[3 * G + g] << 16);  // V scale, zero
    }
  }
  {
    const float ks = h2f(ksh), vs = h2f(vsh);
    const uint32_t kws[4] = {kw.x, kw.y, kw.z, kw.w}, vws[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      kx[e] = (float)(int8_t)(kws[e >> 2] >> (8 * (e & 3))) * ks;
      vx[e] = (float)(int8_t)(vws[e >> 2] >> (8 * (e & 3))) * vs;
    }
  }
  if (PREV) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
  }
#pragma unroll
  for (int k = 0; k < kMaxFastLoops - 1; ++k) {
    if (slot[k] < 0) continue;
    const int bits = c.bits[k + 2];
    const float krs = h2f((uint16_t)meta[k][0]), krz = h2f((uint16_t)(meta[k][0] >> 16));
    const float vrs = h2f((uint16_t)meta[k][1]), vrz = h2f((uint16_t)(meta[k][1] >> 16));
    if (PREV && k + 2 == r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
    }
    if (bits == 4) {
      const uint32_t kq[2] = {kr[k].x, kr[k].y}, vq[2] = {vr[k].x, vr[k].y};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        kx[e] = kx[e] + __builtin_fmaf((float)((kq[e >> 3] >> (4 * (e & 7))) & 15), krs, krz);
        vx[e] = vx[e] + __builtin_fmaf((float)((vq[e >> 3] >> (4 * (e & 7))) & 15), vrs, vrz);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        kx[e] = kx[e] + __builtin_fmaf((float)((kr[k].x >> (2 * e)) & 3), krs, krz);
        vx[e] = vx[e] + __builtin_fmaf((float)((vr[k].x >> (2 * e)) & 3), vrs, vrz);
      }
    }
  }
  // loops beyond the batched range, one lookup at a time
  bool active_r = r >= 2 && r <= kMaxFastLoops && slot[r - 2] >= 0;
  for (int rr = kMaxFastLoops + 1; rr <= r && slot[kMaxFastLoops - 2] >= 0; ++rr) {
    const int t = c.slot[rr][(long long)b * c.S + j];
    if (t < 0) break;
    if (PREV && rr == r) {
#pragma unroll
      for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
      active_r = true;
    }
    const int bits = c.bits[rr], C = d * bits / 8, g = sub >> 1;
    const uint8_t* rrec = res_rec(c, rr, l, b, h, t);
    const uint16_t* mt = (const uint16_t*)(rrec + 2 * C);
    const float krs = h2f(mt[g]), krz = h2f(mt[G + g]), vrs = h2f(mt[2 * G + g]), vrz = h2f(mt[3 * G + g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kc = bits == 4 ? (rrec[sub * 8 + (e >> 1)] >> (4 * (e & 1))) & 15
                               : (rrec[sub * 4 + (e >> 2)] >> (2 * (e & 3))) & 3;
      const int vc = bits == 4 ? (rrec[C + sub * 8 + (e >> 1)] >> (4 * (e & 1))) & 15
                               : (rrec[C + sub * 4 + (e >> 2)] >> (2 * (e & 3))) & 3;
      kx[e] = kx[e] + __builtin_fmaf((float)kc, krs, krz);
      vx[e] = vx[e] + __builtin_fmaf((float)vc, vrs, vrz);
    }
  }
  // a token inactive at loop r has x_hat^(r-1) == x_hat^(r)
  if (PREV && !active_r) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vprev[e] = vx[e];
  }
}

// Loop r >= 2 over the K selected tokens (sel/logits compacted at the front).
template <typename T, bool PRUNED>
__global__ __launch_bounds__(kDecThreads) void k_decode_sparse(DecodeArgs a, float tau) {
  __shared__ GroupState gs;
  __shared__ float csum[PRUNED ? kDecGroups : 1][128];
  __shared__ float psum[kDecGroups];
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
  float q[16];
  load_q16<T>((const T*)a.q + lbh * d, sub, q);
  const float Mprev = a.M[lbh];
  const float lprev = a.lse[lbh];
  float m = -INFINITY, lsum = 0.0f, acc[16], C[16], P = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = C[e] = 0.0f;
  const int32_t* sel = a.sel + lbh * c.S;
  float* logit = a.logits + lbh * c.S;
  for (int t = gid; t < a.K; t += kDecGroups) {
    const int j = sel[t];
    const float old = PRUNED ? logit[t] : 0.0f;
    float kx[16], vx[16], vp[16];
    token16<PRUNED>(c, r, l, b, h, j, sub, kx, vx, vp);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) part = __builtin_fmaf(q[e], kx[e], part);
    const float s = tau * group8_sum(part);
    if (sub == 0) logit[t] = s;  // every lane of the group read the old logit above
    if (PRUNED) {
      const float pj = Mprev * __expf(old - lprev);
      P += pj;
#pragma unroll
      for (int e = 0; e < 16; ++e) C[e] = __builtin_fmaf(pj, vp[e], C[e]);
    }
    const float mn = fmaxf(m, s);
    const float alpha = __expf(m - mn);
    const float p = __expf(s - mn);
    lsum = lsum * alpha + p;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(p, vx[e], acc[e] * alpha);
    m = mn;
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
    if (bf) hipLaunchKernelGGL(k_decode_dense<uint16_t>, dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
    else hipLaunchKernelGGL(k_decode_dense<float>, dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
    return hipGetLastError();
  }
  const int pruned = a.K < a.K_prev;
  hipError_t e;
  if (pruned) {
    const int32_t* cand = (a.r == 2 && a.K_prev == a.c.S) ? nullptr : a.sel;
    e = launch_topk(a.logits, a.c.S, cand, a.c.S, (int)P, a.K_prev, a.K, a.sel, a.c.S, a.logits, a.c.S, st);
    if (e != hipSuccess) return e;
  } else if (a.r == 2) {
    // every position stays selected: sel = 0..S-1 (rows of stride S); the
    // loop-1 logits are already in place
    e = launch_copy_sel(nullptr, (int)P, a.c.S, a.sel, st);
    if (e != hipSuccess) return e;
  }
  if (pruned) {
    if (bf) hipLaunchKernelGGL((k_decode_sparse<uint16_t, true>), dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
    else hipLaunchKernelGGL((k_decode_sparse<float, true>), dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
  } else {
    if (bf) hipLaunchKernelGGL((k_decode_sparse<uint16_t, false>), dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
    else hipLaunchKernelGGL((k_decode_sparse<float, false>), dim3((unsigned)P), dim3(kDecThreads), 0, st, a, tau);
  }
  return hipGetLastError();
}

}  // namespace fl
