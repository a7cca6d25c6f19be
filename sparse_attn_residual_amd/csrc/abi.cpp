// C ABI of the FlashLoop hot path: argument validation, workspace sizing,
// error reporting and kernel dispatch.  Declarations and the meaning of every
// argument are in include/flashloop.h.  Nothing here allocates device memory;
// every check happens before the first launch of a call.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "launch.hpp"

namespace {

thread_local std::string g_err;

fl_status fail(fl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

fl_status hip_fail(hipError_t e, const char* what) {
  return fail(FL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

#define FL_NEED_PTR(p, name)                                                                 \
  do {                                                                                       \
    if (!(p)) return fail(FL_EINVAL, "%s: %s is NULL", fn, name);                            \
    if (!aligned16(p)) return fail(FL_EINVAL, "%s: %s is not 16-byte aligned", fn, name);    \
  } while (0)
// index and mass arrays (int32 / float32 read element-wise): 4-byte alignment
#define FL_NEED_PTR4(p, name)                                                                \
  do {                                                                                       \
    if (!(p)) return fail(FL_EINVAL, "%s: %s is NULL", fn, name);                            \
    if (!aligned4(p)) return fail(FL_EINVAL, "%s: %s is not 4-byte aligned", fn, name);      \
  } while (0)

// Validates the cache geometry and the streams needed by loop r; fills geo.
fl_status check_cache(const char* fn, const fl_cache* c, int r, bool need_res_r, fl::CacheGeo* geo) {
  if (!c) return fail(FL_EINVAL, "%s: cache is NULL", fn);
  if (c->L < 1 || c->B < 1 || c->H < 1 || c->S < 1)
    return fail(FL_EINVAL, "%s: L, B, H, S must be >= 1 (got %d, %d, %d, %d)", fn, c->L, c->B, c->H, c->S);
  if (c->d != 64 && c->d != 128) return fail(FL_EUNSUPPORTED, "%s: head dim %d (supported: 64, 128)", fn, c->d);
  if (c->R < 1 || c->R > FL_MAX_LOOPS) return fail(FL_EINVAL, "%s: R = %d outside [1, %d]", fn, c->R, FL_MAX_LOOPS);
  if (r < 1 || r > c->R) return fail(FL_EINVAL, "%s: loop r = %d outside [1, R = %d]", fn, r, c->R);
  if (c->n[1] != c->S) return fail(FL_EINVAL, "%s: n[1] = %d must equal S = %d", fn, c->n[1], c->S);
  const int hkv = c->Hkv == 0 ? c->H : c->Hkv;
  if (c->T < 0 || c->T > c->S) return fail(FL_EINVAL, "%s: T = %d outside [0, S = %d]", fn, c->T, c->S);
  if (c->fmt != FL_FMT_WORKLOAD && c->fmt != FL_FMT_PAPER)
    return fail(FL_EUNSUPPORTED, "%s: cache format %d (supported: FL_FMT_WORKLOAD, FL_FMT_PAPER)", fn, c->fmt);
  if (c->fmt == FL_FMT_PAPER && c->d != 128)
    return fail(FL_EUNSUPPORTED, "%s: the paper format needs head dim 128 (got %d)", fn, c->d);
  if (hkv < 1 || c->H % hkv != 0)
    return fail(FL_EINVAL, "%s: Hkv = %d must divide H = %d", fn, c->Hkv, c->H);
  if ((long long)c->L * c->B * c->H * c->S > (1LL << 40)) return fail(FL_EUNSUPPORTED, "%s: cache too large", fn);
  // the tile images of one (b, h) are addressed with 32-bit byte offsets
  if (c->S > FL_MAX_S) return fail(FL_EUNSUPPORTED, "%s: S = %d above FL_MAX_S = %d", fn, c->S, FL_MAX_S);
  FL_NEED_PTR(c->base, "cache->base");
  const int last = need_res_r ? r : r - 1;
  for (int rr = 2; rr <= c->R; ++rr) {
    if (c->n[rr] < 1 || c->n[rr] > c->n[rr - 1])
      return fail(FL_EINVAL, "%s: n[%d] = %d must be in [1, n[%d] = %d] (nested sets)", fn, rr, c->n[rr], rr - 1,
                  c->n[rr - 1]);
    if (c->bits[rr] != 2 && c->bits[rr] != 4)
      return fail(FL_EUNSUPPORTED, "%s: bits[%d] = %d (supported: 2, 4)", fn, rr, c->bits[rr]);
  }
  for (int rr = 2; rr <= r; ++rr) {
    char name[32];
    std::snprintf(name, sizeof name, "cache->rows[%d]", rr);
    FL_NEED_PTR4(c->rows[rr], name);
    std::snprintf(name, sizeof name, "cache->slot[%d]", rr);
    FL_NEED_PTR4(c->slot[rr], name);
    if (c->cnt[rr] && !aligned4(c->cnt[rr])) return fail(FL_EINVAL, "%s: cache->cnt[%d] is not 4-byte aligned", fn, rr);
    if (rr <= last) {
      std::snprintf(name, sizeof name, "cache->res[%d]", rr);
      FL_NEED_PTR(c->res[rr], name);
    }
  }
  *geo = fl::CacheGeo{};
  geo->L = c->L; geo->B = c->B; geo->H = c->H; geo->S = c->S; geo->d = c->d; geo->R = c->R;
  geo->Hkv = hkv;
  geo->G = c->H / hkv;
  geo->T = c->T == 0 ? c->S : c->T;
  geo->fmt = c->fmt;
  geo->Sq = c->S > fl::kPTailN ? c->S - fl::kPTailN : 0;
  geo->base = c->base;
  geo->base_rb = fl::base_record_bytes(c->d);
  for (int rr = 1; rr <= c->R; ++rr) {
    geo->n[rr] = c->n[rr];
    geo->bits[rr] = rr == 1 ? 8 : c->bits[rr];
    geo->rows[rr] = c->rows[rr];
    geo->slot[rr] = c->slot[rr];
    geo->cnt[rr] = rr == 1 ? nullptr : c->cnt[rr];
    geo->res[rr] = c->res[rr];
    geo->res_rb[rr] = rr == 1 ? 0 : fl::residual_record_bytes(c->d, c->bits[rr]);
    geo->pm[rr] = rr == 1 ? geo->Sq : c->n[rr];
    geo->pbytes[rr] = fl::paper_stream_bytes(geo->pm[rr]);
  }
  geo->res[1] = c->base;  // loop 1's stream of the paper format
  return FL_OK;
}

fl_status check_dtype(const char* fn, fl_dtype dt) {
  if (dt != FL_F32 && dt != FL_BF16) return fail(FL_EUNSUPPORTED, "%s: dtype %d (supported: FL_F32, FL_BF16)", fn, (int)dt);
  return FL_OK;
}

fl_status check_state(const char* fn, const fl_state* s) {
  if (!s) return fail(FL_EINVAL, "%s: state is NULL", fn);
  FL_NEED_PTR(s->O, "state->O");
  FL_NEED_PTR(s->U, "state->U");
  FL_NEED_PTR4(s->M, "state->M");
  FL_NEED_PTR4(s->lse, "state->lse");
  if (s->lsel && !aligned4(s->lsel)) return fail(FL_EINVAL, "%s: state->lsel is not 4-byte aligned", fn);
  return FL_OK;
}

constexpr int kTopkMax = 32768;  // keys per selection problem (32 per thread)

// ---------------------------------------------------------------- FL_CHECK
// The synchronous validator of the device-side index data (the documented
// preconditions nothing else checks): with FL_CHECK set to anything but "0"
// or "", a call first drains its stream, copies the index arrays it will read
// to the host and checks them; a violation returns FL_EINVAL before any
// launch.  A debugging aid: it costs a synchronization and the copies.
bool check_on() {
  const char* e = std::getenv("FL_CHECK");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

template <typename T>
fl_status fetch(const char* fn, std::vector<T>& out, const void* dev, size_t n, hipStream_t st, const char* what) {
  out.assign(n, T{});
  if (n == 0) return FL_OK;
  const hipError_t e = fl::copy_to_host(out.data(), dev, n * sizeof(T), st);
  if (e != hipSuccess) return fail(FL_EHIP, "%s: FL_CHECK could not read %s: %s", fn, what, hipGetErrorString(e));
  return FL_OK;
}

// Loops 2..last_rows: counts in [1, n[r]] and within loop r-1's count, rows
// strictly ascending in [0, S) and a subset of loop r-1's active set (nested
// sets; loop 1 holds every position).  Loops 2..last_slot: slot[r] is the
// inverse of rows[r] (slot[r][b][rows[r][b][t]] = t) and -1 elsewhere.
// active: if non-NULL, receives the [B][S] membership mask of A_last_rows.
fl_status check_index_sets(const char* fn, const fl_cache* c, int last_rows, int last_slot, hipStream_t st,
                           std::vector<uint8_t>* active = nullptr, std::vector<int32_t>* counts = nullptr,
                           std::vector<int32_t>* rows_out = nullptr) {
  const int B = c->B, S = c->S;
  std::vector<int32_t> prev_cnt(B, S), cnt, rows, slot;
  std::vector<uint8_t> prev_in((size_t)B * S, 1), in((size_t)B * S, 0);
  fl_status s;
  for (int r = 2; r <= last_rows; ++r) {
    const int n = c->n[r];
    char what[48];
    if (c->cnt[r]) {
      std::snprintf(what, sizeof what, "cache->cnt[%d]", r);
      if ((s = fetch(fn, cnt, c->cnt[r], (size_t)B, st, what)) != FL_OK) return s;
    } else {
      cnt.assign(B, n);
    }
    std::snprintf(what, sizeof what, "cache->rows[%d]", r);
    if ((s = fetch(fn, rows, c->rows[r], (size_t)B * n, st, what)) != FL_OK) return s;
    if (r <= last_slot) {
      std::snprintf(what, sizeof what, "cache->slot[%d]", r);
      if ((s = fetch(fn, slot, c->slot[r], (size_t)B * S, st, what)) != FL_OK) return s;
    }
    std::fill(in.begin(), in.end(), (uint8_t)0);
    for (int b = 0; b < B; ++b) {
      const int t = cnt[b];
      if (t < 1 || t > n)
        return fail(FL_EINVAL, "%s: FL_CHECK: sequence %d has %d active rows at loop %d, outside [1, n[%d] = %d]", fn,
                    b, t, r, r, n);
      if (t > prev_cnt[b])
        return fail(FL_EINVAL, "%s: FL_CHECK: sequence %d has %d active rows at loop %d, more than loop %d's %d "
                    "(nested sets)", fn, b, t, r, r - 1, prev_cnt[b]);
      const int32_t* rw = &rows[(size_t)b * n];
      uint8_t* mine = &in[(size_t)b * S];
      const uint8_t* theirs = &prev_in[(size_t)b * S];
      for (int i = 0; i < t; ++i) {
        const int j = rw[i];
        if (j < 0 || j >= S)
          return fail(FL_EINVAL, "%s: FL_CHECK: rows[%d][%d][%d] = %d outside [0, S = %d)", fn, r, b, i, j, S);
        if (i > 0 && j <= rw[i - 1])
          return fail(FL_EINVAL, "%s: FL_CHECK: rows[%d] of sequence %d not strictly ascending at entry %d (%d after %d)",
                      fn, r, b, i, j, rw[i - 1]);
        if (!theirs[j])
          return fail(FL_EINVAL, "%s: FL_CHECK: rows[%d] of sequence %d holds position %d, not active at loop %d "
                      "(nested sets)", fn, r, b, j, r - 1);
        mine[j] = 1;
      }
      if (r <= last_slot) {
        const int32_t* sl = &slot[(size_t)b * S];
        for (int i = 0; i < t; ++i)
          if (sl[rw[i]] != i)
            return fail(FL_EINVAL, "%s: FL_CHECK: slot[%d][%d][%d] = %d, expected %d (rows[%d] entry)", fn, r, b, rw[i],
                        sl[rw[i]], i, r);
        for (int j = 0; j < S; ++j)
          if (sl[j] != -1 && !mine[j])
            return fail(FL_EINVAL, "%s: FL_CHECK: slot[%d][%d][%d] = %d for a position outside loop %d's rows", fn, r,
                        b, j, sl[j], r);
      }
    }
    prev_cnt.swap(cnt);
    prev_in.swap(in);
    if (rows_out && r == last_rows) *rows_out = rows;
  }
  if (active) *active = prev_in;
  if (counts) *counts = prev_cnt;
  return FL_OK;
}

// P rows of `len` int32 entries, `stride` entries apart: each strictly
// ascending within [0, lim).
fl_status check_sel(const char* fn, const int32_t* dev, long long P, int len, long long stride, int lim,
                    hipStream_t st, const char* what) {
  if (P <= 0 || len <= 0) return FL_OK;
  std::vector<int32_t> h((size_t)P * len);
  const hipError_t e = fl::copy_rows_to_host(h.data(), (size_t)len * 4, dev, (size_t)stride * 4, (size_t)len * 4,
                                             (size_t)P, st);
  if (e != hipSuccess) return fail(FL_EHIP, "%s: FL_CHECK could not read %s: %s", fn, what, hipGetErrorString(e));
  for (long long p = 0; p < P; ++p) {
    const int32_t* x = &h[(size_t)p * len];
    for (int i = 0; i < len; ++i) {
      if (x[i] < 0 || x[i] >= lim)
        return fail(FL_EINVAL, "%s: FL_CHECK: %s row %lld entry %d = %d outside [0, %d)", fn, what, p, i, x[i], lim);
      if (i > 0 && x[i] <= x[i - 1])
        return fail(FL_EINVAL, "%s: FL_CHECK: %s row %lld not strictly ascending at entry %d (%d after %d)", fn, what,
                    p, i, x[i], x[i - 1]);
    }
  }
  return FL_OK;
}

}  // namespace

extern "C" {

int fl_abi_version(void) { return FL_ABI_VERSION; }

const char* fl_last_error(void) { return g_err.c_str(); }

size_t fl_base_record_bytes(int d) { return (d == 64 || d == 128) ? (size_t)fl::base_record_bytes(d) : 0; }

size_t fl_stream_bytes(const fl_cache* c, int r) {
  if (!c || r < 1 || r > c->R || r > FL_MAX_LOOPS || (c->d != 64 && c->d != 128)) return 0;
  if (c->fmt == FL_FMT_PAPER) {
    if (c->d != 128) return 0;
    const int Sq = c->S > fl::kPTailN ? c->S - fl::kPTailN : 0;
    return (size_t)fl::paper_stream_bytes(r == 1 ? Sq : c->n[r]);
  }
  if (r == 1) return (size_t)c->S * fl::base_record_bytes(c->d);
  if (c->bits[r] != 2 && c->bits[r] != 4) return 0;
  return (size_t)c->n[r] * fl::residual_record_bytes(c->d, c->bits[r]);
}

size_t fl_residual_record_bytes(int d, int bits) {
  if ((d != 64 && d != 128) || (bits != 2 && bits != 4)) return 0;
  return (size_t)fl::residual_record_bytes(d, bits);
}

namespace {
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
size_t tiles_bytes(const fl_cache* c, int K) {
  if (c->d != 128 || K < 1) return 0;
  fl::CacheGeo g{};
  g.B = c->B;
  g.H = c->H;
  return fl::gather_bytes(g, K);
}
// The mass pass: the candidates' tiles unless it reads the base (r == 2 over
// every position), then the row images of A_r.
size_t mass_pass_bytes(const fl_cache* c, int r, bool base, int K_prev) {
  if (c->d != 128) return 0;
  return (base ? 0 : tiles_bytes(c, K_prev)) + fl::row_img_bytes(c->B, c->H, c->n[r]);
}
// The first-level histogram of the masses the column-mass pass counts for
// the top-K (head dim 128, where that pass is the MFMA one).
size_t hist_bytes(const fl_cache* c) {
  if (c->d != 128) return 0;
  return align256((size_t)c->B * c->H * fl::kHistBins * sizeof(uint32_t));
}
}  // namespace

size_t fl_workspace_bytes(int which, const fl_cache* cache, int r, int K_prev, int K_r) {
  if (!cache || r < 1 || r > cache->R) return 0;
  // loop 1's attention covers every position whatever the budgets say
  if (which == FL_WS_ATTN && r == 1) return tiles_bytes(cache, cache->S);
  if (K_prev < 0 || K_r < 0) return 0;
  if (which == FL_WS_COLSEL) {
    // masses, their first-level histogram, then (in turn) what the mass
    // pass reads and the tiles of the selected columns the cached-mass pass
    // gathers
    if (r > cache->R || r < 2) return 0;
    const bool base = r == 2 && K_prev == cache->S && cache->fmt == FL_FMT_WORKLOAD;
    return align256((size_t)cache->B * cache->H * (size_t)K_prev * sizeof(float)) + hist_bytes(cache) +
           std::max(tiles_bytes(cache, K_r), mass_pass_bytes(cache, r, base, K_prev));
  }
  if (which == FL_WS_ATTN) return tiles_bytes(cache, K_r);
  return 0;
}

fl_status fl_kv_resq(const fl_cache* cache, int r, const void* k, const void* v, fl_dtype dtype, fl_stream stream) {
  const char* fn = "fl_kv_resq";
  g_err.clear();
  fl::CacheGeo geo;
  fl_status s = check_cache(fn, cache, r, true, &geo);
  if (s != FL_OK) return s;
  if ((s = check_dtype(fn, dtype)) != FL_OK) return s;
  FL_NEED_PTR(k, "k");
  FL_NEED_PTR(v, "v");
  hipStream_t st = (hipStream_t)stream;
  // loop r's rows are read here; slot[r] is written here
  if (check_on() && r >= 2 && (s = check_index_sets(fn, cache, r, r - 1, st)) != FL_OK) return s;
  hipError_t e;
  if (r == 1) {
    e = geo.fmt == FL_FMT_PAPER ? fl::launch_paper_quant(geo, 1, k, v, dtype, cache->base, st)
                                : fl::launch_quant_base(geo, k, v, dtype, cache->base, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return FL_OK;
  }
  e = fl::launch_build_slot(geo, r, cache->slot[r], st);
  if (e != hipSuccess) return hip_fail(e, fn);
  e = geo.fmt == FL_FMT_PAPER ? fl::launch_paper_quant(geo, r, k, v, dtype, cache->res[r], st)
                              : fl::launch_quant_res(geo, r, k, v, dtype, cache->res[r], st);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

fl_status fl_kv_append(const fl_cache* cache, int r, int pos, const void* k, const void* v, fl_dtype dtype,
                       fl_stream stream) {
  const char* fn = "fl_kv_append";
  g_err.clear();
  fl::CacheGeo geo;
  fl_status s = check_cache(fn, cache, r, true, &geo);
  if (s != FL_OK) return s;
  if ((s = check_dtype(fn, dtype)) != FL_OK) return s;
  FL_NEED_PTR(k, "k");
  FL_NEED_PTR(v, "v");
  if (pos < 0 || pos >= cache->S) return fail(FL_EINVAL, "%s: pos = %d outside [0, S = %d)", fn, pos, cache->S);
  if (geo.fmt == FL_FMT_PAPER)
    return fail(FL_EUNSUPPORTED, "%s: appending to the paper format (its key groups span 64 tokens)", fn);
  if (r >= 2 && !cache->cnt[r])
    return fail(FL_EINVAL, "%s: appending a row at loop %d needs the per-sequence counts cache->cnt[%d]", fn, r, r);
  if (check_on() && r >= 2) {
    // the sets as they stand, then: pos active at loop r-1 and after every
    // row loop r holds in each sequence that still has room
    std::vector<uint8_t> prev_in;
    std::vector<int32_t> prev_cnt, cnt, rows;
    if ((s = check_index_sets(fn, cache, r - 1, r - 1, (hipStream_t)stream, &prev_in, &prev_cnt)) != FL_OK) return s;
    if ((s = check_index_sets(fn, cache, r, r, (hipStream_t)stream, nullptr, &cnt, &rows)) != FL_OK) return s;
    for (int b = 0; b < cache->B; ++b) {
      if (cnt[b] >= cache->n[r]) continue;
      if (!prev_in[(size_t)b * cache->S + pos])
        return fail(FL_EINVAL, "%s: FL_CHECK: position %d is not active at loop %d in sequence %d (nested sets)", fn,
                    pos, r - 1, b);
      if (rows[(size_t)b * cache->n[r] + cnt[b] - 1] >= pos)
        return fail(FL_EINVAL, "%s: FL_CHECK: position %d does not follow the active rows of loop %d in sequence %d",
                    fn, pos, r, b);
    }
  }
  hipError_t e = fl::launch_append(geo, r, pos, k, v, dtype, cache->base, cache->res[r],
                                   r >= 2 ? const_cast<int32_t*>(cache->rows[r]) : nullptr,
                                   r >= 2 ? cache->slot[r] : nullptr, r >= 2 ? cache->cnt[r] : nullptr,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

fl_status fl_colsel(const fl_cache* cache, int r, const void* q_prev, fl_dtype dtype, const fl_state* state,
                    int K_prev, const int32_t* cand, int K_r, const float* mass_in, float* mass_out, int32_t* sel_out,
                    void* ws, size_t ws_bytes, fl_stream stream) {
  const char* fn = "fl_colsel";
  g_err.clear();
  fl::CacheGeo geo;
  fl_status s = check_cache(fn, cache, r, false, &geo);
  if (s != FL_OK) return s;
  if (r < 2) return fail(FL_EINVAL, "%s: loop r = %d (selection exists for r >= 2)", fn, r);
  if (cache->L != 1) return fail(FL_EINVAL, "%s: prefill state covers one layer (L = %d)", fn, cache->L);
  if ((s = check_dtype(fn, dtype)) != FL_OK) return s;
  if ((s = check_state(fn, state)) != FL_OK) return s;
  FL_NEED_PTR(q_prev, "q_prev");
  FL_NEED_PTR4(sel_out, "sel_out");
  if (K_prev < 1 || K_prev > cache->S) return fail(FL_EINVAL, "%s: K_prev = %d outside [1, S]", fn, K_prev);
  if (!cand && K_prev != cache->S) return fail(FL_EINVAL, "%s: cand is NULL but K_prev = %d != S", fn, K_prev);
  if (cand && !aligned4(cand)) return fail(FL_EINVAL, "%s: cand is not 4-byte aligned", fn);
  if (K_r < 1 || K_r > K_prev) return fail(FL_EINVAL, "%s: K_r = %d outside [1, K_prev = %d]", fn, K_r, K_prev);
  if (mass_in && !aligned4(mass_in)) return fail(FL_EINVAL, "%s: mass_in is not 4-byte aligned", fn);
  if (mass_out && !aligned4(mass_out)) return fail(FL_EINVAL, "%s: mass_out is not 4-byte aligned", fn);
  const bool prune = K_r < K_prev;
  const bool need_mass = (prune && !mass_in) || mass_out;
  float* mass = mass_out;
  const size_t mass_ws = align256((size_t)cache->B * cache->H * (size_t)K_prev * sizeof(float));
  const size_t hist_ws = hist_bytes(cache);
  // what the mass pass reads, then (reusing the space) the tiles of the
  // selected columns the cached-mass pass gathers
  const size_t pass_ws = std::max(prune ? tiles_bytes(cache, K_r) : 0,
                                  need_mass ? mass_pass_bytes(cache, r, r == 2 && !cand && geo.fmt == FL_FMT_WORKLOAD,
                                                              K_prev) : 0);
  // the masses' first-level histogram, when the top-K can start from it
  const bool use_hist = prune && !mass_in && !cand && hist_ws > 0;
  const size_t need = (need_mass && !mass_out ? mass_ws : 0) + (use_hist ? hist_ws : 0) + pass_ws;
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(FL_EINVAL, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(FL_EINVAL, "%s: ws is not 16-byte aligned", fn);
  }
  uint8_t* tiles_ws = (uint8_t*)ws;
  if (need_mass && !mass_out) {
    mass = (float*)ws;
    tiles_ws += mass_ws;
  }
  uint32_t* hist = nullptr;
  if (use_hist) {
    hist = (uint32_t*)tiles_ws;
    tiles_ws += hist_ws;
  }
  if (prune && K_prev > kTopkMax)
    return fail(FL_EUNSUPPORTED, "%s: %d candidates (at most %d)", fn, K_prev, kTopkMax);
  hipStream_t st = (hipStream_t)stream;
  if (check_on()) {
    // rows of loops <= r; the chains and queries of loop r-1
    if ((s = check_index_sets(fn, cache, r, r - 1, st)) != FL_OK) return s;
    if (cand && (s = check_sel(fn, cand, (long long)cache->B * cache->H, K_prev, K_prev, cache->S, st, "cand")) != FL_OK)
      return s;
    if (prune && mass_in) {
      std::vector<float> m;
      if ((s = fetch(fn, m, mass_in, (size_t)cache->B * cache->H * K_prev, st, "mass_in")) != FL_OK) return s;
      for (size_t i = 0; i < m.size(); ++i)
        if (std::isnan(m[i])) return fail(FL_EINVAL, "%s: FL_CHECK: mass_in[%zu] is NaN", fn, i);
    }
  }
  fl::AttnArgs a{};
  a.c = geo;
  a.r = r;
  a.dt = dtype;
  a.q = q_prev;
  a.O = state->O; a.U = state->U; a.M = state->M; a.lse = state->lse;
  a.lsel = state->lsel;
  hipError_t e;
  bool hist_built = false;
  if (need_mass) {
    e = fl::launch_mass(a, cand, K_prev, mass, tiles_ws, st, hist, &hist_built);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  const int P = cache->B * cache->H;
  if (!prune) {
    e = fl::launch_copy_sel(cand, P, K_prev, sel_out, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    // same columns as loop r-1: their loop r-1 log-sum-exp is loop r-1's lse
    if (state->lsel) {
      e = fl::copy_d2d_async(state->lsel, state->lse, (size_t)P * cache->S * sizeof(float), st);
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    return FL_OK;
  }
  const float* keys = mass_in ? mass_in : mass;
  e = fl::launch_topk(keys, K_prev, cand, K_prev, P, K_prev, K_r, sel_out, K_r, nullptr, 0, st,
                      hist_built ? (const int32_t*)hist : nullptr, fl::kHistBins);
  if (e != hipSuccess) return hip_fail(e, fn);
  a.K = K_r;
  a.sel = sel_out;
  e = fl::launch_um(a, tiles_ws, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

fl_status fl_loop_attn(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_r, const int32_t* sel,
                       const fl_state* state, void* ws, size_t ws_bytes, fl_stream stream) {
  const char* fn = "fl_loop_attn";
  g_err.clear();
  fl::CacheGeo geo;
  fl_status s = check_cache(fn, cache, r, true, &geo);
  if (s != FL_OK) return s;
  if (cache->L != 1) return fail(FL_EINVAL, "%s: prefill state covers one layer (L = %d)", fn, cache->L);
  if ((s = check_dtype(fn, dtype)) != FL_OK) return s;
  if ((s = check_state(fn, state)) != FL_OK) return s;
  FL_NEED_PTR(q, "q");
  if (r >= 2) {
    FL_NEED_PTR4(sel, "sel");
    if (K_r < 1 || K_r > cache->S) return fail(FL_EINVAL, "%s: K_r = %d outside [1, S]", fn, K_r);
  }
  {
    // the tile images of every attended column (K_r has been checked when r >= 2; loop 1 attends all S)
    const size_t need = dtype == FL_BF16 ? tiles_bytes(cache, r == 1 ? cache->S : K_r) : 0;
    if (need > 0 && (!ws || ws_bytes < need))
      return fail(FL_EINVAL, "%s: workspace of %zu bytes needed (got %zu)", fn, need, ws ? ws_bytes : (size_t)0);
    if (need > 0 && !aligned16(ws)) return fail(FL_EINVAL, "%s: ws is not 16-byte aligned", fn);
  }
  if (check_on() && r >= 2) {
    if ((s = check_index_sets(fn, cache, r, r, (hipStream_t)stream)) != FL_OK) return s;
    if ((s = check_sel(fn, sel, (long long)cache->B * cache->H, K_r, K_r, cache->S, (hipStream_t)stream, "sel")) !=
        FL_OK)
      return s;
  }
  fl::AttnArgs a{};
  a.c = geo;
  a.r = r;
  a.dt = dtype;
  a.q = q;
  a.K = r >= 2 ? K_r : 0;
  a.sel = r >= 2 ? sel : nullptr;
  a.O = state->O; a.U = state->U; a.M = state->M; a.lse = state->lse;
  a.lsel = state->lsel;
  hipError_t e = fl::launch_attn(a, (uint8_t*)ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

fl_status fl_loop_decode(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_prev, int K_r,
                         const fl_dstate* state, void* ws, size_t ws_bytes, fl_stream stream) {
  (void)ws;
  (void)ws_bytes;
  const char* fn = "fl_loop_decode";
  g_err.clear();
  fl::CacheGeo geo;
  fl_status s = check_cache(fn, cache, r, true, &geo);
  if (s != FL_OK) return s;
  if (cache->d != 128) return fail(FL_EUNSUPPORTED, "%s: head dim %d (decode supports 128)", fn, cache->d);
  if ((s = check_dtype(fn, dtype)) != FL_OK) return s;
  if (!state) return fail(FL_EINVAL, "%s: state is NULL", fn);
  FL_NEED_PTR(state->O, "state->O");
  FL_NEED_PTR(state->U, "state->U");
  FL_NEED_PTR4(state->M, "state->M");
  FL_NEED_PTR4(state->lse, "state->lse");
  FL_NEED_PTR4(state->logits, "state->logits");
  FL_NEED_PTR4(state->sel, "state->sel");
  FL_NEED_PTR(q, "q");
  if ((long long)cache->L * cache->B * cache->H > 0x7FFFFFFFLL)
    return fail(FL_EUNSUPPORTED, "%s: too many (layer, sequence, head) triples", fn);
  if (r >= 2) {
    if (K_prev < 1 || K_prev > geo.T) return fail(FL_EINVAL, "%s: K_prev = %d outside [1, T = %d]", fn, K_prev, geo.T);
    if (r == 2 && K_prev != geo.T) return fail(FL_EINVAL, "%s: at r = 2 K_prev must be T = %d", fn, geo.T);
    if (K_r < 1 || K_r > K_prev) return fail(FL_EINVAL, "%s: K_r = %d outside [1, K_prev = %d]", fn, K_r, K_prev);
    if (K_r < K_prev && K_prev > kTopkMax)
      return fail(FL_EUNSUPPORTED, "%s: %d candidates (at most %d)", fn, K_prev, kTopkMax);
  }
  if (check_on() && r >= 2) {
    if ((s = check_index_sets(fn, cache, r, r, (hipStream_t)stream)) != FL_OK) return s;
    // loop r >= 3 ranks (or keeps) the previous loop's selection
    if (r >= 3 && (s = check_sel(fn, state->sel, (long long)cache->L * cache->B * cache->H, K_prev, cache->S, geo.T,
                                 (hipStream_t)stream, "state->sel")) != FL_OK)
      return s;
  }
  fl::DecodeArgs a{};
  a.c = geo;
  a.r = r;
  a.dt = dtype;
  a.q = q;
  a.K_prev = K_prev;
  a.K = K_r;
  a.O = state->O; a.U = state->U; a.M = state->M; a.lse = state->lse;
  a.logits = state->logits;
  a.sel = state->sel;
  hipError_t e = fl::launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

fl_status fl_select_active(int B, int S, int D, const void* h_prev, const void* h_cur, fl_dtype dtype, int n_prev,
                           const int32_t* rows_prev, int k, int32_t* rows_out, float* score_out, fl_stream stream) {
  const char* fn = "fl_select_active";
  g_err.clear();
  if (B < 1 || S < 1) return fail(FL_EINVAL, "%s: B, S must be >= 1 (got %d, %d)", fn, B, S);
  if (D < 8 || D % 8 != 0) return fail(FL_EUNSUPPORTED, "%s: hidden size %d (a positive multiple of 8)", fn, D);
  fl_status s = check_dtype(fn, dtype);
  if (s != FL_OK) return s;
  FL_NEED_PTR(h_prev, "h_prev");
  FL_NEED_PTR(h_cur, "h_cur");
  FL_NEED_PTR4(rows_out, "rows_out");
  FL_NEED_PTR4(score_out, "score_out");
  if (n_prev < 1 || n_prev > S) return fail(FL_EINVAL, "%s: n_prev = %d outside [1, S = %d]", fn, n_prev, S);
  if (!rows_prev && n_prev != S) return fail(FL_EINVAL, "%s: rows_prev is NULL but n_prev = %d != S", fn, n_prev);
  if (rows_prev && !aligned4(rows_prev)) return fail(FL_EINVAL, "%s: rows_prev is not 4-byte aligned", fn);
  if (k < 1 || k > n_prev) return fail(FL_EINVAL, "%s: k = %d outside [1, n_prev = %d]", fn, k, n_prev);
  if (k < n_prev && n_prev > kTopkMax)
    return fail(FL_EUNSUPPORTED, "%s: %d candidates (at most %d)", fn, n_prev, kTopkMax);
  if ((long long)B * S * D > (1LL << 40)) return fail(FL_EUNSUPPORTED, "%s: hidden states too large", fn);
  if (check_on() && rows_prev &&
      (s = check_sel(fn, rows_prev, B, n_prev, n_prev, S, (hipStream_t)stream, "rows_prev")) != FL_OK)
    return s;
  hipError_t e = fl::launch_active(B, S, D, h_prev, h_cur, dtype, rows_prev, n_prev, k, rows_out, score_out,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return FL_OK;
}

}  // extern "C"

namespace fl {

// Hooks of the allocation-free entry point (noalloc.hip): the workspace
// fl_loop_attn checks for, and the per-thread error message.
size_t attn_workspace_need(const fl_cache* cache, int r, int K_r, fl_dtype dtype) {
  if (!cache || dtype != FL_BF16) return 0;
  return tiles_bytes(cache, r == 1 ? cache->S : K_r);
}

fl_status report(fl_status s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace fl
