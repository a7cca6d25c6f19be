// CPU driver of the C ABI's validation layer (abi.cpp linked against
// stub_launch.cpp), built with AddressSanitizer by tests/test_abi.py.
// Host arrays stand in for device memory: the stub launch layer copies them
// with memcpy and only counts launches.  Exit status 0 and a final "PASS"
// line when every case behaves; the first failing case is printed.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "flashloop.h"

extern int g_launches;

static int g_cases = 0;

#define EXPECT(cond, ...)                                   \
  do {                                                      \
    ++g_cases;                                              \
    if (!(cond)) {                                          \
      std::printf("FAIL line %d: ", __LINE__);              \
      std::printf(__VA_ARGS__);                             \
      std::printf(" [%s]\n", fl_last_error());              \
      std::exit(1);                                         \
    }                                                       \
  } while (0)

// 256-byte aligned host buffer of n elements
template <typename T>
struct Buf {
  T* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t count) : n(count) {
    p = static_cast<T*>(std::aligned_alloc(256, ((count * sizeof(T) + 255) / 256 + 1) * 256));
    std::memset(p, 0, count * sizeof(T));
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

// One consistent index set: B sequences, S positions, loops 1..3 with the
// given capacities and per-sequence counts, slots the inverse of the rows.
struct Sets {
  int B, S;
  int n[4];
  Buf<int32_t> rows2, rows3, slot2, slot3, cnt2, cnt3;
  Sets(int B_, int S_, int n2, int n3, unsigned seed)
      : B(B_), S(S_), n{0, S_, n2, n3}, rows2((size_t)B_ * n2), rows3((size_t)B_ * n3), slot2((size_t)B_ * S_),
        slot3((size_t)B_ * S_), cnt2(B_), cnt3(B_) {
    std::mt19937 g(seed);
    for (int b = 0; b < B; ++b) {
      std::vector<int> all(S);
      for (int j = 0; j < S; ++j) all[j] = j;
      std::shuffle(all.begin(), all.end(), g);
      std::vector<int> a2(all.begin(), all.begin() + n2);
      std::sort(a2.begin(), a2.end());
      std::vector<int> pick(a2);
      std::shuffle(pick.begin(), pick.end(), g);
      std::vector<int> a3(pick.begin(), pick.begin() + n3);
      std::sort(a3.begin(), a3.end());
      for (int j = 0; j < S; ++j) slot2.p[(size_t)b * S + j] = slot3.p[(size_t)b * S + j] = -1;
      for (int i = 0; i < n2; ++i) {
        rows2.p[(size_t)b * n2 + i] = a2[i];
        slot2.p[(size_t)b * S + a2[i]] = i;
      }
      for (int i = 0; i < n3; ++i) {
        rows3.p[(size_t)b * n3 + i] = a3[i];
        slot3.p[(size_t)b * S + a3[i]] = i;
      }
      cnt2.p[b] = n2;
      cnt3.p[b] = n3;
    }
  }
  void fill(fl_cache& c, uint8_t* base, uint8_t* res, bool counts) {
    c.n[1] = S;
    c.n[2] = n[2];
    c.n[3] = n[3];
    c.rows[2] = rows2.p;
    c.rows[3] = rows3.p;
    c.slot[2] = slot2.p;
    c.slot[3] = slot3.p;
    c.base = base;
    c.res[2] = c.res[3] = res;
    c.cnt[2] = counts ? cnt2.p : nullptr;
    c.cnt[3] = counts ? cnt3.p : nullptr;
  }
};

static fl_cache make_cache(int d, int B, int H, int S, int L) {
  fl_cache c;
  std::memset(&c, 0, sizeof c);
  c.L = L;
  c.B = B;
  c.H = H;
  c.S = S;
  c.d = d;
  c.R = 3;
  c.bits[1] = 8;
  c.bits[2] = 4;
  c.bits[3] = 2;
  return c;
}

static bool has_check_msg() { return std::strstr(fl_last_error(), "FL_CHECK") != nullptr; }

int main() {
  const int B = 2, H = 2, S = 64, n2 = 30, n3 = 12;
  Buf<uint8_t> base(1 << 20), res(1 << 20), kv(1 << 20), ws(1 << 22);
  Buf<float> O(1 << 16), U(1 << 16), M(1 << 12), lse(1 << 12), mass(1 << 12), massin((size_t)B * H * S);
  Buf<int32_t> sel2((size_t)B * H * 10), sel3((size_t)B * H * 5);
  fl_state st{O.p, U.p, M.p, lse.p, nullptr};
  for (int p = 0; p < B * H; ++p) {
    for (int i = 0; i < 10; ++i) sel2.p[p * 10 + i] = 3 * i + 2;
    for (int i = 0; i < 5; ++i) sel3.p[p * 5 + i] = 6 * i + 2;
  }

  // ---- off by default: bad index data is not looked at
  unsetenv("FL_CHECK");
  {
    Sets s(B, S, n2, n3, 1);
    fl_cache c = make_cache(64, B, H, S, 1);
    s.fill(c, base.p, res.p, false);
    std::swap(s.rows2.p[0], s.rows2.p[1]);
    const int before = g_launches;
    EXPECT(fl_kv_resq(&c, 2, kv.p, kv.p, FL_F32, nullptr) == FL_OK, "unchecked resq");
    EXPECT(g_launches > before, "unchecked resq launched");
  }

  setenv("FL_CHECK", "1", 1);
  // ---- valid data passes every checked call
  {
    Sets s(B, S, n2, n3, 2);
    fl_cache c = make_cache(64, B, H, S, 1);
    s.fill(c, base.p, res.p, true);
    int before = g_launches;
    EXPECT(fl_kv_resq(&c, 2, kv.p, kv.p, FL_F32, nullptr) == FL_OK, "valid resq 2");
    EXPECT(fl_kv_resq(&c, 3, kv.p, kv.p, FL_F32, nullptr) == FL_OK, "valid resq 3");
    EXPECT(fl_colsel(&c, 2, kv.p, FL_F32, &st, S, nullptr, 10, nullptr, mass.p, sel2.p, nullptr, 0, nullptr) == FL_OK,
           "valid colsel 2");
    EXPECT(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr) == FL_OK, "valid attn 2");
    EXPECT(fl_colsel(&c, 3, kv.p, FL_F32, &st, 10, sel2.p, 5, nullptr, mass.p, sel3.p, nullptr, 0, nullptr) == FL_OK,
           "valid colsel 3");
    EXPECT(fl_loop_attn(&c, 3, kv.p, FL_F32, 5, sel3.p, &st, nullptr, 0, nullptr) == FL_OK, "valid attn 3");
    for (int i = 0; i < B * H * S; ++i) massin.p[i] = (float)(i % 7);
    EXPECT(fl_colsel(&c, 2, kv.p, FL_F32, &st, S, nullptr, 10, massin.p, nullptr, sel2.p, nullptr, 0, nullptr) ==
               FL_OK, "valid colsel with mass_in");
    EXPECT(g_launches > before, "valid calls launched");
  }

  // ---- each violation: FL_EINVAL, an FL_CHECK message, nothing launched
  auto refused = [](fl_status st_, const char* what) {
    EXPECT(st_ == FL_EINVAL && has_check_msg(), "%s: status %d", what, (int)st_);
  };
  {
    Sets s(B, S, n2, n3, 3);
    fl_cache c = make_cache(64, B, H, S, 1);
    s.fill(c, base.p, res.p, true);
    const int before = g_launches;
    // loop-2 rows not ascending
    std::swap(s.rows2.p[n2 + 3], s.rows2.p[n2 + 4]);
    refused(fl_kv_resq(&c, 2, kv.p, kv.p, FL_F32, nullptr), "unsorted rows");
    refused(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr), "unsorted rows (attn)");
    std::swap(s.rows2.p[n2 + 3], s.rows2.p[n2 + 4]);
    // a loop-2 row outside [0, S)
    const int keep = s.rows2.p[n2 - 1];
    s.rows2.p[n2 - 1] = S;
    refused(fl_kv_resq(&c, 2, kv.p, kv.p, FL_F32, nullptr), "row out of range");
    s.rows2.p[n2 - 1] = keep;
    // loop-3 rows not a subset of loop 2's: a position outside A_2, order kept
    {
      int j = 0;
      std::vector<char> in2(S, 0);
      for (int i = 0; i < n2; ++i) in2[s.rows2.p[i]] = 1;
      while (in2[j]) ++j;
      const int old = s.rows3.p[0];
      std::vector<int> v(s.rows3.p, s.rows3.p + n3);
      v[0] = j;
      std::sort(v.begin(), v.end());
      std::vector<int> saved(s.rows3.p, s.rows3.p + n3);
      std::copy(v.begin(), v.end(), s.rows3.p);
      refused(fl_kv_resq(&c, 3, kv.p, kv.p, FL_F32, nullptr), "rows not nested");
      std::copy(saved.begin(), saved.end(), s.rows3.p);
      (void)old;
    }
    // counts: more rows at loop 3 than at loop 2, a zero count
    s.cnt2.p[1] = n3 - 1;
    refused(fl_kv_resq(&c, 3, kv.p, kv.p, FL_F32, nullptr), "count above the previous loop's");
    s.cnt2.p[1] = n2;
    s.cnt3.p[0] = 0;
    refused(fl_kv_resq(&c, 3, kv.p, kv.p, FL_F32, nullptr), "zero count");
    s.cnt3.p[0] = n3;
    s.cnt2.p[0] = n2 + 1;
    refused(fl_kv_resq(&c, 2, kv.p, kv.p, FL_F32, nullptr), "count above capacity");
    s.cnt2.p[0] = n2;
    // slot of loop 2 not the inverse of its rows
    {
      int32_t* sl = s.slot2.p + S;  // sequence 1
      const int j = s.rows2.p[n2 + 5];
      sl[j] = 6;
      refused(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr), "wrong slot");
      sl[j] = 5;
      int free_j = 0;
      while (sl[free_j] >= 0) ++free_j;
      sl[free_j] = 0;
      refused(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr), "slot of an inactive position");
      sl[free_j] = -1;
    }
    // selections: unsorted, out of range; candidates unsorted; NaN keys
    std::swap(sel2.p[12], sel2.p[13]);
    refused(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr), "unsorted sel");
    refused(fl_colsel(&c, 3, kv.p, FL_F32, &st, 10, sel2.p, 5, nullptr, mass.p, sel3.p, nullptr, 0, nullptr),
            "unsorted cand");
    std::swap(sel2.p[12], sel2.p[13]);
    const int keep_s = sel2.p[39];
    sel2.p[39] = S;
    refused(fl_loop_attn(&c, 2, kv.p, FL_F32, 10, sel2.p, &st, nullptr, 0, nullptr), "sel out of range");
    sel2.p[39] = keep_s;
    for (int i = 0; i < B * H * S; ++i) massin.p[i] = (float)(i % 7);
    massin.p[77] = std::nanf("");
    refused(fl_colsel(&c, 2, kv.p, FL_F32, &st, S, nullptr, 10, massin.p, nullptr, sel2.p, nullptr, 0, nullptr),
            "NaN mass_in");
    EXPECT(g_launches == before, "refused calls launched %d kernels", g_launches - before);
  }
  // ---- decode (head dim 128): the previous loop's selection as candidates
  {
    Sets s(B, S, n2, n3, 4);
    const int L = 2;
    fl_cache c = make_cache(128, B, H, S, L);
    s.fill(c, base.p, res.p, false);
    Buf<int32_t> dsel((size_t)L * B * H * S);
    for (int p = 0; p < L * B * H; ++p)
      for (int i = 0; i < 10; ++i) dsel.p[(size_t)p * S + i] = 5 * i + 1;
    fl_dstate ds{O.p, U.p, M.p, lse.p, mass.p, dsel.p};
    int before = g_launches;
    EXPECT(fl_loop_decode(&c, 3, kv.p, FL_BF16, 10, 5, &ds, nullptr, 0, nullptr) == FL_OK, "valid decode 3");
    EXPECT(g_launches > before, "decode launched");
    before = g_launches;
    std::swap(dsel.p[(size_t)3 * S + 4], dsel.p[(size_t)3 * S + 5]);
    refused(fl_loop_decode(&c, 3, kv.p, FL_BF16, 10, 5, &ds, nullptr, 0, nullptr), "unsorted decode candidates");
    std::swap(dsel.p[(size_t)3 * S + 4], dsel.p[(size_t)3 * S + 5]);
    c.T = 40;  // candidates must lie below T
    refused(fl_loop_decode(&c, 3, kv.p, FL_BF16, 10, 5, &ds, nullptr, 0, nullptr), "decode candidate beyond T");
    EXPECT(g_launches == before, "refused decode launched");
  }
  // ---- appending: the new position must follow the rows and be active a loop earlier
  {
    Sets s(B, S, n2, n3, 5);
    fl_cache c = make_cache(64, B, H, S, 1);
    s.fill(c, base.p, res.p, true);
    s.cnt2.p[0] = s.cnt2.p[1] = n2 - 1;  // room for one row per sequence
    for (int b = 0; b < B; ++b) s.slot2.p[(size_t)b * S + s.rows2.p[(size_t)b * n2 + n2 - 1]] = -1;
    s.cnt3.p[0] = s.cnt3.p[1] = 1;
    for (int b = 0; b < B; ++b)
      for (int i = 1; i < n3; ++i) s.slot3.p[(size_t)b * S + s.rows3.p[(size_t)b * n3 + i]] = -1;
    const int before = g_launches;
    const int last0 = s.rows2.p[n2 - 2], last1 = s.rows2.p[n2 + n2 - 2];
    const int early = std::min(last0, last1);
    refused(fl_kv_append(&c, 2, early, kv.p, kv.p, FL_F32, nullptr), "append before the rows");
    EXPECT(g_launches == before, "refused append launched");
    int pos = std::max(last0, last1) + 1;
    if (pos < S) {
      EXPECT(fl_kv_append(&c, 2, pos, kv.p, kv.p, FL_F32, nullptr) == FL_OK, "valid append");
    }
  }
  // ---- active-set selection: the previous rows ascending
  {
    Buf<int32_t> prev((size_t)B * 16);
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < 16; ++i) prev.p[b * 16 + i] = 3 * i;
    EXPECT(fl_select_active(B, S, 16, kv.p, kv.p, FL_F32, 16, prev.p, 4, sel3.p, mass.p, nullptr) == FL_OK,
           "valid select");
    std::swap(prev.p[20], prev.p[21]);
    refused(fl_select_active(B, S, 16, kv.p, kv.p, FL_F32, 16, prev.p, 4, sel3.p, mass.p, nullptr),
            "unsorted rows_prev");
  }
  // ---- argument errors (the messages are formatted into fixed buffers)
  {
    fl_cache c = make_cache(96, B, H, S, 1);
    EXPECT(fl_kv_resq(&c, 1, kv.p, kv.p, FL_F32, nullptr) == FL_EUNSUPPORTED, "head dim");
    fl_cache c1 = make_cache(128, B, H, S, 1);
    c1.R = 1;
    c1.n[1] = S;
    c1.base = base.p;
    for (int kr : {-1, 0, 7})
      EXPECT(fl_loop_attn(&c1, 1, kv.p, FL_BF16, kr, nullptr, &st, nullptr, 0, nullptr) == FL_EINVAL &&
                 std::strstr(fl_last_error(), "workspace"),
             "loop-1 workspace with K_r = %d", kr);
    EXPECT(fl_loop_attn(&c1, 1, kv.p, FL_BF16, -1, nullptr, &st, ws.p,
                        fl_workspace_bytes(FL_WS_ATTN, &c1, 1, -1, -1), nullptr) == FL_OK,
           "loop-1 with a sized workspace");
    EXPECT(fl_kv_resq(nullptr, 1, kv.p, kv.p, FL_F32, nullptr) == FL_EINVAL, "null cache");
  }
  std::printf("PASS %d cases\n", g_cases);
  return 0;
}
