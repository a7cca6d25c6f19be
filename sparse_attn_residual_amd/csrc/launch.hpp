// Host-side launchers of the FlashLoop kernels, called by the C ABI layer
// (abi.cpp) after it has validated every argument.  Each returns the HIP
// status of its launches.
#pragma once

#include "common.hpp"

namespace fl {

// ---- opt-in kernel timing (fl_timing_enable): while the calling thread has
// it on, a launch through FL_LAUNCH records an event on its stream before and
// after the kernel and files the pair under the kernel's name.
struct TimedLaunch {
  TimedLaunch(const char* name, hipStream_t st);
  ~TimedLaunch();
  hipStream_t st;
  int slot;
};
#define FL_LAUNCH(kernel, grid, block, lds, st, ...)                 \
  do {                                                               \
    fl::TimedLaunch fl_timed_(#kernel, st);                          \
    hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);   \
  } while (0)

// ---- fl_kv_resq
hipError_t launch_quant_base(const CacheGeo& c, const void* k, const void* v, fl_dtype dt, uint8_t* base,
                             hipStream_t st);
hipError_t launch_build_slot(const CacheGeo& c, int r, int32_t* slot, hipStream_t st);
// The paper's format: the streams of loop r (base at r == 1) from k, v.
hipError_t launch_paper_quant(const CacheGeo& c, int r, const void* k, const void* v, fl_dtype dt, uint8_t* out,
                              hipStream_t st);
// One new token at position pos, loop r, from k, v [L][B][Hkv][d]: r == 1 the
// base records; r >= 2 row cnt[r][b] of every sequence, then the counts.
hipError_t launch_append(const CacheGeo& c, int r, int pos, const void* k, const void* v, fl_dtype dt,
                         uint8_t* base, uint8_t* res, int32_t* rows, int32_t* slot, int32_t* cnt, hipStream_t st);
hipError_t launch_quant_res(const CacheGeo& c, int r, const void* k, const void* v, fl_dtype dt, uint8_t* res,
                            hipStream_t st);

// ---- selection (top-K of keys per problem; ties to the lower position).
// keys [P][key_stride] (first n valid), cand [P][cand_stride] or NULL (iota);
// writes sel_out [P][sel_stride] ascending and, if keys_out is set, the keys
// of the selected entries in the same order.  In place (keys_out == keys,
// sel_out == cand) is allowed: every block reads its inputs before writing.
// given_hist: rows of hist_stride entries, one per problem, whose first
// kHistBins entries hold the problem's histogram of keys by the top 11 bits
// of their order keys (cand NULL, n <= 32768); the search starts from it.
// It may be sel_out itself (every row read before any is written).
hipError_t launch_topk(const float* keys, long long key_stride, const int32_t* cand, long long cand_stride,
                       int P, int n, int K, int32_t* sel_out, long long sel_stride, float* keys_out,
                       long long keys_out_stride, hipStream_t st, const int32_t* given_hist = nullptr,
                       long long hist_stride = 0);
// sel[p][t] = cand ? cand[p][t] : t for t < K
hipError_t launch_copy_sel(const int32_t* cand, int P, int K, int32_t* sel, hipStream_t st, long long sel_stride = 0);

// ---- prefill attention family (one layer: l = 0).
struct AttnArgs {
  CacheGeo c;
  int r;                 // loop whose chain / state is used
  fl_dtype dt;
  const void* q;         // [B][H][nq][d], rows of loop r (r == 1: all S)
  int K;                 // number of selected columns (r >= 2)
  const int32_t* sel;    // [B][H][K] or NULL (dense loop 1)
  float* O;
  float* U;
  float* M;
  float* lse;
  float* lsel;           // NULL: mass-rescaled combine; else the mixed-logit ablation
};
// Loop r attention (dense when r == 1, sparse otherwise).  ws: workspace of
// gather_bytes(c, K) bytes for the gathered column tiles (sparse loops).
hipError_t launch_attn(const AttnArgs& a, uint8_t* ws, hipStream_t st);
// Cached mass and reused part for loop r: reads loop r-1 state, q_prev and
// chains to r-1; rows A_r; columns sel (S_r).  ws as for launch_attn.
hipError_t launch_um(const AttnArgs& a, uint8_t* ws, hipStream_t st);
// Bytes of one 64-column tile image and of one 64-row query image of the
// matrix-core kernels (attn_mfma.hip lays them out).
constexpr int kTileImgBytes = 36 * 1024;
constexpr int kRowImgBytes = 18 * 1024;
// Bytes of the gathered tiles of K selected columns (head dim 128).
inline size_t gather_bytes(const CacheGeo& c, int K) {
  return (size_t)c.B * c.H * (size_t)((K + 63) / 64) * kTileImgBytes;
}
// Bytes of the 64-row images of n rows per (b, h) that the mass pass streams.
inline size_t row_img_bytes(int B, int H, int n) { return (size_t)B * H * (size_t)((n + 63) / 64) * kRowImgBytes; }
// Column mass of the candidates cand (NULL: all S) over rows A_r with loop
// r-1's probabilities.  ws (head dim 128, bf16): gather_bytes(c, K_prev)
// bytes when the candidates are gathered (cand != NULL or r > 2), then
// row_img_bytes(B, H, n_r).
// hist (or NULL): [B*H][kHistBins] space for the masses' first-level
// histogram; *hist_built says whether it was filled.
hipError_t launch_mass(const AttnArgs& a, const int32_t* cand, int K_prev, float* mass, uint8_t* ws,
                       hipStream_t st, uint32_t* hist = nullptr, bool* hist_built = nullptr);

// ---- next active set: scores [B][n_prev] (relative hidden-state change of
// the candidates rows_prev, NULL: positions 0..n_prev-1), then the top k of
// each sequence into rows_out [B][k], ascending.
hipError_t launch_active(int B, int S, int D, const void* h_prev, const void* h_cur, fl_dtype dt,
                         const int32_t* rows_prev, int n_prev, int k, int32_t* rows_out, float* score,
                         hipStream_t st);

// ---- memory operations of the ABI layer (no kernels)
// Synchronous copies to host memory after the stream has drained (the
// FL_CHECK validator): bytes contiguous, or `rows` rows of `width` bytes.
hipError_t copy_to_host(void* dst, const void* src, size_t bytes, hipStream_t st);
hipError_t copy_rows_to_host(void* dst, size_t dst_pitch, const void* src, size_t src_pitch, size_t width,
                             size_t rows, hipStream_t st);
// Device-to-device copy on the stream.
hipError_t copy_d2d_async(void* dst, const void* src, size_t bytes, hipStream_t st);

// ---- the allocation-free entry point (abi.cpp)
// Workspace bytes fl_loop_attn requires for these arguments (0 when none).
size_t attn_workspace_need(const fl_cache* cache, int r, int K_r, fl_dtype dtype);
// Sets the calling thread's error message; returns s.
fl_status report(fl_status s, const char* msg);

// ---- decode
struct DecodeArgs {
  CacheGeo c;
  int r;
  fl_dtype dt;
  const void* q;     // [L][B][H][d]
  int K_prev, K;
  float* O;
  float* U;
  float* M;
  float* lse;
  float* logits;     // [L][B][H][S]
  int32_t* sel;      // [L][B][H][S]
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

}  // namespace fl
