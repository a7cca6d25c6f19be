/*
 * flashloop.h — C ABI of the FlashLoop loop-attention hot path on MI355X (gfx950).
 *
 * What the library computes (FlashLoop: Fast and Memory-Efficient Looped
 * Transformers via Lazy Updates; paperlayer.ai abstract page, "p1" below, with
 * its sections; the flozi-tech guide, "guide"):
 *   A looped model applies one shared block R times, H^(r) = F(H^(r-1)), and
 *   keeps a separate (K^(r), V^(r)) for every loop (guide §1; p1 §3).  The
 *   library implements the attention of that block across loops:
 *     - the cross-loop KV cache: a quantized loop-1 base plus quantized
 *       residuals against the reconstructed previous loop, stored for active
 *       tokens only (p1 §4.3, §D.3)            -> fl_kv_resq
 *     - loop-aware column selection: rank the candidate key columns by the
 *       attention mass loop r-1 gave them over the rows loop r recomputes,
 *       keep the top K, cache their mass (p1 §4.2, §D.2)   -> fl_colsel
 *     - sparse loop-r attention: recompute the active rows (p1 §4.1, §D.1)
 *       only against the selected columns and rescale the softmax by their
 *       cached mass, reusing every other column's contribution (p1 §4.2;
 *       guide §3: a low-rank fix of the previous output, eq. 3) -> fl_loop_attn
 *     - the decode step over the packed streams, with the selection fused in
 *       (p1 App. G)                                -> fl_loop_decode
 *
 * Notation: loops r = 1..R; A_r = active rows of a sequence (A_1 = all rows,
 * A_r ⊆ A_{r-1}, shared by every head and layer), n_r = |A_r|; S_r = selected
 * columns of a (b, h) (S_1 = all), K_r = |S_r|, S_r ⊆ S_{r-1}; tau = fp32(1/sqrt(d)).
 * With J_i = {j in S_r : j <= i} and P^(r-1) the probabilities loop r-1 left:
 *   M^r_i = sum_{J_i} P^(r-1)_ij,     U^r_i = O^(r-1)_i - sum_{J_i} P^(r-1)_ij v~^(r-1)_j,
 *   O^r_i = U^r_i + M^r_i * sum_{J_i} softmax_{J_i}(tau q^r_i . k~^r_j) v~^r_j,
 *   lse^r_i = log sum_{J_i} exp(tau q^r_i . k~^r_j).
 * k~, v~ are the reconstructions (rounded to bf16 for bf16 prefill inputs).
 *
 * Conventions for every call:
 *   - All array arguments are device pointers to caller-owned memory.  Index
 *     arrays (rows, slot, cand, sel), masses, M and lse must be 4-byte
 *     aligned; every other array 16-byte aligned.  No call allocates memory
 *     or keeps a pointer after it returns (fl_loop_attn_noalloc's scratch is
 *     a device array the library itself holds).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and do not synchronize.  They are reentrant and thread safe.
 *   - Every argument is validated before anything is launched; on error the
 *     call returns a nonzero fl_status, launches nothing and writes nothing;
 *     fl_last_error() then describes the error (per thread).  No C++ exception
 *     crosses this boundary.
 *   - Device-data preconditions are documented, and checked only on request:
 *     rows strictly ascending and nested, counts within their bounds, slots
 *     the inverse of the rows, selections strictly ascending, finite inputs,
 *     |x| < 8e6 and |x^(r) - x_hat^(r-1)| < 65504 (the ranges of the fp16
 *     scales and zeros).  With the environment variable
 *     FL_CHECK set (to anything but "" or "0"), every call first drains its
 *     stream, copies the index arrays it reads to the host and checks them;
 *     a violation returns FL_EINVAL before anything is launched.  This costs
 *     a synchronization and the copies: a debugging aid.
 *   - FL_TILES=lds (environment, a measurement aid) makes the sparse loops'
 *     attention build its tiles from the packed records in LDS in every row
 *     block instead of reading the tile images built once per loop (the
 *     default; same results bit for bit, measured slower).
 */
#ifndef FLASHLOOP_H
#define FLASHLOOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FL_ABI_VERSION 1
#define FL_MAX_LOOPS 16
/* Longest sequence a cache may hold (2^21 tokens): the prefill kernels address
 * one head's dequantized 64-column tiles (36 KB each) with 32-bit offsets.
 * Larger S: FL_EUNSUPPORTED from every call that takes the cache. */
#define FL_MAX_S (1 << 21)

typedef enum fl_status {
  FL_OK = 0,
  FL_EINVAL = 1,        /* bad pointer, size, loop index or budget */
  FL_EUNSUPPORTED = 2,  /* valid but not implemented: d, bits, dtype, size */
  FL_EHIP = 3           /* a HIP launch or runtime call failed */
} fl_status;

typedef enum fl_dtype {
  FL_F32 = 0,   /* float32 inputs; attention operands are the fp32 reconstructions */
  FL_BF16 = 1   /* bfloat16 inputs; prefill operands rounded to bf16 (matrix cores) */
} fl_dtype;

/* A stream handle: a hipStream_t passed through as an opaque pointer. */
typedef void* fl_stream;

/*
 * The packed cross-loop KV cache of L layers (p1 §4.3 and §D.3; p1 App. G:
 * the engine keeps the base and the residuals as packed streams).  Index r of every
 * loop array is the loop number (index 0 is unused).
 *
 *   L, B, H, S, d, R   layers, sequences, query heads, tokens, head dim (64
 *                      or 128), loops (1..FL_MAX_LOOPS)
 *   Hkv                key/value heads (0: H).  H must be a multiple of it;
 *                      query head h reads KV head h / (H / Hkv) (grouped-query
 *                      attention, a serving variant the pages leave open).
 *                      Queries, states, masses and selections are per query
 *                      head; the streams below are per KV head.
 *   n[r]               active rows per sequence at loop r (n[1] == S); with
 *                      cnt[r] set, the capacity per sequence: the stride of
 *                      rows[r], of the loop-r streams and of loop-r queries
 *   cnt[r]             NULL, or [B] int32 device array: |A_r| of each sequence
 *                      (ragged batches, a serving variant).  Each count must
 *                      lie in [1, n[r]] and in [cnt[r+1][b], cnt[r-1][b]]
 *                      (nested sets; checked under FL_CHECK); rows past a
 *                      sequence's count are neither read nor written.
 *                      fl_kv_append writes them.
 *   T                  tokens a decode step attends, positions [0, T) (0: S);
 *                      S is then the capacity in positions.
 *   fmt                FL_FMT_WORKLOAD (the records below) or FL_FMT_PAPER
 *                      (the paper's own format, head dim 128; see below).
 *
 * FL_FMT_PAPER (p1 App. E: INT4 asymmetric group-wise quantization, group
 * 64, for the base and every residual; post-RoPE keys per channel, values
 * per token; the 64 most recent tokens in BF16).  Sq = max(0, S - 64)
 * positions are quantized, [Sq, S) is the tail.  Each (layer, sequence, KV
 * head) owns, per loop, one stream of fl_stream_bytes(cache, r) bytes:
 *   m entries of 144 bytes (loop 1: m = Sq positions; loop r: m = n[r], the
 *   compact rows): K codes 64 B | V codes 64 B (4-bit, dim 2i in the low
 *   nibble of byte i) | V scale, zero fp16 of dims 0-63, then of 64-127 | 8
 *   zero bytes;
 *   ceil(m / 64) key blocks of 512 bytes: fp16 scales of channels 0..127,
 *   then their fp16 zeros, for entries [64 k, 64 k + 64) (a key group is one
 *   channel over 64 consecutive entries; loop r >= 2: the active rows below
 *   Sq, which come first in rows[r]);
 *   64 tail slots of 512 bytes: K then V of position Sq + slot in bf16 (the
 *   loop's own values of an active tail token).
 * Per group: z = fp16 rounded down of the minimum, s = fp16 rounded up of
 * ((max - z) / 15), c = clamp(rint((x - z) / s), 0, 15) (0 when s == 0),
 * x_hat = fma(c, s, z); loop 1 quantizes x, loop r >= 2 x^(r) - x_hat^(r-1).
 *   bits[r]            residual code width of loop r: 4 or 2 (bits[1] == 8)
 *   rows[r]            [B][n_r] int32, strictly ascending positions of A_r
 *                      (rows[1] unused: every row)
 *   slot[r]            [B][S] int32: index of position j in rows[r], or -1.
 *                      Written by fl_kv_resq(r); read by the other calls.
 *   base               [L][B][Hkv][S] base records (fl_base_record_bytes(d) each)
 *   res[r]             [L][B][Hkv][n_r] residual records of loop r
 *                      (fl_residual_record_bytes(d, bits[r]) each), in rows[r]
 *                      order
 *
 * Base record of one (token, head), G = d/32 groups of 32 dims:
 *   [0,d) K codes int8 | [d,2d) V codes int8 | K scales fp16 x G | V scales fp16 x G
 *   | zero padding to a multiple of 16 bytes          (d = 128: 272 bytes)
 *   x_hat = code * scale (exact in fp32); codes in [-127, 127].
 * Residual record, b bits, C = d*b/8:
 *   [0,C) K codes | [C,2C) V codes | K scales | K zeros | V scales | V zeros
 *   (fp16 x G each) | padding to 16 bytes        (d = 128: 160 bytes at 4 bits, 96 at 2)
 *   4-bit: element 2k in the low nibble of byte k, 2k+1 in the high nibble;
 *   2-bit: element 4k+t in bits 2t..2t+1 of byte k.
 *   delta_hat = fma(code, scale, zero) rounded once to fp32; x_hat^(r) =
 *   x_hat^(r-1) + delta_hat in fp32.  Tokens outside A_r keep x_hat^(r-1).
 */
typedef struct fl_cache {
  int L, B, H, S, d, R;
  int n[FL_MAX_LOOPS + 1];
  int bits[FL_MAX_LOOPS + 1];
  const int32_t* rows[FL_MAX_LOOPS + 1];
  int32_t* slot[FL_MAX_LOOPS + 1];
  uint8_t* base;
  uint8_t* res[FL_MAX_LOOPS + 1];
  int Hkv;
  int32_t* cnt[FL_MAX_LOOPS + 1];
  int T;
  int fmt;
} fl_cache;

/* Per-row prefill state, position indexed (one layer: the cache's L must be 1).
 *   O, U  [B][H][S][d] float32     output and reused part
 *   M     [B][H][S] float32        cached mass of the selected columns
 *   lse   [B][H][S] float32        log-sum-exp of the last recomputation
 *                                  (-inf when a row had no column left)
 *   lsel  [B][H][S] float32 or NULL.  NULL: the method's mass-rescaled
 *         combine (above).  Non-NULL selects the exact mixed-logit combine,
 *         an ablation (p1 §4.2 names the renormalization the method avoids):
 *         fl_colsel's cached-mass pass also stores
 *           L^r_i = log sum_{J_i} exp(tau q^(r-1)_i . k~^(r-1)_j)
 *         and fl_loop_attn forms one softmax over loop r's logits on J_i and
 *         the logits loop r-1's distribution held elsewhere:
 *           O^r_i = (U^r_i + M^r_i rho_i A_i) / (1 - M^r_i + M^r_i rho_i),
 *           rho_i = exp(lse^r_i - L^r_i), A_i = softmax_{J_i}(...) v~^r,
 *         then keeps O = U + M A with M = M^r rho / D, U = U^r / D (D the
 *         denominator), so loop r's probabilities M e^{x - lse} on J_i are
 *         those of the combined softmax.  Rows with M^r_i = 0 combine as in
 *         the mass-rescaled rule.  Both calls of a loop must use the same
 *         setting.  Decode always uses the mass-rescaled combine. */
typedef struct fl_state {
  float* O;
  float* U;
  float* M;
  float* lse;
  float* lsel;
} fl_state;

/* Decode state of one new token per (layer, sequence, head).
 *   O, U    [L][B][H][d] float32
 *   M, lse  [L][B][H] float32
 *   logits  [L][B][H][S] float32: after loop 1 the logits of all S cached
 *           tokens; after loop r >= 2 the logits of the K_r selected tokens,
 *           compacted to the front in the order of sel
 *   sel     [L][B][H][S] int32: after loop r >= 2 the K_r selected token
 *           positions, ascending, at the front */
typedef struct fl_dstate {
  float* O;
  float* U;
  float* M;
  float* lse;
  float* logits;
  int32_t* sel;
} fl_dstate;

/* ABI version of the loaded library (FL_ABI_VERSION). */
int fl_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  The pointer
 * stays valid until the next library call on the same thread. */
const char* fl_last_error(void);

/* Record sizes in bytes (see fl_cache); 0 for unsupported d or bits. */
size_t fl_base_record_bytes(int d);
size_t fl_residual_record_bytes(int d, int bits);

#define FL_FMT_WORKLOAD 0
#define FL_FMT_PAPER 1

/* Bytes of one (layer, sequence, KV head) stream of loop r (r == 1: the base
 * records of all S positions; r >= 2: n[r] residual records), in the cache's
 * format; 0 for an invalid cache or r. */
size_t fl_stream_bytes(const fl_cache* cache, int r);

/* Workspace sizes in bytes for the calls that take one.
 *   which = FL_WS_COLSEL: fl_colsel at loop r with K_prev candidates
 *   which = FL_WS_ATTN:   fl_loop_attn at loop r
 *   which = FL_WS_DECODE: fl_loop_decode at loop r
 * A call may be given a larger workspace; 0 means none is needed.  For
 * FL_WS_COLSEL at r == 2 with K_prev == S the size assumes cand == NULL (the
 * mass pass reads the base records directly). */
#define FL_WS_COLSEL 1
#define FL_WS_ATTN 2
#define FL_WS_DECODE 3
size_t fl_workspace_bytes(int which, const fl_cache* cache, int r, int K_prev, int K_r);

/*
 * fl_kv_resq — quantize and pack loop r's keys and values (p1 §4.3 and §D.3;
 * guide §3: residuals X^(r) - X_hat^(r-1) of the active tokens only).
 *   r == 1: k, v are [L][B][Hkv][S][d] (dtype); writes cache->base.
 *           Per group of 32: s = fp16 rounded up of (max|x| / 127) (fp32
 *           divide); code = clamp(rint(x / s), -127, 127), 0 when s == 0.
 *   r >= 2: k, v are [L][B][Hkv][n_r][d] in rows[r] order (the loop-r values of
 *           the active rows); writes cache->res[r] and cache->slot[r].
 *           delta = x - x_hat^(r-1) (fp32); z = fp16 rounded down of min(delta);
 *           s = fp16 rounded up of ((max(delta) - z) / (2^b - 1));
 *           code = clamp(rint((delta - z) / s), 0, 2^b - 1), 0 when s == 0.
 *           Needs the streams of loops 1..r-1 (and slot[2..r-1]) in place.
 * Codes, scales and zeros are bit-exact functions of the inputs.
 */
fl_status fl_kv_resq(const fl_cache* cache, int r, const void* k, const void* v, fl_dtype dtype,
                     fl_stream stream);

/*
 * fl_kv_append — decode: write one new token's loop-r keys and values into the
 * cache (p1 §4.3; the token being decoded is active in every loop and attends
 * itself, so its records must be in place before fl_loop_decode(r)).
 *   k, v   [L][B][Hkv][d] (dtype): the token's loop-r values
 *   pos    its position, the same in every sequence, 0 <= pos < S
 *   r == 1: writes the base records of pos.
 *   r >= 2: needs cache->cnt[r]; in every sequence b whose count
 *           t = cnt[r][b] is below n[r], pos becomes row t (rows[r][b][t] =
 *           pos, slot[r][b][pos] = t), record t of res[r] receives the
 *           residual against x_hat^(r-1) of pos, and cnt[r][b] becomes t + 1.
 *           A sequence at capacity is left unchanged.  pos must exceed the
 *           sequence's active rows, and loops 1..r-1 of pos must be in place.
 * The records are those fl_kv_resq writes for the same token (same codes).
 * Raise cache->T past pos (host side) before decoding it.
 */
fl_status fl_kv_append(const fl_cache* cache, int r, int pos, const void* k, const void* v, fl_dtype dtype,
                       fl_stream stream);

/*
 * fl_colsel — loop-aware column selection for loop r >= 2 of one layer
 * (p1 §4.2: the previous loop's attention picks the top-K key columns, and a
 * later loop may keep a subset of them; p1 §D.2: the chosen positions are
 * kept together with their share of the full distribution).
 *   q_prev   [B][H][n_{r-1}][d] (dtype): loop r-1 queries in rows[r-1] order
 *   state    the fl_state left by loop r-1 (O, lse, M read; U, M written)
 *   cand     [B][H][K_prev] int32 ascending: S_{r-1}; NULL means every
 *            position (then K_prev must equal S)
 *   K_r      budget, 1 <= K_r <= K_prev
 *   mass_in  [B][H][K_prev] float32 or NULL: column masses to rank instead of
 *            computing them (lets a caller reproduce a selection exactly)
 *   mass_out [B][H][K_prev] float32 or NULL: receives the computed mass
 *            c_j = sum_{i in A_r, i >= j} P^(r-1)_ij, in fp32, accumulated in
 *            a fixed order (deterministic)
 *   sel_out  [B][H][K_r] int32: S_r, the K_r candidates first under
 *            (mass descending, position ascending), written ascending
 *   ws       workspace of fl_workspace_bytes(FL_WS_COLSEL, ...) bytes
 * When K_r == K_prev the selection is the candidate set itself; sel_out gets
 * a copy and U, M are left as they are (they already hold M^r, U^r); with
 * state->lsel set, lsel receives a copy of lse (which then holds L^r).
 * A selection that prunes (K_r < K_prev) takes at most 32768 candidates
 * (K_prev <= 32768; FL_EUNSUPPORTED beyond); keys must not be NaN.
 * Otherwise M^r and U^r of the rows in A_r are written into state.
 * The mass pass runs when it is needed for the selection or mass_out is set.
 */
fl_status fl_colsel(const fl_cache* cache, int r, const void* q_prev, fl_dtype dtype, const fl_state* state,
                    int K_prev, const int32_t* cand, int K_r, const float* mass_in, float* mass_out,
                    int32_t* sel_out, void* ws, size_t ws_bytes, fl_stream stream);

/*
 * fl_loop_attn — loop-r attention of one layer (prefill), over the packed
 * cache streams (p1 App. G: attention works from the packed streams; p1 §4.4:
 * the chosen tokens and keys are gathered into dense tiles).
 *   r == 1: q [B][H][S][d]; dense causal attention of every row:
 *           O = softmax(tau q k~^T) v~, lse; sets M = 1 and U = 0.
 *   r >= 2: q [B][H][n_r][d] in rows[r] order; sel [B][H][K_r] = S_r from
 *           fl_colsel.  For i in A_r with J_i non-empty: O_i = U_i +
 *           M_i * softmax_{J_i}(...) v~ and lse_i; rows with J_i empty get
 *           lse_i = -inf and keep O_i.  Rows outside A_r are not touched.
 * The cache must hold the streams of loops 1..r (fl_kv_resq(r) done).
 */
fl_status fl_loop_attn(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_r,
                       const int32_t* sel, const fl_state* state, void* ws, size_t ws_bytes,
                       fl_stream stream);

/*
 * fl_loop_attn_noalloc — fl_loop_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as fl_loop_attn without the
 * workspace: the tile images go to a device array of FL_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends (its
 * address is looked up on the first call on each device).  The call
 * allocates nothing.  A call that would need more scratch than the array
 * holds returns FL_EUNSUPPORTED (fl_workspace_bytes(FL_WS_ATTN, ...) gives the
 * need; at most 64 MiB: e.g. the sparse loops of a 32K, 16-head layer, or a
 * dense loop 1 of B * H * ceil(S / 64) <= 1820 tiles).  All calls on one GPU
 * share the array: calls that overlap on one GPU (concurrent streams or
 * threads) race and must be serialized by the caller.
 */
#define FL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fl_status fl_loop_attn_noalloc(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_r,
                               const int32_t* sel, const fl_state* state, fl_stream stream);

/*
 * fl_loop_decode — loop r of one decode step for every (layer, sequence,
 * head) of the cache (guide §1 and Cell 1: decode is bound by reading the
 * cache; p1 App. G: packed streams read directly, fused sparse decode
 * selection).  The new token attends all S cached tokens (its own K/V is
 * already cached) and is active at every loop.  Operands are the fp32
 * reconstructions.
 *   q      [L][B][H][d] (dtype): the loop-r query of the new token
 *   r == 1: O, lse, logits of all S tokens; M = 1, U = 0.
 *   r >= 2: S_r = top K_r of the K_prev candidates (state.sel, or every
 *           position when r == 2 and K_prev == S) ranked by their stored
 *           loop r-1 logits (ties: lower position first); when K_r < K_prev,
 *           M = sum_{S_r} P^(r-1)_j and U = O - sum_{S_r} P^(r-1)_j v^(r-1)_j
 *           with P^(r-1)_j = M exp(logit_j - lse); then
 *           O = U + M softmax_{S_r}(tau q.k^r) v^r, lse, and the new logits
 *           and selection are compacted into state.logits / state.sel.
 *   K_prev S when r == 2, else the K of the previous loop; 1 <= K_r <= K_prev.
 *   A loop that prunes (K_r < K_prev) takes at most 32768 candidates
 *   (FL_EUNSUPPORTED beyond).
 */
fl_status fl_loop_decode(const fl_cache* cache, int r, const void* q, fl_dtype dtype, int K_prev, int K_r,
                         const fl_dstate* state, void* ws, size_t ws_bytes, fl_stream stream);

/*
 * fl_select_active — the next loop's active-token set (p1 §4.1 and §D.1:
 * after the dense early loops, later loops recompute only nested active-token
 * sets of budget k(r), and tokens outside them reuse their hidden and KV
 * states; the guide's §3 summary: the tokens updated by the previous loop are
 * ranked by their normalized hidden-state change and the top k kept).
 *   h_prev, h_cur [B][S][D] (dtype): hidden states of every position before
 *            and after the loop just run (rows outside rows_prev are not read)
 *   rows_prev [B][n_prev] int32 ascending: the active set of that loop; NULL
 *            means every position (then n_prev must equal S)
 *   k        budget, 1 <= k <= n_prev; a pruning call (k < n_prev) takes at
 *            most 32768 candidates (FL_EUNSUPPORTED beyond)
 *   rows_out [B][k] int32: the k candidates of largest change (ties: lower
 *            position first), written ascending — the next rows[r] of fl_cache
 *   score_out [B][n_prev] float32: the change of every candidate, in
 *            rows_prev order: ||h_cur - h_prev||_2 / ||h_prev||_2 accumulated in
 *            fp32 (0 for an unmoved token, +inf for a move from a zero state)
 * D must be a positive multiple of 8; h_prev and h_cur 16-byte aligned.
 */
fl_status fl_select_active(int B, int S, int D, const void* h_prev, const void* h_cur, fl_dtype dtype, int n_prev,
                           const int32_t* rows_prev, int k, int32_t* rows_out, float* score_out, fl_stream stream);

/*
 * Kernel timing, a measurement aid outside the method: while a thread has it
 * enabled (on != 0), every kernel that thread's library calls launch is
 * bracketed by two HIP events recorded on the kernel's stream.
 * fl_timing_collect waits for the recorded launches, writes up to max
 * (kernel name, milliseconds) pairs in launch order into names / ms, clears
 * the thread's list (records beyond max are dropped) and returns how many it
 * wrote.  Names are the launch expression's text, truncated to
 * FL_TIMING_NAME - 1 characters.  Off by default; when on it costs two event
 * records per launch, and the events are created on first use and reused
 * (so it is not for callers that must not create runtime objects).
 */
#define FL_TIMING_NAME 48
void fl_timing_enable(int on);
int fl_timing_collect(char (*names)[FL_TIMING_NAME], float* ms, int max);

#ifdef __cplusplus
}
#endif

#endif /* FLASHLOOP_H */
