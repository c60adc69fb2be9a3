/*
 * f4kv.h -- C ABI of the F4 paged-attention library for MI355X (gfx950).
 *
 * Paged grouped-query attention over a 4-bit symmetric block-scaled KV cache
 * ("F4": values (nibble - 8) * scale, 32 values per 16-byte row, one fp16
 * scale per 32 values), with statically YaRN-rotated keys, split across page
 * chunks and folded by log-sum-exp.
 *
 * Sources for what each call computes:
 *   [MRS]  mistral.rs PR #2375 "YaRN rope scaling, 4-bit F4 packed KV cache,
 *          and hybrid paged attention", sections "Changes by area" items 1-2
 *          and "Known limitations".
 *   [IGN]  ignis docs, configuration / context-and-speculation: the
 *          --model-rope-scaling, --model-adapt-context-step and
 *          --model-prefill-chunk rows.
 *   [FT]   FreeToken issue #568, "Proposed solution" item 2 (device windows
 *          folded by log2-sum-exp) and "What problem does this solve" item 1.
 *   [AE]   aeliusai "hybrid-attention-economics", "What a token of context
 *          costs" (4 KV heads of key length 256).
 *
 * Conventions (all entry points):
 *   - Every call returns an int status (F4KV_OK or an error below).  On error
 *     nothing has been enqueued and f4kv_last_error() names the reason
 *     (thread-local, valid until the next call from the same thread).
 *   - All array arguments are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory.  Parameter structs are host
 *     memory, read only during the call.
 *   - Work is enqueued on `stream` (0 = the null stream); no call waits for the
 *     device.  Faults surface at the caller's next synchronisation.
 *   - Shapes and pointers are validated on the host before any launch.  Values
 *     that live on the device (context lengths, page ids, slot ids) cannot be
 *     checked there: out-of-range entries are skipped by the kernels (never
 *     read or written out of bounds), and the results for them are undefined.
 *   - Calls on one stream are ordered; calls on different streams that touch
 *     the same buffers race like any other kernels.
 *
 * Cache layout (one layer; P pages of 64 tokens, H kv heads, D = head_dim):
 *   k_nib   uint8   [P][H][D/32][64][16]  bytes (c, t): block c of token t;
 *                                         byte m holds element 2m (low nibble)
 *                                         and 2m+1 (high nibble) of the block
 *   k_scale fp16    [P][H][64][D/32]      scale of block c of token t
 *   v_nib   uint8   [P][H][8][D/4][16]    unit (c, j): tokens 8c..8c+7 x dims
 *                                         4j..4j+3; byte 4k+2r+h holds dims
 *                                         4j+2h (low) and 4j+2h+1 (high) of
 *                                         token 8c+2k+r
 *   v_scale fp16    [P][H][64][D/32]      one scale per 32 values, like K; or,
 *                   [P][H][64]            with v_scale_per_token = 1, one
 *                                         scale per token and V head (the V
 *                                         format of [MRS item 2]), taken from
 *                                         the absmax of the token's whole V
 *                                         row
 *   Logical value of element e of block c of token t: (nibble - 8) * scale.
 *   Token i of a sequence lives in page page_table[i / 64], slot i % 64.
 */
#ifndef F4KV_H
#define F4KV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define F4KV_ABI_VERSION 5

enum {
  F4KV_OK = 0,
  F4KV_ERR_INVALID = 1,      /* a null/misaligned pointer or an argument out of range */
  F4KV_ERR_UNSUPPORTED = 2,  /* valid, but a shape these kernels do not implement     */
  F4KV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_size */
  F4KV_ERR_LAUNCH = 4        /* the HIP runtime refused a launch                       */
};

enum { F4KV_F32 = 0, F4KV_BF16 = 1 };

/* ABI version of the loaded library (F4KV_ABI_VERSION it was built with). */
int f4kv_abi_version(void);

/* Reason for the last non-zero status returned on this thread ("" if none). */
const char* f4kv_last_error(void);

/*
 * YaRN parameters [MRS item 1; IGN --model-rope-scaling].
 *   theta       rope base (> 1)
 *   rotary_dim  channels rotated, even, > 0 (the rest pass through)
 *   factor      1 = plain RoPE; otherwise YaRN with factor in (1, 64]
 *   orig_ctx    trained context the correction dims refer to (> 0)
 *   beta_fast / beta_slow   correction-dim betas (beta_fast > beta_slow > 0)
 *   mscale      table scale; <= 0 derives it: 1 for factor 1, otherwise
 *               1 + 0.1 ln(factor) (net 1.0199427025 at factor 1.220703125)
 */
typedef struct {
  double theta;
  int32_t rotary_dim;
  double factor;
  int32_t orig_ctx;
  double beta_fast;
  double beta_slow;
  double mscale;
} f4kv_yarn_params;

/*
 * One layer's paged F4 cache (layout above).  All four pointers are device
 * memory aligned to 16 bytes.  page_size must be 64 [IGN
 * --model-adapt-context-step: pages are multiples of 64 tokens]; head_dim a
 * multiple of 32.  v_scale_per_token selects the V scale granularity: 0 = one
 * fp16 scale per 32 values (as K), 1 = one per token and V head; every entry
 * point reads and writes the cache in the layout it names.
 */
typedef struct {
  uint8_t* k_nib;
  uint16_t* k_scale;
  uint8_t* v_nib;
  uint16_t* v_scale;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t v_scale_per_token;
} f4kv_cache;

/* Bytes of each of the four cache arrays for the given geometry and V scale
 * granularity (host helper, no device work).  Any output pointer may be NULL.
 * Returns the total, or 0 for an invalid geometry. */
size_t f4kv_cache_bytes(int32_t num_pages, int32_t num_kv_heads, int32_t head_dim, int32_t v_scale_per_token,
                        size_t* k_nib, size_t* k_scale, size_t* v_nib, size_t* v_scale);

/*
 * yarn_rope_table [MRS item 1; IGN --model-rope-scaling; FT problem item 1]
 * Rows of the static YaRN table for n positions:
 *   cos_out[i][p] = m * cos(pos[i] * theta'_p), sin_out likewise, p < rotary_dim/2,
 * where theta'_p blends theta^(-2p/rotary_dim) and that divided by the factor
 * with a linear ramp between the beta_fast / beta_slow correction dims
 * (floored / ceiled, clamped to [0, rotary_dim - 1]).  Angles and the
 * trigonometry are evaluated in fp64; outputs are rounded to fp32.
 *   positions  int32 [n], each in [0, 2^24)   (values outside give undefined rows)
 *   cos_out, sin_out  fp32 [n][rotary_dim/2]
 */
int yarn_rope_table(const f4kv_yarn_params* params, const int32_t* positions, int32_t n,
                    float* cos_out, float* sin_out, hipStream_t stream);

/*
 * yarn_rope_apply [MRS item 1: partial rotary; IMROPE-to-NEOX equivalence]
 * NEOX rotation of the first rotary_dim channels of every head of every row:
 *   y[t][h][i]      = x[t][h][i] * c[t][i] - x[t][h][i + r/2] * s[t][i]
 *   y[t][h][i + r/2] = x[t][h][i + r/2] * c[t][i] + x[t][h][i] * s[t][i]
 * for i < r/2 (r = rotary_dim); channels >= r are copied.  Arithmetic in fp64,
 * one rounding to the output type (bf16: nearest-even via fp32).
 *   cos_rows, sin_rows fp32 [T][r/2];  x, y [T][H][D] of dtype F4KV_F32 or
 *   F4KV_BF16 (y may equal x: in place).  x, y aligned to 4 bytes.
 */
int yarn_rope_apply(const float* cos_rows, const float* sin_rows,
                    const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                    int32_t T, int32_t H, int32_t D, int32_t rotary_dim, hipStream_t stream);

/*
 * kv_cache_write_f4 [MRS item 2: reshape_and_cache writes symmetric 4-bit
 * (nibble - 8) * scale; "Known limitations": per-value bound max_abs/16]
 * Quantises k and v (fp32 [T][H][D], 16-byte aligned) into the cache slots
 * slot_mapping[t] = page * 64 + offset (-1 skips the token; live entries must
 * be distinct, else the result is undefined).  Per token, kv head and
 * 32-value block (for V with v_scale_per_token: per token and kv head, the
 * absmax taken over the whole V row):
 *   s = fp16_nearest_even(min(absmax * 0.125, 65504)),
 *   code = clamp(nearest_even(x / s), -8, 7) with the exact quotient
 *   (s == 0: every code 0), nibble = code + 8.
 * One thread owns whole blocks: no byte is written by two threads.
 */
int kv_cache_write_f4(const f4kv_cache* cache, const float* k, const float* v,
                      const int32_t* slot_mapping, int32_t T, hipStream_t stream);

/*
 * paged_attn_decode_f4 [MRS item 2: paged attention dequantises F4 cells
 * inline; FT item 2: windows folded by log-sum-exp; AE: grouped KV heads]
 * One query row per sequence.  For sequence b, query head h, KV head
 * g = h / (Hq / H) and window w:
 *   s_t = sm_scale * q[b][h] . k_t over the window's tokens t of [0, ctx_b),
 *   out_m = max s_t,  out_l = sum exp(s_t - out_m),
 *   out   = sum exp(s_t - out_m) v_t / out_l
 * (natural-log units).  Window w covers tokens [w*window_tokens,
 * (w+1)*window_tokens); num_windows == 1 with window_tokens == 0 means the
 * whole context.  An empty window gives (-inf, 0, 0), the identity of
 * lse_merge.  Internally each window is split further across the GPU and
 * folded with the same merge.
 *   q             bf16 [B][Hq][D] (already rotated), 16-byte aligned
 *   page_table    int32 [B][max_pages]
 *   context_lens  int32 [B], each in [0, max_context_len]
 *   max_context_len  host bound, <= max_pages * 64
 *   window_tokens    multiple of 64 (0 only with num_windows == 1)
 *   out    fp32 [W][B][Hq][D] (16-byte aligned); out_m, out_l fp32 [W][B][Hq] or NULL
 *   workspace   device scratch of at least paged_attn_decode_f4_workspace_size()
 *               bytes (16-byte aligned); may be NULL when that size is 0
 * Supported: D == 256, Hq / H in {1, 2, 4, 8}.
 */
size_t paged_attn_decode_f4_workspace_size(int32_t B, int32_t Hq, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_context_len,
                                           int32_t num_windows, int32_t window_tokens);
int paged_attn_decode_f4(const f4kv_cache* cache, const uint16_t* q,
                         const int32_t* page_table, const int32_t* context_lens,
                         int32_t B, int32_t Hq, int32_t max_pages, int32_t max_context_len,
                         int32_t num_windows, int32_t window_tokens, float sm_scale,
                         float* out, float* out_m, float* out_l,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * paged_attn_decode_f4_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same computation, arguments and outputs as
 * paged_attn_decode_f4, without the workspace: its partial states, work list
 * and query operands live in a fixed 8 MiB device array of the library (one
 * per GPU, held until the process ends; its address is looked up on the first
 * call on each device).  The call allocates and frees nothing.  Calls whose
 * workspace (paged_attn_decode_f4_workspace_size) exceeds 8 MiB are refused
 * with F4KV_ERR_UNSUPPORTED before any launch.  Nothing in the array carries
 * from one call to the next (every call writes what it reads), but all calls
 * on one GPU share it: calls that can overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.
 */
int paged_attn_decode_f4_noalloc(const f4kv_cache* cache, const uint16_t* q,
                                 const int32_t* page_table, const int32_t* context_lens,
                                 int32_t B, int32_t Hq, int32_t max_pages, int32_t max_context_len,
                                 int32_t num_windows, int32_t window_tokens, float sm_scale,
                                 float* out, float* out_m, float* out_l, hipStream_t stream);

/*
 * paged_attn_decode_step_f4 [MRS items 1 and 2: the keys are rotated before
 * they are quantised into the cache, the queries at attention time; FT item 2]
 * One decode step of a layer in one call: the new token of each sequence is
 * rotated and written, then each sequence's query attends over its cache, the
 * new token included.  Equivalent, bit for bit, to
 *   yarn_rope_apply(cos_rows, sin_rows, q  -> bf16 q_rot,  T = B, H = Hq)
 *   yarn_rope_apply(cos_rows, sin_rows, k_new -> fp32 k_rot, T = B, H = num_kv_heads)
 *   kv_cache_write_f4(cache, k_rot, v_new, slots, T = B)
 *   paged_attn_decode_f4(cache, q_rot, ...)
 * with the rotation, the write and the query preparation in one launch (the
 * decode's own), so the step costs the decode's launches only.
 *   cos_rows, sin_rows  fp32 [B][rotary_dim / 2]: row b is the table row of
 *                       sequence b's new token (yarn_rope_table at its position)
 *   rotary_dim          even, in (0, head_dim]; channels from it on pass through
 *   q                   bf16 [B][Hq][D], not yet rotated, 16-byte aligned
 *   k_new, v_new        fp32 [B][num_kv_heads][D], k not yet rotated, 16-byte aligned
 *   slots               int32 [B]: cache slot (page * 64 + offset) of each new
 *                       token; -1 (or a slot outside the pool) writes nothing.
 *                       context_lens must already count the new token.
 *   other arguments, the workspace (paged_attn_decode_f4_workspace_size) and
 *   the outputs as paged_attn_decode_f4.
 * The inputs q, k_new and v_new are not modified.
 */
int paged_attn_decode_step_f4(const f4kv_cache* cache, const float* cos_rows, const float* sin_rows,
                              int32_t rotary_dim, const uint16_t* q, const float* k_new,
                              const float* v_new, const int32_t* slots,
                              const int32_t* page_table, const int32_t* context_lens,
                              int32_t B, int32_t Hq, int32_t max_pages, int32_t max_context_len,
                              int32_t num_windows, int32_t window_tokens, float sm_scale,
                              float* out, float* out_m, float* out_l,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * paged_attn_decode_rows_f4 [IGN --spec-draft-tokens / --spec-draft-rows: a
 * verify round takes up to 8 query rows of a lane; MRS item 2; FT item 2]
 * Decode of R query rows per sequence (1 <= R <= 8), as one round of
 * speculative verification: row r of sequence b is the query at position
 * context_lens[b] - R + r and attends to tokens [0, context_lens[b] - R + r]
 * of each window, with the states and windows of paged_attn_decode_f4 (a row
 * before position 0 gives (-inf, 0, 0)).  R == 1 is paged_attn_decode_f4.
 *   q      bf16 [B][R][Hq][D] (already rotated), 16-byte aligned
 *   out    fp32 [W][B][R][Hq][D];  out_m, out_l fp32 [W][B][R][Hq] or NULL
 *   other arguments as paged_attn_decode_f4; the workspace size comes from
 *   paged_attn_decode_rows_f4_workspace_size().
 * The rows of a KV head's query heads are processed together, up to 8 per
 * pass over the pages (Hq / H * R rows; more take several passes).  With
 * Hq / H == 4, R >= 5 and one window over the whole context (num_windows == 1,
 * window_tokens == 0), a verification round is a short causal prefill: the
 * rows then run on the prefill kernel (fp16 matrix cores with exact splits,
 * one pass over the pages for all R rows), within the same tolerance.
 */
size_t paged_attn_decode_rows_f4_workspace_size(int32_t B, int32_t R, int32_t Hq, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_context_len,
                                                int32_t num_windows, int32_t window_tokens);
int paged_attn_decode_rows_f4(const f4kv_cache* cache, const uint16_t* q,
                              const int32_t* page_table, const int32_t* context_lens,
                              int32_t B, int32_t R, int32_t Hq, int32_t max_pages, int32_t max_context_len,
                              int32_t num_windows, int32_t window_tokens, float sm_scale,
                              float* out, float* out_m, float* out_l,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * lse_merge [FT item 2: partial windows folded by log-sum-exp]
 * Folds C partial states per row:  M = max_c m_c,  w_c = l_c exp(m_c - M),
 *   L = sum w_c,  out = sum w_c o_c / L;  rows with every l_c == 0 give
 *   (-inf, 0, 0).
 *   m, l  fp32 [C][R];  o fp32 [C][R][D];  out fp32 [R][D];
 *   out_m, out_l fp32 [R] or NULL.   D a multiple of 4, pointers 16-byte aligned.
 */
int lse_merge(const float* m, const float* l, const float* o, int32_t C, int32_t R, int32_t D,
              float* out, float* out_m, float* out_l, hipStream_t stream);

/*
 * paged_attn_prefill_f4 [IGN --model-prefill-chunk: chunk widths; FT item 2:
 * a prefill attends within a device window; MRS item 2: F4 cells dequantised
 * inline]
 * Writes the chunk's own keys and values (when k_new/v_new are non-NULL, as
 * kv_cache_write_f4 at positions pos0 .. pos0+T-1 through page_table), then
 * computes causal attention of T query rows at positions pos0 + i over cache
 * tokens [0, pos0 + i] of one sequence:
 *   out[i][h] = softmax_t(sm_scale * q[i][h] . k_t) . v_t ;  out_m, out_l as in
 *   decode (natural-log units).
 *   q            bf16 [T][Hq][D] (already rotated), 16-byte aligned
 *   k_new, v_new fp32 [T][H][D] or both NULL (cache already holds them)
 *   page_table   int32 [max_pages] of this sequence; pos0 + T <= max_pages * 64
 *   out          fp32 [T][Hq][D];  out_m, out_l fp32 [T][Hq] or NULL
 *   workspace    at least paged_attn_prefill_f4_workspace_size() bytes
 * Supported: D == 256, Hq / H == 4.  The products run in fp16 on MFMA with
 * fp32 accumulation, so cache values must lie within fp16 range (|x| < 65504,
 * which holds whenever the written keys/values did).  The query rows enter
 * fp16 in groups of 32 (8 consecutive positions x the 4 query heads of a KV
 * head), each group scaled by one power of two that brings its largest |q|
 * into [2^10, 2^11): exact for groups whose largest |q| lies in
 * [2^-54, 2^75); elements below 2^-27 of their group's largest |q| round to
 * fp16's subnormal step.  Any finite sm_scale, including 0 and negative
 * values.
 */
size_t paged_attn_prefill_f4_workspace_size(int32_t T, int32_t Hq, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t pos0);
int paged_attn_prefill_f4(const f4kv_cache* cache, const uint16_t* q,
                          const float* k_new, const float* v_new,
                          const int32_t* page_table, int32_t max_pages,
                          int32_t T, int32_t Hq, int32_t pos0, float sm_scale,
                          float* out, float* out_m, float* out_l,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * paged_attn_prefill_f4_fp8 [IGN --model-prefill-attention: the prompt
 * attention over a 4-bit-cache chunk in 8 bits, Q.K^T in INT8 and P.V in E4M3]
 * The computation of paged_attn_prefill_f4 (same arguments, layouts, state
 * outputs, workspace size and errors) with 8-bit products, for a query row r
 * at position p over cache tokens [0, p]:
 *   - q to INT8 with one power-of-two scale per row, sigma = 2^(e - 7) where
 *     max |q| < 2^e, round half to even, clamped to [-127, 127];
 *   - each cached key to INT8 with one power-of-two scale per token,
 *     tau = 2^(E - 4), E = (exponent field of the token's largest fp16 block
 *     scale) - 14, code * scale / tau rounded to nearest, ties to even
 *     (within [-128, 112]);
 *   - x = (Qi . Kt) sigma tau qk in log2 units, qk = fp32(sm_scale log2(e));
 *   - per 32-token group (half a page) of a row, G = ceil(max x) and the
 *     weights P8 = e4m3(2^(x - G)) (OCP E4M3, nearest even) carrying 2^G;
 *   - per 32-token group and 32-channel block, values V8 = e4m3(code * scale
 *     / 2^F) carrying 2^F, F = (exponent field of the largest V scale) - 19;
 *   - out = sum P8 2^G V8 2^F / sum 2^x (unquantised denominator).
 * The result is within a few percent of the exact attention (E4M3 keeps 3
 * mantissa bits: ~4% of the output RMS on N(0,1) data); it is the faster
 * choice where that is acceptable.
 */
int paged_attn_prefill_f4_fp8(const f4kv_cache* cache, const uint16_t* q,
                              const float* k_new, const float* v_new,
                              const int32_t* page_table, int32_t max_pages,
                              int32_t T, int32_t Hq, int32_t pos0, float sm_scale,
                              float* out, float* out_m, float* out_l,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * gather_kv_cache_f4 [MRS item 2: the cache's gather path gains an F4 variant]
 * Dequantises the cached keys and values of B sequences into contiguous rows:
 * token i of sequence b, for i < cu_seq_lens[b + 1] - cu_seq_lens[b], becomes
 * row cu_seq_lens[b] + i of k_out and v_out, every value (nibble - 8) * scale
 * (exact in fp32; bf16 outputs rounded to nearest-even).  A token whose page
 * id is out of range gives a zero row; rows at or past total_tokens are not
 * written.
 *   page_table   int32 [B][max_pages]
 *   cu_seq_lens  int32 [B + 1] (device): row offsets, cu_seq_lens[0] = 0,
 *                non-decreasing, each length at most max_pages * 64, and
 *                cu_seq_lens[B] <= total_tokens
 *   k_out, v_out [total_tokens][H][D] of out_dtype (F4KV_BF16 or F4KV_F32),
 *                16-byte aligned
 * Supported: D == 256; B <= 65535; max_pages * H < 2^31.
 */
int gather_kv_cache_f4(const f4kv_cache* cache, const int32_t* page_table, const int32_t* cu_seq_lens,
                       int32_t B, int32_t max_pages, int32_t total_tokens, void* k_out, void* v_out,
                       int32_t out_dtype, hipStream_t stream);

/*
 * Device-side checks (a debugging aid).  Context lengths, page ids, slot ids
 * and row offsets live in device memory, where the host cannot validate them;
 * the kernels skip out-of-range entries rather than read or write out of
 * bounds.  f4kv_device_checks(1) makes every following call (on any thread)
 * first launch a small check kernel on its stream that ORs the flags below
 * into a word of the current device; f4kv_device_check_word(&w) waits for the
 * device, returns that word and clears it.  f4kv_device_checks(0) (the
 * default) launches nothing.  Checked: every context length in
 * [0, max_context_len] (decode); the page ids of every live page (tokens
 * below the context length, or pos0 + T for prefill, or the row count for
 * the gather) in [0, num_pages); every slot id -1 or in [0, num_pages * 64)
 * (the writer; distinctness is not checked); cu_seq_lens starting at 0,
 * non-decreasing, lengths at most max_pages * 64, cu_seq_lens[B] <=
 * total_tokens (the gather).
 */
enum {
  F4KV_CHECK_CONTEXT = 1,  /* a context length outside [0, max_context_len] */
  F4KV_CHECK_PAGE = 2,     /* a live page id outside [0, num_pages)         */
  F4KV_CHECK_SLOT = 4,     /* a slot id neither -1 nor a slot of the pool    */
  F4KV_CHECK_ROWS = 8      /* cu_seq_lens not a valid list of row offsets    */
};
int f4kv_device_checks(int32_t on);
int f4kv_device_check_word(uint32_t* word);

/*
 * Kernel timing (a measurement aid of this library, not an operation of the
 * method).  f4kv_timing_start(kernel, max_launches) makes every following call
 * that launches `kernel` record a pair of HIP events on its stream right
 * around that one launch, for up to max_launches launches (the events are
 * created here, on the current device; no device memory is allocated).
 * f4kv_timing_stop(kernel, &total_ms, &launches) waits for the recorded
 * events, returns the summed kernel time and the number of timed launches, and
 * ends the timing.  Launches beyond max_launches are not timed.
 *   kernel  F4KV_KERNEL_DECODE: the split-K attention kernel of
 *           paged_attn_decode_f4 and paged_attn_decode_rows_f4 (not its query
 *           preparation or fold);
 *           F4KV_KERNEL_PREFILL: the attention kernel of paged_attn_prefill_f4,
 *           which also runs the verification rounds of paged_attn_decode_rows_f4
 *           that go to it (R >= 5, see there).
 *           F4KV_KERNEL_PREFILL_FP8: that of paged_attn_prefill_f4_fp8.
 * Timing one kernel from two host threads at once is not supported.
 */
enum { F4KV_KERNEL_DECODE = 0, F4KV_KERNEL_PREFILL = 1, F4KV_KERNEL_PREFILL_FP8 = 2 };
int f4kv_timing_start(int32_t kernel, int32_t max_launches);
int f4kv_timing_stop(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* F4KV_H */
