/*
 * attnq8 -- scaled-dot-product GQA attention over an int8 block-32 KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Two shapes of the same operation:
 *
 *  - the speculative-decode verifier: a run of sequential query rows after a
 *    context; each workgroup owns every query vector of a row group that reads
 *    one KV head and shares each K/V scan across them, writing split-context
 *    partials that a reducer merges ("perf(gfx1100): share Q8 KV scans across
 *    verifier rows", Summary);
 *  - chunked causal prompt attention over a long int8 context with online
 *    softmax and the V scale folded into the probabilities ("hip: gfx12 (RDNA4)
 *    WMMA kernel for the int8-KV QSA prompt attention", What and How).
 *
 * Operation (both shapes).  For query row r at position pos_r, Q head h and
 * KV head g = h / (n_q_heads / n_kv_heads):
 *     Khat[t][j] = f32(k_scales[g][t][j/32]) * k_codes[g][t][j]   (same for V)
 *     s_t = sm_scale * sum_j q[r][h][j] * Khat[t][j],  t = 0 .. pos_r
 *     out[r][h][:] = sum_t exp(s_t - max s) Vhat[t][:] / sum_t exp(s_t - max s)
 *
 * Memory layouts (row-major, all buffers are DEVICE memory owned by the caller):
 *     q          [n_rows][n_q_heads][head_dim]      fp32 or fp16 (q_dtype)
 *     k_codes    [n_kv_heads][kv_stride][head_dim]  int8
 *     k_scales   [n_kv_heads][kv_stride][head_dim/32] fp16 bit patterns
 *     v_codes, v_scales: as K
 *     out        [n_rows][n_q_heads][head_dim]      fp32
 * A block is 32 consecutive head_dim elements of one (KV head, token) with one
 * fp16 scale.  head_dim is 64, 128 or 256.
 *
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream),
 * never synchronise, never allocate device memory and keep no device state
 * (except attn_verify_q8_static's scratch array, below), so they may be
 * captured into a HIP graph.  Every argument check runs on the host
 * before anything is launched; on failure nothing is launched and a negative
 * status is returned.  A device fault surfaces at the caller's next
 * synchronisation, as for any HIP launch.  There is one code path per call: no
 * fallback kernels.
 */
#ifndef ATTNQ8_H
#define ATTNQ8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTNQ8_OK = 0,
  ATTNQ8_EINVAL = -1,      /* a size, count or pointer argument is out of range or NULL */
  ATTNQ8_EUNSUPPORTED = -2,/* the current device is not gfx950, or the shape is not served */
  ATTNQ8_EALIGN = -3,      /* a pointer is not aligned as documented */
  ATTNQ8_EWORKSPACE = -4,  /* workspace smaller than attn_verify_q8_workspace_bytes() */
  ATTNQ8_EHIP = -5         /* the HIP runtime reported an error while launching */
};

enum { ATTNQ8_F32 = 0, ATTNQ8_F16 = 1 };

/* ---------------------------------------------------------------------------
 * Verify attention ("perf(gfx1100): share Q8 KV scans across verifier rows",
 * Summary and Kernel evidence).
 *
 * Row i of the n_rows query rows sits at position ctx_len + i and sees keys
 * 0 .. ctx_len + i (the cache already holds the rows' own keys).  Rows are
 * taken rows_per_group at a time; one workgroup holds every (row, Q head) of a
 * group that reads one KV head -- rows_per_group * n_q_heads / n_kv_heads
 * query vectors, at most 128 -- and splits the group's visible context into
 * n_splits ranges of whole 32-key tiles.  rows_per_group = 0 picks the largest
 * group of at most 64 query vectors (at least one row); n_splits = 0 picks
 * attn_verify_q8_splits().  The grouping and split count change only the
 * rounding of the result.
 *
 * Output: split-context partials in `workspace`, merged by
 * attn_reduce_partials().  Workspace layout (fp32, 16-byte aligned):
 *     o  [n_splits][n_rows][n_q_heads][head_dim]
 *     ml [n_splits][n_rows][n_q_heads][2]          (m, l), after o
 * With x_t = s_t * log2(e) (base-2 units), a split's partial over the keys it
 * covers that the row sees is   l = sum 2^(x_t - m),  o = sum 2^(x_t - m) Vhat_t
 * for a reference m near the largest x_t (not necessarily equal to it); a
 * split with no visible key holds m = -inf, l = 0, o = 0.
 *
 * Requirements: n_q_heads % n_kv_heads == 0; n_kv_heads <= 65535 (also for
 * the prompt and the fp16-cache calls); 1 <= n_rows <= 32;
 * ctx_len >= 0; ctx_len + n_rows <= kv_stride; q, codes and workspace 16-byte
 * aligned, scales 4-byte aligned; workspace_bytes >=
 * attn_verify_q8_workspace_bytes(n_rows, n_q_heads, head_dim, n_splits after
 * auto selection).  sm_scale = 0 means 1/sqrt(head_dim).
 * ------------------------------------------------------------------------- */
int attn_verify_q8_splits(int n_q_heads, int n_kv_heads, int head_dim, int ctx_len,
                          int n_rows, int rows_per_group);
size_t attn_verify_q8_workspace_bytes(int n_rows, int n_q_heads, int head_dim,
                                      int n_splits);
int attn_verify_q8(const void* q, int q_dtype,
                   const int8_t* k_codes, const uint16_t* k_scales,
                   const int8_t* v_codes, const uint16_t* v_scales,
                   int n_q_heads, int n_kv_heads, int head_dim,
                   int kv_stride, int ctx_len, int n_rows,
                   int rows_per_group, int n_splits,
                   void* workspace, size_t workspace_bytes,
                   float sm_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Reducer: merge the partials of attn_verify_q8 ("partials layout and reducer",
 * "perf(gfx1100): share Q8 KV scans across verifier rows", Summary):
 *     M = max of m over splits with l > 0
 *     out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
 * in a fixed split order (run-to-run bitwise reproducible).  `workspace` holds
 * the layout above for the given n_splits; out is fp32
 * [n_rows][n_q_heads][head_dim], 16-byte aligned; n_rows * n_q_heads at most
 * INT_MAX, 1 <= n_splits <= 65535.  Every (row, head) must have at least one
 * split with l > 0.
 * ------------------------------------------------------------------------- */
int attn_reduce_partials(const void* workspace, size_t workspace_bytes,
                         int n_rows, int n_q_heads, int head_dim, int n_splits,
                         float* out, void* stream);

/* ---------------------------------------------------------------------------
 * attn_verify_q8_static: for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc -- and so cannot provide attn_verify_q8's workspace.  It runs
 * attn_verify_q8 and then attn_reduce_partials on `stream` with the split
 * partials in a scratch array the library keeps in device memory
 * (ATTNQ8_STATIC_SCRATCH_BYTES on every GPU it runs on, held until the process
 * ends), and writes the normalised fp32 output to `out`
 * [n_rows][n_q_heads][head_dim] (16-byte aligned).  It calls no allocator.
 *
 * Arguments and requirements as attn_verify_q8; n_splits = 0 takes
 * attn_verify_q8_splits() capped to what the scratch holds
 * (ATTNQ8_STATIC_SCRATCH_BYTES / attn_verify_q8_workspace_bytes(n_rows,
 * n_q_heads, head_dim, 1) splits); an explicit n_splits beyond that, or a
 * shape of which not even one split fits, returns ATTNQ8_EWORKSPACE with
 * nothing launched.  With the same split count the output is bitwise the
 * output of attn_verify_q8 followed by attn_reduce_partials.
 *
 * Every call on one GPU uses that GPU's single scratch array: calls that
 * overlap on one GPU (on different streams or host threads without ordering)
 * race and may return wrong results.  Calls ordered on one stream are safe.
 * ------------------------------------------------------------------------- */
#define ATTNQ8_STATIC_SCRATCH_BYTES (32u << 20)
int attn_verify_q8_static(const void* q, int q_dtype,
                          const int8_t* k_codes, const uint16_t* k_scales,
                          const int8_t* v_codes, const uint16_t* v_scales,
                          int n_q_heads, int n_kv_heads, int head_dim,
                          int kv_stride, int ctx_len, int n_rows,
                          int rows_per_group, int n_splits,
                          float sm_scale, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Prompt attention ("hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA prompt
 * attention", What, How and Measurements).
 *
 * Query i of the n_queries rows sits at position q_pos0 + i and sees keys
 * 0 .. q_pos0 + i (causal).  Requirements: q_pos0 >= 0,
 * q_pos0 + n_queries <= kv_len <= kv_stride, n_queries >= 1; q and out
 * 16-byte aligned; codes 16-byte, scales 4-byte aligned.  Writes the
 * normalised result to `out`.  sm_scale = 0 means 1/sqrt(head_dim).
 * ------------------------------------------------------------------------- */
int attn_prompt_q8(const void* q, int q_dtype,
                   const int8_t* k_codes, const uint16_t* k_scales,
                   const int8_t* v_codes, const uint16_t* v_scales,
                   int n_q_heads, int n_kv_heads, int head_dim,
                   int kv_stride, int kv_len, int q_pos0, int n_queries,
                   float sm_scale, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * The same two attention shapes over an fp16 K/V cache ("hip: gfx12 (RDNA4)
 * WMMA kernel for the int8-KV QSA prompt attention", What: fp16 KV pools stay
 * with the earlier kernel; the operation is the one above with Khat = K and
 * Vhat = V, no scales).
 *
 * k, v: fp16 bit patterns [n_kv_heads][kv_stride][head_dim], 16-byte aligned.
 * Every other argument, the workspace layout, the reducer and the errors are
 * those of attn_verify_q8 / attn_prompt_q8, with one limit more: at head_dim
 * 256 a row group holds at most 96 query vectors (rows_per_group * n_q_heads /
 * n_kv_heads <= 96; the automatic grouping stays within it), else
 * ATTNQ8_EUNSUPPORTED.  Sizes and splits come from attn_verify_q8_splits and
 * attn_verify_q8_workspace_bytes.
 * ------------------------------------------------------------------------- */
int attn_verify_f16kv(const void* q, int q_dtype,
                      const uint16_t* k, const uint16_t* v,
                      int n_q_heads, int n_kv_heads, int head_dim,
                      int kv_stride, int ctx_len, int n_rows,
                      int rows_per_group, int n_splits,
                      void* workspace, size_t workspace_bytes,
                      float sm_scale, void* stream);
int attn_prompt_f16kv(const void* q, int q_dtype,
                      const uint16_t* k, const uint16_t* v,
                      int n_q_heads, int n_kv_heads, int head_dim,
                      int kv_stride, int kv_len, int q_pos0, int n_queries,
                      float sm_scale, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * KV append: quantise n_tokens new K (and V) rows into the cache at positions
 * pos0 .. pos0 + n_tokens - 1 of every KV head.  The format is the pages' Q8
 * KV block ("perf(gfx1100): share Q8 KV scans across verifier rows", Summary;
 * the Q8_0 block of "[Engine] perf(hip): optimize MTP draft, shared expert,
 * and verify/sampler head kernels on RDNA4", Problem and result item 2 and
 * Verification & Parity Evidence).  For each block of 32 consecutive head_dim
 * elements of one (token, KV head) row:
 *     scale = fp16(amax / 127)   amax = max |x|; fp32 divide, round to nearest
 *                                even into fp16 (+inf above the fp16 range)
 *     code  = clamp(round_half_away_from_zero(x / scale), -127, 127),
 *             x / scale an fp32 divide by the stored scale; scale 0 -> codes 0
 * The results are bit-exact (they equal the exactly rounded quotients).
 *
 * Layouts: k, v [n_tokens][n_kv_heads][head_dim] fp32 or fp16 (x_dtype), 16-byte
 * aligned, finite values; the cache planes as for the attention calls (codes
 * [n_kv_heads][kv_stride][head_dim] int8, 16-byte aligned; scales
 * [n_kv_heads][kv_stride][head_dim/32] fp16 bit patterns, 4-byte aligned).
 * Only the n_tokens positions of each head are written.  head_dim is any
 * multiple of 32 up to 4096.  Pass v, v_codes and v_scales all NULL to
 * quantise K alone.  n_tokens = 0 launches nothing (the row pointers may then
 * be NULL; the cache pointers are still checked).  Requires pos0 >= 0 and
 * pos0 + n_tokens <= kv_stride; the input rows must not overlap the cache.
 * ------------------------------------------------------------------------- */
int attn_kv_append_q8(const void* k, const void* v, int x_dtype,
                      int n_tokens, int n_kv_heads, int head_dim,
                      int8_t* k_codes, uint16_t* k_scales,
                      int8_t* v_codes, uint16_t* v_scales,
                      int kv_stride, int pos0, void* stream);

/* ---------------------------------------------------------------------------
 * Verify head: the greedy token and its probability for each row of logits
 * ("[Engine] perf(hip): optimize MTP draft, shared expert, and verify/sampler
 * head kernels on RDNA4", Problem and result item 1, Summary item 1 and
 * Verification & Parity Evidence: T rows of 248,320 fp32 logits, ties, NaN
 * and -inf entries, 1..8 rows on one scratch).  Per row x[0 .. vocab-1]:
 *     token[r]    = the smallest i with x[i] = max of the non-NaN entries;
 *                   -1 when every entry is NaN (-inf is an ordinary value)
 *     top_prob[r] = 1 / sum_i exp(x[i] - x[token]) over the non-NaN entries
 *                   (-inf entries add 0); NaN when no entry is finite
 * +inf entries are outside the contract.  top_prob is computed in fp32 with a
 * fixed merge order (run-to-run bitwise identical); its relative error is a
 * few 1e-6.
 *
 * Layouts: logits fp32, row r at logits + r * row_stride (row_stride >= vocab,
 * in elements; 4-byte alignment); token int32 [n_rows]; top_prob fp32
 * [n_rows] or NULL.  The workspace (16-byte aligned, at least
 * attn_verify_head_workspace_bytes(n_rows, vocab) bytes) holds one ticket per
 * row at fixed offsets in its first 4,096 bytes, then per-block states (24
 * bytes each, for about 256 blocks over all rows): it must be zero-filled
 * before its first use, and every completed call leaves it zero again, so one
 * workspace (sized for the largest call; the size grows with n_rows) serves
 * any sequence of calls of any shape on one stream.  Calls that share
 * a workspace must not run concurrently.  1 <= n_rows <= 1024, vocab >= 1.
 * ------------------------------------------------------------------------- */
size_t attn_verify_head_workspace_bytes(int n_rows, int vocab);
int attn_verify_head_greedy(const float* logits, int n_rows, int vocab,
                            long long row_stride, int* token, float* top_prob,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics.
 *
 * attnq8_selftest_i8_to_f16: run the device's int8 -> fp16 code conversion
 * (exact, "hip: gfx12 (RDNA4) WMMA kernel for the int8-KV QSA prompt
 * attention", How) over all 65,536 byte pairs: for p in [0, 65536), out[2p]
 * and out[2p+1] receive the fp16 bit patterns of the signed bytes (p & 255)
 * and (p >> 8).  out is a device buffer of 131,072 uint16 values.
 *
 * attnq8_stream_read: a plain read of `bytes` bytes at `buf` with 16-byte
 * vector loads, the practical read-bandwidth ceiling against which the
 * attention kernels' HBM rates are also reported.  buf is a device pointer,
 * 16-byte aligned, and bytes a multiple of 16 (0 is allowed); sink is a
 * device buffer of ATTNQ8_STREAM_SINK_WORDS uint32 words, each written with
 * the XOR of the 32-bit words one workgroup read, so the XOR of the sink is
 * the XOR of every word of the buffer.  Errors: ATTNQ8_EINVAL for a null
 * buffer (with bytes > 0) or sink, ATTNQ8_EALIGN for a misaligned buffer or
 * a size that is not a multiple of 16; nothing is launched then.
 *
 * attnq8_status_string: a static description of a status code.
 * attnq8_last_path: a static per-thread description of the kernel variant,
 * grid and split count the calling thread's last successful call launched
 * (the same idea as the expert kernels' report of which path ran: "Faster
 * grouped and per-hit Q2_0 expert kernels, bitwise identical", What it does).
 * Diagnostic only; it never changes which kernel runs.
 * ------------------------------------------------------------------------- */
int attnq8_selftest_i8_to_f16(uint16_t* out, void* stream);
#define ATTNQ8_STREAM_SINK_WORDS 1024
int attnq8_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
const char* attnq8_status_string(int status);
const char* attnq8_last_path(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQ8_H */
