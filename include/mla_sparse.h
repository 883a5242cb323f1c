/*
 * mla_sparse.h — C ABI of the MI355X (gfx950) sparse latent attention library.
 *
 * The library computes DeepSeek-V3.2-Exp's sparse latent attention in its
 * absorbed form for 128 heads that share one latent cache ("Mix and project"
 * page, Explanation: the decode-branch code; "Key heads" page, Explanation: folding
 * W_UK into the query gives the same scores):
 *
 *   1. q_c[h]   = q_nope[h] . W_UK[h]                (512 per head)
 *   2. s[h, t]  = (q_c[h] . c_t + q_pe[h] . kR_t) * softmax_scale
 *   3. s[h, t]  = -inf for every position t not in the top-k list
 *   4. A        = softmax_t(s);  O~[h] = sum_t A[h, t] c_t
 *   5. out[h]   = O~[h] . W_UV[h]^T                  (128 per head)
 *
 * where c_t is the cached, normalised 512-wide latent and kR_t the cached
 * 64-wide rotary key of position t ("KV compression" page, Explanation: 576
 * cached values per position; "Rotated shared key" page, shape [B, T, 64]).
 *
 * Fixed model widths: 128 heads, latent 512, rotary 64, q_nope 128, value 128.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller, row-major,
 *   16-byte aligned.  The library allocates no device memory, never
 *   synchronises the stream, and launches all work asynchronously on `stream`.
 * - `dtype` (mla_dtype) is the element type of every floating tensor of the
 *   call (queries, caches, weights, output).  MLA_BF16 computes with bf16
 *   MFMA and float32 accumulation; MLA_F32 computes in float32 throughout.
 * - W_UK and W_UV are [128 heads, 128, 512] in [h, d, c] order: the per-head
 *   view [128, 256, 512] of the model's wkv_b weight ([out, in] storage),
 *   first 128 rows of each head = W_UK, last 128 = W_UV.
 * - Index lists are int32.  An entry < 0 is an empty slot and selects
 *   nothing.  Valid entries must be distinct and lie in [0, T) (a repeated
 *   position would be counted twice; the model's scatter_ mask would count it
 *   once).  This is a precondition that only mla_validate_indices checks; an
 *   entry >= T is never read and is treated as an empty slot.
 * - A query whose selection is empty gets an all-zero output.
 * - Arguments are checked on the host before anything is launched; a failed
 *   check returns its error code and launches nothing.  A failed kernel
 *   launch returns MLA_ERR_HIP.
 */
#ifndef MLA_SPARSE_H
#define MLA_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from libmla_sparse.so. */
#ifndef MLA_API
#define MLA_API __attribute__((visibility("default")))
#endif

#define MLA_N_HEADS 128
#define MLA_D_LATENT 512
#define MLA_D_ROPE 64
#define MLA_D_NOPE 128
#define MLA_D_V 128
#define MLA_MAX_T 2097148   /* largest cache length T (positions per sequence) */

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL = 1,      /* a required pointer is NULL */
    MLA_ERR_SHAPE = 2,     /* a size is out of range (B, S, T, k < 1, k > T, T > MLA_MAX_T, ...) */
    MLA_ERR_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
    MLA_ERR_DTYPE = 4,     /* dtype is not an mla_dtype value */
    MLA_ERR_WORKSPACE = 5, /* workspace NULL/misaligned or smaller than the size query */
    MLA_ERR_INDEX = 6,     /* reserved for index errors reported by mla_validate_indices */
    MLA_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
MLA_API const char* mla_status_string(int status);

/* ABI revision of this header; bumps on any signature change. */
MLA_API int mla_abi_version(void);

/*
 * Decode: one new query per batch row against that row's cache.
 * ("Mix and project" page, Explanation, decode-branch code: no causal mask, all
 *  cached positions [0, T) are visible, the index mask keeps the top-k list.)
 *
 *   q_nope   [B, 128, 128]   q_pe [B, 128, 64] (already rotated)
 *   kv_cache [B, ld_T, 512]  pe_cache [B, ld_T, 64]; rows 0..T-1 are used
 *   topk_idx [B, k] int32    positions in [0, T) (order irrelevant), <0 = empty
 *   w_uk, w_uv [128, 128, 512]
 *   out      [B, 128, 128]   written, never read
 *   softmax_scale: multiplies the scores (the model uses 192 ** -0.5)
 *   workspace: device scratch of at least
 *              mla_sparse_decode_workspace_size(B, T, k, dtype) bytes, 256-byte
 *              aligned; contents on entry are ignored.  Concurrent calls need
 *              distinct workspaces.
 */
MLA_API size_t mla_sparse_decode_workspace_size(int B, int T, int k, int dtype);

MLA_API mla_status mla_sparse_decode(const void* q_nope, const void* q_pe,
                      const void* kv_cache, const void* pe_cache,
                      const int32_t* topk_idx,
                      const void* w_uk, const void* w_uv, void* out,
                      int B, int T, int ld_T, int k, float softmax_scale, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, arguments, checks and errors as
 * mla_sparse_decode, with the workspace taken from a fixed array of
 * MLA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on, from the first such call until the process ends.  The call itself
 * allocates nothing.
 *
 * Returns MLA_ERR_WORKSPACE when mla_sparse_decode_workspace_size(B, T, k,
 * dtype) exceeds MLA_NOALLOC_SCRATCH_BYTES (B = 64, k = 2048 in bf16 needs
 * 41.3 MiB and fits; large k at small B, or float32, may not).  Every call on
 * one device shares that device's array, which keeps the last call's
 * contents: calls that overlap on one device (different streams, or threads
 * without ordering) race and corrupt each other's results; calls queued on
 * one stream are ordered and safe.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (48 * 1024 * 1024)

MLA_API mla_status mla_sparse_decode_noalloc(const void* q_nope, const void* q_pe,
                                             const void* kv_cache, const void* pe_cache,
                                             const int32_t* topk_idx,
                                             const void* w_uk, const void* w_uv, void* out,
                                             int B, int T, int ld_T, int k, float softmax_scale,
                                             int dtype, hipStream_t stream);

/*
 * Prefill chunk in latent form: S consecutive queries of ONE sequence against
 * its cache.  Query s sits at absolute position start_pos + s and ignores any
 * listed position greater than that (the causal mask the model adds in its
 * prefill branch, "Key heads" page, Explanation, prefill-branch code).
 *
 *   q_nope [S, 128, 128], q_pe [S, 128, 64]
 *   kv_cache [T, 512], pe_cache [T, 64]   (start_pos + S <= T)
 *   topk_idx [S, k] int32, -1 padded     out [S, 128, 128]
 */
MLA_API size_t mla_sparse_prefill_chunk_workspace_size(int S, int T, int k, int dtype);

MLA_API mla_status mla_sparse_prefill_chunk(const void* q_nope, const void* q_pe,
                             const void* kv_cache, const void* pe_cache,
                             const int32_t* topk_idx,
                             const void* w_uk, const void* w_uv, void* out,
                             int S, int T, int k, int start_pos, float softmax_scale, int dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Output projection, the step after the attention ("Mix and project" page,
 * All 4 steps: o = reshape(O), Delta = o W_O; Parameters: 16,384 x 7,168;
 * code: the head outputs flattened and passed through the output linear
 * layer, the only step that mixes heads):
 *
 *   out[b, n] = sum_k o[b, k] * w_o[n, k],  k = 128 * head + value
 *
 *   o    [B, 128, 128]  per-head outputs (what mla_sparse_decode writes)
 *   w_o  [7168, 16384]  the output layer's weight in its [out, in] storage
 *   out  [B, 7168]      written, never read
 *
 * bf16: MFMA with float32 accumulation; the 16,384 inputs are taken in eight
 * ranges whose float32 partial sums go to the workspace (256-byte aligned,
 * mla_output_projection_workspace_size(B, dtype) bytes, contents ignored) and
 * are then added and rounded once to bf16 (deterministic).  float32: float32
 * throughout, no workspace (size 0; NULL accepted).  Errors: MLA_ERR_NULL,
 * MLA_ERR_SHAPE (B < 1), MLA_ERR_ALIGN, MLA_ERR_DTYPE, MLA_ERR_WORKSPACE,
 * MLA_ERR_HIP.
 */
#define MLA_D_MODEL 7168

MLA_API size_t mla_output_projection_workspace_size(int B, int dtype);

MLA_API mla_status mla_output_projection(const void* o, const void* w_o, void* out, int B, int dtype,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 wkv_b dequantisation: the decode branch dequantises the stored wkv_b
 * once when it carries a scale, views it [heads, 256, 512] and takes the first
 * 128 rows of each head as W_UK and the last 128 as W_UV ("Mix and project"
 * page, Explanation, decode-branch code; FP8 block scales: "Key heads" page,
 * Parameters, the note under the table).  The pages do not give the format;
 * this library reads it as OCP E4M3 codes (1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9; the code
 * with all exponent and mantissa bits set is NaN; no infinities) and one
 * float32 scale per 128 x 128 block:
 *
 *   w[r, c] = value(codes[r, c]) * scales[r / 128, c / 128]
 *   w_uk[h, d, c] = w[256 h + d, c],  w_uv[h, d, c] = w[256 h + 128 + d, c]
 *
 *   codes   [32768, 512] uint8 (16-byte aligned)
 *   scales  [256, 4] float32, row-major by block
 *   w_uk, w_uv [128, 128, 512] bf16, written (value times scale in float32,
 *           rounded once to bf16); the inputs mla_sparse_decode takes
 *
 * Errors: MLA_ERR_NULL, MLA_ERR_ALIGN, MLA_ERR_HIP.
 */
MLA_API mla_status mla_wkv_b_dequant(const void* codes, const float* scales, void* w_uk, void* w_uv,
                                     hipStream_t stream);

/*
 * Cache append: the step that fills the caches the attention reads
 * ("KV compression" page, Explanation and code: one joint down-projection
 * gives the 512-wide latent and the 64-wide rotary key, split after the
 * product; the latent goes through its RMSNorm; the rotary key is rotated;
 * the model caches these 576 values per position.  "Rotated shared key"
 * page: the rotary function, with interleaved feature pairs as the key path
 * calls it).  For each of B sequences and S new positions:
 *
 *   c   = kv_a_out[b, s, 0:512] / sqrt(mean(kv_a_out[b, s, 0:512]^2) + eps) * norm_weight
 *   kR  = kv_a_out[b, s, 512:576] with pair i (features 2i, 2i+1) taken as
 *         re + j im and multiplied by cos_sin[s, i, 0] + j cos_sin[s, i, 1]
 *   kv_cache[b, start_pos + s] = c,  pe_cache[b, start_pos + s] = kR
 *
 *   kv_a_out    [B, S, 576]    the down-projection's output, in `dtype`
 *   norm_weight [512]          the latent RMSNorm's gains, in `dtype`
 *   cos_sin     [S, 32, 2]     float32: cos and sin of the rotary angle of each
 *                              pair at each new position (the caller's
 *                              frequency table, sliced to those positions)
 *   kv_cache    [B, ld_T, 512], pe_cache [B, ld_T, 64], in `dtype`: rows
 *               start_pos .. start_pos+S-1 are written, no other row is touched
 *   eps         the RMSNorm epsilon (>= 0; the pages do not give its value)
 *
 * Arithmetic in float32, results rounded to `dtype`.  Errors: MLA_ERR_NULL,
 * MLA_ERR_SHAPE (B or S < 1, start_pos < 0, start_pos + S > ld_T, eps < 0 or
 * not finite), MLA_ERR_ALIGN, MLA_ERR_DTYPE, MLA_ERR_HIP.
 */
MLA_API mla_status mla_cache_append(const void* kv_a_out, const void* norm_weight, const float* cos_sin,
                                    void* kv_cache, void* pe_cache, int B, int S, int start_pos, int ld_T,
                                    float eps, int dtype, hipStream_t stream);

/*
 * Prefill chunk in the explicit form the pages print for prefill ("Key heads"
 * page, Explanation: the prefill-branch code: the latent is up-projected into
 * per-head content keys and values, each head's key joins its content part
 * with the shared rotary key, scores are scaled, masked by the index list and
 * the causal mask, normalised and used to mix the values).  Same arguments,
 * layouts, readings and result as mla_sparse_prefill_chunk (which computes
 * the absorbed form); bf16 only (MLA_ERR_DTYPE otherwise).
 *
 * Computation: the keys and values of positions 0 .. min(start_pos + S, T) - 1
 * are up-projected into the workspace ([positions, 128, 256] bf16), the index
 * lists become a bitmap of selected positions per query, and blocks of 128
 * queries attend, head by head, over every position up to their last query's,
 * with unselected positions masked.  The workspace must hold
 * mla_sparse_prefill_explicit_workspace_size(S, T, k, start_pos, dtype) bytes
 * (0 for invalid arguments or a dtype other than MLA_BF16).
 */
MLA_API size_t mla_sparse_prefill_explicit_workspace_size(int S, int T, int k, int start_pos, int dtype);

MLA_API mla_status mla_sparse_prefill_explicit(const void* q_nope, const void* q_pe,
                                               const void* kv_cache, const void* pe_cache,
                                               const int32_t* topk_idx,
                                               const void* w_uk, const void* w_uv, void* out,
                                               int S, int T, int k, int start_pos, float softmax_scale,
                                               int dtype, void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/*
 * Debug check of index lists (off the hot path).  For each of `rows` lists of
 * width k: every entry must be in [0, T), or < 0 when allow_pad != 0, and the
 * non-negative entries of a list must be distinct.  Writes into *d_flag
 * (device int, caller-owned) the bitwise OR of 1 (entry out of range) and
 * 2 (repeated entry); 0 means valid.  *d_flag is overwritten, asynchronously.
 */
MLA_API mla_status mla_validate_indices(const int32_t* idx, int rows, int k, int T, int allow_pad,
                         int* d_flag, hipStream_t stream);

/*
 * Diagnostics of the last decode or prefill call that used `workspace`, with
 * the same row count (B or S), k and dtype: copies, asynchronously on
 * `stream`, two ints into d_out[0..1] (device memory, caller-owned, 4-byte
 * aligned):
 *
 *   d_out[0]  index-list splits the attention kernel ran a second time.  The
 *             softmax ("Mix and project" page, All 4 steps: A = softmax,
 *             O~ = A c^KV) is computed per split of an index list against a
 *             reference score per head, taken from the split's first tile of
 *             32 positions with a selected one.  When a later score beats it
 *             by about 60 in log2 units (so that the probabilities could leave
 *             the float range), the bf16 path discards the split's pass and
 *             runs it again: once to find each head's largest score, then in
 *             full with that as the reference.  The float32 path keeps a
 *             running maximum instead and reports 0.
 *   d_out[1]  reserved; always 0.
 *
 * Off the hot path; the next call does not read them.
 */
MLA_API mla_status mla_read_diagnostics(const void* workspace, int rows, int k, int dtype,
                                        int* d_out, hipStream_t stream);

/*
 * Timing hook.  When `begin` and `end` are non-NULL (events the caller has
 * created, with timing enabled), the next decode or prefill call has the
 * dispatch of its attention kernel record `begin` when the kernel starts and
 * `end` when it completes (hipExtLaunchKernel), then forgets both: their
 * interval is the kernel's own duration, without the cost of separate event
 * records.  Passing NULLs cancels a pending request.  Process-wide, not
 * thread-safe; intended for benchmarks.
 */
MLA_API mla_status mla_set_attention_events(hipEvent_t begin, hipEvent_t end);

#ifdef __cplusplus
}
#endif

#endif /* MLA_SPARSE_H */
