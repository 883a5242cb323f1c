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
 * Debug check of index lists (off the hot path).  For each of `rows` lists of
 * width k: every entry must be in [0, T), or < 0 when allow_pad != 0, and the
 * non-negative entries of a list must be distinct.  Writes into *d_flag
 * (device int, caller-owned) the bitwise OR of 1 (entry out of range) and
 * 2 (repeated entry); 0 means valid.  *d_flag is overwritten, asynchronously.
 */
MLA_API mla_status mla_validate_indices(const int32_t* idx, int rows, int k, int T, int allow_pad,
                         int* d_flag, hipStream_t stream);

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
