"""Plain fp64 CPU oracle of DeepSeek-V3.2-Exp sparse latent attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
calls it and shares no code with it.

What it computes, and where the pages define it
------------------------------------------------
The oracle follows the *explicit* (non-absorbed) form that the model source
uses for its prefill branch ("Key heads" page, Explanation: the code of the
prefill branch, repeated on the "Rotated shared key" page):

1. ``wkv_b`` is one matrix whose per-head view is [128, 256, 512]; the first
   128 rows of each head are W_UK and the last 128 are W_UV ("Mix and project",
   Explanation, decode-branch code; "Key heads", Explanation: one matrix gives content
   keys and values, split after the product).
2. Each cached latent row is up-projected, ``kv = c . wkv_b^T``, viewed
   [rows, 128, 256] and split into per-head content keys k_nope (128) and
   values v (128).
3. Per-head keys join the content part with the one rotary key shared by all
   heads: K_i = [K^C_i ; k^R] ("Key heads", equation K_i = [K^C_i; k^R]).
4. Queries join q_nope and q_pe; scores are q . K scaled by
   ``softmax_scale = qk_head_dim ** -0.5`` = 1/sqrt(192) ("Key heads", Explanation,
   the attention module's constructor).
5. The index mask is -inf everywhere except at the listed positions, where it
   is 0 (``full(-inf).scatter_(..., topk, 0)``); prefill adds the causal mask
   ("Mix and project" and "Key heads" code).  Listing a position twice is the
   same as listing it once (set semantics of the scatter).
6. Softmax over positions, then the weights mix the per-head values.

Readings taken where the pages are silent (each also listed with the design
notes):
* an index of -1 marks an empty slot and selects nothing;
* a query whose selection is empty gets an all-zero output (PyTorch would give
  NaN from a softmax over only -inf);
* softmax is the stable form: subtract the row maximum, exponentiate, divide
  by the sum; exp(-inf) is exactly 0;
* decode has no causal mask (the decode branch passes no mask); prefill query
  s sits at absolute position start_pos + s and sees positions <= that.

A second form, :func:`decode_absorbed`, restates the decode branch of the
pages (W_UK folded into the query, scores against the cached latent, W_UV
applied after the mix).  It exists only to check the pages' claim that the
folded form gives the same scores.

All arithmetic is float64.  bf16 inputs arrive as uint16 bit patterns and are
widened exactly.
"""
from __future__ import annotations

import numpy as np

N_HEADS = 128        # n_heads
D_LATENT = 512       # kv_lora_rank
D_ROPE = 64          # qk_rope_head_dim
D_NOPE = 128         # qk_nope_head_dim
D_V = 128            # v_head_dim
D_QK = D_NOPE + D_ROPE   # qk_head_dim = 192
SOFTMAX_SCALE = D_QK ** -0.5


# --------------------------------------------------------------------------
# input widening
# --------------------------------------------------------------------------
def to_f64(x: np.ndarray) -> np.ndarray:
    """Widen an input tensor to float64 exactly.

    uint16 arrays are bf16 bit patterns: shifting them into the high half of a
    float32 word gives the same real number, which float64 holds exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# the explicit form, step by step
# --------------------------------------------------------------------------
def stack_wkv_b(w_uk: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Rebuild wkv_b as the model stores it: [n_heads * 256, 512] ([out, in]).

    Head h owns output rows 256*h .. 256*h+255; the first 128 are W_UK[h] and
    the last 128 are W_UV[h] (per-head view [128, 256, 512], sliced [:, :128]
    and [:, -128:] in the decode code of "Mix and project").
    """
    w_uk = to_f64(w_uk)
    w_uv = to_f64(w_uv)
    per_head = np.concatenate([w_uk, w_uv], axis=1)          # [128, 256, 512]
    return per_head.reshape(N_HEADS * (D_NOPE + D_V), D_LATENT)


def up_project(latent_rows: np.ndarray, wkv_b: np.ndarray):
    """kv = wkv_b(c): per-position, per-head content keys and values.

    ``latent_rows`` [R, 512] -> (k_nope [R, 128, 128], v [R, 128, 128]).
    The linear layer multiplies by the transposed [out, in] weight.
    """
    kv = latent_rows @ wkv_b.T                                # [R, 32768]
    kv = kv.reshape(latent_rows.shape[0], N_HEADS, D_NOPE + D_V)
    return kv[..., :D_NOPE], kv[..., D_NOPE:]


def join_keys(k_nope: np.ndarray, k_rope: np.ndarray) -> np.ndarray:
    """K_i = [K^C_i ; k^R]: per-head content key then the shared rotary key.

    ``k_nope`` [R, 128, 128], ``k_rope`` [R, 64] -> keys [R, 128, 192].
    """
    R = k_nope.shape[0]
    shared = np.broadcast_to(k_rope[:, None, :], (R, N_HEADS, D_ROPE))
    return np.concatenate([k_nope, shared], axis=-1)


def join_query(q_nope: np.ndarray, q_pe: np.ndarray) -> np.ndarray:
    """q = cat(q_nope, q_pe): [128, 128] and [128, 64] -> [128, 192]."""
    return np.concatenate([q_nope, q_pe], axis=-1)


def scores(q: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s[h, t] = (q[h] . K[t, h]) * scale; q [128, 192], keys [R, 128, 192]."""
    return np.einsum("hd,thd->ht", q, keys) * scale


def index_mask(T: int, idx_row: np.ndarray, causal_limit: int | None = None) -> np.ndarray:
    """Additive mask over positions [0, T).

    0 at every listed position (set semantics: a repeat changes nothing),
    -inf elsewhere; entries < 0 are empty slots.  With ``causal_limit`` the
    causal term adds -inf at every position greater than it.
    """
    mask = np.full(T, -np.inf)
    listed = np.asarray(idx_row)
    listed = listed[listed >= 0]
    if listed.size and listed.max() >= T:
        raise ValueError("index beyond the cache")
    mask[listed] = 0.0
    if causal_limit is not None:
        causal = np.zeros(T)
        causal[causal_limit + 1:] = -np.inf
        mask = mask + causal
    return mask


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Stable softmax along the last axis; a row of only -inf gives zeros."""
    top = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(top)
    top = np.where(empty, 0.0, top)
    e = np.exp(s - top)
    total = np.sum(e, axis=-1, keepdims=True)
    total = np.where(total == 0.0, 1.0, total)
    return e / total


def mix_values(weights: np.ndarray, v: np.ndarray) -> np.ndarray:
    """out[h, d] = sum_t A[h, t] * v[t, h, d]; weights [128, R], v [R, 128, 128]."""
    return np.einsum("ht,thd->hd", weights, v)


# --------------------------------------------------------------------------
# one query, explicit form
# --------------------------------------------------------------------------
def attend_explicit(q_nope, q_pe, latent, rope, w_uk, w_uv, idx_row,
                    scale=SOFTMAX_SCALE, causal_limit=None, return_weights=False):
    """Explicit-form attention of one query over every cached row.

    ``latent`` [T, 512] and ``rope`` [T, 64] are the cached rows; the mask keeps
    the listed rows (and, with ``causal_limit``, only rows <= it).
    Returns out [128, 128] (and the weights [128, T] if asked).
    """
    latent = to_f64(latent)
    rope = to_f64(rope)
    wkv_b = stack_wkv_b(w_uk, w_uv)
    k_nope, v = up_project(latent, wkv_b)
    keys = join_keys(k_nope, rope)
    q = join_query(to_f64(q_nope), to_f64(q_pe))
    s = scores(q, keys, scale)
    s = s + index_mask(latent.shape[0], idx_row, causal_limit)[None, :]
    a = softmax_rows(s)
    out = mix_values(a, v)
    return (out, a) if return_weights else out


def selected_rows(idx_row: np.ndarray, T: int, causal_limit: int | None = None) -> np.ndarray:
    """The set of positions a query sees: listed, non-empty, <= the causal limit."""
    listed = np.asarray(idx_row)
    listed = listed[listed >= 0]
    if listed.size and listed.max() >= T:
        raise ValueError("index beyond the cache")
    if causal_limit is not None:
        listed = listed[listed <= causal_limit]
    return np.unique(listed)


def attend_explicit_gather(q_nope, q_pe, latent, rope, w_uk, w_uv, idx_row,
                           scale=SOFTMAX_SCALE, causal_limit=None):
    """Same result as :func:`attend_explicit`, computed over the visible rows only.

    Rows outside the selection get weight exactly 0 in the full form, so
    dropping them changes nothing but the work; this is what makes full-size
    checks affordable.  ``latent``/``rope`` may be indexable lazily (any array
    supporting fancy indexing by row).
    """
    T = latent.shape[0]
    rows = selected_rows(idx_row, T, causal_limit)
    if rows.size == 0:
        return np.zeros((N_HEADS, D_V))
    sub_latent = to_f64(latent[rows])
    sub_rope = to_f64(rope[rows])
    wkv_b = stack_wkv_b(w_uk, w_uv)
    k_nope, v = up_project(sub_latent, wkv_b)
    keys = join_keys(k_nope, sub_rope)
    q = join_query(to_f64(q_nope), to_f64(q_pe))
    a = softmax_rows(scores(q, keys, scale))
    return mix_values(a, v)


# --------------------------------------------------------------------------
# batched entry points
# --------------------------------------------------------------------------
def decode(inputs: dict, rows=None, gather=True, scale=SOFTMAX_SCALE) -> np.ndarray:
    """Decode output [n, 128, 128] for batch rows ``rows`` (default all).

    ``inputs`` holds q_nope [B,128,128], q_pe [B,128,64], kv_cache [B,T,512],
    pe_cache [B,T,64], topk_idx [B,k], w_uk, w_uv [128,128,512].  Decode has no
    causal mask: every cached position is visible.
    """
    B = inputs["q_nope"].shape[0]
    rows = range(B) if rows is None else rows
    fn = attend_explicit_gather if gather else attend_explicit
    outs = [fn(inputs["q_nope"][b], inputs["q_pe"][b], inputs["kv_cache"][b],
               inputs["pe_cache"][b], inputs["w_uk"], inputs["w_uv"],
               inputs["topk_idx"][b], scale=scale) for b in rows]
    return np.stack(outs)


def prefill(inputs: dict, rows=None, start_pos: int = 0, gather=True,
            scale=SOFTMAX_SCALE) -> np.ndarray:
    """Prefill-chunk output [n, 128, 128] for query rows ``rows`` (default all).

    One sequence: kv_cache [T,512], pe_cache [T,64], queries q_nope [S,128,128],
    q_pe [S,128,64], topk_idx [S,k] (-1 = empty slot).  Query s sits at
    absolute position start_pos + s and sees listed positions <= that.
    """
    S = inputs["q_nope"].shape[0]
    rows = range(S) if rows is None else rows
    kv, pe = inputs["kv_cache"], inputs["pe_cache"]
    if not gather:
        outs = [attend_explicit(inputs["q_nope"][s], inputs["q_pe"][s], kv, pe,
                                inputs["w_uk"], inputs["w_uv"], inputs["topk_idx"][s],
                                scale=scale, causal_limit=start_pos + s) for s in rows]
        return np.stack(outs)
    # Up-project each visible cache row once for all requested queries.
    rows = list(rows)
    T = kv.shape[0]
    visible = [selected_rows(inputs["topk_idx"][s], T, start_pos + s) for s in rows]
    union = np.unique(np.concatenate(visible)) if visible else np.zeros(0, np.int64)
    wkv_b = stack_wkv_b(inputs["w_uk"], inputs["w_uv"])
    k_nope, v = up_project(to_f64(kv[union]), wkv_b)
    keys = join_keys(k_nope, to_f64(pe[union]))
    pos = {int(t): i for i, t in enumerate(union)}
    outs = []
    for s, vis in zip(rows, visible):
        if vis.size == 0:
            outs.append(np.zeros((N_HEADS, D_V)))
            continue
        sel = np.array([pos[int(t)] for t in vis])
        q = join_query(to_f64(inputs["q_nope"][s]), to_f64(inputs["q_pe"][s]))
        a = softmax_rows(scores(q, keys[sel], scale))
        outs.append(mix_values(a, v[sel]))
    return np.stack(outs)


# --------------------------------------------------------------------------
# the folded (absorbed) decode form, used only to check the pages' claim
# --------------------------------------------------------------------------
def absorbed_scores(q_nope, q_pe, latent, rope, w_uk, scale=SOFTMAX_SCALE):
    """Decode-branch scores: W_UK folded into the query, scored on the latent.

    q_c[h, c] = sum_d q_nope[h, d] W_UK[h, d, c]; s[h, t] = (q_c[h] . c_t +
    q_pe[h] . k^R_t) * scale ("Mix and project", Explanation, decode-branch code).
    """
    q_c = np.einsum("hd,hdc->hc", to_f64(q_nope), to_f64(w_uk))
    return (q_c @ to_f64(latent).T + to_f64(q_pe) @ to_f64(rope).T) * scale


def decode_absorbed(q_nope, q_pe, latent, rope, w_uk, w_uv, idx_row, scale=SOFTMAX_SCALE):
    """Decode branch as the pages write it: fold, score, mask, softmax, mix, unfold.

    O~ = A . c^KV (latent mix), then O[h, d] = sum_c O~[h, c] W_UV[h, d, c].
    """
    latent64 = to_f64(latent)
    s = absorbed_scores(q_nope, q_pe, latent64, rope, w_uk, scale)
    s = s + index_mask(latent64.shape[0], idx_row)[None, :]
    a = softmax_rows(s)
    mixed = a @ latent64                                      # [128, 512]
    return np.einsum("hc,hdc->hd", mixed, to_f64(w_uv))


def explicit_scores(q_nope, q_pe, latent, rope, w_uk, w_uv, scale=SOFTMAX_SCALE):
    """Unmasked explicit-form scores [128, T] (rebuilt per-head keys)."""
    wkv_b = stack_wkv_b(w_uk, w_uv)
    k_nope, _ = up_project(to_f64(latent), wkv_b)
    keys = join_keys(k_nope, to_f64(rope))
    return scores(join_query(to_f64(q_nope), to_f64(q_pe)), keys, scale)


# --------------------------------------------------------------------------
# cache append: the step that produces the cached latent and rotary key
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * weight.

    The latent RMSNorm ("KV compression" page, Parameters: 512 learned gains;
    code: kv = self.kv_norm(kv)).  The pages do not show its epsilon; it is a
    caller-supplied reading.
    """
    x = to_f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * to_f64(weight)


def rotate_pairs(x: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """Interleaved rotary embedding of the last axis.

    Feature pairs (x[2i], x[2i+1]) are the real and imaginary parts of one
    complex number, which is multiplied by cos(theta_i) + j sin(theta_i)
    ("Rotated shared key" page, the rotary function with its default
    interleaved layout, as the key path calls it).  ``cos_sin`` [..., D/2, 2]
    holds (cos theta_i, sin theta_i) and broadcasts against x's leading axes.
    """
    x = to_f64(x)
    re, im = x[..., 0::2], x[..., 1::2]
    c, s = to_f64(cos_sin)[..., 0], to_f64(cos_sin)[..., 1]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def cache_append(kv_a_out, norm_weight, cos_sin, kv_cache, pe_cache, start_pos: int, eps: float):
    """New cache contents after appending S positions of B sequences.

    kv_a_out [B, S, 576]: the joint down-projection's output, latent (512)
    then rotary key (64), split after the product ("KV compression" page,
    Explanation).  The latent is RMS-normalised with the gains norm_weight
    [512]; the rotary key is rotated with cos_sin [S, 32, 2] (the angles of
    positions start_pos .. start_pos+S-1).  Both are written to rows
    start_pos .. start_pos+S-1 of kv_cache [B, T, 512] and pe_cache [B, T, 64]
    (the model caches these 576 values per position); every other row keeps
    its value.  Returns (kv_cache, pe_cache) as float64 copies.
    """
    a = to_f64(kv_a_out)
    S = a.shape[1]
    kv = to_f64(kv_cache).copy()
    pe = to_f64(pe_cache).copy()
    kv[:, start_pos:start_pos + S] = rms_norm(a[..., :D_LATENT], norm_weight, eps)
    pe[:, start_pos:start_pos + S] = rotate_pairs(a[..., D_LATENT:], to_f64(cos_sin)[None])
    return kv, pe


# --------------------------------------------------------------------------
# output projection: the step after the path
# --------------------------------------------------------------------------
D_MODEL = 7168       # model width


def output_projection(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Delta = o W_O: the 128 heads' outputs joined and projected to the model width.

    ``o`` [B, 128, 128] is the per-head output O_i; it is flattened head by
    head into [B, 16384] (o = reshape(O), "Mix and project" page, All 4
    steps; the code flattens the head and value axes).  ``w_o`` is stored as
    the model's linear layer stores it, [7168 out, 16384 in], so the product
    is o . w_o^T -> [B, 7168].
    """
    o = to_f64(o)
    return o.reshape(o.shape[0], N_HEADS * D_V) @ to_f64(w_o).T


# --------------------------------------------------------------------------
# FP8 wkv_b: the decode branch dequantises the stored wkv_b once when it
# carries a scale and caches the result ("Mix and project", Explanation,
# decode-branch code); the pages name FP8 block scales ("Key heads",
# Parameters, the note under the table) but not their format.  Reading:
# OCP E4M3 codes -- 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
# exponent 0 holds the subnormals m * 2^-9; the code with every exponent and
# mantissa bit set is NaN; there are no infinities -- and one scale per
# 128 x 128 block of the [rows, cols] weight.
# --------------------------------------------------------------------------
FP8_BLOCK = 128


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 byte, exactly, in float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    # normal: (1 + m/8) * 2^(e - 7) = (8 + m) * 2^(e - 10); subnormal: (m/8) * 2^(1 - 7)
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    val = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, val)


def fp8_block_dequant(codes: np.ndarray, scales: np.ndarray, block: int = FP8_BLOCK) -> np.ndarray:
    """weight[r, c] = value(codes[r, c]) * scales[r // block, c // block], float64."""
    codes = np.asarray(codes)
    R, C = codes.shape
    s = to_f64(scales)
    assert s.shape == (-(-R // block), -(-C // block)), "one scale per block"
    full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:R, :C]
    return fp8_e4m3_decode(codes) * full


def wkv_b_dequant(codes: np.ndarray, scales: np.ndarray):
    """The dequantised wkv_b [128 * 256, 512] split per head into W_UK and W_UV.

    The decode branch views the weight as [heads, 256, 512] and takes the first
    qk_nope_head_dim rows of each head as W_UK and the rest as W_UV ("Mix and
    project", Explanation, decode-branch code).  Returns two [128, 128, 512].
    """
    w = fp8_block_dequant(codes, scales).reshape(N_HEADS, D_NOPE + D_V, D_LATENT)
    return w[:, :D_NOPE], w[:, D_NOPE:]
