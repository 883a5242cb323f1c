"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here runs on the CPU.  The independent references are:
* numbers the pages print (tests/golden/page_shapes.json);
* the pages' own claim that the folded decode form gives the same scores (I1);
* softmax invariants (I2) and set semantics shown by brute force (I4);
* closed forms (C1 single row, C2 zero query, C3 identity weights that reduce
  the method to textbook multi-head attention);
* torch's CPU ``scaled_dot_product_attention`` in float64 on keys and values
  built from the definition k^C = c^KV W_UK (C4), a library routine that
  shares nothing with the oracle's stacked-matrix route;
* the bf16 format definition for the input widening.
The mutation tests at the end plant one plausible mistake at a time in the
oracle and check that some pin fails.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import mla_oracle as om

H, DL, DR, DN, DV = 128, 512, 64, 128, 128
SCALE = 192 ** -0.5


def rand_case(T, seed, q_scale=1.0):
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((T, DL))
    lat /= np.sqrt(np.mean(lat * lat, axis=1, keepdims=True))
    rope = rng.standard_normal((T, DR))
    qn = rng.standard_normal((H, DN)) * q_scale
    qp = rng.standard_normal((H, DR)) * q_scale
    w_uk = rng.standard_normal((H, DN, DL)) / np.sqrt(512)
    w_uv = rng.standard_normal((H, DV, DL)) / np.sqrt(512)
    return qn, qp, lat, rope, w_uk, w_uv


# ---------------------------------------------------------------- references
def sdpa_reference(qn, qp, lat, rope, w_uk, w_uv, rows, scale=SCALE, causal_limit=None):
    """torch SDPA (CPU, float64) over keys/values built from k^C = c W_UK, v = c W_UV."""
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    lat_t, rope_t = t(lat)[rows], t(rope)[rows]
    k_c = torch.einsum("tc,hdc->htd", lat_t, t(w_uk))          # [H, R, 128]
    v = torch.einsum("tc,hdc->htd", lat_t, t(w_uv))            # [H, R, 128]
    k = torch.cat([k_c, rope_t.unsqueeze(0).expand(H, -1, -1)], dim=-1)   # [H, R, 192]
    q = torch.cat([t(qn), t(qp)], dim=-1).unsqueeze(1)          # [H, 1, 192]
    out = F.scaled_dot_product_attention(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0),
                                         scale=scale)
    return out[0, :, 0, :].numpy()


def textbook_mha(q, k, v, scale, allowed):
    """Plain multi-head attention of one query: q [H,E], k [T,H,E], v [T,H,Ev]."""
    out = np.zeros((q.shape[0], v.shape[-1]))
    for h in range(q.shape[0]):
        s = np.array([q[h] @ k[t, h] * scale for t in allowed])
        w = np.exp(s - s.max())
        w /= w.sum()
        out[h] = sum(w[i] * v[t, h] for i, t in enumerate(allowed))
    return out


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


# ---------------------------------------------------------------- page pins
def test_page_shape_pins(repo_root):
    g = json.load(open(os.path.join(repo_root, "tests", "golden", "page_shapes.json")))
    val = lambda key: g[key]["value"]
    assert oracle.N_HEADS == val("n_heads")
    assert oracle.D_QK == val("key_features_per_head")
    assert oracle.D_LATENT == val("kv_latent_width")
    assert oracle.D_ROPE == val("rotary_key_width")
    # W_UK is 512 x (heads * nope width): the parameter count pins D_NOPE per head.
    assert oracle.D_LATENT * oracle.N_HEADS * oracle.D_NOPE == val("key_content_up_projection_params")
    assert val("model_width") * oracle.D_ROPE == val("rotary_key_projection_params")
    assert (val("key_content_up_projection_params") + val("rotary_key_projection_params")
            == val("key_heads_instance_total"))
    assert val("model_width") * oracle.D_LATENT == val("kv_down_projection_params")
    assert oracle.D_LATENT == val("kv_latent_rmsnorm_params")
    # W_O input width is heads * value width: pins D_V.
    assert oracle.N_HEADS * oracle.D_V * val("model_width") == val("output_projection_params")
    assert 1536 * oracle.N_HEADS * oracle.D_ROPE == val("query_rotary_up_projection_params")
    assert oracle.D_LATENT + oracle.D_ROPE == val("cached_values_per_position")
    assert oracle.N_HEADS * (oracle.D_QK + oracle.D_V) == val("explicit_kv_values_per_position")
    assert 1000 + 1 == val("decode_page_keys_at_p1000")
    # the stacked wkv_b has [heads * (nope + v), latent] = [32768, 512]
    w = om.stack_wkv_b(np.zeros((H, DN, DL)), np.zeros((H, DV, DL)))
    assert w.shape == (32768, 512)
    assert w[:, :].size // 2 == val("key_content_up_projection_params")


def test_softmax_scale_is_inverse_sqrt_head_dim():
    # softmax_scale = qk_head_dim ** -0.5, qk_head_dim = 128 + 64 (Key heads, code).
    assert oracle.SOFTMAX_SCALE == pytest.approx(1.0 / np.sqrt(192.0), rel=0, abs=1e-16)


def test_bf16_widening_matches_format_definition():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x4049],
                    dtype=np.uint16)
    want = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, np.inf, -np.inf, 0.0, -0.0,
                     2.0 * (1 + 0x49 / 128.0)])
    got = om.to_f64(bits)
    assert np.array_equal(got, want)
    assert np.signbit(got[7])


# ---------------------------------------------------------------- invariants
def test_I1_absorbed_scores_equal_explicit_scores():
    qn, qp, lat, rope, w_uk, w_uv = rand_case(40, 1)
    s_exp = om.explicit_scores(qn, qp, lat, rope, w_uk, w_uv)
    s_abs = om.absorbed_scores(qn, qp, lat, rope, w_uk)
    assert rel_err(s_abs, s_exp) <= 1e-12
    idx = np.array([0, 3, 7, 11, 20, 39])
    o_exp = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, idx)
    o_abs = om.decode_absorbed(qn, qp, lat, rope, w_uk, w_uv, idx)
    assert rel_err(o_abs, o_exp) <= 1e-12


def test_I2_softmax_rows_sum_to_one():
    qn, qp, lat, rope, w_uk, w_uv = rand_case(33, 2, q_scale=3.0)
    idx = np.arange(0, 33, 2)
    _, a = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, idx, return_weights=True)
    assert np.all(a >= 0)
    assert np.max(np.abs(a.sum(axis=1) - 1.0)) <= 1e-12
    # extreme logits stay finite and normalised
    s = np.array([[1e300, -1e300, 0.0], [-np.inf, 5.0, -np.inf]])
    p = om.softmax_rows(s)
    assert np.all(np.isfinite(p)) and np.allclose(p.sum(axis=1), 1.0)


def test_I3_all_positions_selected_equals_unmasked_attention():
    qn, qp, lat, rope, w_uk, w_uv = rand_case(24, 3)
    full = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, np.arange(24))
    ref = sdpa_reference(qn, qp, lat, rope, w_uk, w_uv, np.arange(24))
    assert rel_err(full, ref) <= 1e-12


def test_I4_brute_force_subsets_of_six_positions():
    T = 6
    qn, qp, lat, rope, w_uk, w_uv = rand_case(T, 4, q_scale=2.0)
    poison = lat.copy()
    poison_r = rope.copy()
    for r in range(1, T + 1):
        for subset in itertools.combinations(range(T), r):
            S = np.array(subset)
            out, a = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, S, return_weights=True)
            outside = np.setdiff1d(np.arange(T), S)
            assert np.all(a[:, outside] == 0.0)
            ref = sdpa_reference(qn, qp, lat, rope, w_uk, w_uv, S)
            assert rel_err(out, ref) <= 1e-12
            # order of the list does not matter, repeats do not count twice
            shuffled = np.random.default_rng(r).permutation(np.concatenate([S, S[:1]]))
            out2 = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, shuffled)
            assert rel_err(out2, out) <= 1e-14
            # unselected rows never reach the result
            g = om.attend_explicit_gather(qn, qp, lat, rope, w_uk, w_uv, S)
            poison[:] = lat
            poison_r[:] = rope
            poison[outside] = 1e30
            poison_r[outside] = -1e30
            g2 = om.attend_explicit_gather(qn, qp, poison, poison_r, w_uk, w_uv, S)
            assert np.array_equal(g, g2)
            f2 = om.attend_explicit(qn, qp, poison, poison_r, w_uk, w_uv, S)
            assert rel_err(f2, out) <= 1e-12
            assert rel_err(g, out) <= 1e-12


def test_gather_form_equals_full_form_on_sparse_selection():
    T = 300
    qn, qp, lat, rope, w_uk, w_uv = rand_case(T, 5)
    idx = np.sort(np.random.default_rng(5).choice(T, 77, replace=False))
    a = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, idx)
    b = om.attend_explicit_gather(qn, qp, lat, rope, w_uk, w_uv, idx)
    assert rel_err(b, a) <= 1e-12


# ---------------------------------------------------------------- closed forms
def test_C1_single_selected_row_is_projected_latent():
    T = 9
    qn, qp, lat, rope, w_uk, w_uv = rand_case(T, 6)
    for i in (0, 4, 8):
        want = np.stack([w_uv[h] @ lat[i] for h in range(H)])
        for qs in (1.0, 10.0):
            out = om.attend_explicit(qn * qs, qp * qs, lat, rope, w_uk, w_uv, np.array([i]))
            assert rel_err(out, want) <= 1e-13


def test_C2_zero_query_gives_uniform_mean():
    T = 17
    _, _, lat, rope, w_uk, w_uv = rand_case(T, 7)
    S = np.array([1, 2, 5, 9, 16])
    mean = lat[S].mean(axis=0)
    want = np.stack([w_uv[h] @ mean for h in range(H)])
    out = om.attend_explicit(np.zeros((H, DN)), np.zeros((H, DR)), lat, rope, w_uk, w_uv, S)
    assert rel_err(out, want) <= 1e-13


def test_C3_identity_weights_reduce_to_textbook_attention():
    T = 12
    qn, qp, lat, rope, _, _ = rand_case(T, 8)
    eye = np.zeros((H, 128, DL))
    eye[:, :, :128] = np.eye(128)
    S = [0, 2, 3, 7, 11]
    k = np.concatenate([np.repeat(lat[:, None, :128], H, axis=1),
                        np.repeat(rope[:, None, :], H, axis=1)], axis=-1)   # [T,H,192]
    v = np.repeat(lat[:, None, :128], H, axis=1)
    q = np.concatenate([qn, qp], axis=-1)
    want = textbook_mha(q, k, v, SCALE, S)
    out = om.attend_explicit(qn, qp, lat, rope, eye, eye, np.array(S))
    assert rel_err(out, want) <= 1e-13


def test_C4_dense_case_matches_library_attention():
    qn, qp, lat, rope, w_uk, w_uv = rand_case(64, 9)
    out = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, np.arange(64))
    ref = sdpa_reference(qn, qp, lat, rope, w_uk, w_uv, np.arange(64))
    assert rel_err(out, ref) <= 1e-12


def test_empty_selection_reads_as_zero_output():
    qn, qp, lat, rope, w_uk, w_uv = rand_case(5, 10)
    out = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, np.array([-1, -1]))
    assert np.array_equal(out, np.zeros((H, DV)))
    out = om.attend_explicit_gather(qn, qp, lat, rope, w_uk, w_uv, np.array([], dtype=np.int32))
    assert np.array_equal(out, np.zeros((H, DV)))


# ---------------------------------------------------------------- batched decode
def decode_batch_case(seed=14, B=3, T=20, k=7):
    """B batch rows, each with its own cache, queries and index list."""
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((B, T, DL))
    lat /= np.sqrt(np.mean(lat * lat, axis=2, keepdims=True))
    return {"q_nope": rng.standard_normal((B, H, DN)), "q_pe": rng.standard_normal((B, H, DR)),
            "kv_cache": lat, "pe_cache": rng.standard_normal((B, T, DR)),
            "topk_idx": np.stack([np.sort(rng.choice(T, k, replace=False)) for _ in range(B)]),
            "w_uk": rng.standard_normal((H, DN, DL)) / np.sqrt(512),
            "w_uv": rng.standard_normal((H, DV, DL)) / np.sqrt(512)}


def test_D1_batched_decode_pairs_rows_and_honours_scale():
    # The batched entry point every decode parity check uses: batch row b's queries meet
    # row b's own cache and index list ("Mix and project", decode-branch code: one query per
    # sequence, scores against that sequence's cache), under the caller's scale.  Each row
    # is compared with torch's CPU SDPA on keys and values built from the definition.
    inp = decode_batch_case()
    scale = 0.7
    rows = [2, 0]
    got = om.decode(inp, rows=rows, scale=scale)
    assert got.shape == (2, H, DV)
    for i, b in enumerate(rows):
        ref = sdpa_reference(inp["q_nope"][b], inp["q_pe"][b], inp["kv_cache"][b],
                             inp["pe_cache"][b], inp["w_uk"], inp["w_uv"], inp["topk_idx"][b],
                             scale=scale)
        assert rel_err(got[i], ref) <= 1e-12
    full = om.decode(inp, rows=rows, scale=scale, gather=False)
    assert rel_err(full, got) <= 1e-12
    # default rows: every batch row, in order; default scale 1/sqrt(192)
    every = om.decode(inp)
    assert every.shape == (3, H, DV)
    ref1 = sdpa_reference(inp["q_nope"][1], inp["q_pe"][1], inp["kv_cache"][1], inp["pe_cache"][1],
                          inp["w_uk"], inp["w_uv"], inp["topk_idx"][1])
    assert rel_err(every[1], ref1) <= 1e-12


# ---------------------------------------------------------------- prefill pins
def prefill_case(T, S, start_pos, seed, k):
    qn0, qp0, lat, rope, w_uk, w_uv = rand_case(T, seed)
    rng = np.random.default_rng(seed + 100)
    qn = rng.standard_normal((S, H, DN))
    qp = rng.standard_normal((S, H, DR))
    idx = np.full((S, k), -1, dtype=np.int32)
    for s in range(S):
        p = start_pos + s
        n = min(p + 1, k)
        pick = np.arange(p + 1) if p + 1 <= k else np.append(rng.choice(p, k - 1, replace=False), p)
        idx[s, :n] = np.sort(pick)
    return {"q_nope": qn, "q_pe": qp, "kv_cache": lat, "pe_cache": rope, "topk_idx": idx,
            "w_uk": w_uk, "w_uv": w_uv}


def test_prefill_full_causal_equals_library_causal_attention():
    T = S = 10
    inp = prefill_case(T, S, 0, 11, k=T)
    out = om.prefill(inp, gather=False)
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    lat = t(inp["kv_cache"])
    k_c = torch.einsum("tc,hdc->htd", lat, t(inp["w_uk"]))
    v = torch.einsum("tc,hdc->htd", lat, t(inp["w_uv"]))
    k = torch.cat([k_c, t(inp["pe_cache"]).unsqueeze(0).expand(H, -1, -1)], dim=-1)
    q = torch.cat([t(inp["q_nope"]), t(inp["q_pe"])], dim=-1).transpose(0, 1)   # [H, S, 192]
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                         scale=SCALE)[0].transpose(0, 1).numpy()
    assert rel_err(out, ref) <= 1e-12


def test_prefill_sparse_causal_gather_and_full_agree_and_match_decode():
    T, S, start = 40, 8, 30
    inp = prefill_case(T, S, start, 12, k=12)
    full = om.prefill(inp, start_pos=start, gather=False)
    gat = om.prefill(inp, start_pos=start, gather=True)
    assert rel_err(gat, full) <= 1e-12
    for s in range(S):
        p = start + s
        # same query as a decode over the first p+1 cached rows
        dec = om.attend_explicit(inp["q_nope"][s], inp["q_pe"][s], inp["kv_cache"][:p + 1],
                                 inp["pe_cache"][:p + 1], inp["w_uk"], inp["w_uv"],
                                 inp["topk_idx"][s])
        assert rel_err(full[s], dec) <= 1e-12


def test_prefill_ignores_listed_positions_beyond_the_query():
    T = 16
    qn, qp, lat, rope, w_uk, w_uv = rand_case(T, 13)
    listed = np.array([0, 3, 5, 9, 14, -1, -1])
    p = 6
    a = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, listed, causal_limit=p)
    b = om.attend_explicit(qn, qp, lat, rope, w_uk, w_uv, np.array([0, 3, 5]))
    assert rel_err(a, b) <= 1e-14


# ---------------------------------------------------------------- mutations
def _pins_all_pass(stop_at_first=False):
    """Run the value pins; return the names of those that fail (only the first one with
    ``stop_at_first``)."""
    failed = []
    for name, fn in [("I1", test_I1_absorbed_scores_equal_explicit_scores),
                     ("I3", test_I3_all_positions_selected_equals_unmasked_attention),
                     ("C1", test_C1_single_selected_row_is_projected_latent),
                     ("C2", test_C2_zero_query_gives_uniform_mean),
                     ("C3", test_C3_identity_weights_reduce_to_textbook_attention),
                     ("C4", test_C4_dense_case_matches_library_attention),
                     ("P1", test_prefill_full_causal_equals_library_causal_attention),
                     ("P3", test_prefill_ignores_listed_positions_beyond_the_query),
                     ("D1", test_D1_batched_decode_pairs_rows_and_honours_scale)]:
        try:
            fn()
        except AssertionError:
            failed.append(name)
            if stop_at_first:
                break
    return failed


MUTATIONS = {
    # W_UK and W_UV exchanged when the stacked matrix is built
    "swap_uk_uv": ("stack_wkv_b", lambda orig: (lambda a, b: orig(b, a))),
    # rotary part of the key dropped
    "drop_rope_key": ("join_keys", lambda orig: (lambda kn, kr: orig(kn, np.zeros_like(kr)))),
    # rotary part of the query dropped
    "drop_rope_query": ("join_query", lambda orig: (lambda qn, qp: orig(qn, np.zeros_like(qp)))),
    # scale by 1/sqrt(128) instead of 1/sqrt(192)
    "wrong_scale": ("scores", lambda orig: (lambda q, k, s: orig(q, k, 128 ** -0.5))),
    # heads and features split in the wrong order after the up-projection
    "head_split_transposed": ("up_project", lambda orig: (
        lambda c, w: _bad_split(c, w))),
    # softmax with the sign of the logits flipped
    "softmax_sign": ("softmax_rows", lambda orig: (lambda s: orig(-s))),
    # mixing weights transposed over heads
    "mix_wrong_head": ("mix_values", lambda orig: (
        lambda a, v: np.einsum("ht,thd->hd", a, v[:, ::-1, :]))),
    # causal bound off by one (query cannot see itself)
    "causal_off_by_one": ("index_mask", lambda orig: (
        lambda T, idx, lim=None: orig(T, idx, None if lim is None else lim - 1))),
    # batched decode pairs row b's queries with the next row's cache and index list
    "decode_row_pairing": ("decode", lambda orig: (
        lambda inp, rows=None, gather=True, scale=SCALE: orig(
            dict(inp, kv_cache=np.roll(inp["kv_cache"], 1, axis=0),
                 pe_cache=np.roll(inp["pe_cache"], 1, axis=0),
                 topk_idx=np.roll(inp["topk_idx"], 1, axis=0)), rows=rows, gather=gather,
            scale=scale))),
    # batched decode ignores the caller's scale
    "decode_drops_scale": ("decode", lambda orig: (
        lambda inp, rows=None, gather=True, scale=SCALE: orig(inp, rows=rows, gather=gather))),
    # batched decode ignores the requested rows and returns every batch row
    "decode_ignores_rows": ("decode", lambda orig: (
        lambda inp, rows=None, gather=True, scale=SCALE: orig(inp, gather=gather, scale=scale))),
}


def _bad_split(c, w):
    kv = c @ w.T
    kv = kv.reshape(c.shape[0], DN + DV, H).transpose(0, 2, 1)
    return kv[..., :DN], kv[..., DN:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, make = MUTATIONS[name]
    orig = getattr(om, attr)
    monkeypatch.setattr(om, attr, make(orig))
    failed = _pins_all_pass(stop_at_first=True)
    assert failed, f"mutation {name} slipped past every pin"


def test_pins_pass_without_mutation():
    assert _pins_all_pass() == []
