"""The seeded input generators: determinism, index structure, bf16 rounding."""
import numpy as np

import synth
from synth.generators import DecodeConfig, PrefillConfig


def test_bf16_round_to_nearest_even():
    # exact halfway cases round to the even neighbour, others to nearest
    # 1.0, halfway below even, halfway above odd, just past halfway, -2.5, large, subnormal
    vals = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0xC0200000, 0x7F61B1E6,
                     0x000116C2], dtype=np.uint32).view(np.float32)
    got = synth.bf16_round_bits(vals)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F62, 0x0001], dtype=np.uint16)
    assert np.array_equal(got, want)
    nan = synth.bf16_round_bits(np.array([np.nan], dtype=np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def test_decode_generation_is_deterministic_and_row_addressable():
    cfg = DecodeConfig(99, "t", B=3, T=300, k=50, dtype="bf16")
    a = synth.decode_inputs(cfg, seed=7)
    b = synth.decode_inputs(cfg, seed=7)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    kv1, pe1 = synth.decode_batch_row(cfg, 1, seed=7)
    assert np.array_equal(kv1, a["kv_cache"][1]) and np.array_equal(pe1, a["pe_cache"][1])
    c = synth.decode_inputs(cfg, seed=8)
    assert not np.array_equal(a["q_nope"], c["q_nope"])
    assert a["kv_cache"].dtype == np.uint16 and a["topk_idx"].dtype == np.int32


def test_decode_indices_structure():
    cfg = DecodeConfig(98, "t", B=4, T=1000, k=64, dtype="bf16")
    inp = synth.decode_inputs(cfg, seed=3, with_cache=False)
    for row in inp["topk_idx"]:
        assert row.shape == (64,)
        assert np.all(np.diff(row) > 0)            # sorted, distinct
        assert row[-1] == cfg.T - 1                # newest position always kept
        assert row[0] >= 0 and row[-1] < cfg.T
    dense = DecodeConfig(97, "d", B=1, T=70, k=70, dtype="f32")
    inp = synth.decode_inputs(dense, seed=3, with_cache=False)
    assert np.array_equal(inp["topk_idx"][0], np.arange(70))


def test_query_sets_differ_but_cache_does_not():
    cfg = DecodeConfig(96, "t", B=2, T=200, k=20, dtype="bf16")
    q0 = synth.decode_query_set(cfg, 0, set_id=0)
    q1 = synth.decode_query_set(cfg, 0, set_id=1)
    assert not np.array_equal(q0[0], q1[0]) and not np.array_equal(q0[2], q1[2])


def test_latent_rows_are_rms_normalised_before_rounding():
    cfg = DecodeConfig(95, "t", B=1, T=64, k=64, dtype="f32")
    kv, _ = synth.decode_batch_row(cfg, 0)
    rms = np.sqrt(np.mean(kv.astype(np.float64) ** 2, axis=1))
    assert np.allclose(rms, 1.0, atol=1e-5)


def test_weight_scale():
    cfg = DecodeConfig(94, "t", B=1, T=8, k=8, dtype="f32")
    w_uk, w_uv = synth.weights(cfg)
    assert w_uk.shape == (128, 128, 512) and w_uv.shape == (128, 128, 512)
    assert abs(np.var(w_uk) * 512 - 1.0) < 0.01 and abs(np.var(w_uv) * 512 - 1.0) < 0.01


def test_prefill_indices_structure():
    cfg = PrefillConfig(93, "p", S=40, T=40, k=16, start_pos=0, dtype="bf16")
    qn, qp, idx = synth.prefill_query_rows(cfg, range(cfg.S))
    assert idx.shape == (40, 16)
    for t, row in enumerate(idx):
        n = min(t + 1, 16)
        valid = row[row >= 0]
        assert valid.size == n and np.all(row[n:] == -1)
        assert np.all(np.diff(valid) > 0) and valid[-1] == t and valid.max() <= t
        if t + 1 <= 16:
            assert np.array_equal(valid, np.arange(t + 1))
    one = synth.prefill_query_rows(cfg, [25])
    assert np.array_equal(one[2][0], idx[25]) and np.array_equal(one[0][0], qn[25])


def test_named_configs_match_stated_shapes():
    c = synth.CONFIGS
    assert (c["tiny_dense_f32"].B, c["tiny_dense_f32"].T, c["tiny_dense_f32"].k) == (1, 64, 64)
    assert (c["page_dense_bf16"].T, c["page_dense_bf16"].k) == (1001, 1001)
    assert (c["sparse_b32_t8k"].B, c["sparse_b32_t8k"].T, c["sparse_b32_t8k"].k) == (32, 8192, 2048)
    assert (c["sparse_b64_t32k"].B, c["sparse_b64_t32k"].T, c["sparse_b64_t32k"].k) == (64, 32768, 2048)
    p = c["prefill_s4096"]
    assert (p.S, p.T, p.k, p.start_pos) == (4096, 4096, 2048, 0)
    assert sum(p.valid_count(s) for s in range(p.S)) == 6292480


def test_fp8_wkv_b_inputs():
    d = synth.fp8_wkv_b_inputs()
    c, s = d["codes"], d["scales"]
    assert c.shape == (128 * 256, 512) and c.dtype == np.uint8
    assert s.shape == (256, 4) and s.dtype == np.float32
    assert not np.any((c == 0x7F) | (c == 0xFF))            # no NaN codes
    assert len(np.unique(c)) == 254
    assert np.all((s >= 2.0 ** -14) & (s <= 2.0 ** -4))
    assert np.array_equal(synth.fp8_wkv_b_inputs()["codes"], c)   # seeded
