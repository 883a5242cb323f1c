"""Pins of the oracle's FP8 wkv_b dequantisation.

The pages fix what is done (the decode branch dequantises wkv_b once when it
carries a scale, then views it [heads, 256, 512] and splits each head into
W_UK and W_UV) but not the FP8 format; the oracle reads it as OCP E4M3 codes
with one scale per 128 x 128 block.  Independent references: torch's own
float8_e4m3fn conversion of every code (a library routine), the format's
defining values (largest normal 448, smallest normal 2^-6, smallest
subnormal 2^-9, NaN codes, signed zero), and closed forms that fix the block
indexing and the per-head split.
"""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as om

H, DN, DV, C = 128, 128, 128, 512


def all_codes():
    return np.arange(256, dtype=np.uint8)


def test_F1_every_code_matches_library_conversion():
    got = om.fp8_e4m3_decode(all_codes())
    ref = torch.from_numpy(all_codes()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))   # -0.0 for 0x80


def test_F2_defining_values():
    d = om.fp8_e4m3_decode
    assert d([0x38])[0] == 1.0
    assert d([0x7E])[0] == 448.0 and d([0xFE])[0] == -448.0       # largest normal
    assert d([0x08])[0] == 2.0 ** -6                               # smallest normal
    assert d([0x01])[0] == 2.0 ** -9                               # smallest subnormal
    assert d([0x07])[0] == 7 * 2.0 ** -9                           # largest subnormal
    assert d([0x00])[0] == 0.0 and np.signbit(d([0x80])[0])
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])       # the only NaN codes
    assert np.count_nonzero(np.isnan(d(all_codes()))) == 2          # no infinities either
    assert np.all(np.isfinite(d(all_codes())[[i for i in range(256) if i not in (0x7F, 0xFF)]]))
    # 16 values per binade: consecutive normal codes step by 2^(e - 10)
    v = d(np.arange(0x08, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_B1_one_scale_per_block():
    R, Cc = 300, 260                                   # ragged: 3 x 3 blocks, partial last ones
    codes = np.full((R, Cc), 0x38, np.uint8)           # every value 1.0
    scales = np.exp2(np.arange(9, dtype=np.float64)).reshape(3, 3)
    w = om.fp8_block_dequant(codes, scales)
    for i in range(3):
        for j in range(3):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            assert np.all(blk == scales[i, j]), (i, j)
    scales2 = scales.copy()
    scales2[1, 2] = 1000.0                             # one block's scale changes one block
    diff = om.fp8_block_dequant(codes, scales2) != w
    assert diff[128:256, 256:].all() and np.count_nonzero(diff) == 128 * (Cc - 256)


def test_S1_per_head_split():
    codes = np.zeros((H * (DN + DV), C), np.uint8)
    codes[3 * 256 + 130, 7] = 0x38                     # head 3, stacked row 130 -> W_UV row 2
    codes[5 * 256 + 4, 9] = 0x40                       # head 5, stacked row 4 -> W_UK row 4 (2.0)
    scales = np.ones((H * 256 // 128, C // 128))
    w_uk, w_uv = om.wkv_b_dequant(codes, scales)
    assert w_uk.shape == (H, DN, C) and w_uv.shape == (H, DV, C)
    assert w_uv[3, 2, 7] == 1.0 and np.count_nonzero(w_uv) == 1
    assert w_uk[5, 4, 9] == 2.0 and np.count_nonzero(w_uk) == 1


def _bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 0x7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 11.0))
    return np.where(c & 0x80, -v, v)


def _subnormal_as_normal(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 0x7
    v = (8 + m) * np.exp2(e - 10.0)
    v = np.where(c & 0x80, -v, v)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _nan_as_number(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 0x7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    return np.where(c & 0x80, -v, v)


_orig_decode = om.fp8_e4m3_decode
_orig_block = om.fp8_block_dequant

MUTATIONS = {
    "exponent_bias_8": ("fp8_e4m3_decode", _bias8),
    "subnormals_as_normals": ("fp8_e4m3_decode", _subnormal_as_normal),
    "nan_code_as_480": ("fp8_e4m3_decode", _nan_as_number),
    # scales indexed [col block][row block]
    "scales_transposed": ("fp8_block_dequant", lambda codes, scales, block=128: _orig_block(
        codes, np.asarray(scales).T.reshape(np.asarray(scales).shape), block)),
    # W_UV taken from the first half of each head
    "halves_swapped": ("wkv_b_dequant", lambda codes, scales: tuple(reversed(
        _orig_block(codes, scales).reshape(H, 256, C).reshape(H, 2, 128, C).transpose(1, 0, 2, 3)))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(om, attr, fn)
    failed = 0
    for t in (test_F1_every_code_matches_library_conversion, test_F2_defining_values,
              test_B1_one_scale_per_block, test_S1_per_head_split):
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed, name
