"""Pins of the oracle's cache append (latent RMSNorm, rotary key, cache write).

The independent references are torch's CPU routines in float64 (rms_norm, and
complex multiplication through view_as_complex, which is how the pages'
rotary function is written), closed forms of the two operations and the
layout facts the pages fix: the joint down-projection's 576 outputs are the
512-wide latent then the 64-wide rotary key, and the key path rotates
interleaved feature pairs.  Planted mistakes at the end show that each pin
bites.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_oracle as om

DL, DR = 512, 64


def rand_append(B=2, S=5, T=12, seed=0):
    rng = np.random.default_rng(seed)
    return dict(kv_a_out=rng.standard_normal((B, S, DL + DR)) * 3.0,
                norm_weight=rng.standard_normal(DL),
                cos_sin=_angles(rng.uniform(-np.pi, np.pi, (S, DR // 2))),
                kv_cache=rng.standard_normal((B, T, DL)),
                pe_cache=rng.standard_normal((B, T, DR)))


def _angles(theta):
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- RMSNorm
def test_R1_rms_norm_matches_library_routine():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((7, DL)) * 5, rng.standard_normal(DL)
    for eps in (0.0, 1e-6, 0.5):
        ref = F.rms_norm(torch.from_numpy(x), (DL,), torch.from_numpy(w), eps).numpy()
        assert rel(om.rms_norm(x, w, eps), ref) <= 1e-13


def test_R2_rms_norm_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, DL)) * 7
    one = np.ones(DL)
    y = om.rms_norm(x, one, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-13)   # unit RMS
    assert rel(om.rms_norm(x * 123.0, one, 0.0), y) <= 1e-14                        # scale invariant
    w = rng.standard_normal(DL)
    assert rel(om.rms_norm(x, w, 0.0), y * w) <= 1e-14                              # gains elementwise
    # eps adds to the mean square: a row of constant c maps to c / sqrt(c^2 + eps)
    c, eps = 0.3, 0.07
    assert rel(om.rms_norm(np.full((1, DL), c), one, eps), np.full((1, DL), c / np.sqrt(c * c + eps))) <= 1e-14


# ---------------------------------------------------------------- rotary key
def test_P1_rotary_matches_complex_multiplication():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 6, DR))
    cs = _angles(rng.uniform(-4, 4, (6, DR // 2)))
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(3, 6, DR // 2, 2).contiguous())
    f = torch.polar(torch.ones(6, DR // 2, dtype=torch.float64),
                    torch.from_numpy(np.arctan2(cs[..., 1], cs[..., 0])))
    ref = torch.view_as_real(xc * f).flatten(2).numpy()
    assert rel(om.rotate_pairs(x, cs), ref) <= 1e-14


def test_P2_rotary_closed_forms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, DR))
    pair_norm = lambda v: np.hypot(v[..., 0::2], v[..., 1::2])                      # noqa: E731
    th = rng.uniform(-3, 3, DR // 2)
    y = om.rotate_pairs(x, _angles(th))
    assert rel(pair_norm(y), pair_norm(x)) <= 1e-14                                 # rotations keep length
    assert np.array_equal(om.rotate_pairs(x, _angles(np.zeros(DR // 2))), x)        # angle 0
    th2 = rng.uniform(-3, 3, DR // 2)
    assert rel(om.rotate_pairs(y, _angles(th2)), om.rotate_pairs(x, _angles(th + th2))) <= 1e-13
    # a quarter turn maps each pair (a, b) to (-b, a); features 2i and 2i+1 form pair i
    q = om.rotate_pairs(x, _angles(np.full(DR // 2, np.pi / 2)))
    assert np.allclose(q[..., 0::2], -x[..., 1::2], atol=1e-15)
    assert np.allclose(q[..., 1::2], x[..., 0::2], atol=1e-15)
    e = np.zeros(DR)
    e[6] = 1.0                                                                      # pair 3, real part
    q = om.rotate_pairs(e, _angles(np.full(DR // 2, np.pi / 2)))
    assert abs(q[7] - 1.0) < 1e-15 and np.count_nonzero(np.abs(q) > 1e-15) == 1


# ---------------------------------------------------------------- the write
def test_A1_append_writes_only_its_rows():
    inp = rand_append(B=2, S=5, T=12)
    start, eps = 4, 1e-6
    kv, pe = om.cache_append(inp["kv_a_out"], inp["norm_weight"], inp["cos_sin"], inp["kv_cache"],
                             inp["pe_cache"], start, eps)
    keep = np.r_[0:start, start + 5:12]
    assert np.array_equal(kv[:, keep], inp["kv_cache"][:, keep])
    assert np.array_equal(pe[:, keep], inp["pe_cache"][:, keep])
    a = inp["kv_a_out"]
    ref_kv = F.rms_norm(torch.from_numpy(a[..., :DL]), (DL,), torch.from_numpy(inp["norm_weight"]), eps).numpy()
    assert rel(kv[:, start:start + 5], ref_kv) <= 1e-13
    xc = torch.view_as_complex(torch.from_numpy(a[..., DL:]).reshape(2, 5, DR // 2, 2).contiguous())
    f = torch.polar(torch.ones(5, DR // 2, dtype=torch.float64),
                    torch.from_numpy(np.arctan2(inp["cos_sin"][..., 1], inp["cos_sin"][..., 0])))
    assert rel(pe[:, start:start + 5], torch.view_as_real(xc * f[None]).flatten(2).numpy()) <= 1e-13


def test_A2_latent_first_rotary_last():
    # a position whose down-projection output is nonzero only in its last 64 features gets a
    # zero latent row and a rotated rotary row
    inp = rand_append(B=1, S=1, T=3)
    a = np.zeros((1, 1, DL + DR))
    a[0, 0, DL:] = np.arange(1, DR + 1)
    kv, pe = om.cache_append(a, inp["norm_weight"], inp["cos_sin"], inp["kv_cache"], inp["pe_cache"], 1, 1e-6)
    assert np.array_equal(kv[0, 1], np.zeros(DL))
    assert np.count_nonzero(pe[0, 1]) == DR


# ---------------------------------------------------------------- mutations
def _pins():
    failed = []
    for name, fn in [("R1", test_R1_rms_norm_matches_library_routine), ("R2", test_R2_rms_norm_closed_forms),
                     ("P1", test_P1_rotary_matches_complex_multiplication), ("P2", test_P2_rotary_closed_forms),
                     ("A1", test_A1_append_writes_only_its_rows), ("A2", test_A2_latent_first_rotary_last)]:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def _non_interleaved(x, cs):
    x = om.to_f64(x)
    h = x.shape[-1] // 2
    re, im = x[..., :h], x[..., h:]
    c, s = om.to_f64(cs)[..., 0], om.to_f64(cs)[..., 1]
    return np.concatenate([re * c - im * s, re * s + im * c], axis=-1)


MUTATIONS = {
    # pairs taken as (x[i], x[i + 32]) instead of (x[2i], x[2i+1])
    "rotary_not_interleaved": ("rotate_pairs", lambda orig: _non_interleaved),
    # rotation by -theta
    "rotary_wrong_sign": ("rotate_pairs", lambda orig: (
        lambda x, cs: orig(x, np.stack([om.to_f64(cs)[..., 0], -om.to_f64(cs)[..., 1]], axis=-1)))),
    # the learned gains dropped
    "norm_without_gains": ("rms_norm", lambda orig: (lambda x, w, eps: orig(x, np.ones_like(om.to_f64(w)), eps))),
    # epsilon added outside the square root
    "norm_eps_outside_sqrt": ("rms_norm", lambda orig: (
        lambda x, w, eps: om.to_f64(x) / (np.sqrt(np.mean(om.to_f64(x) ** 2, axis=-1, keepdims=True)) + eps)
        * om.to_f64(w))),
    # split taken with the rotary key first
    "split_rotary_first": ("cache_append", lambda orig: (
        lambda a, w, cs, kv, pe, sp, eps: orig(np.concatenate([om.to_f64(a)[..., DR:], om.to_f64(a)[..., :DR]], -1),
                                               w, cs, kv, pe, sp, eps))),
    # written one row late
    "append_off_by_one": ("cache_append", lambda orig: (
        lambda a, w, cs, kv, pe, sp, eps: orig(a, w, cs, kv, pe, sp + 1, eps))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_append_mistake_is_caught(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(om, attr, make(getattr(om, attr)))
    assert _pins(), f"mutation {name} slipped past every pin"


def test_append_pins_pass_without_mutation():
    assert _pins() == []
