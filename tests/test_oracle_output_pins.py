"""Pins of the oracle's output projection Delta = o W_O.

Independent references: the parameter count the page prints for W_O
(tests/golden/page_shapes.json), torch's CPU linear layer in float64 (the
model applies W_O as a linear layer to the flattened head outputs), and
closed forms that fix the head-major flattening and the [out, in] storage.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as om

H, DV, DM = 128, 128, 7168
N = 96          # output rows used in the value pins (the projection treats every row alike)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_W1_shapes_match_the_page(repo_root):
    g = json.load(open(os.path.join(repo_root, "tests", "golden", "page_shapes.json")))
    assert H * DV * om.D_MODEL == g["output_projection_params"]["value"]
    assert om.D_MODEL == g["model_width"]["value"]


def test_W2_matches_library_linear_layer():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((3, H, DV))
    w = rng.standard_normal((N, H * DV)) / 128
    ref = torch.nn.functional.linear(torch.from_numpy(o).flatten(1), torch.from_numpy(w)).numpy()
    assert rel(om.output_projection(o, w), ref) <= 1e-12


def test_W3_head_major_flattening_and_storage():
    # o nonzero only at (head 5, value 17): every output n is w_o[n, 5 * 128 + 17]
    rng = np.random.default_rng(2)
    w = rng.standard_normal((N, H * DV))
    o = np.zeros((1, H, DV))
    o[0, 5, 17] = 2.0
    assert np.array_equal(om.output_projection(o, w)[0], 2.0 * w[:, 5 * DV + 17])
    # w_o with a single nonzero column picks one input feature for one output
    w1 = np.zeros((N, H * DV))
    w1[70, 3 * DV + 4] = 1.0
    o = rng.standard_normal((2, H, DV))
    out = om.output_projection(o, w1)
    assert np.array_equal(out[:, 70], o[:, 3, 4]) and np.count_nonzero(out) == 2


MUTATIONS = {
    # value-major flattening instead of head-major
    "flatten_value_major": lambda o, w: om.to_f64(o).transpose(0, 2, 1).reshape(o.shape[0], -1) @ om.to_f64(w).T,
    # the [out, in] storage read as [in, out]
    "storage_read_as_in_out": lambda o, w: om.to_f64(o).reshape(o.shape[0], -1) @ om.to_f64(w).reshape(
        H * DV, -1),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_projection_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(om, "output_projection", MUTATIONS[name])
    failed = 0
    for fn in (test_W2_matches_library_linear_layer, test_W3_head_major_flattening_and_storage):
        try:
            fn()
        except AssertionError:
            failed += 1
    assert failed, name
