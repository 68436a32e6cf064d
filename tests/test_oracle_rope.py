"""Pins of the oracle's inverse rotary embedding with per-head FP8
quantisation (oracle/rope.py).

Compared with: a hand-worked example (tests/golden/inv_rope_hand.json); the
same rotation written as complex multiplication in float64 (z * e^(-i theta));
the forward rotary embedding written independently, which the inverse must
undo; the two pair layouts, which differ only by a permutation of features;
pass-through of the features beyond R; and the pinned per-row FP8 quantiser,
which the per-head codes must equal for unrotated rows.
"""

import json
import os

import numpy as np
import pytest
import torch

from moe_layer_05_amd import workloads
from oracle import fp8, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "inv_rope_hand.json")


def test_hand_example():
    g = json.load(open(GOLDEN))
    x = np.array(g["x"], np.float32)
    pos = np.array(g["positions"])
    for case in g["cases"]:
        R = case["R"]
        table = np.array(g["cos_sin_R%d" % R], np.float32)
        y = rope.inv_rope(x, pos, table, R, case["interleaved"])
        assert np.array_equal(y, np.array(case["rotated"], np.float32)), case
        codes, scales = rope.inv_rope_fp8_quant_per_head(x, pos, table, R, case["interleaved"])
        assert np.array_equal(codes, np.array(case["codes"], np.uint8)), case
        assert np.array_equal(scales, np.array(case["scales"], np.float32)), case


def _case(T=6, NH=3, D=32, R=32, seed=0, max_pos=1000):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, NH, D)).astype(np.float32)
    pos = rng.integers(0, max_pos, T)
    table = workloads.rope_table(max_pos, R).numpy()
    return x, pos, table


def _angles(pos, R, base=10000.0):
    i = np.arange(R // 2)
    return np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * i / R)[None, :]


@pytest.mark.parametrize("interleaved", [False, True])
def test_equals_complex_rotation(interleaved):
    """Pairs as complex numbers z = x1 + i x2: the inverse embedding is
    z * e^(-i theta) (float64), which the float32 oracle matches within its
    rounding (a few ulp of |z|)."""
    T, NH, D, R = 7, 4, 64, 48
    x, pos, table = _case(T, NH, D, R)
    y = rope.inv_rope(x, pos, table, R, interleaved).astype(np.float64)
    f, s = rope.pair_index(D, R, interleaved)
    z = x[:, :, f].astype(np.float64) + 1j * x[:, :, s].astype(np.float64)
    ang = _angles(pos, R)[:, None, :]
    want = z * np.exp(-1j * ang)
    got = y[:, :, f] + 1j * y[:, :, s]
    # the table entries are float32 roundings of cos / sin (2^-24 relative)
    # and each product and sum rounds once: within 2^-21 of |z|
    assert (np.abs(got - want) <= 2.0 ** -21 * np.abs(z) + 1e-30).all()
    assert np.array_equal(y[:, :, R:] if not interleaved else y[:, :, R:], x[:, :, R:])


def _forward_rope(x, pos, R, interleaved):
    """The rotary embedding itself, by the angle +theta (float64), written
    without the oracle: x1' = x1 cos - x2 sin, x2' = x2 cos + x1 sin."""
    x = np.asarray(x, np.float64)
    out = x.copy()
    ang = _angles(pos, R)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    if interleaved:
        x1, x2 = x[..., 0:R:2], x[..., 1:R:2]
        out[..., 0:R:2] = x1 * c - x2 * s
        out[..., 1:R:2] = x2 * c + x1 * s
    else:
        h = R // 2
        x1, x2 = x[..., :h], x[..., h:R]
        out[..., :h] = x1 * c - x2 * s
        out[..., h:R] = x2 * c + x1 * s
    return out


@pytest.mark.parametrize("interleaved", [False, True])
def test_undoes_the_rotary_embedding(interleaved):
    T, NH, D, R = 5, 2, 32, 32
    x, pos, table = _case(T, NH, D, R, seed=3)
    rotated = _forward_rope(x, pos, R, interleaved).astype(np.float32)
    back = rope.inv_rope(rotated, pos, table, R, interleaved)
    assert np.abs(back - x).max() <= 2.0 ** -20 * np.abs(x).max()


def test_layouts_differ_by_a_feature_permutation():
    """Interleaved pairs (2i, 2i+1) on x equal half-layout pairs (i, i + R/2)
    on x with its rotated features reordered, then reordered back."""
    T, NH, D, R = 4, 2, 40, 32
    x, pos, table = _case(T, NH, D, R, seed=5)
    perm = np.concatenate([np.arange(0, R, 2), np.arange(1, R, 2), np.arange(R, D)])
    y_int = rope.inv_rope(x, pos, table, R, interleaved=True)
    y_half = rope.inv_rope(x[:, :, perm], pos, table, R, interleaved=False)
    inv = np.argsort(perm)
    assert np.array_equal(y_half[:, :, inv], y_int)


def test_position_zero_is_plain_per_head_quantisation():
    """cos 1, sin 0: the heads pass unchanged, so the codes and scales are the
    row quantiser's on x itself, one row per (token, head)."""
    T, NH, D, R = 3, 5, 64, 64
    x, _, table = _case(T, NH, D, R)
    pos = np.zeros(T, dtype=np.int64)
    assert np.array_equal(rope.inv_rope(x, pos, table, R), x)
    for fmt in ("e4m3", "e5m2"):
        codes, scales = rope.inv_rope_fp8_quant_per_head(x, pos, table, R, fmt=fmt)
        rc, rs = fp8.quantize_rows(x.reshape(T * NH, D), fmt)
        assert np.array_equal(codes.reshape(T * NH, D), rc)
        assert np.array_equal(scales.reshape(-1), rs)


def test_partial_rotary_passes_features_through():
    T, NH, D, R = 4, 2, 96, 32
    x, pos, table = _case(T, NH, D, R, seed=9)
    for inter in (False, True):
        y = rope.inv_rope(x, pos, table, R, inter)
        assert np.array_equal(y[:, :, R:], x[:, :, R:])
        assert not np.array_equal(y[:, :, :R], x[:, :, :R])


def test_rotation_keeps_pair_norms():
    T, NH, D, R = 6, 3, 64, 64
    x, pos, table = _case(T, NH, D, R, seed=11)
    y = rope.inv_rope(x, pos, table, R).astype(np.float64)
    f, s = rope.pair_index(D, R, False)
    n0 = np.hypot(x[:, :, f], x[:, :, s])
    n1 = np.hypot(y[:, :, f], y[:, :, s])
    assert np.abs(n1 - n0).max() <= 2.0 ** -20 * n0.max()


def test_per_head_scale_and_code_bound():
    """Each (token, head) scale is amax / 448 of its rotated row; each code
    times its scale lies within half a grid step (at most 2^-4 relative) of
    the rotated value."""
    T, NH, D, R = 5, 4, 128, 128
    x, pos, table = _case(T, NH, D, R, seed=2)
    y = rope.inv_rope(x, pos, table, R)
    codes, scales = rope.inv_rope_fp8_quant_per_head(x, pos, table, R)
    amax = np.abs(y).max(axis=2).astype(np.float32)
    assert np.array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))
    back = fp8.decode(codes) * scales[:, :, None].astype(np.float64)
    err = np.abs(back - y)
    assert (err <= 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * scales[:, :, None]).all()


def test_rope_table_matches_closed_form():
    t = workloads.rope_table(64, 16).numpy()
    ang = _angles(np.arange(64), 16)
    assert np.array_equal(t[:, :8], np.cos(ang).astype(np.float32))
    assert np.array_equal(t[:, 8:], np.sin(ang).astype(np.float32))
    assert (t[0, :8] == 1).all() and (t[0, 8:] == 0).all()


def test_heads_generator_positions():
    cfg = workloads.ROPE_CONFIGS["inv_rope_tp8"]
    d = workloads.make_heads(cfg, 8)
    assert d["x"].shape == (8, cfg.NH, cfg.D) and d["x"].dtype == torch.bfloat16
    assert ((d["positions"] >= 0) & (d["positions"] < cfg.max_pos)).all()
    p = workloads.make_heads(cfg, 100)["positions"]
    assert torch.equal(p, torch.arange(100))
