"""Pins for oracle.project (the QKV projection, rotary embedding, block means and int8 codes its
epilogue emits) against facts fixed outside it: explicit loops for the product, the rotation as a
complex multiplication and hand-worked angles, the generator's independent quantiser and hand-worked
codes, and exact bf16 rounding cases."""
import math

import numpy as np
import pytest
import torch

import gen
from oracle import project as op


def test_product_and_head_split_by_loops():
    rng = np.random.default_rng(0)
    S, D, d, Hq, Hkv = 4, 3, 4, 2, 1
    X = np.round(rng.standard_normal((S, D)) * 4) / 4          # exactly representable in bf16
    W = np.round(rng.standard_normal(((Hq + 2 * Hkv) * d, D)) * 4) / 4
    out = op.project(X, W, Hq, Hkv, b=2, d=d)
    for name, h0, nh in (("q", 0, Hq), ("k", Hq, Hkv), ("v", Hq + Hkv, Hkv)):
        for h in range(nh):
            for t in range(S):
                for c in range(d):
                    y = sum(X[t, k] * W[(h0 + h) * d + c, k] for k in range(D))
                    assert out[name][h, t, c] == op.bf16_round(np.array([y]))[0]
    # block means over b = 2 tokens
    np.testing.assert_array_equal(out["qbar"][1, 1], (out["q"][1, 2] + out["q"][1, 3]) / 2)


def test_rope_is_a_complex_rotation():
    rng = np.random.default_rng(1)
    S, d = 5, 8
    x = rng.standard_normal((S, d))
    ang = rng.uniform(-3, 3, (S, d // 2))
    y = op.rope(x, np.cos(ang), np.sin(ang))
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, : d // 2], z.real, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y[:, d // 2:], z.imag, rtol=1e-14, atol=1e-14)
    # a quarter turn maps (1, 0) to (0, 1); a zero angle is the identity
    q = op.rope(np.array([[1.0, 0.0, 0.0, 0.0]]), np.array([[0.0, 1.0]]), np.array([[1.0, 0.0]]))
    np.testing.assert_allclose(q, [[0.0, 0.0, 1.0, 0.0]], atol=0)
    np.testing.assert_array_equal(op.rope(x, np.ones((S, d // 2)), np.zeros((S, d // 2))), x)


def test_rope_tables_follow_the_base():
    cos, sin = gen.rope_tables(7, 128, 500000.0)
    t, c = 5, 3
    theta = t * 500000.0 ** (-2.0 * c / 128)
    assert abs(cos[t, c] - math.cos(theta)) < 1e-7 and abs(sin[t, c] - math.sin(theta)) < 1e-7
    assert cos.shape == (7, 64) and np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


def test_quantize_by_hand_and_against_the_generator():
    codes, s = op.quantize(np.array([[127.0, -63.5, 0.5, 1.5], [0.0, 0.0, 0.0, 0.0], [2.54, -1.27, 0.0, 0.01]]))
    assert s[0] == 1.0 and codes[0].tolist() == [127, -64, 0, 2]            # halves to even
    assert s[1] == 1.0 and codes[1].tolist() == [0, 0, 0, 0]
    assert s[2] == np.float32(np.float32(2.54) / np.float32(127.0)) and codes[2].tolist() == [127, -64, 0, 0]
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((300, 128)) * rng.uniform(0.1, 10, (300, 1))).astype(np.float32)
    c1, s1 = op.quantize(x)
    c2, s2 = gen.quantize_rows(x)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


def test_bf16_round_ties_to_even():
    one = 1.0
    vals = np.array([one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -20, -(one + 2.0 ** -8)])
    got = op.bf16_round(vals)
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0])


def test_projection_of_planted_values_is_the_identity_without_rotation():
    """W = [I; I; I] per head and X = the values: the projection returns X rounded, its block means
    and its codes."""
    rng = np.random.default_rng(3)
    S, d = 8, 4
    X = rng.standard_normal((S, d))
    W = np.concatenate([np.eye(d)] * 3)
    out = op.project(X, W, 1, 1, b=4, d=d)
    for name in ("q", "k", "v"):
        np.testing.assert_array_equal(out[name][0], op.bf16_round(X))
    np.testing.assert_allclose(out["kbar"][0], op.bf16_round(X).reshape(2, 4, d).mean(axis=1), rtol=0, atol=1e-15)
