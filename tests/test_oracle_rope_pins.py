"""Pins of the oracle's partial RoPE and mixed-precision entry store.

Each check is independent of the oracle's own arithmetic: a complex-number
formulation of the rotation, the rotation group laws, hand-computed values,
the relative-position property of rotary encodings, and the encoders'
definitions ("Ch 05 · HCA — 长上下文的全景镜", section on partial RoPE;
"混合压缩注意力双方案解析：CSA与HCA技术对比与选型指南", section 3).
"""

import numpy as np
import pytest
import torch

import oracle


def _complex_rope(X, pos, r, base=10000.0):
    """Rotation as multiplication of x_j + i x_{j+1} by e^{i pos theta_k}."""
    X = np.asarray(X, dtype=np.float64)
    c = X.shape[1]
    z = X[:, c - r::2] + 1j * X[:, c - r + 1::2]
    theta = base ** (-np.arange(r // 2) * 2.0 / r)
    z = z * np.exp(1j * np.outer(pos, theta))
    out = X.copy()
    out[:, c - r::2] = z.real
    out[:, c - r + 1::2] = z.imag
    return out


def _data(E=7, c=32, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((E, c)), rng.uniform(0, 70000, E)


def test_rope_equals_complex_multiplication():
    X, pos = _data()
    for r in (4, 16, 32):
        np.testing.assert_allclose(oracle.rope_partial(X, pos, r), _complex_rope(X, pos, r), rtol=0, atol=1e-12)
    # a different base too
    np.testing.assert_allclose(oracle.rope_partial(X, pos, 8, base=500.0), _complex_rope(X, pos, 8, base=500.0),
                               rtol=0, atol=1e-12)


def test_rope_leaves_position_free_dims_and_norms():
    X, pos = _data()
    Y = oracle.rope_partial(X, pos, 16)
    assert np.array_equal(Y[:, :16], X[:, :16])
    n0 = X[:, 16::2] ** 2 + X[:, 17::2] ** 2
    n1 = Y[:, 16::2] ** 2 + Y[:, 17::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    assert np.array_equal(oracle.rope_partial(X, np.zeros(len(X)), 16), X)      # position 0 is the identity


def test_rope_group_laws_and_relative_positions():
    X, pos = _data()
    p2 = np.linspace(-50, 3000, len(X))
    np.testing.assert_allclose(oracle.rope_partial(oracle.rope_partial(X, pos, 16), p2, 16),
                               oracle.rope_partial(X, pos + p2, 16), atol=1e-9)
    # q . k after rotation depends only on the position difference
    q, k = X[:1], X[1:2]
    for shift in (0.0, 17.5, 12345.0):
        dq = oracle.rope_partial(q, [300.0 + shift], 32)
        dk = oracle.rope_partial(k, [120.5 + shift], 32)
        if shift == 0.0:
            ref = float((dq @ dk.T)[0, 0])
        assert abs(float((dq @ dk.T)[0, 0]) - ref) < 1e-9


def test_rope_hand_values():
    # r = 4 on c = 4: theta_0 = 1, theta_1 = 10000^(-1/2) = 0.01
    X = np.array([[1.0, 0.0, 1.0, 0.0]])
    Y = oracle.rope_partial(X, [np.pi / 2], 4)
    np.testing.assert_allclose(Y, [[0.0, 1.0, np.cos(np.pi / 200), np.sin(np.pi / 200)]], atol=1e-15)


def test_entry_positions_are_block_centres():
    assert np.array_equal(oracle.entry_positions([0, 10, 18], 4), [1.5, 5.5, 1.5, 5.5])
    assert np.array_equal(oracle.entry_positions([0, 10, 18], 4, [100, 7]), [101.5, 105.5, 8.5, 12.5])
    assert np.array_equal(oracle.entry_positions([0, 300], 128), [63.5, 191.5])
    assert oracle.entry_positions([0, 3, 3], 4).size == 0


def test_mixed_store_parts():
    X, pos = _data(E=9, c=64, seed=3)
    codes, scales, rope = oracle.rope_mixed_store(X, pos, 16)
    assert codes.shape == (9, 48) and codes.dtype == np.uint8 and rope.shape == (9, 16)
    # position-free part: per-entry scale over its 48 dims, decode within one E4M3 step
    amax = np.abs(X[:, :48]).max(axis=1)
    np.testing.assert_allclose(scales, amax / 448.0, rtol=1e-15)
    dec = oracle.fp8_e4m3_decode(codes) * scales[:, None]
    rel = np.abs(dec - X[:, :48]) / np.abs(X[:, :48])
    assert np.all(rel <= 2.0 ** -4 + 1e-12)               # half an E4M3 step (2^-3) at any normal magnitude
    # rotated part: torch's bf16 rounding of the complex-number rotation
    want = torch.from_numpy(_complex_rope(X, pos, 16)[:, 48:]).to(torch.bfloat16).double().numpy()
    assert np.array_equal(rope, want)


@pytest.mark.parametrize("mutant", ["sign", "half_split", "freq"])
def test_planted_rope_mistakes_are_caught(mutant):
    X, pos = _data(c=16)
    r = 16

    def bad(X, pos):
        X = np.array(X, dtype=np.float64, copy=True)
        for k in range(r // 2):
            if mutant == "half_split":               # pairs (k, k + r/2) instead of adjacent dims
                j0, j1 = k, k + r // 2
            else:
                j0, j1 = 2 * k, 2 * k + 1
            th = 10000.0 ** (-2.0 * k / r) if mutant != "freq" else 10000.0 ** (-1.0 * k / r)
            a = pos * th
            x, y = X[:, j0].copy(), X[:, j1].copy()
            s = -1.0 if mutant == "sign" else 1.0
            X[:, j0] = x * np.cos(a) - s * y * np.sin(a)
            X[:, j1] = s * x * np.sin(a) + y * np.cos(a)
        return X

    assert not np.allclose(bad(X, pos), _complex_rope(X, pos, r), atol=1e-6)
