"""Pins of the QK-Norm / RoPE oracle (CPU only): closed forms, a second formulation of the rotation with
complex numbers, the invariants a rotary embedding must have, and planted mistakes that each fail one of
them."""

import math

import numpy as np
import pytest

import oracle
from oracle.qknorm_rope import rope_angles_ref


# ---------------------------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    w = np.array([0.5, 2.0, -1.0, 3.0])
    # alternating signs of one magnitude: the root mean square is that magnitude
    x = np.array([[1.0, -1.0, 1.0, -1.0]])
    np.testing.assert_allclose(oracle.rms_norm_ref(x, w, 0.0), x * w, rtol=0, atol=1e-15)
    # a constant row of any positive scale normalises to the weight itself
    for t in (1e-3, 1.0, 7.5, 1e4):
        np.testing.assert_allclose(oracle.rms_norm_ref(np.full((1, 4), t), w, 0.0), w[None], rtol=1e-14)
    # eps inside the root: mean square 1 plus eps 3 gives a divisor of exactly 2
    np.testing.assert_allclose(oracle.rms_norm_ref(np.ones((1, 2)), np.ones(2), 3.0), [[0.5, 0.5]], atol=0)
    # an all-zero row stays zero (no division by zero with eps > 0)
    assert np.all(oracle.rms_norm_ref(np.zeros((2, 8)), np.ones(8), 1e-6) == 0)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 16)) * rng.uniform(0.1, 10, size=(5, 3, 1))
    y = oracle.rms_norm_ref(x, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)    # unit mean square
    np.testing.assert_allclose(oracle.rms_norm_ref(4.0 * x, np.ones(16), 0.0), y, rtol=1e-12)  # scale-free
    # each head on its own: normalising heads separately equals normalising the [N, H, hd] array
    for h in range(3):
        np.testing.assert_array_equal(oracle.rms_norm_ref(x[:, h], np.ones(16), 0.0), y[:, h])


# ---------------------------------------------------------------------------------------------- RoPE

def _rope_complex(x, positions, theta):
    """The same rotation written as complex multiplication: z_i = x_i + j x_{i+hd/2} times e^{j angle_i}."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    h = hd // 2
    z = x[..., :h] + 1j * x[..., h:]
    freq = np.array([theta ** (-(2.0 * i) / hd) for i in range(h)])
    rot = np.exp(1j * np.outer(np.asarray(positions, dtype=np.float64), freq))[:, None, :]
    zr = z * rot
    return np.concatenate([zr.real, zr.imag], axis=-1)


def test_rope_closed_forms():
    # position 0 is the identity
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 2, 8))
    np.testing.assert_array_equal(oracle.rope_ref(x, [0, 0, 0], 1e4), x)
    # head_dim 2, position 1: (1, 0) turns by one radian
    y = oracle.rope_ref(np.array([[[1.0, 0.0]]]), [1], 1e6)
    np.testing.assert_allclose(y[0, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    # head_dim 4, theta 10000: the second pair turns 100 times slower (10000^(-1/2) = 0.01)
    ang = rope_angles_ref([100], 4, 1e4)
    np.testing.assert_allclose(ang, [[100.0, 1.0]], rtol=1e-14)
    y = oracle.rope_ref(np.array([[[0.0, 1.0, 0.0, 0.0]]]), [100], 1e4)  # element 1 pairs with element 3
    np.testing.assert_allclose(y[0, 0], [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-14)


def test_rope_matches_complex_formulation():
    rng = np.random.default_rng(2)
    for hd in (2, 8, 128):
        x = rng.standard_normal((6, 3, hd))
        pos = rng.integers(0, 40000, size=6)
        np.testing.assert_allclose(oracle.rope_ref(x, pos, 1e6), _rope_complex(x, pos, 1e6), atol=1e-11)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    hd = 64
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    # rotation: each (i, i + hd/2) pair keeps its length
    y = oracle.rope_ref(q, [1234], 1e6)
    np.testing.assert_allclose(y[..., :32] ** 2 + y[..., 32:] ** 2, q[..., :32] ** 2 + q[..., 32:] ** 2, rtol=1e-12)
    # composition: turning by p1 then by p2 is turning by p1 + p2
    np.testing.assert_allclose(oracle.rope_ref(oracle.rope_ref(q, [300], 1e6), [77], 1e6),
                               oracle.rope_ref(q, [377], 1e6), atol=1e-12)
    # relative positions: <R(p) q, R(p') k> depends on p - p' only
    def dot(p, pk):
        return float(np.sum(oracle.rope_ref(q, [p], 1e6) * oracle.rope_ref(k, [pk], 1e6)))
    base = dot(10, 3)
    for shift in (1, 100, 20000):
        assert dot(10 + shift, 3 + shift) == pytest.approx(base, rel=1e-9, abs=1e-9)


def test_qk_norm_rope_composition():
    """Step 4 then step 5, with v untouched by both; q and k each use their own weight."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 16, 128))
    k = rng.standard_normal((4, 8, 128))
    wq = rng.uniform(0.5, 1.5, 128)
    wk = rng.uniform(0.5, 1.5, 128)
    pos = [0, 5, 6, 4095]
    qo, ko = oracle.qk_norm_rope_ref(q, k, pos, wq, wk, 1e-6, 1e6)
    np.testing.assert_allclose(qo, oracle.rope_ref(oracle.rms_norm_ref(q, wq, 1e-6), pos, 1e6), atol=0)
    np.testing.assert_allclose(ko, oracle.rope_ref(oracle.rms_norm_ref(k, wk, 1e-6), pos, 1e6), atol=0)
    # position 0 rows are the normalised vectors themselves
    np.testing.assert_allclose(qo[0], oracle.rms_norm_ref(q[0], wq, 1e-6), atol=0)


# ---------------------------------------------------------------------------------------------- planted mistakes

def _rope_interleaved(x, positions, theta):  # pairs (2i, 2i+1) instead of (i, i + hd/2)
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    ang = rope_angles_ref(positions, hd, theta)[:, None, :]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_sign_flipped(x, positions, theta):
    return oracle.rope_ref(x, -np.asarray(positions), theta)


def _rope_wrong_freq(x, positions, theta):  # exponent -i/hd
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    h = hd // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None, None] * (float(theta) ** (-np.arange(h) / hd))[None, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * np.cos(ang) - x2 * np.sin(ang), x2 * np.cos(ang) + x1 * np.sin(ang)], axis=-1)


@pytest.mark.parametrize("wrong", [_rope_interleaved, _rope_sign_flipped, _rope_wrong_freq])
def test_planted_rope_mistakes_fail_the_pins(wrong):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 3, 8))
    pos = rng.integers(1, 5000, size=6)
    assert not np.allclose(wrong(x, pos, 1e6), _rope_complex(x, pos, 1e6), atol=1e-6)


def test_planted_rmsnorm_mistakes_fail_the_pins():
    x = np.ones((1, 2))
    w = np.ones(2)
    no_weight = lambda x, w, e: oracle.rms_norm_ref(x, np.ones_like(w), e)
    eps_outside = lambda x, w, e: np.asarray(x) / (np.sqrt(np.mean(np.asarray(x) ** 2, -1, keepdims=True)) + e) * w
    assert not np.allclose(eps_outside(x, w, 3.0), [[0.5, 0.5]])
    wq = np.array([0.5, 2.0, -1.0, 3.0])
    assert not np.allclose(no_weight(np.full((1, 4), 2.0), wq, 0.0), wq[None])
