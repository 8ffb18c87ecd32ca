"""Pins for the oracle's rotary embedding (CPU only).

The pages say only that rotary embeddings are applied to queries and keys ("Show HN:
NanoEuler", section 2; "Tiny Hackable CUDA Language Model Implementation", section 1).  The
reading pinned here: adjacent pairs (2i, 2i+1), theta_i = base^(-2i/D), angle (pos0+t)*theta_i,
inverse = rotation by the negated angle.  Each test below would fail for a plausible mistake:
a wrong sign (rotation direction), wrong pairing, wrong frequency exponent, a dropped pos0.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_unit_rotations.json")


def _rng(seed):
    return np.random.default_rng(seed)


def test_d2_is_complex_multiplication():
    # For D = 2 the single pair has theta = 1: RoPE is multiplication by e^{i (pos0 + t)}.
    x = _rng(1).standard_normal((2, 9, 3, 2))
    for pos0 in (0, 5):
        y = oracle.rope(x, base=10000.0, pos0=pos0)
        z = x[..., 0] + 1j * x[..., 1]
        t = np.arange(9)[None, :, None] + pos0
        w = z * np.exp(1j * t)
        np.testing.assert_allclose(y[..., 0], w.real, rtol=0, atol=1e-14)
        np.testing.assert_allclose(y[..., 1], w.imag, rtol=0, atol=1e-14)
        yi = oracle.rope(x, base=10000.0, pos0=pos0, inverse=True)
        wi = z * np.exp(-1j * t)
        np.testing.assert_allclose(yi[..., 0], wi.real, rtol=0, atol=1e-14)
        np.testing.assert_allclose(yi[..., 1], wi.imag, rtol=0, atol=1e-14)


def test_golden_unit_rotations():
    doc = json.load(open(GOLDEN))
    assert len(doc["cases"]) >= 5
    for c in doc["cases"]:
        D, t, i = c["D"], c["t"], c["pair"]
        x = np.zeros((1, t + 1, 2, D))
        x[0, t, 0, 2 * i] = 1.0          # head 0: e_{2i}
        x[0, t, 1, 2 * i + 1] = 1.0      # head 1: e_{2i+1}
        y = oracle.rope(x, base=c["base"])
        e0 = np.zeros(D)
        e0[2 * i], e0[2 * i + 1] = c["cos"], c["sin"]
        e1 = np.zeros(D)
        e1[2 * i], e1[2 * i + 1] = -c["sin"], c["cos"]
        np.testing.assert_allclose(y[0, t, 0], e0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(y[0, t, 1], e1, rtol=0, atol=1e-13)


def test_identity_at_position_zero():
    x = _rng(2).standard_normal((2, 1, 4, 16))
    np.testing.assert_array_equal(oracle.rope(x), x)


def test_norm_preserved_per_pair_and_row():
    x = _rng(3).standard_normal((2, 33, 3, 32))
    y = oracle.rope(x, base=10000.0, pos0=11)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.max(np.abs(nx - ny) / nx) < 1e-14
    assert np.max(np.abs(np.linalg.norm(x, axis=-1) - np.linalg.norm(y, axis=-1))) < 1e-13


def test_inverse_round_trip():
    x = _rng(4).standard_normal((2, 40, 2, 64))
    for base in (10000.0, 500000.0):
        y = oracle.rope(x, base=base, pos0=3)
        back = oracle.rope(y, base=base, pos0=3, inverse=True)
        np.testing.assert_allclose(back, x, rtol=0, atol=1e-13)


def test_relative_position_property():
    # <R_m q, R_n k> = <R_{m-n} q, k>: the score depends only on the offset m - n.
    r = _rng(5)
    D = 16
    q = r.standard_normal((1, 1, 1, D))
    k = r.standard_normal((1, 1, 1, D))
    for m, n in ((7, 3), (100, 41), (5, 5), (2, 9)):
        qm = oracle.rope(q, pos0=m)
        kn = oracle.rope(k, pos0=n)
        lhs = float(np.sum(qm * kn))
        if m >= n:
            rhs = float(np.sum(oracle.rope(q, pos0=m - n) * k))
        else:
            rhs = float(np.sum(q * oracle.rope(k, pos0=n - m)))
        assert abs(lhs - rhs) < 1e-12


def test_pos0_is_a_shift_of_t():
    x = _rng(6).standard_normal((1, 12, 2, 8))
    y_shift = oracle.rope(x[:, 4:], pos0=4)
    y_full = oracle.rope(x)
    np.testing.assert_allclose(y_shift, y_full[:, 4:], rtol=0, atol=1e-13)


def test_pairs_do_not_mix_and_frequencies_decrease():
    # A unit vector in pair i stays in pair i; higher pairs rotate more slowly.
    D, t = 12, 3
    angles = []
    for i in range(D // 2):
        x = np.zeros((1, t + 1, 1, D))
        x[0, t, 0, 2 * i] = 1.0
        y = oracle.rope(x)[0, t, 0]
        mask = np.ones(D, bool)
        mask[2 * i:2 * i + 2] = False
        assert np.all(y[mask] == 0.0)
        angles.append(np.arctan2(y[2 * i + 1], y[2 * i]) % (2 * np.pi))
    # pair 0 has theta = 1 (angle 3 rad); later pairs strictly slower (all angles < pi here)
    assert abs(angles[0] - 3.0) < 1e-14
    assert all(a > b for a, b in zip(angles, angles[1:]))


def test_odd_head_dim_rejected():
    with pytest.raises(ValueError):
        oracle.rope(np.zeros((1, 2, 1, 3)))
