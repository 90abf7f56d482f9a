"""Pins for the RoPE oracle (CPU only).

Each check ties ``oracle.rope`` to something other than itself: hand-derived
values, the complex-number form of the rotation, the textbook 2-D rotation,
invariants the method guarantees, and the exact permutation between the two
pairing conventions.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.conftest import GOLDEN


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_inv_freq_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "rope_inv_freq_d4.json")))
    got = oracle.inv_freq(g["head_dim"], g["theta"])
    np.testing.assert_allclose(got, g["inv_freq"], rtol=1e-15, atol=0)
    assert oracle.inv_freq(2, 123.0).tolist() == [1.0]


def test_inv_freq_geometric_and_endpoint():
    # theta^(-2i/D): ratio between neighbours is theta^(-2/D); one step past the
    # last pair would reach exactly 1/theta.
    D, th = 128, 10000.0
    f = oracle.inv_freq(D, th)
    assert f[0] == 1.0
    r = f[1:] / f[:-1]
    np.testing.assert_allclose(r, np.full_like(r, th ** (-2.0 / D)), rtol=1e-13)
    np.testing.assert_allclose(f[-1] * th ** (-2.0 / D), 1.0 / th, rtol=1e-13)


def test_position_zero_is_identity():
    x = _rng(1).standard_normal((3, 5, 64))
    np.testing.assert_array_equal(oracle.rotate(x, np.zeros((3, 5)), 10000.0), x)


@pytest.mark.parametrize("pos,factor", [(1, 1.0), (7, 1.0), (7, 2.0), (4095, 1.0), (8192, 2.0)])
def test_d2_is_plane_rotation(pos, factor):
    # D = 2: one pair, frequency 1, so the vector turns by pos/factor radians.
    a, b = 0.3, -1.7
    z = complex(a, b) * cmath.exp(1j * (pos / factor))
    got = oracle.rotate(np.array([a, b]), np.array(pos), 10000.0, factor)
    assert abs(got[0] - z.real) < 1e-12 and abs(got[1] - z.imag) < 1e-12


@pytest.mark.parametrize("D", [4, 8, 64, 128])
def test_half_pairing_is_complex_product(D):
    # Pair i = (x[i], x[i+D/2]) as the complex number x[i] + 1j x[i+D/2],
    # multiplied by exp(1j * pos * theta^(-2i/D)).
    th = 10000.0
    x = _rng(D).standard_normal(D)
    for pos in (0, 1, 5, 127, 4096):
        got = oracle.rotate(x, np.array(pos), th)
        for i in range(D // 2):
            w = th ** (-2.0 * i / D)
            z = complex(x[i], x[i + D // 2]) * cmath.exp(1j * pos * w)
            assert abs(got[i] - z.real) < 1e-9 and abs(got[i + D // 2] - z.imag) < 1e-9


def test_interleaved_pairing_is_complex_product():
    D, th = 16, 500.0
    x = _rng(3).standard_normal(D)
    got = oracle.rotate(x, np.array(9), th, style="interleaved")
    for i in range(D // 2):
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * 9 * th ** (-2.0 * i / D))
        assert abs(got[2 * i] - z.real) < 1e-12 and abs(got[2 * i + 1] - z.imag) < 1e-12


def test_half_and_interleaved_differ_by_a_fixed_permutation():
    # perm takes an interleaved vector to the half-split layout.
    D = 32
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    x = _rng(4).standard_normal((6, D))
    pos = np.arange(6) * 37
    a = oracle.rotate(x, pos, 10000.0, style="interleaved")
    b = oracle.rotate(x[:, perm], pos, 10000.0, style="half")[:, inv]
    np.testing.assert_array_equal(a, b)


def test_norm_is_preserved():
    x = _rng(5).standard_normal((4, 33, 8, 128))
    pos = _rng(6).integers(0, 9000, size=(4, 33, 1))
    y = oracle.rotate(x, pos, 10000.0, 2.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


@pytest.mark.parametrize("factor", [1.0, 2.0])
def test_dot_product_depends_only_on_offset(factor):
    rng = _rng(7)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(0, 0), (5, 2), (100, 3000), (4000, 17)]:
        base = oracle.rotate(q, np.array(m), 10000.0, factor) @ oracle.rotate(k, np.array(n), 10000.0, factor)
        for t in (1, 64, 999):
            sh = oracle.rotate(q, np.array(m + t), 10000.0, factor) @ oracle.rotate(k, np.array(n + t), 10000.0, factor)
            assert abs(sh - base) < 1e-10


def test_linear_factor_divides_positions():
    # factor 2 at position 2m is exactly factor 1 at position m.
    x = _rng(8).standard_normal((10, 128))
    m = np.arange(10) * 411
    np.testing.assert_array_equal(oracle.rotate(x, 2 * m, 10000.0, 2.0), oracle.rotate(x, m, 10000.0, 1.0))
    # and is not factor 1 at 2m (the factor is really applied)
    assert not np.allclose(oracle.rotate(x, 2 * m, 10000.0, 2.0), oracle.rotate(x, 2 * m, 10000.0, 1.0))


def test_rope_apply_defaults_and_heads():
    rng = _rng(9)
    B, S, Hq, Hkv, D = 2, 7, 4, 2, 16
    q, k = rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D))
    qa, ka = oracle.rope_apply(q, k, None, 10000.0)
    pos = np.broadcast_to(np.arange(S), (B, S))
    qb, kb = oracle.rope_apply(q, k, pos, 10000.0)
    np.testing.assert_array_equal(qa, qb)
    np.testing.assert_array_equal(ka, kb)
    # every head of a token turns by the same angles
    for h in range(Hq):
        np.testing.assert_array_equal(qa[:, :, h], oracle.rotate(q[:, :, h], pos, 10000.0))
    # inputs untouched
    assert not np.shares_memory(qa, q)
