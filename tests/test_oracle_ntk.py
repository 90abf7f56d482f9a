"""Pins of the NTK-aware RoPE base scaling (oracle/ntk.py) to the method's
defining properties, not to its formula: the highest-frequency pair keeps its
angle, the lowest-frequency pair turns as linear interpolation by the scale
would turn it, scale 1 changes nothing, the dynamic form is the identity up
to the trained length and continuous there, and a hand-computed case."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("D", [4, 64, 128, 256])
@pytest.mark.parametrize("alpha", [1.5, 2.0, 8.0, 0.5])
@pytest.mark.parametrize("theta", [1e4, 5e5])
def test_frequency_endpoints(D, alpha, theta):
    t2 = oracle.ntk_theta(theta, D, alpha)
    f0, f1 = oracle.inv_freq(D, theta), oracle.inv_freq(D, t2)
    assert f1[0] == 1.0 and f0[0] == 1.0                      # highest frequency untouched
    assert f1[-1] == pytest.approx(f0[-1] / alpha, rel=1e-12)  # lowest one divided by the scale
    r = np.diff(f1 / f0) * (1 if alpha >= 1 else -1)
    assert np.all(r <= 1e-15)                                  # in between: ratios move monotonically


@pytest.mark.parametrize("alpha", [2.0, 4.0])
def test_lowest_pair_matches_linear_interpolation(alpha):
    """At position alpha * p the lowest-frequency pair has the angle it had at
    p without scaling -- what linear interpolation by alpha does to every pair."""
    D, theta = 128, 1e4
    p = np.array([0, 1, 100, 4095])
    a_ntk = oracle.angles(alpha * p, D, oracle.ntk_theta(theta, D, alpha))
    a_lin = oracle.angles(alpha * p, D, theta, linear_factor=alpha)
    a_ref = oracle.angles(p, D, theta)
    np.testing.assert_allclose(a_ntk[:, -1], a_ref[:, -1], rtol=1e-12, atol=0)
    np.testing.assert_allclose(a_lin[:, -1], a_ref[:, -1], rtol=1e-12, atol=0)
    np.testing.assert_allclose(a_ntk[:, 0], alpha * p, rtol=0, atol=0)  # the highest pair is not interpolated


def test_scale_one_and_hand_value():
    assert oracle.ntk_theta(1e4, 128, 1.0) == 1e4
    # D = 4: theta' = theta * alpha^(4/2); alpha = 4 -> 16 theta
    assert oracle.ntk_theta(100.0, 4, 4.0) == 1600.0
    f = oracle.inv_freq(4, 1600.0)
    assert f[1] == pytest.approx(oracle.inv_freq(4, 100.0)[1] / 4, rel=1e-15)


def test_dynamic_form():
    D, theta, L0 = 128, 1e4, 4096
    for L in (1, 100, L0):
        assert oracle.dynamic_ntk_theta(theta, D, 2.0, L, L0) == theta
    # continuous at the trained length
    assert oracle.dynamic_ntk_theta(theta, D, 2.0, L0 + 1, L0) == pytest.approx(theta, rel=1e-3)
    # with factor 1 the scale is L / L0
    assert oracle.dynamic_ntk_theta(theta, D, 1.0, 2 * L0, L0) == oracle.ntk_theta(theta, D, 2.0)
    # factor f at L = 2 L0: scale 2f - (f - 1) = f + 1
    assert oracle.dynamic_ntk_theta(theta, D, 4.0, 2 * L0, L0) == pytest.approx(oracle.ntk_theta(theta, D, 5.0),
                                                                                 rel=1e-15)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.ntk_theta(1e4, 2, 2.0)
    with pytest.raises(ValueError):
        oracle.ntk_theta(1e4, 127, 2.0)
    with pytest.raises(ValueError):
        oracle.ntk_theta(1e4, 128, 0.0)
