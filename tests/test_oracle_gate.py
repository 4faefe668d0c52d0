"""Pins of the oracle's confidence gate (README, "How it fits": confidence gate, tau = 0.60)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import gate as G


def test_confidence_is_softmax_max():
    rng = np.random.default_rng(0)
    lg = (rng.standard_normal((7, 1000)) * np.array([0.1, 1, 3, 5, 8, 12, 20])[:, None]).astype(np.float32)
    ref = softmax(lg.astype(np.float64), axis=1).max(axis=1)
    assert np.allclose(G.confidence(lg), ref, rtol=1e-12, atol=0)


def test_closed_forms():
    V = 4096
    assert G.confidence(np.zeros((1, V), np.float32))[0] == pytest.approx(1.0 / V, rel=1e-15)
    two = np.full((1, V), -np.inf, np.float32)
    two[0, 5] = two[0, 9] = 3.0
    assert G.confidence(two)[0] == 0.5
    one = np.full((1, V), -50.0, np.float32)
    one[0, 7] = 50.0
    assert G.confidence(one)[0] == pytest.approx(1.0, abs=1e-40)
    # shifting every logit of a row leaves the confidence unchanged
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((3, 333)).astype(np.float32)
    assert np.allclose(G.confidence(lg), G.confidence(lg + np.float32(4.0)), rtol=1e-6)


def test_flags_threshold():
    V = 10
    lg = np.zeros((3, V), np.float32)
    lg[1, 0] = np.log(9 * 1.5, dtype=np.float64)   # p_max = 13.5 / 22.5 = 0.6 exactly in real arithmetic
    lg[2, 0] = 10.0
    conf = G.confidence(lg)
    flags = G.gate_flags(lg, 0.60)
    assert flags[0] == 1 and flags[2] == 0
    assert flags[1] == (1 if conf[1] < np.float32(0.60) else 0)
