"""Pins for the oracle's entropy functions (closed forms, the InfoKV worked
example, Renyi-family limits and bounds)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import egs_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "window_mean_example.json")


def test_one_hot_has_zero_entropy():
    # EntropyInfer Sec. 3.1: concentrated attention -> low entropy; a one-hot
    # row is the limit with H = 0 for every order.
    p = np.zeros(17)
    p[5] = 1.0
    assert O.shannon(p) == 0.0
    for a in (0.5, 2.0, 3.0):
        assert abs(O.renyi(p, a)) < 1e-15


@pytest.mark.parametrize("n", [1, 2, 3, 64, 1000])
def test_uniform_has_log_n_entropy(n):
    p = np.full(n, 1.0 / n)
    assert abs(O.shannon(p) - math.log(n)) < 1e-12
    for a in (0.5, 2.0, 3.0):
        assert abs(O.renyi(p, a) - math.log(n)) < 1e-12


def test_worked_window_mean_example():
    g = json.load(open(GOLDEN))
    a = O.window_mean(np.array(g["rows"]))
    np.testing.assert_allclose(a, g["mean"], atol=1e-15)
    assert abs(a.sum() - 1.0) < 1e-15
    assert abs(O.shannon(a) - g["shannon"]) < 1e-12
    assert abs(O.renyi(a, 2.0) - g["renyi2"]) < 1e-12


def test_renyi_tends_to_shannon():
    rng = np.random.default_rng(1)
    for _ in range(20):
        p = rng.dirichlet(np.full(50, 0.3))
        h1 = O.shannon(p)
        for a in (1 - 1e-6, 1 + 1e-6):
            assert abs(O.renyi(p, a) - h1) < 1e-5
        assert O.renyi(p, 1.0) == h1


def test_renyi_non_increasing_in_order():
    # EntroPrefill Sec. 3.2: H_1 >= H_alpha >= H_2 for 1 <= alpha <= 2; the
    # family is non-increasing in alpha (van Erven & Harremoes).
    rng = np.random.default_rng(2)
    for _ in range(50):
        p = rng.dirichlet(np.full(40, 0.2))
        hs = [O.renyi(p, a) for a in (0.5, 1.0, 1.5, 2.0, 3.0)]
        assert all(hs[i] >= hs[i + 1] - 1e-12 for i in range(len(hs) - 1))


def test_collision_bounds():
    # EntroPrefill Sec. 3.2: 1/n <= sum p^2 <= 1, hence 0 <= H_2 <= ln n.
    rng = np.random.default_rng(3)
    for n in (2, 7, 100):
        for _ in range(20):
            p = rng.dirichlet(np.full(n, 0.5))
            h2 = O.renyi(p, 2.0)
            assert -1e-12 <= h2 <= math.log(n) + 1e-12
            assert abs(h2 + math.log(np.sum(p * p))) < 1e-12


def test_shannon_known_value_two_point():
    # H(1/4, 3/4) = ln 4 - (3/4) ln 3 (closed form).
    assert abs(O.shannon([0.25, 0.75]) - (math.log(4) - 0.75 * math.log(3))) < 1e-14


def test_renyi_rejects_bad_orders():
    for a in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            O.renyi([0.5, 0.5], a)
