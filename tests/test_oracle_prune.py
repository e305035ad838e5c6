"""Pins for chunk pruning (EntroPrefill Sec. 3.1-3.2, 4.1-4.2): the uniform
null, the priority bound of Sec. 3.2, the pooled measure against the decode
retention's group scores, the row-chunk masses by loops, the greedy proposer's
feasibility and scan order, and weak duality of the certificate by brute force."""
import itertools
import math

import numpy as np

from oracle import egs_oracle as O


def _chunks(rng, T, W, k):
    cuts = np.sort(rng.choice(np.arange(8, T - W), 2 * k, replace=False))
    return [(int(cuts[2 * i]), int(cuts[2 * i + 1])) for i in range(k)]


def test_uniform_null_gives_unit_ratio():
    # Sec. 3.2: under the uniform null M_i = pi_i, p_hat = 1/n_i and l_i = 1;
    # then kappa_i = -1 for chunks of two or more tokens.
    T = 100
    chunks = [(5, 25), (30, 31), (40, 90)]
    mu = np.full(T, 1.0 / T)
    S, ell, kap, M = O.prune_priorities(mu, chunks, eps_s=0.2, lam=0.7)
    N = sum(e - b for b, e in chunks)
    np.testing.assert_allclose(M, [(e - b) / N for b, e in chunks], atol=1e-15)
    np.testing.assert_allclose(ell, 1.0, atol=1e-15)
    np.testing.assert_allclose(kap, [-1.0, 0.0, -1.0], atol=1e-15)
    np.testing.assert_allclose(S, [-0.7, 0.0, -0.7], atol=1e-15)


def test_priority_bound_of_sec_3_2():
    # S_i - S_j >= ln(l_i / l_j) - lambda for every pair, kappa in [-1, 0]
    rng = np.random.default_rng(0)
    for _ in range(40):
        T = 300
        mu = rng.random(T) ** 6
        mu /= mu.sum()
        chunks = _chunks(rng, T, 10, 8)
        lam = float(rng.uniform(0, 2))
        S, ell, kap, _ = O.prune_priorities(mu, chunks, float(rng.uniform(0.01, 1)), lam)
        assert np.all(kap <= 1e-15) and np.all(kap >= -1 - 1e-12)
        for i in range(len(S)):
            for j in range(len(S)):
                assert S[i] - S[j] >= math.log(ell[i] / ell[j]) - lam - 1e-12


def test_pooled_measure_is_the_mean_of_group_scores():
    rng = np.random.default_rng(1)
    Hq, Hkv, W, d, T = 6, 3, 5, 8, 60
    q = rng.standard_normal((Hq, W, d))
    k = rng.standard_normal((Hkv, T, d))
    mu, A = O.prune_pooled_measure(q, k, n_sink=2, zeta=0.4, tau=0.8)
    want = np.mean([O.kv_retain_slice(q[g * 2:(g + 1) * 2], k[g], 2, 1, 1, kind=O.RENYI,
                                      alpha=2.0, zeta=0.4, tau=0.8)[1] for g in range(Hkv)],
                   axis=0)
    np.testing.assert_allclose(mu, want, atol=1e-14)
    assert abs(mu.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(A.sum(axis=2), 1.0, atol=1e-12)


def test_row_chunk_mass_loops():
    rng = np.random.default_rng(2)
    A = rng.random((3, 4, 50))
    chunks = [(2, 9), (9, 10), (20, 41)]
    m = O.prune_row_chunk_mass(A, chunks)
    for h in range(3):
        for u in range(4):
            for i, (b, e) in enumerate(chunks):
                s = 0.0
                for j in range(b, e):
                    s += A[h, u, j]
                assert abs(m[h * 4 + u, i] - s) < 1e-12


def test_greedy_feasibility_and_order():
    rng = np.random.default_rng(3)
    for _ in range(200):
        k, R = int(rng.integers(1, 12)), int(rng.integers(1, 6))
        n = rng.integers(1, 20, k)
        m = rng.random((R, k)) * 0.3
        S = np.round(rng.standard_normal(k), 1)          # ties on S are common
        eps, m0 = float(rng.uniform(0.05, 0.9)), int(rng.integers(0, 3))
        target = int(rng.integers(1, 120))
        rem, tok = O.prune_greedy(S, n, m, eps, m0, target)
        assert tok == int(n[rem].sum())
        assert np.all(m[:, rem].sum(axis=1) <= eps + 1e-12)
        assert rem.sum() <= max(k - m0, 0)
        order = sorted(range(k), key=lambda i: (S[i], -n[i], i))
        # scanned in order until the target is met; every chunk it passed over
        # would break a constraint when added to the final set
        stop = len(order)
        run = 0
        for pos, i in enumerate(order):
            if run >= target or rem.sum() >= k - m0 and not rem[i]:
                stop = pos
                break
            if rem[i]:
                run += n[i]
        for i in order[:stop]:
            if not rem[i]:
                assert np.any(m[:, rem].sum(axis=1) + m[:, i] > eps)


def test_certificate_weak_duality_by_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(60):
        k, R = int(rng.integers(1, 9)), int(rng.integers(1, 4))
        n = rng.integers(1, 15, k)
        m = rng.random((R, k)) * 0.4
        eps, m0 = float(rng.uniform(0.05, 1.0)), int(rng.integers(0, 3))
        best = 0
        for x in itertools.product([0, 1], repeat=k):
            x = np.array(x, dtype=bool)
            if x.sum() <= k - m0 and np.all(m[:, x].sum(axis=1) <= eps):
                best = max(best, int(n[x].sum()))
        _, tok = O.prune_greedy(np.zeros(k), n, m, eps, m0, 10 ** 9)
        assert tok <= best
        for _ in range(5):
            y, t = float(rng.uniform(0, 50)), float(rng.uniform(0, 10))
            assert O.prune_certificate(n, m, eps, m0, y, t) >= best - 1e-9
            ya = rng.uniform(0, 50, R)                 # one price per row
            assert O.prune_certificate(n, m, eps, m0, ya, t) >= best - 1e-9
        # zero prices and t = 0 give the trivial bound N; a scalar price is
        # the same as that price on every row
        assert O.prune_certificate(n, m, eps, m0, 0.0, 0.0) == float(n.sum())
        assert abs(O.prune_certificate(n, m, eps, m0, 3.5, 1.0)
                   - O.prune_certificate(n, m, eps, m0, np.full(R, 3.5), 1.0)) < 1e-9


def test_certificate_by_hand():
    # two rows, three chunks: n = (4, 2, 5), eps = 0.5, m0 = 1, y = (1, 2), t = 1
    m = np.array([[0.2, 0.1, 0.4],
                  [0.3, 0.0, 0.1]])
    n = np.array([4, 2, 5])
    # sum_a y_a eps = 1.5; t (k - m0) = 2; priced masses (0.8, 0.1, 0.6);
    # hinges [4 - 0.8 - 1]+ = 2.2, [2 - 0.1 - 1]+ = 0.9, [5 - 0.6 - 1]+ = 3.4
    assert abs(O.prune_certificate(n, m, 0.5, 1, np.array([1.0, 2.0]), 1.0)
               - (1.5 + 2.0 + 2.2 + 0.9 + 3.4)) < 1e-12


def test_streaming_paths_agree_with_the_stacked_rows():
    # rows=False (no A kept) and single-head rows give the same values as the
    # stacked computation; each observer row is a causal softmax over T keys
    rng = np.random.default_rng(5)
    Hq, Hkv, W, d, T = 6, 2, 7, 16, 90
    q = rng.standard_normal((Hq, W, d))
    k = rng.standard_normal((Hkv, T, d))
    mu, A = O.prune_pooled_measure(q, k, n_sink=3)
    mu2, none = O.prune_pooled_measure(q, k, n_sink=3, rows=False)
    assert none is None
    np.testing.assert_array_equal(mu, mu2)
    for h in range(Hq):
        np.testing.assert_array_equal(O.prune_head_rows(q, k, h), A[h])
    u = 2                                         # observer u sits at T - W + u
    z = k[1] @ q[4, u] / math.sqrt(d)
    z[T - W + u + 1:] = -np.inf
    p = np.exp(z - z.max())
    np.testing.assert_allclose(A[4, u], p / p.sum(), atol=1e-15)


def test_priorities_hand_example_with_smoothing():
    # EntroPrefill Sec. 3.2 worked by hand (reading: p is mu on the candidate
    # tokens renormalised, uniform null pi_i = n_i / N).
    # mu = (0.2, 0.4, 0.24, 0.08, 0.08), candidates c_0 = {1, 2}, c_1 = {3, 4}:
    # Z = 0.8, p = (0.5, 0.3 | 0.1, 0.1), N = 4, n = (2, 2), pi = (1/2, 1/2),
    # M = (0.8, 0.2).  With eps_s = 0.1, eps_s pi_i / n_i = 0.025 and
    # eps_s pi_i = 0.05:
    #   chunk 0: p_hat = (0.525, 0.325) / 0.85 = (21/34, 13/34),
    #            l = 0.85 / (1.1 * 0.5) = 17/11, sum p_hat^2 = 610/1156,
    #            kappa = ln(610/1156) / ln 2;
    #   chunk 1: p_hat = (1/2, 1/2), l = 0.25 / 0.55 = 5/11, kappa = -1.
    # Without smoothing chunk 0 would have p_hat = (5/8, 3/8) and l = 8/5.
    mu = np.array([0.2, 0.4, 0.24, 0.08, 0.08])
    chunks = [(1, 3), (3, 5)]
    lam = 0.5
    S, ell, kap, M = O.prune_priorities(mu, chunks, eps_s=0.1, lam=lam)
    k0 = math.log(610 / 1156) / math.log(2.0)
    np.testing.assert_allclose(M, [0.8, 0.2], atol=1e-15)
    np.testing.assert_allclose(ell, [17 / 11, 5 / 11], atol=1e-15)
    np.testing.assert_allclose(kap, [k0, -1.0], atol=1e-15)
    np.testing.assert_allclose(S, [math.log(17 / 11) + lam * k0, math.log(5 / 11) - lam],
                               atol=1e-15)


def test_priorities_hand_example_unequal_chunks():
    # A one-token chunk beside a three-token chunk (kappa = 0 for n = 1):
    # mu = (0.6, 0.1, 0.2, 0.1) all candidates, c_0 = {0}, c_1 = {1, 2, 3};
    # N = 4, pi = (1/4, 3/4), M = (0.6, 0.4).  eps_s = 0.2:
    #   chunk 0: l = (0.6 + 0.05) / (1.2 * 0.25) = 13/6, S = ln(13/6);
    #   chunk 1: eps_s pi_1 = 0.15, per token 0.05;
    #            p_hat = (0.15, 0.25, 0.15) / 0.55 = (3, 5, 3)/11,
    #            l = 0.55 / (1.2 * 0.75) = 11/18, sum p_hat^2 = 43/121,
    #            kappa = ln(43/121) / ln 3.
    mu = np.array([0.6, 0.1, 0.2, 0.1])
    S, ell, kap, M = O.prune_priorities(mu, [(0, 1), (1, 4)], eps_s=0.2, lam=2.0)
    k1 = math.log(43 / 121) / math.log(3.0)
    np.testing.assert_allclose(M, [0.6, 0.4], atol=1e-15)
    np.testing.assert_allclose(ell, [13 / 6, 11 / 18], atol=1e-15)
    np.testing.assert_allclose(kap, [0.0, k1], atol=1e-15)
    np.testing.assert_allclose(S, [math.log(13 / 6), math.log(11 / 18) + 2.0 * k1], atol=1e-15)
