"""Pins for page-level retention (EntroPrefill Sec. 7): page maxima, the
page-keep lemma, the reduction to token-level retention, union bounds."""
import numpy as np

from oracle import egs_oracle as O


def _dist(rng, L, spikes=6):
    """A probability vector with a few large entries and a diffuse rest."""
    p = rng.random(L) ** 4
    hot = rng.choice(L, spikes, replace=False)
    p[hot] += rng.uniform(2.0, 40.0, spikes) * p.sum() / spikes
    return p / p.sum()


def test_page_scores_loop():
    rng = np.random.default_rng(0)
    p = rng.random(37)
    got = O.page_scores(p, 5)
    assert got.size == 8                       # ceil(37 / 5), last page holds 2 tokens
    for i in range(8):
        m = -1.0
        for t in range(i * 5, min(37, i * 5 + 5)):
            m = max(m, p[t])
        assert got[i] == m


def test_forced_pages():
    # L = 20, S = 4: sinks 0..2 touch page 0, recent 15..19 touch pages 3 and 4
    assert O.forced_pages(20, 4, 3, 5) == {0, 3, 4}
    assert O.forced_pages(20, 4, 0, 0) == set()
    assert O.forced_pages(20, 4, 5, 1) == {0, 1, 4}


def test_page_keep_lemma():
    # Sec. 7: a candidate token with mass above 1/(K+1) always keeps its page;
    # otherwise K competing pages would each hold a token at least as heavy, and
    # together with it exceed total mass 1.
    rng = np.random.default_rng(1)
    hits = 0
    for trial in range(300):
        L = int(rng.integers(40, 400))
        S = int(rng.integers(1, 9))
        K = int(rng.integers(1, 6))
        n_sink, n_recent = int(rng.integers(0, 5)), int(rng.integers(0, 9))
        p = _dist(rng, L, spikes=int(rng.integers(1, 8)))
        kept = set(O.page_select(p, S, n_sink, n_recent, K))
        forced = O.forced_pages(L, S, n_sink, n_recent)
        for t in np.nonzero(p > 1.0 / (K + 1))[0]:
            if t // S not in forced:
                hits += 1
                assert t // S in kept, (trial, t)
    assert hits > 50


def test_page_size_one_is_token_retention():
    # With one token per page the page rule is the token-level keep rule
    # (sinks, recent, top n_keep of the middle under (-score, index)).
    rng = np.random.default_rng(2)
    for _ in range(20):
        L = int(rng.integers(30, 200))
        n_sink, n_recent, n_keep = 3, 7, int(rng.integers(1, 15))
        p = _dist(rng, L)
        p[rng.integers(L)] = p[rng.integers(L)]      # a tie
        want = list(range(n_sink)) + [n_sink + t for t in O.select_topk(p[n_sink:L - n_recent],
                                                                         n_keep)]
        want = sorted(want + list(range(L - n_recent, L)))
        assert O.page_select(p, 1, n_sink, n_recent, n_keep) == want


def test_selection_is_the_best_by_brute_force():
    # every kept candidate page beats every dropped one under (-I, index)
    rng = np.random.default_rng(3)
    for _ in range(50):
        L, S, K = int(rng.integers(20, 120)), int(rng.integers(1, 6)), int(rng.integers(1, 8))
        p = np.round(_dist(rng, L), 3)                 # rounding makes ties common
        I = O.page_scores(p, S)
        forced = O.forced_pages(L, S, 2, 3)
        kept = set(O.page_select(p, S, 2, 3, K))
        cand = [i for i in range(I.size) if i not in forced]
        ksel = [i for i in cand if i in kept]
        assert len(ksel) == min(K, len(cand))
        assert forced <= kept
        for a in ksel:
            for b in cand:
                if b not in kept:
                    assert (I[a] > I[b]) or (I[a] == I[b] and a < b)


def test_union_bounds_and_identity():
    # Sec. 7: K <= |union| <= min(m K, N_P) over m members (here with the
    # forced pages F added to every member: |F| + K <= |U| <= min(|F| + m K, N_P))
    rng = np.random.default_rng(4)
    B, Hkv, r, L, S, K = 2, 3, 4, 300, 8, 5
    scores = np.stack([[_dist(rng, L) for _ in range(Hkv * r)] for _ in range(B)])
    n_pages = -(-L // S)
    F = len(O.forced_pages(L, S, 4, 16))
    heads = O.page_retain(scores, S, 4, 16, K, O.PAGE_HEAD_UNION, r=r)
    for b in range(B):
        for g in range(Hkv):
            u = heads[b][g]
            assert F + K <= len(u) <= min(F + r * K, n_pages)
            for h in range(g * r, (g + 1) * r):
                assert set(O.page_select(scores[b, h], S, 4, 16, K)) <= set(u)
    grp = O.page_retain(scores[:, :Hkv], S, 4, 16, K, O.PAGE_GROUP)
    lay = O.page_retain(scores[:, :Hkv], S, 4, 16, K, O.PAGE_LAYER_UNION)
    for b in range(B):
        assert lay[b][0] == sorted(set().union(*grp[b]))
        assert F + K <= len(lay[b][0]) <= min(F + Hkv * K, n_pages)
    # identical members: the union is the single set
    same = np.repeat(scores[:, :1], 3, axis=1)
    one = O.page_retain(same, S, 4, 16, K, O.PAGE_LAYER_UNION)
    for b in range(B):
        assert one[b][0] == O.page_select(same[b, 0], S, 4, 16, K)
