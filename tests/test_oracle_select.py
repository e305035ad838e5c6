"""Pins for top-k block selection: sorting-library brute force and planted recall."""
import numpy as np

from oracle import egs_oracle as O
from entropy_guided_sparse_amd import synth


def test_select_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(0)
    for n in (1, 5, 33, 200):
        for _ in range(10):
            s = np.round(rng.random(n) * 8) / 8.0        # many exact ties
            for k in {0, 1, n // 3, n}:
                order = np.lexsort((np.arange(n), -s))   # primary -score, then index
                assert O.select_topk(s, k) == sorted(order[:k].tolist())


def test_select_blocks_layout_and_clamping():
    rng = np.random.default_rng(1)
    Hq, LS, LB, N = 3, 64, 16, 256
    CS, CB = N // LS, N // LB
    abar = np.full((Hq, CS, CB), -1.0)
    for s in range(CS):
        cb = (s + 1) * LS // LB
        abar[:, s, :cb] = rng.dirichlet(np.ones(cb), size=Hq)
    budget = np.array([[1, 2, 3, 4], [4, 8, 12, 16], [100, 100, 100, 100]])
    idx, cnt = O.select_blocks(abar, budget, LS, LB, k_max=20)
    for h in range(Hq):
        for s in range(CS):
            cb = (s + 1) * LS // LB
            c = int(cnt[h, s])
            assert c == min(budget[h, s], cb)
            row = idx[h, s]
            assert np.all(row[c:] == -1)
            assert np.all(np.diff(row[:c]) > 0)
            assert np.all(row[:c] < cb)
            order = np.lexsort((np.arange(cb), -abar[h, s, :cb]))
            assert row[:c].tolist() == sorted(order[:c].tolist())


def test_planted_hot_blocks_recalled():
    cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    inp = synth.make_prefill(cfg, seed=0)
    abar, E = O.entropy_score(inp.q, inp.k, cfg.segment_size, cfg.block_size, cfg.probe_len)
    _, k = O.allocate_budget(E, cfg.segment_size, cfg.block_size, O.MODE_FIXED, frac=0.25)
    idx, cnt = O.select_blocks(abar, k, cfg.segment_size, cfg.block_size)
    for h in range(cfg.n_q_heads):
        for s in range(cfg.n_segments):
            sel = set(idx[h, s, :cnt[h, s]].tolist())
            if inp.rigid_hs[h, s]:
                assert 0 in sel                       # the planted sink block
            else:
                assert set(inp.hot_blocks[(h, s)].tolist()) <= sel
