"""Pins for latent decoding (EntropyInfer Sec. 4.3 and App. B): the schedule,
reduction to dense decoding when nothing is evicted, and the point of the
method, that generated tokens in the observation window change what is kept."""
import math

import numpy as np

from oracle import egs_oracle as O


def test_schedule():
    due = lambda nd, iv, T: [s for s in range(1, T + 1) if O.latent_due(s, nd, iv)]
    assert due(5, 8, 30) == [5, 13, 21, 29]
    assert due(5, 0, 30) == [5]
    assert due(0, 8, 30) == [8, 16, 24]
    assert due(40, 8, 30) == []


def _dense(q, K, V):
    z = K @ q / math.sqrt(q.size)
    p = np.exp(z - z.max())
    return (p / p.sum()) @ V


def _steps(rng, T, B, Hq, Hkv, d):
    return [(rng.standard_normal((B, Hq, d)), rng.standard_normal((B, Hkv, d)),
             rng.standard_normal((B, Hkv, d))) for _ in range(T)]


def test_no_eviction_is_dense_decoding():
    rng = np.random.default_rng(0)
    B, Hq, Hkv, d, L0, W, T = 2, 4, 2, 8, 40, 4, 12
    k0, v0 = rng.standard_normal((B, Hkv, L0, d)), rng.standard_normal((B, Hkv, L0, d))
    win = rng.standard_normal((B, Hq, W, d))
    steps = _steps(rng, T, B, Hq, Hkv, d)
    for (n_delay, n_keep) in [(T + 5, 3), (3, 10_000)]:     # never due / keeps everything
        outs, events = O.latent_decode(k0, v0, win, steps, 2, 4, n_keep, n_delay, 4)
        for s in range(T):
            for b in range(B):
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    K = np.vstack([k0[b, g]] + [steps[t][1][b, g][None] for t in range(s + 1)])
                    V = np.vstack([v0[b, g]] + [steps[t][2][b, g][None] for t in range(s + 1)])
                    np.testing.assert_allclose(outs[s, b, h], _dense(steps[s][0][b, h], K, V),
                                               atol=1e-12)
        for _, ev in events:
            for (keep, _) in ev.values():
                assert np.array_equal(keep, np.arange(len(keep)))


def test_compaction_keeps_order_and_later_tokens_see_the_compacted_cache():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, d, L0, W, T = 1, 2, 1, 8, 30, 4, 9
    k0, v0 = rng.standard_normal((B, Hkv, L0, d)), rng.standard_normal((B, Hkv, L0, d))
    win = rng.standard_normal((B, Hq, W, d))
    steps = _steps(rng, T, B, Hq, Hkv, d)
    outs, events = O.latent_decode(k0, v0, win, steps, 2, 4, 5, 4, 0)
    (s, ev), = events
    assert s == 4
    keep, _ = ev[(0, 0)]
    assert len(keep) == 2 + 5 + 4 and np.all(np.diff(keep) > 0)
    K = np.vstack([k0[0, 0]] + [steps[t][1][0, 0][None] for t in range(4)])[keep]
    V = np.vstack([v0[0, 0]] + [steps[t][2][0, 0][None] for t in range(4)])[keep]
    for t in range(4, T):                   # after the compression: kept + new entries
        K = np.vstack([K, steps[t][1][0, 0][None]])
        V = np.vstack([V, steps[t][2][0, 0][None]])
        for h in range(Hq):
            np.testing.assert_allclose(outs[t, 0, h], _dense(steps[t][0][0, h], K, V), atol=1e-12)


def test_generated_queries_change_what_is_kept():
    # A key that only the generated tokens attend to: ranking with the prompt
    # window alone evicts it, the latent window (generated queries included)
    # keeps it.
    rng = np.random.default_rng(2)
    d, L0, W = 16, 64, 4
    e = np.zeros(d)
    e[0] = 1.0
    k0 = 0.3 * rng.standard_normal((1, 1, L0, d))
    k0[0, 0, :, 0] = 0.0
    k0[0, 0, 20] = 6.0 * e                   # the key the generated tokens need
    v0 = rng.standard_normal((1, 1, L0, d))
    win = rng.standard_normal((1, 1, W, d))
    win[..., 0] = 0.0                        # prompt observers ignore direction e
    # prompt-only ranking (compression right after prefill)
    keep_pf, _, _ = O.kv_retain_slice(win[0, 0][None], k0[0, 0], 1, 2, 3)
    assert 20 not in keep_pf
    steps = []
    for _ in range(W):
        q = rng.standard_normal((1, 1, d))
        q[0, 0, 0] = 0.0
        q[0, 0] += 6.0 * e                   # generated queries look for e
        steps.append((q, 0.3 * rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))))
    _, events = O.latent_decode(k0, v0, win, steps, 1, 2, 3, W, 0)
    (_, ev), = events
    assert 20 in ev[(0, 0)][0]
