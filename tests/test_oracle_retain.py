"""Pins for decode-time KV retention and decode attention."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import egs_oracle as O
from entropy_guided_sparse_amd import synth


def _causal_probs(q, k):
    """Attention probabilities of observers at positions L-W..L-1 from torch's
    float64 SDPA with identity values (rows of A)."""
    r, W, d = q.shape
    L = k.shape[0]
    pos = L - W + np.arange(W)
    mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(np.tile(k, (r, 1, 1)))[None]
    vt = torch.from_numpy(np.tile(np.eye(L), (r, 1, 1)))[None]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None])[0].numpy()


def test_zeta_one_is_plain_window_mean():
    rng = np.random.default_rng(0)
    r, W, d, L = 4, 8, 16, 300
    q = rng.standard_normal((r, W, d))
    k = rng.standard_normal((L, d))
    keep, mu, H = O.kv_retain_slice(q, k, 4, 16, 32, zeta=1.0)
    A = _causal_probs(q, k)
    ref = A.mean(axis=1).mean(axis=0)
    np.testing.assert_allclose(mu, ref, atol=1e-14)
    cand = np.arange(4, L - 16)
    top = cand[np.lexsort((cand, -ref[cand]))[:32]]
    assert keep.tolist() == sorted(list(range(4)) + top.tolist() + list(range(L - 16, L)))


def test_raw_mode_is_single_gemv():
    rng = np.random.default_rng(1)
    r, W, d, L = 4, 8, 16, 200
    q = rng.standard_normal((r, W, d))
    k = rng.standard_normal((L, d))
    _, mu, _ = O.kv_retain_slice(q, k, 2, 8, 20, raw=True)
    np.testing.assert_allclose(mu, k @ (q.sum(axis=(0, 1)) / math.sqrt(d)), atol=1e-11)


def test_mass_sums_to_one_and_weights_floor():
    rng = np.random.default_rng(2)
    r, W, d, L = 4, 8, 16, 256
    q = 3.0 * rng.standard_normal((r, W, d))
    k = rng.standard_normal((L, d))
    for zeta in (0.1, 0.5, 0.9):
        _, mu, H = O.kv_retain_slice(q, k, 4, 16, 32, zeta=zeta, tau=0.7)
        assert abs(mu.sum() - 1.0) < 1e-12
        w = O.head_weights(H, zeta, 0.7)
        assert abs(w.sum() - 1.0) < 1e-14
        assert np.all(w >= zeta / r - 1e-15)


def test_equal_entropies_give_uniform_weights():
    rng = np.random.default_rng(3)
    r, W, d, L = 4, 8, 16, 128
    q1 = rng.standard_normal((1, W, d))
    q = np.repeat(q1, r, axis=0)
    k = rng.standard_normal((L, d))
    _, mu, H = O.kv_retain_slice(q, k, 4, 16, 8, zeta=0.3)
    np.testing.assert_allclose(O.head_weights(H, 0.3, 1.0), 0.25, atol=1e-15)
    A = _causal_probs(q1, k)
    np.testing.assert_allclose(mu, A[0].mean(axis=0), atol=1e-14)


def test_sink_isolated_entropy_closed_form():
    # One observer at position L-1 and identical keys: attention is uniform over
    # L keys, so the sink-isolated distribution is uniform over L - n_sink
    # positions and every Renyi order gives ln(L - n_sink).
    rng = np.random.default_rng(4)
    r, d, L = 2, 16, 100
    q = rng.standard_normal((r, 1, d))
    k = np.tile(rng.standard_normal(d), (L, 1))
    for kind, a in ((O.SHANNON, 2.0), (O.RENYI, 2.0), (O.RENYI, 0.5)):
        _, mu, H = O.kv_retain_slice(q, k, 4, 8, 10, kind=kind, alpha=a)
        np.testing.assert_allclose(H, math.log(L - 4), atol=1e-12)
        np.testing.assert_allclose(mu, 1.0 / L, atol=1e-15)


def test_keep_everything_when_budget_covers_cache():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 8))
    k = rng.standard_normal((40, 8))
    keep, _, _ = O.kv_retain_slice(q, k, 4, 16, 20)
    assert keep.tolist() == list(range(40))


def test_infokv_alpha_zero_ranks_by_token_entropy():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 4, 8))
    k = rng.standard_normal((64, 8))
    te = rng.random(64) * 3.0
    keep, mu, _ = O.kv_retain_slice(q, k, 2, 4, 10, info_alpha=0.0, token_entropy=te)
    cand = np.arange(2, 60)
    top = cand[np.lexsort((cand, -te[cand]))[:10]]
    assert keep.tolist() == sorted([0, 1] + top.tolist() + [60, 61, 62, 63])
    np.testing.assert_allclose(mu, np.exp(te) / np.exp(te).sum(), atol=1e-15)


def test_planted_keys_retained_small_decode():
    cfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
    inp = synth.make_decode(cfg, seed=0, batch=2, cache_len=8192)
    out = O.kv_retain(inp.q_obs, inp.k, inp.v, 4, 256, 512)
    for (b, g), (keep, kk, vv, mu, H) in out.items():
        assert len(keep) == 4 + 256 + 512
        assert set(inp.planted[b, g].tolist()) <= set(keep.tolist())
        np.testing.assert_array_equal(kk, inp.k[b, g][keep])


def test_decode_attention_keep_all_is_dense_sdpa():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, n = 2, 4, 2, 16, 50
    qn = rng.standard_normal((B, Hq, d))
    kk = rng.standard_normal((B, Hkv, n, d))
    vv = rng.standard_normal((B, Hkv, n, d))
    o = O.sparse_decode_attn(qn, kk, vv)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(qn)[:, :, None], torch.from_numpy(np.repeat(kk, 2, axis=1)),
        torch.from_numpy(np.repeat(vv, 2, axis=1)))[:, :, 0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_head_weights_hand_examples():
    # EntroPrefill Sec. 3.1 head weights worked by hand.  r = 2, zeta = 1/2.
    # tau = 1, H = (0, ln 2): v = (1, 1/2) / (3/2) = (2/3, 1/3), so
    # w = 1/4 + (1/2)(2/3, 1/3) = (7/12, 5/12).
    np.testing.assert_allclose(O.head_weights([0.0, math.log(2.0)], 0.5, 1.0),
                               [7 / 12, 5 / 12], atol=1e-15)
    # tau = 2, H = (0, ln 4): the temperature divides, exp(-ln 4 / 2) = 1/2,
    # so v and w are again (2/3, 1/3) and (7/12, 5/12).  (Multiplying by tau
    # would give v = (16/17, 1/17); a positive sign would favour head 1.)
    np.testing.assert_allclose(O.head_weights([0.0, math.log(4.0)], 0.5, 2.0),
                               [7 / 12, 5 / 12], atol=1e-15)
    # r = 4, zeta = 0.2, tau = 1/2, H = (ln 3, 0, ln 3, ln 3) / 2:
    # exp(-H / tau) = (1/3, 1, 1/3, 1/3), sum 2, v = (1/6, 1/2, 1/6, 1/6),
    # w = 0.05 + 0.8 v = (11/60, 9/20, 11/60, 11/60).
    h3 = math.log(3.0) / 2
    np.testing.assert_allclose(O.head_weights([h3, 0.0, h3, h3], 0.2, 0.5),
                               [11 / 60, 9 / 20, 11 / 60, 11 / 60], atol=1e-15)


def test_head_weight_lower_bound_of_sec_3_1():
    # EntroPrefill Sec. 3.1: a head whose entropy lies at least Delta below each
    # of its s - 1 siblings gets w >= zeta/r + (1 - zeta)/(1 + (s - 1) e^{-Delta/tau})
    # (divide the denominator of its softmax weight by its own term; every
    # sibling's term is then at most e^{-Delta/tau}).  Equality holds when every
    # sibling sits exactly Delta above it.
    rng = np.random.default_rng(11)
    for _ in range(300):
        r = int(rng.integers(2, 9))
        zeta = float(rng.uniform(0.0, 1.0))
        tau = float(rng.uniform(0.1, 5.0))
        delta = float(rng.uniform(0.0, 3.0))
        hs = int(rng.integers(0, r))
        Hs = float(rng.uniform(0.0, 4.0))
        H = Hs + delta + rng.exponential(1.0, r) * (rng.random() < 0.7)
        H[hs] = Hs
        bound = zeta / r + (1 - zeta) / (1 + (r - 1) * math.exp(-delta / tau))
        w = O.head_weights(H, zeta, tau)
        assert w[hs] >= bound - 1e-13
        H_eq = np.full(r, Hs + delta)
        H_eq[hs] = Hs
        assert abs(O.head_weights(H_eq, zeta, tau)[hs] - bound) < 1e-13


def test_head_weights_high_temperature_limit():
    # As tau grows the tempered softmax flattens: w -> 1/r for any entropies
    # (|w_h - 1/r| <= (1 - zeta) (e^{spread/tau} - 1) for spread = max H - min H).
    rng = np.random.default_rng(12)
    for r in (2, 4, 7):
        H = rng.uniform(0.0, 6.0, r)
        spread = float(H.max() - H.min())
        for tau in (1e3, 1e6):
            w = O.head_weights(H, 0.3, tau)
            assert np.all(np.abs(w - 1.0 / r) <= 0.7 * math.expm1(spread / tau) + 1e-15)
        # and at small tau all the non-floor weight goes to the lowest entropy
        w = O.head_weights(H, 0.3, 1e-3)
        lo = int(np.argmin(H))
        np.testing.assert_allclose(w, 0.3 / r + 0.7 * (np.arange(r) == lo), atol=1e-12)
