"""GPU parity of page-level retention (EntroPrefill Sec. 7) against the oracle,
through the C ABI: page lists and counts are integer outputs, so they must be
bit-exact (both sides compare the same float32 page maxima)."""
import numpy as np
import pytest
import torch

from _parity import dev_tensor, log
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _scores(rng, B, X, L, ties=False):
    """Per-member token distributions: a diffuse rest, a few spikes; with
    `ties`, values rounded so that equal page maxima are common."""
    p = rng.random((B, X, L)) ** 4
    for b in range(B):
        for x in range(X):
            hot = rng.choice(L, 6, replace=False)
            p[b, x, hot] += rng.uniform(2.0, 40.0, 6) * p[b, x].sum() / 6
    p /= p.sum(axis=2, keepdims=True)
    if ties:
        p = np.round(p * 2000.0) / 2000.0
    return p.astype(np.float32)


def _check(api, B, Hq, Hkv, L, S, n_sink, n_recent, K, mode, seed=0, ties=False, scores=None):
    r = Hq // Hkv
    X = Hq if mode == api.L.EGS_PAGE_HEAD_UNION else Hkv
    log(f"[pages] B={B} Hq={Hq} Hkv={Hkv} L={L} S={S} sink={n_sink} recent={n_recent} K={K} "
        f"mode={mode} ties={ties}")
    if scores is None:
        scores = _scores(np.random.default_rng(seed), B, X, L, ties)
    shape = api.DecodeShape(B, Hq, Hkv, 128, L, min(64, L), n_sink, n_recent, 0)
    ts = torch.from_numpy(scores).cuda()
    idx, cnt = api.page_retain(shape, ts, S, K, mode)
    torch.cuda.synchronize()
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    want = O.page_retain(scores.astype(np.float64), S, n_sink, n_recent, K, mode, r=r)
    for b in range(B):
        for y, pages in enumerate(want[b]):
            n = int(g_cnt[b, y])
            assert n == len(pages), (b, y, n, len(pages))
            assert g_idx[b, y, :n].tolist() == pages, (b, y)
            assert np.all(g_idx[b, y, n:] == -1)
    return scores, g_idx, g_cnt


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_pages_basic(api, mode):
    _check(api, 2, 8, 2, 4096, 16, 4, 256, 32, mode, seed=1)


@pytest.mark.parametrize("case", ["ragged_last_page", "sinks_span_pages", "page_of_one",
                                  "keep_none", "keep_all", "no_forced", "forced_overlap",
                                  "ties"])
def test_pages_edges(api, case):
    B, Hq, Hkv = 2, 6, 3
    kw = dict(ragged_last_page=dict(L=1000, S=24, n_sink=4, n_recent=7, K=5),
              sinks_span_pages=dict(L=2048, S=8, n_sink=30, n_recent=40, K=9),
              page_of_one=dict(L=3000, S=1, n_sink=4, n_recent=100, K=200),
              keep_none=dict(L=2048, S=32, n_sink=4, n_recent=64, K=0),
              keep_all=dict(L=2048, S=32, n_sink=4, n_recent=64, K=1000),
              no_forced=dict(L=2048, S=16, n_sink=0, n_recent=0, K=11),
              forced_overlap=dict(L=100, S=16, n_sink=60, n_recent=50, K=2),
              ties=dict(L=4096, S=16, n_sink=4, n_recent=256, K=40))[case]
    for mode in (0, 1, 2):
        _check(api, B, Hq, Hkv, kw["L"], kw["S"], kw["n_sink"], kw["n_recent"], kw["K"], mode,
               seed=2, ties=(case == "ties"))


def test_page_of_one_matches_token_retention(api):
    # page size 1 under GROUP is the token-level keep rule of kv_retain
    B, Hq, Hkv, L = 2, 8, 2, 4096
    rng = np.random.default_rng(5)
    sc = _scores(rng, B, Hkv, L)
    _, g_idx, g_cnt = _check(api, B, Hq, Hkv, L, 1, 4, 256, 512, 0, scores=sc)
    for b in range(B):
        for g in range(Hkv):
            top = O.select_topk(sc[b, g, 4:L - 256].astype(np.float64), 512)
            want = sorted(list(range(4)) + [4 + t for t in top] + list(range(L - 256, L)))
            assert g_idx[b, g, :g_cnt[b, g]].tolist() == want


def test_pages_from_kv_retain_scores(api):
    # the group scores mu of kv_retain feed the page rule; the keep lemma holds
    cfg = synth.DecodeConfig("pages", 2, 8, 2, 128, 4096, 64, 4, 256, 512)
    inp = synth.make_decode(cfg, seed=4)
    shape = api.DecodeShape(2, 8, 2, 128, 4096, 64, 4, 256, 512)
    prm = api.RetainParams(entropy_kind=api.L.EGS_SHANNON, zeta=0.5, tau=1.0)
    qo, k, v = (dev_tensor(x, "bf16") for x in (inp.q_obs_store, inp.k_store, inp.v_store))
    res = api.kv_retain(shape, prm, qo, k, v, want_scores=True, gather=False)
    torch.cuda.synchronize()
    mu = res["scores"].cpu().numpy()
    S, K = 16, 24
    for mode in (api.L.EGS_PAGE_GROUP, api.L.EGS_PAGE_LAYER_UNION):
        _, g_idx, g_cnt = _check(api, 2, 8, 2, 4096, S, 4, 256, K, mode, scores=mu)
        if mode == api.L.EGS_PAGE_GROUP:
            forced = O.forced_pages(4096, S, 4, 256)
            for b in range(2):
                for g in range(2):
                    kept = set(g_idx[b, g, :g_cnt[b, g]].tolist())
                    for t in np.nonzero(mu[b, g] > 1.0 / (K + 1))[0]:
                        assert t // S in kept or t // S in forced


def test_pages_full_decode_workload(api):
    """Batch 8, 32/8 heads, 128k cache: GROUP and LAYER_UNION on the GPU's
    kv_retain scores, HEAD_UNION on seeded per-head scores; two batch
    elements are checked against the oracle."""
    L_ = api.L
    cfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
    inp = synth.make_decode(cfg, seed=0)
    B, Hq, Hkv, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.cache_len
    shape = api.DecodeShape(B, Hq, Hkv, cfg.head_dim, L, cfg.n_obs, cfg.n_sink, cfg.n_recent,
                            cfg.n_keep)
    prm = api.RetainParams(entropy_kind=L_.EGS_SHANNON, zeta=0.5, tau=1.0)
    qo, k = (dev_tensor(x, "bf16") for x in (inp.q_obs_store, inp.k_store))
    res = api.kv_retain(shape, prm, qo, k, k, want_scores=True, gather=False)
    torch.cuda.synchronize()
    del qo, k
    mu = res["scores"]
    S, K = 16, 256
    heads = torch.from_numpy(_scores(np.random.default_rng(9), B, Hq, L)).cuda()
    for mode, ts in ((L_.EGS_PAGE_GROUP, mu), (L_.EGS_PAGE_LAYER_UNION, mu),
                     (L_.EGS_PAGE_HEAD_UNION, heads)):
        log(f"[pages full] mode={mode}")
        idx, cnt = api.page_retain(shape, ts, S, K, mode)
        torch.cuda.synchronize()
        for b in (0, B - 1):
            want = O.page_retain(ts[b:b + 1].cpu().numpy().astype(np.float64), S, cfg.n_sink,
                                 cfg.n_recent, K, mode, r=Hq // Hkv)[0]
            for y, pages in enumerate(want):
                n = int(cnt[b, y])
                assert n == len(pages)
                assert idx[b, y, :n].cpu().tolist() == pages
