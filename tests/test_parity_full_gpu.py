"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times (its budget policies and k_max), through the C ABI.

The oracle computes every observation row, entropy, budget and block list of a
layer (they are small), and the attention / retention outputs on seeded
samples of (head, query block) pairs and (batch, KV group) slices, which it
computes one by one."""
import numpy as np
import pytest
import torch

from _parity import (ATTN_MAX_ABS, ATTN_REL_L2, ENTROPY_ATOL, SCORE_ATOL, attn_errors,
                     dev_tensor, list_violations, log, prefill_shape)
from bench import k_max_for, prefill_policy
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _attn_samples(cfg, E_rigid, rng, n_rand=10):
    """(h, b) pairs: the heaviest query block of a rigid and a dynamic head, the
    first block, a segment boundary, plus seeded random pairs."""
    Hq, CB, bps = cfg.n_q_heads, cfg.n_blocks, cfg.segment_size // cfg.block_size
    rig = [h for h in range(Hq) if E_rigid[h]]
    dyn = [h for h in range(Hq) if not E_rigid[h]]
    pairs = [(dyn[0] if dyn else 0, CB - 1), (rig[0] if rig else Hq - 1, CB - 1),
             (0, 0), (Hq - 1, bps), (Hq // 2, CB - bps)]
    for _ in range(n_rand):
        pairs.append((int(rng.integers(Hq)), int(rng.integers(CB))))
    return pairs


@pytest.mark.parametrize("name,kind", [("llama3-8b-32k", 0), ("qwen-64k", 0),
                                       ("llama3-8b-128k", 0), ("llama3-8b-128k", 1)])
def test_full_prefill_workload(api, name, kind):
    cfg = synth.PREFILL_CONFIGS[name]
    L = api.L
    log(f"[full prefill parity] {name} kind={kind}")
    inp = synth.make_prefill(cfg, seed=0)
    shape = prefill_shape(api, cfg)
    pol = prefill_policy(api, cfg)
    LS, LB, CB = cfg.segment_size, cfg.block_size, cfg.n_blocks
    k_max = k_max_for(pol, api, CB, LB)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    v = dev_tensor(inp.v_store, cfg.dtype)
    scores, E = api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0)
    rigid, budget = api.allocate_budget(shape, pol, E)
    idx, cnt = api.select_blocks(shape, scores, budget, k_max)
    out, lse = api.sparse_prefill_attn(shape, q, k, v, idx, cnt, return_lse=True)
    torch.cuda.synchronize()
    g_scores, g_E = scores.cpu().numpy(), E.cpu().numpy()
    g_rigid = rigid.cpu().numpy().astype(bool)
    g_budget = budget.cpu().numpy()
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    del q, k, v

    r_scores, r_E = O.entropy_score(inp.q, inp.k, LS, LB, cfg.probe_len, kind=kind, alpha=2.0)
    ds, dE = float(np.abs(g_scores - r_scores).max()), float(np.abs(g_E - r_E).max())
    log(f"  scores max|d|={ds:.3e} entropy max|d|={dE:.3e}")
    assert ds <= SCORE_ATOL and dE <= ENTROPY_ATOL
    pk = dict(frac=pol.frac, frac_rigid=pol.frac_rigid, frac_dynamic=pol.frac_dynamic,
              frac_min=pol.frac_min, frac_max=pol.frac_max,
              entropy_threshold=pol.entropy_threshold, base_tokens=pol.base_tokens,
              alg3_alpha=pol.alg3_alpha, alg3_delta_t=pol.alg3_delta_t)
    o_rigid, o_budget = O.allocate_budget(g_E.astype(np.float64), LS, LB, pol.mode, **pk)
    np.testing.assert_array_equal(g_rigid, o_rigid)
    np.testing.assert_array_equal(g_budget, o_budget)
    # every list is bit-exact against the oracle's selection on the GPU scores
    o_idx, o_cnt = O.select_blocks(g_scores.astype(np.float64), g_budget, LS, LB, k_max=k_max)
    np.testing.assert_array_equal(g_cnt, o_cnt)
    np.testing.assert_array_equal(g_idx, o_idx)
    bad = list_violations(g_idx, g_cnt, r_scores, g_budget, LS, LB)
    assert not bad, bad[:5]
    # the planted rigid heads are found (two-level workloads)
    if pol.mode == L.EGS_BUDGET_TWO_LEVEL:
        np.testing.assert_array_equal(g_rigid, inp.rigid_hs.all(axis=1))

    g_out = out[:, :, :]  # stays on the device; copy the sampled rows only
    rng = np.random.default_rng(1)
    num = den = 0.0
    worst = 0.0
    for (h, b) in _attn_samples(cfg, g_rigid, rng):
        ro, rl = O.sparse_prefill_attn_rows(inp.q, inp.k, inp.v, g_idx, g_cnt, h, b, LS, LB)
        go = g_out[h, b * LB:(b + 1) * LB].float().cpu().numpy()
        gl = lse[h, b * LB:(b + 1) * LB].cpu().numpy()
        worst = max(worst, float(np.abs(go - ro).max()))
        num += float(((go - ro) ** 2).sum())
        den += float((ro ** 2).sum())
        assert float((np.abs(gl - rl) - 2e-6 * np.abs(rl)).max()) <= 1e-3, (h, b)
    rel = (num / den) ** 0.5
    log(f"  sampled attention max|d|={worst:.3e} relL2={rel:.3e}")
    assert worst <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


def test_full_decode_retention(api):
    cfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
    log(f"[full decode parity] {cfg.name}")
    inp = synth.make_decode(cfg, seed=0)
    B, Hq, Hkv, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.cache_len
    r = Hq // Hkv
    shape = api.DecodeShape(B, Hq, Hkv, cfg.head_dim, L, cfg.n_obs, cfg.n_sink, cfg.n_recent,
                            cfg.n_keep)
    prm = api.RetainParams(entropy_kind=api.L.EGS_SHANNON, zeta=0.5, tau=1.0)
    qo, k, v, qn = (dev_tensor(x, "bf16") for x in (inp.q_obs_store, inp.k_store, inp.v_store,
                                                   inp.q_new_store))
    res = api.kv_retain(shape, prm, qo, k, v, want_scores=True)
    out = api.sparse_decode_attn(shape, qn, res["k_out"], res["v_out"])
    torch.cuda.synchronize()
    keep = res["keep_idx"].cpu().numpy()
    H = res["head_entropy"].cpu().numpy()
    mu = res["scores"]
    del qo, k, v
    band = 1e-4 / L
    for (b, g) in [(0, 0), (B - 1, Hkv - 1), (3, 5)]:
        o_keep, o_mu, o_H = O.kv_retain_slice(inp.q_obs[b, g * r:(g + 1) * r], inp.k[b, g],
                                              cfg.n_sink, cfg.n_recent, cfg.n_keep)
        g_mu = mu[b, g].cpu().numpy().astype(np.float64)
        err = float((np.abs(g_mu - o_mu) / (1e-4 * np.abs(o_mu) + 1e-5 / L)).max())
        dH = float(np.abs(H[b, g * r:(g + 1) * r] - o_H).max())
        log(f"  slice ({b},{g}): mu error/bound={err:.3e} head entropy max|d|={dH:.3e}")
        assert err <= 1.0 and dH <= ENTROPY_ATOL
        # keep set: bit-exact on the GPU's own scores, band rule on the oracle's
        top = O.select_topk(g_mu[cfg.n_sink:L - cfg.n_recent], cfg.n_keep)
        want = sorted(list(range(cfg.n_sink)) + [cfg.n_sink + t for t in top]
                      + list(range(L - cfg.n_recent, L)))
        np.testing.assert_array_equal(keep[b, g], np.asarray(want))
        cand = np.arange(cfg.n_sink, L - cfg.n_recent)
        sel = np.isin(cand, keep[b, g])
        sc = o_mu[cand]
        c = np.sort(sc)[::-1][cfg.n_keep - 1]
        assert not np.any((sc > c + band) & ~sel) and not np.any((sc < c - band) & sel)
        # every planted high-mass key is retained
        assert set(inp.planted[b, g].tolist()) <= set(keep[b, g].tolist())
        # the gather is a copy
        kk = res["k_out"][b, g].cpu()
        assert torch.equal(kk, torch.from_numpy(inp.k_store[b, g][keep[b, g]]).view(torch.bfloat16))
    # decode attention on the GPU's kept entries, sampled batches
    for b in (0, B - 1):
        kk = res["k_out"][b:b + 1].float().cpu().numpy()
        vv = res["v_out"][b:b + 1].float().cpu().numpy()
        ref = O.sparse_decode_attn(inp.q_new[b:b + 1], kk, vv)
        ma, rel = attn_errors(out[b:b + 1].float().cpu().numpy(), ref)
        log(f"  decode attention batch {b}: max|d|={ma:.3e} relL2={rel:.3e}")
        assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


def test_full_maxmin_observation_rows(api):
    """[EI] Alg. 1-2 representatives on the 128k layer: every observation row
    and entropy against the oracle."""
    cfg = synth.PREFILL_CONFIGS["llama3-8b-128k"]
    log(f"[full maxmin parity] {cfg.name}")
    inp = synth.make_prefill(cfg, seed=0)
    shape = prefill_shape(api, cfg)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    scores, E = api.entropy_score(shape, q, k, pool=api.L.EGS_POOL_MAXMIN)
    torch.cuda.synchronize()
    g_scores, g_E = scores.cpu().numpy(), E.cpu().numpy()
    del q, k
    r_scores, r_E = O.entropy_score(inp.q, inp.k, cfg.segment_size, cfg.block_size,
                                    cfg.probe_len, pool="maxmin")
    ds, dE = float(np.abs(g_scores - r_scores).max()), float(np.abs(g_E - r_E).max())
    log(f"  scores max|d|={ds:.3e} entropy max|d|={dE:.3e}")
    assert ds <= SCORE_ATOL and dE <= ENTROPY_ATOL
