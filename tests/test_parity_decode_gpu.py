"""GPU parity of decode-time KV retention (kv_retain) and decode attention
(sparse_decode_attn) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from _parity import ATTN_MAX_ABS, ATTN_REL_L2, ENTROPY_ATOL, attn_errors, dev_tensor, log
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu

# Retention band: the group score mu is a probability over the cache, so it is
# compared on the uniform-normalised scale L * mu (1 = uniform); entries this
# close to the cutoff may swap.  Raw-mode scores are compared on the scale of
# the largest |score|.
RETAIN_BAND = 1e-4
# mu comes from fp32 logits of exact bf16 products (|z| <= ~50 here, so
# |dz| ~ 1e-5) and exp2 / fp32 sums: its relative error is ~2e-5 where the
# mass is concentrated.  Bound: |d mu| <= MU_RTOL * mu + MU_ATOL_NORM / L.
MU_RTOL = 1e-4
MU_ATOL_NORM = 1e-5


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _cfg(B=2, Hq=8, Hkv=2, d=128, L=4096, W=64, n_sink=4, n_recent=256, n_keep=512):
    return synth.DecodeConfig("decode-small", B, Hq, Hkv, d, L, W, n_sink, n_recent, n_keep)


def _keep_band_ok(keep, mu_ref, n_sink, n_recent, n_keep, band):
    L = mu_ref.size
    if n_sink + n_recent + n_keep >= L:
        return keep.tolist() == list(range(L))
    got = set(keep.tolist())
    if len(got) != n_sink + n_recent + n_keep or list(keep) != sorted(keep):
        return False
    if not set(range(n_sink)) <= got or not set(range(L - n_recent, L)) <= got:
        return False
    cand = np.arange(n_sink, L - n_recent)
    sel = np.isin(cand, list(got))
    if n_keep == 0:
        return not sel.any()
    sc = mu_ref[cand]
    c = np.sort(sc)[::-1][n_keep - 1]
    return not (np.any((sc > c + band) & ~sel) or np.any((sc < c - band) & sel))


def run_retain(api, cfg, seed=0, kind=0, alpha=2.0, zeta=0.5, tau=1.0, raw=0, info_alpha=1.0,
               with_entropy=False, slices=None, inp=None):
    log(f"[retain parity] B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} d={cfg.head_dim} "
        f"L={cfg.cache_len} W={cfg.n_obs} sink={cfg.n_sink} recent={cfg.n_recent} "
        f"keep={cfg.n_keep} kind={kind} raw={raw} info={info_alpha} seed={seed}")
    if inp is None:
        inp = synth.make_decode(cfg, seed)
    B, Hq, Hkv, L = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.cache_len
    r = Hq // Hkv
    shape = api.DecodeShape(B, Hq, Hkv, cfg.head_dim, L, cfg.n_obs, cfg.n_sink, cfg.n_recent,
                            cfg.n_keep)
    prm = api.RetainParams(entropy_kind=kind, renyi_alpha=alpha, zeta=zeta, tau=tau,
                           raw_logit_mode=raw, info_alpha=info_alpha)
    qo, k, v, qn = (dev_tensor(x, "bf16") for x in (inp.q_obs_store, inp.k_store, inp.v_store,
                                                   inp.q_new_store))
    te = None
    te_np = None
    if with_entropy:
        te_np = (np.random.default_rng(seed + 100).random((B, L)) * 4.0).astype(np.float32)
        te = torch.from_numpy(te_np).cuda()
    res = api.kv_retain(shape, prm, qo, k, v, token_entropy=te, want_scores=True)
    out = api.sparse_decode_attn(shape, qn, res["k_out"], res["v_out"])
    torch.cuda.synchronize()
    keep = res["keep_idx"].cpu().numpy()
    mu = res["scores"].cpu().numpy()
    H = res["head_entropy"].cpu().numpy()
    k_out = res["k_out"].cpu()
    todo = slices if slices is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    worst_mu = worst_H = 0.0
    for (b, g) in todo:
        o_keep, o_mu, o_H = O.kv_retain_slice(
            inp.q_obs[b, g * r:(g + 1) * r], inp.k[b, g], cfg.n_sink, cfg.n_recent, cfg.n_keep,
            kind=kind, alpha=alpha, zeta=zeta, tau=tau, raw=bool(raw), info_alpha=info_alpha,
            token_entropy=None if te_np is None else te_np[b])
        if raw:
            scale = np.abs(o_mu).max()
            dmu = np.abs(mu[b, g] - o_mu).max() / scale
            band = RETAIN_BAND * scale
            assert dmu <= 1e-5, dmu
        else:
            err = np.abs(mu[b, g] - o_mu)
            dmu = float((err / (MU_RTOL * np.abs(o_mu) + MU_ATOL_NORM / L)).max())
            band = RETAIN_BAND / L
            assert dmu <= 1.0, dmu
            dH = np.abs(H[b, g * r:(g + 1) * r] - o_H).max()
            worst_H = max(worst_H, dH)
            assert dH <= ENTROPY_ATOL, dH
        worst_mu = max(worst_mu, dmu)
        # bit-exact selection on the GPU's own scores, band rule on the oracle's
        g_keep = keep[b, g]
        sel_on_gpu_mu = _select_on(mu[b, g].astype(np.float64), cfg)
        np.testing.assert_array_equal(g_keep, sel_on_gpu_mu)
        assert _keep_band_ok(g_keep, o_mu, cfg.n_sink, cfg.n_recent, cfg.n_keep, band)
        # gather is a pure copy
        assert torch.equal(k_out[b, g], torch.from_numpy(inp.k_store[b, g][g_keep]).view(torch.bfloat16))
    log(f"  mu error / bound={worst_mu:.3e}  head entropy max|d|={worst_H:.3e}")
    # decode attention on the GPU's own kept entries
    kk = res["k_out"].float().cpu().numpy()
    vv = res["v_out"].float().cpu().numpy()
    ref = O.sparse_decode_attn(inp.q_new, kk, vv)
    ma, rel = attn_errors(out.float().cpu().numpy(), ref)
    log(f"  decode attention max|d|={ma:.3e} relL2={rel:.3e}")
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2
    return dict(inp=inp, keep=keep, mu=mu, H=H, out=out)


def _select_on(mu, cfg):
    L = mu.size
    if cfg.n_sink + cfg.n_recent + cfg.n_keep >= L:
        return np.arange(L)
    top = O.select_topk(mu[cfg.n_sink:L - cfg.n_recent], cfg.n_keep)
    keep = list(range(cfg.n_sink)) + [cfg.n_sink + t for t in top] + \
        list(range(L - cfg.n_recent, L))
    return np.asarray(sorted(keep))


def test_retain_small_default(api):
    res = run_retain(api, _cfg())
    inp = res["inp"]
    for b in range(2):
        for g in range(2):
            assert set(inp.planted[b, g].tolist()) <= set(res["keep"][b, g].tolist())


def test_retain_renyi2(api):
    run_retain(api, _cfg(), seed=1, kind=api.L.EGS_RENYI, alpha=2.0)


def test_retain_zeta_one_tau(api):
    run_retain(api, _cfg(), seed=2, zeta=1.0, tau=0.3)


def test_retain_raw_mode(api):
    run_retain(api, _cfg(), seed=3, raw=1)


def test_retain_infokv_fusion(api):
    run_retain(api, _cfg(), seed=4, info_alpha=0.9, with_entropy=True)


def test_retain_keep_all(api):
    run_retain(api, _cfg(L=700, n_keep=600), seed=5)


def test_retain_no_top_entries(api):
    run_retain(api, _cfg(L=2048, n_keep=0, n_recent=64, n_sink=0), seed=6)


@pytest.mark.parametrize("W", [1, 40, 128])
def test_retain_observer_windows(api, W):
    run_retain(api, _cfg(W=W, L=3000, n_recent=max(W, 16), n_keep=300), seed=7)


def test_retain_wide_group_d64(api):
    # 7 query heads per KV head (two 4-head groups per workgroup row)
    run_retain(api, _cfg(B=1, Hq=14, Hkv=2, d=64, L=5000, n_keep=700), seed=8)


def test_decode_attention_keep_all_is_dense(api):
    cfg = _cfg(B=2, L=1500, n_keep=2000)
    res = run_retain(api, cfg, seed=9)
    inp = res["inp"]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(inp.q_new.astype(np.float64))[:, :, None],
        torch.from_numpy(np.repeat(inp.k, 4, axis=1).astype(np.float64)),
        torch.from_numpy(np.repeat(inp.v, 4, axis=1).astype(np.float64)))[:, :, 0].numpy()
    ma, rel = attn_errors(res["out"].float().cpu().numpy(), ref)
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


def test_retain_all_scores_tied(api):
    """Zero keys make every observer's attention uniform over its visible keys,
    so all candidates (all visible to every observer) tie exactly: the keep set
    is the first n_keep candidates by index, on the GPU as in the oracle."""
    B, Hq, Hkv, d, L, W = 1, 4, 1, 128, 4096, 64
    n_sink, n_recent, n_keep = 4, 256, 300
    log(f"[retain ties] L={L} keep={n_keep}")
    rng = np.random.default_rng(11)
    q_obs = synth.round_to_bf16(rng.standard_normal((B, Hq, W, d)).astype(np.float32))
    k = np.zeros((B, Hkv, L, d), dtype=np.int16)
    v = synth.round_to_bf16(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    shape = api.DecodeShape(B, Hq, Hkv, d, L, W, n_sink, n_recent, n_keep)
    res = api.kv_retain(shape, api.RetainParams(), dev_tensor(q_obs, "bf16"),
                        dev_tensor(k, "bf16"), dev_tensor(v, "bf16"), want_scores=True)
    torch.cuda.synchronize()
    keep = res["keep_idx"].cpu().numpy()[0, 0]
    want = np.array(list(range(n_sink)) + list(range(n_sink, n_sink + n_keep)) +
                    list(range(L - n_recent, L)))
    np.testing.assert_array_equal(keep, want)
    o_keep, o_mu, _ = O.kv_retain_slice(synth.bf16_bits_to_f32(q_obs)[0], np.zeros((L, d)),
                                        n_sink, n_recent, n_keep)
    np.testing.assert_array_equal(o_keep, want)


# The launcher splits the kept entries into pieces of 192 to 1024 entries, the
# size chosen from n_total and batch x KV groups (64 here); these n_total reach
# every size it can pick: 193 -> 192, 257 -> 256, 321 -> 320, 2561 -> 384,
# 3137 -> 448, 4000 -> 512, 4033 -> 576, 4481 -> 640, 4929 -> 704, 5377 -> 768,
# 5825 -> 832, 6273 -> 896, 6721 -> 960, 1 -> 1024.
@pytest.mark.parametrize("n_total", [1, 193, 257, 321, 2561, 3137, 4000, 4033, 4481, 4929,
                                     5377, 5825, 6273, 6721])
def test_decode_attention_every_split_size(api, n_total):
    B, Hq, Hkv, d = 8, 32, 8, 128
    log(f"[decode attention splits] B={B} Hq={Hq} Hkv={Hkv} d={d} n_total={n_total}")
    rng = np.random.default_rng(1000 + n_total)
    qb = synth.round_to_bf16(rng.standard_normal((B, Hq, d)).astype(np.float32))
    kb = synth.round_to_bf16(rng.standard_normal((B, Hkv, n_total, d)).astype(np.float32))
    vb = synth.round_to_bf16(rng.standard_normal((B, Hkv, n_total, d)).astype(np.float32))
    # a few entries with large logits so that each head's softmax is peaked
    kf = synth.bf16_bits_to_f32(kb).copy()
    qf = synth.bf16_bits_to_f32(qb)
    for b in range(B):
        for g in range(Hkv):
            t = int(rng.integers(n_total))
            kf[b, g, t] += 3.0 * qf[b, g * (Hq // Hkv)]
    kb = synth.round_to_bf16(kf)
    shape = api.DecodeShape(B, Hq, Hkv, d, max(n_total, 1), 1, 0, 0, 0)
    out = api.sparse_decode_attn(shape, dev_tensor(qb, "bf16"), dev_tensor(kb, "bf16"),
                                 dev_tensor(vb, "bf16"))
    torch.cuda.synchronize()
    ref = O.sparse_decode_attn(synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(kb),
                               synth.bf16_bits_to_f32(vb))
    ma, rel = attn_errors(out.float().cpu().numpy(), ref)
    log(f"  max|d|={ma:.3e} relL2={rel:.3e}")
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


@pytest.mark.parametrize("L,n_keep", [(65536, 300), (70001, 5000), (70001, 0), (66000, 66000)])
def test_retain_split_topk_edges(api, L, n_keep):
    """Cache rows of 65,536 entries and more take the select split over many
    workgroups (per-chunk digit histograms, then chunked compaction).  Zero
    keys tie every candidate exactly, so the keep set is the sinks, the first
    n_keep candidates by index and the recent window; n_keep = 0 keeps sinks
    and recent only, and n_keep >= L keeps everything (as the oracle)."""
    B, Hq, Hkv, d, W = 1, 4, 1, 128, 64
    n_sink, n_recent = 4, 256
    log(f"[retain split top-k] L={L} keep={n_keep}")
    rng = np.random.default_rng(13)
    q_obs = synth.round_to_bf16(rng.standard_normal((B, Hq, W, d)).astype(np.float32))
    k = np.zeros((B, Hkv, L, d), dtype=np.int16)
    v = synth.round_to_bf16(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    shape = api.DecodeShape(B, Hq, Hkv, d, L, W, n_sink, n_recent, n_keep)
    res = api.kv_retain(shape, api.RetainParams(), dev_tensor(q_obs, "bf16"),
                        dev_tensor(k, "bf16"), dev_tensor(v, "bf16"))
    torch.cuda.synchronize()
    keep = res["keep_idx"].cpu().numpy()[0, 0]
    if n_sink + n_recent + n_keep >= L:
        want = np.arange(L)
    else:
        want = np.array(list(range(n_sink)) + list(range(n_sink, n_sink + n_keep)) +
                        list(range(L - n_recent, L)))
    np.testing.assert_array_equal(keep, want)
    o_keep, _, _ = O.kv_retain_slice(synth.bf16_bits_to_f32(q_obs)[0], np.zeros((L, d)),
                                     n_sink, n_recent, n_keep)
    np.testing.assert_array_equal(o_keep, want)
    # the kept rows are gathered bit for bit
    got_v = res["v_out"].cpu().view(torch.int16).numpy().view(np.uint16)[0, 0]
    np.testing.assert_array_equal(got_v, v[0, 0][want].view(np.uint16))
