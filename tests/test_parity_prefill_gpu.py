"""GPU parity of the prefill path (entropy_score -> allocate_budget ->
select_blocks -> sparse_prefill_attn) against the float64 oracle, through
the C ABI, on seeded inputs small enough for the oracle to run in full."""
import math

import numpy as np
import pytest
import torch

from _parity import (ATTN_MAX_ABS, ATTN_REL_L2, ENTROPY_ATOL, SCORE_ATOL, attn_errors,
                     dev_tensor, list_violations, log, prefill_shape)
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _policy(api, mode, **kw):
    return api.BudgetPolicy(mode=mode, **kw)


def _oracle_budget(E, cfg, pol):
    return O.allocate_budget(E, cfg.segment_size, cfg.block_size, pol.mode, frac=pol.frac,
                             frac_rigid=pol.frac_rigid, frac_dynamic=pol.frac_dynamic,
                             frac_min=pol.frac_min, frac_max=pol.frac_max,
                             entropy_threshold=pol.entropy_threshold,
                             base_tokens=pol.base_tokens, alg3_alpha=pol.alg3_alpha,
                             alg3_delta_t=pol.alg3_delta_t)


def run_pipeline(api, cfg, pol, seed=0, kind=0, alpha=2.0, attn_blocks=None, inp=None):
    log(f"[prefill parity] {cfg.name} seed={seed} kind={kind} mode={pol.mode} "
        f"Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} d={cfg.head_dim} N={cfg.seq_len} "
        f"LB={cfg.block_size} LS={cfg.segment_size} P={cfg.probe_len} {cfg.dtype}")
    if inp is None:
        inp = synth.make_prefill(cfg, seed)
    shape = prefill_shape(api, cfg)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    v = dev_tensor(inp.v_store, cfg.dtype)
    LS, LB = cfg.segment_size, cfg.block_size
    CB = cfg.seq_len // LB

    scores, E = api.entropy_score(shape, q, k, kind=kind, renyi_alpha=alpha)
    rigid, budget = api.allocate_budget(shape, pol, E)
    idx, cnt = api.select_blocks(shape, scores, budget, CB)
    out, lse = api.sparse_prefill_attn(shape, q, k, v, idx, cnt, return_lse=True)
    torch.cuda.synchronize()
    g_scores = scores.cpu().numpy()
    g_E = E.cpu().numpy()
    g_rigid = rigid.cpu().numpy().astype(bool)
    g_budget = budget.cpu().numpy()
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()

    # steps 1-5
    r_scores, r_E = O.entropy_score(inp.q, inp.k, LS, LB, cfg.probe_len, kind=kind, alpha=alpha)
    ds = np.abs(g_scores - r_scores).max()
    dE = np.abs(g_E - r_E).max()
    log(f"  scores max|d|={ds:.3e}  entropy max|d|={dE:.3e}")
    assert ds <= SCORE_ATOL
    assert dE <= ENTROPY_ATOL
    # steps 6-7: bit-exact on identical entropies
    o_rigid, o_budget = _oracle_budget(g_E.astype(np.float64), cfg, pol)
    np.testing.assert_array_equal(g_rigid, o_rigid)
    np.testing.assert_array_equal(g_budget, o_budget)
    # step 8: bit-exact on identical scores, band rule against the oracle's scores
    o_idx, o_cnt = O.select_blocks(g_scores.astype(np.float64), g_budget, LS, LB, k_max=CB)
    np.testing.assert_array_equal(g_cnt, o_cnt)
    np.testing.assert_array_equal(g_idx, o_idx)
    bad = list_violations(g_idx, g_cnt, r_scores, g_budget, LS, LB)
    assert not bad, bad[:5]
    # steps 9-10 on the GPU's own lists
    g_out = out.float().cpu().numpy()
    g_lse = lse.cpu().numpy()
    if attn_blocks is None:
        r_out, r_lse = O.sparse_prefill_attn(inp.q, inp.k, inp.v, g_idx, g_cnt, LS, LB)
        ma, rel = attn_errors(g_out, r_out)
        dl = np.abs(g_lse - r_lse) - 2e-6 * np.abs(r_lse)
    else:
        ma, rel, dl = 0.0, 0.0, np.zeros(1)
        num = den = 0.0
        for (h, b) in attn_blocks:
            ro, rl = O.sparse_prefill_attn_rows(inp.q, inp.k, inp.v, g_idx, g_cnt, h, b, LS, LB)
            go = g_out[h, b * LB:(b + 1) * LB]
            ma = max(ma, float(np.abs(go - ro).max()))
            num += float(((go - ro) ** 2).sum())
            den += float((ro ** 2).sum())
            dl = np.maximum(dl.max(), (np.abs(g_lse[h, b * LB:(b + 1) * LB] - rl)
                                       - 2e-6 * np.abs(rl)).max())
        rel = math.sqrt(num / den)
    log(f"  attention max|d|={ma:.3e} relL2={rel:.3e} lse excess={float(np.max(dl)):.3e}")
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2
    assert float(np.max(dl)) <= 1e-3
    return dict(inp=inp, scores=g_scores, E=g_E, budget=g_budget, idx=g_idx, cnt=g_cnt,
                out=out, lse=g_lse, r_scores=r_scores, r_E=r_E, q=q, k=k, v=v, shape=shape)


def test_tiny_fp32_workload_fixed_quarter(api):
    cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    res = run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.25))
    assert res["budget"].tolist() == [[2, 4, 6, 8]] * 4
    # planted structure recovered on the GPU
    inp = res["inp"]
    for h in range(cfg.n_q_heads):
        for s in range(cfg.n_segments):
            sel = set(res["idx"][h, s, :res["cnt"][h, s]].tolist())
            if inp.rigid_hs[h, s]:
                assert 0 in sel
            else:
                assert set(inp.hot_blocks[(h, s)].tolist()) <= sel


def test_tiny_fp32_workload_alg3(api):
    cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_ALG3, base_tokens=512.0,
                                   entropy_threshold=1e-5))


def test_tiny_generic_shape_bf16(api):
    cfg = synth.small_prefill_config(head_dim=16, seq_len=256, block_size=16, segment_size=64,
                                     probe_len=8)
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.5), seed=1)


def test_tiny_generic_shape_fp32(api):
    cfg = synth.small_prefill_config(head_dim=16, seq_len=256, block_size=16, segment_size=64,
                                     probe_len=8, dtype="f32")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.5), seed=2)


def test_mfma_d128_two_level_several_tiles(api):
    cfg = synth.small_prefill_config(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8192,
                                     block_size=128, segment_size=2048, probe_len=64,
                                     head_types="fraction", hot_count="8", hot_dist="zipf1.2")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.05,
                                   frac_dynamic=0.3, entropy_threshold=0.5), seed=0)


def test_mfma_d128_renyi2(api):
    cfg = synth.small_prefill_config(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8192,
                                     block_size=128, segment_size=2048, probe_len=64,
                                     head_types="fraction", hot_count="8", hot_dist="zipf1.2")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.05,
                                   frac_dynamic=0.3, entropy_threshold=0.5), seed=1,
                 kind=api.L.EGS_RENYI, alpha=2.0)


def test_mfma_d64_block64_proportional_ragged_probe(api):
    cfg = synth.small_prefill_config(n_q_heads=6, n_kv_heads=3, head_dim=64, seq_len=4096,
                                     block_size=64, segment_size=512, probe_len=40,
                                     head_types="per_segment", hot_count="poisson4")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_PROPORTIONAL, frac_min=0.02,
                                   frac_max=0.5), seed=3)


def test_mfma_d128_block64(api):
    cfg = synth.small_prefill_config(n_q_heads=4, n_kv_heads=1, head_dim=128, seq_len=4096,
                                     block_size=64, segment_size=1024, probe_len=64,
                                     head_types="fraction", hot_count="2")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.3), seed=4)


def test_mfma_d64_block128(api):
    cfg = synth.small_prefill_config(n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=4096,
                                     block_size=128, segment_size=1024, probe_len=33,
                                     head_types="fraction", hot_count="2")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.4), seed=5)


# The attention's work queues: one per (XCD, head of the KV group), 8 r of
# them, while 8 r fits the 128 counters the workspace holds; r = 16 uses every
# counter, r = 17 falls back to one queue (H_kv * C_B is a multiple of 8 in
# both, so only r decides).
@pytest.mark.parametrize("n_q_heads", [32, 34])
def test_mfma_work_queue_edges(api, n_q_heads):
    cfg = synth.small_prefill_config(n_q_heads=n_q_heads, n_kv_heads=2, head_dim=128,
                                     seq_len=2048, block_size=64, segment_size=1024,
                                     probe_len=32, head_types="fraction", hot_count="2")
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.3), seed=12)


@pytest.mark.parametrize("case", ["one_block_segments", "single_segment", "probe_whole",
                                  "probe_one", "no_xcd_remap"])
def test_degenerate_shapes(api, case):
    kw = dict(n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=1024, block_size=64,
              segment_size=256, probe_len=32, head_types="fraction", hot_count="2")
    if case == "one_block_segments":      # C_B(s) = s + 1
        kw.update(segment_size=64, probe_len=16, seq_len=512)
    elif case == "single_segment":
        kw.update(segment_size=1024)
    elif case == "probe_whole":
        kw.update(probe_len=256)
    elif case == "probe_one":
        kw.update(probe_len=1)
    elif case == "no_xcd_remap":          # H_kv * C_B not a multiple of 8
        kw.update(n_q_heads=3, n_kv_heads=1, head_dim=128, seq_len=768, block_size=128)
    cfg = synth.small_prefill_config(**kw)
    run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.5), seed=6)


def test_full_budget_equals_dense_attention(api):
    cfg = synth.small_prefill_config(n_q_heads=4, n_kv_heads=2, head_dim=128, seq_len=2048,
                                     block_size=128, segment_size=512, probe_len=64,
                                     head_types="fraction", hot_count="2")
    res = run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=1.0), seed=7)
    inp = res["inp"]
    dense = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(inp.q.astype(np.float64))[None],
        torch.from_numpy(np.repeat(inp.k, 2, axis=0).astype(np.float64))[None],
        torch.from_numpy(np.repeat(inp.v, 2, axis=0).astype(np.float64))[None],
        is_causal=True)[0].numpy()
    ma, rel = attn_errors(res["out"].float().cpu().numpy(), dense)
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


def test_empty_lists_attend_diagonal_only(api):
    cfg = synth.small_prefill_config(n_q_heads=4, n_kv_heads=2, head_dim=128, seq_len=2048,
                                     block_size=128, segment_size=512, probe_len=64,
                                     head_types="fraction", hot_count="2")
    inp = synth.make_prefill(cfg, 8)
    shape = prefill_shape(api, cfg)
    q, k, v = (dev_tensor(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    CS, CB = cfg.n_segments, cfg.n_blocks
    idx = torch.full((4, CS, 3), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((4, CS), dtype=torch.int32, device="cuda")
    out = api.sparse_prefill_attn(shape, q, k, v, idx, cnt)
    torch.cuda.synchronize()
    r_out, _ = O.sparse_prefill_attn(inp.q, inp.k, inp.v, idx.cpu().numpy(), cnt.cpu().numpy(),
                                     cfg.segment_size, cfg.block_size)
    ma, rel = attn_errors(out.float().cpu().numpy(), r_out)
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2


@pytest.mark.parametrize("jump", [8.0, 60.0])
def test_logit_jumps_after_the_first_block(api, jump):
    # Every block listed, ascending.  Keys of some blocks are scaled by `jump`,
    # so rows meet logits far above the maximum of their first block: x8 (up
    # to ~35 in log2 units) makes the MFMA kernel raise its running maximum
    # mid-list and rescale O; x60 (~260) lies beyond the fp32 range of the
    # probabilities, so the rescale factor underflows to zero and the earlier
    # blocks drop out, as they do in float64.  Both must match the oracle.
    Hq, Hkv, d, N, LB, LS = 4, 2, 128, 2048, 128, 512
    CS, CB = N // LS, N // LB
    rng = np.random.default_rng(31)
    q = rng.standard_normal((Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((Hkv, N, d)).astype(np.float32)
    for g, blk in ((0, 3), (1, 5), (1, 9)):
        k[g, blk * LB:(blk + 1) * LB] *= jump
    qt, kt, vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    q64, k64, v64 = (x.double().numpy() for x in (qt, kt, vt))
    log(f"[prefill parity] logit jump x{jump} Hq={Hq} Hkv={Hkv} d={d} N={N} LB={LB} LS={LS}")
    cfg = synth.small_prefill_config(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, seq_len=N,
                                     block_size=LB, segment_size=LS, probe_len=64)
    shape = prefill_shape(api, cfg)
    idx = np.full((Hq, CS, CB), -1, dtype=np.int32)
    cnt = np.zeros((Hq, CS), dtype=np.int32)
    for s_ in range(CS):
        cb = (s_ + 1) * LS // LB
        idx[:, s_, :cb] = np.arange(cb)
        cnt[:, s_] = cb
    out, lse = api.sparse_prefill_attn(shape, qt.cuda(), kt.cuda(), vt.cuda(),
                                       torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                                       return_lse=True)
    torch.cuda.synchronize()
    r_out, r_lse = O.sparse_prefill_attn(q64, k64, v64, idx, cnt, LS, LB)
    ma, rel = attn_errors(out.float().cpu().numpy(), r_out)
    g_lse = lse.cpu().numpy()
    dl = float((np.abs(g_lse - r_lse) - 2e-6 * np.abs(r_lse)).max())
    log(f"  attention max|d|={ma:.3e} relL2={rel:.3e} lse excess={dl:.3e}")
    assert np.isfinite(g_lse).all()
    assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2
    assert dl <= 1e-3


def test_select_zero_and_clamped_budgets(api):
    cfg = synth.small_prefill_config(n_q_heads=2, n_kv_heads=1, head_dim=64, seq_len=1024,
                                     block_size=64, segment_size=256, probe_len=32,
                                     head_types="fraction", hot_count="2")
    shape = prefill_shape(api, cfg)
    CS, CB = cfg.n_segments, cfg.n_blocks
    rng = np.random.default_rng(9)
    sc = np.full((2, CS, CB), -1.0, dtype=np.float32)
    for s in range(CS):
        cb = (s + 1) * 4
        sc[:, s, :cb] = np.round(rng.random((2, cb)) * 4) / 4   # heavy ties
    bud = np.array([[0, 1, 100, 7], [4, 8, 12, 16]], dtype=np.int32)
    idx, cnt = api.select_blocks(shape, torch.from_numpy(sc).cuda(), torch.from_numpy(bud).cuda(), 10)
    torch.cuda.synchronize()
    o_idx, o_cnt = O.select_blocks(sc.astype(np.float64), bud, cfg.segment_size, cfg.block_size,
                                   k_max=10)
    np.testing.assert_array_equal(cnt.cpu().numpy(), o_cnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)


def test_outputs_are_deterministic(api):
    cfg = synth.small_prefill_config(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=4096,
                                     block_size=128, segment_size=1024, probe_len=64,
                                     head_types="fraction", hot_count="2")
    inp = synth.make_prefill(cfg, 10)
    shape = prefill_shape(api, cfg)
    q, k, v = (dev_tensor(x, "bf16") for x in (inp.q_store, inp.k_store, inp.v_store))
    pol = _policy(api, api.L.EGS_BUDGET_TWO_LEVEL)
    outs = []
    for _ in range(2):
        sc, E = api.entropy_score(shape, q, k)
        _, bud = api.allocate_budget(shape, pol, E)
        idx, cnt = api.select_blocks(shape, sc, bud, cfg.n_blocks)
        o = api.sparse_prefill_attn(shape, q, k, v, idx, cnt)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (sc, E, bud, idx, cnt, o)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def run_maxmin(api, cfg, seed=0, kind=0, alpha=2.0):
    """MAXMIN observation rows ([EI] Alg. 1-2) against the oracle, then the
    budget and selection steps on them."""
    log(f"[maxmin parity] {cfg.name} seed={seed} kind={kind} Hq={cfg.n_q_heads} "
        f"Hkv={cfg.n_kv_heads} d={cfg.head_dim} N={cfg.seq_len} LB={cfg.block_size} "
        f"LS={cfg.segment_size} {cfg.dtype}")
    inp = synth.make_prefill(cfg, seed)
    shape = prefill_shape(api, cfg)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    LS, LB = cfg.segment_size, cfg.block_size
    CB = cfg.seq_len // LB
    scores, E = api.entropy_score(shape, q, k, kind=kind, renyi_alpha=alpha,
                                  pool=api.L.EGS_POOL_MAXMIN)
    pol = _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.3)
    rigid, budget = api.allocate_budget(shape, pol, E)
    idx, cnt = api.select_blocks(shape, scores, budget, CB)
    torch.cuda.synchronize()
    g_scores, g_E = scores.cpu().numpy(), E.cpu().numpy()
    r_scores, r_E = O.entropy_score(inp.q, inp.k, LS, LB, cfg.probe_len, kind=kind,
                                    alpha=alpha, pool="maxmin")
    ds = float(np.abs(g_scores - r_scores).max())
    dE = float(np.abs(g_E - r_E).max())
    log(f"  scores max|d|={ds:.3e}  entropy max|d|={dE:.3e}")
    assert ds <= SCORE_ATOL and dE <= ENTROPY_ATOL
    o_rigid, o_budget = _oracle_budget(g_E.astype(np.float64), cfg, pol)
    np.testing.assert_array_equal(budget.cpu().numpy(), o_budget)
    o_idx, o_cnt = O.select_blocks(g_scores.astype(np.float64), o_budget, LS, LB, k_max=CB)
    np.testing.assert_array_equal(cnt.cpu().numpy(), o_cnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)


@pytest.mark.parametrize("case", ["tiny_f32", "tiny_f32_renyi", "d16_bf16", "d16_f32",
                                  "d128_two_chunks", "d64_block64", "d32_ragged_chunk",
                                  "one_block_segments"])
def test_maxmin_observation_rows(api, case):
    if case.startswith("tiny_f32"):
        cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    else:
        kw = dict(d16_bf16=dict(head_dim=16, seq_len=256, block_size=16, segment_size=64),
                  d16_f32=dict(head_dim=16, seq_len=256, block_size=16, segment_size=64,
                               dtype="f32"),
                  # L_S = 2048: two pooled query chunks of 1024 rows per segment
                  d128_two_chunks=dict(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8192,
                                       block_size=128, segment_size=2048,
                                       head_types="fraction", hot_count="8",
                                       hot_dist="zipf1.2"),
                  d64_block64=dict(n_q_heads=6, n_kv_heads=3, head_dim=64, seq_len=4096,
                                   block_size=64, segment_size=512,
                                   head_types="per_segment", hot_count="poisson4"),
                  # L_S / L_B = 3: query chunks of 48 rows, fewer than the row phases
                  d32_ragged_chunk=dict(head_dim=32, seq_len=576, block_size=16,
                                        segment_size=48, probe_len=16),
                  one_block_segments=dict(segment_size=64, probe_len=16, seq_len=512))[case]
        cfg = synth.small_prefill_config(**kw)
    kind = api.L.EGS_RENYI if case.endswith("renyi") else api.L.EGS_SHANNON
    run_maxmin(api, cfg, seed=7, kind=kind)


@pytest.mark.parametrize("LB,N,LS", [(64, 65536, 8192), (128, 131072, 16384)])
def test_mfma_lists_longer_than_one_lds_stage(api, LB, N, LS):
    # FIXED 60% of the causal blocks: the last segment lists 615 of its 1,024
    # blocks and the one before it 538 of 896, more than the 512 entries the
    # MFMA attention kernel stages in LDS at a time, so every query block of
    # those segments walks its list across a refill (EntropyInfer Alg. 3 lets
    # budgets reach 3 B_h, App. A eq. (3)).  Sampled query blocks of both
    # segments, every head, against the oracle on the GPU's lists.
    cfg = synth.small_prefill_config(name="long-lists", n_q_heads=4, n_kv_heads=2,
                                     head_dim=128, seq_len=N, block_size=LB, segment_size=LS,
                                     probe_len=64)
    CB, bps = N // LB, LS // LB
    blocks = [(h, b) for h in range(4)
              for b in (CB - 1, CB - bps, CB - bps // 2, CB - bps - 1)]
    res = run_pipeline(api, cfg, _policy(api, api.L.EGS_BUDGET_FIXED, frac=0.6), seed=4,
                       attn_blocks=blocks)
    assert res["cnt"][:, -1].min() == 615 and res["cnt"][:, -2].min() == 538
