"""The whole path under HIP graph capture: every call enqueues on the caller's
stream, allocates nothing and never synchronises the host, so a prefill layer
(entropy_score -> allocate_budget -> select_blocks -> sparse_prefill_attn) and
a decode step (kv_retain -> sparse_decode_attn) can each be captured once and
replayed.  Every replay must reproduce the eager outputs bit for bit; outputs
are cleared eagerly, with synchronisations, between replays."""
import numpy as np
import pytest
import torch

from _parity import dev_tensor, log, prefill_shape
from entropy_guided_sparse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _capture(fn):
    # warm up on a side stream of default priority, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, refs, n=3):
    for rep in range(n):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, refs)):
            assert torch.equal(t, r), f"replay {rep}: output {i} differs from the eager run"


def test_prefill_layer_graph_replays(api):
    L = api.L
    cfg = synth.small_prefill_config(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8192,
                                     block_size=128, segment_size=2048, probe_len=64,
                                     head_types="fraction", hot_count="8", hot_dist="zipf1.2")
    log(f"[graph] prefill {cfg.name} Hq={cfg.n_q_heads} N={cfg.seq_len}")
    inp = synth.make_prefill(cfg, 0)
    shape = prefill_shape(api, cfg)
    q, k, v = (dev_tensor(x, cfg.dtype) for x in (inp.q_store, inp.k_store, inp.v_store))
    Hq, CS, CB = cfg.n_q_heads, cfg.n_segments, cfg.n_blocks
    dev = q.device
    pol = api.BudgetPolicy(mode=L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.05, frac_dynamic=0.3,
                           entropy_threshold=0.5)
    scores = torch.empty((Hq, CS, CB), dtype=torch.float32, device=dev)
    E = torch.empty((Hq, CS), dtype=torch.float32, device=dev)
    rigid = torch.empty((Hq,), dtype=torch.int8, device=dev)
    budget = torch.empty((Hq, CS), dtype=torch.int32, device=dev)
    idx = torch.empty((Hq, CS, CB), dtype=torch.int32, device=dev)
    cnt = torch.empty((Hq, CS), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((Hq, cfg.seq_len), dtype=torch.float32, device=dev)
    import ctypes
    sc = shape.c()
    ws = torch.empty(L.LIB.egs_entropy_score_workspace(ctypes.byref(sc)), dtype=torch.uint8,
                     device=dev)
    aws = torch.empty(max(256, L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc))),
                      dtype=torch.uint8, device=dev)

    def layer():
        api.entropy_score(shape, q, k, block_scores=scores, entropy=E, workspace=ws)
        api.allocate_budget(shape, pol, E, head_is_rigid=rigid, budget=budget)
        api.select_blocks(shape, scores, budget, CB, block_idx=idx, block_cnt=cnt)
        api.sparse_prefill_attn(shape, q, k, v, idx, cnt, out=out, lse=lse, workspace=aws)

    outs = [scores, E, rigid, budget, idx, cnt, out, lse]
    layer()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    assert int(cnt.sum()) > 0
    g = _capture(layer)
    _replays_match(g, outs, refs)


def test_decode_step_graph_replays(api):
    L = api.L
    B, Hq, Hkv, d, Lc, W = 2, 8, 2, 128, 4096, 64
    cfg = synth.DecodeConfig("graph", B, Hq, Hkv, d, Lc, W, 4, 256, 512, "bf16", 0.01)
    log(f"[graph] decode B={B} Hq={Hq} L={Lc}")
    inp = synth.make_decode(cfg, seed=3)
    shape = api.DecodeShape(B, Hq, Hkv, d, Lc, W, 4, 256, 512)
    prm = api.RetainParams(entropy_kind=L.EGS_SHANNON, zeta=0.5, tau=1.0)
    qo, k, v, qn = (dev_tensor(x, "bf16") for x in (inp.q_obs_store, inp.k_store, inp.v_store,
                                                   inp.q_new_store))
    import ctypes
    dsc = shape.c()
    n_total = api.kv_retain_total(shape)
    dws = torch.empty(L.LIB.egs_kv_retain_workspace(ctypes.byref(dsc)), dtype=torch.uint8,
                      device=qo.device)
    aws = torch.empty(max(256, L.LIB.egs_sparse_decode_attn_workspace(ctypes.byref(dsc),
                                                                      n_total)),
                      dtype=torch.uint8, device=qo.device)
    out = torch.empty_like(qn)
    held = {}

    def step():
        res = api.kv_retain(shape, prm, qo, k, v, workspace=dws, want_scores=True)
        api.sparse_decode_attn(shape, qn, res["k_out"], res["v_out"], out=out, workspace=aws)
        held["res"] = res

    step()
    torch.cuda.synchronize()
    r0 = held["res"]
    refs = [r0["keep_idx"].clone(), r0["k_out"].clone(), r0["v_out"].clone(),
            r0["head_entropy"].clone(), r0["scores"].clone(), out.clone()]
    g = _capture(step)
    r = held["res"]   # the tensors the captured calls write into
    outs = [r["keep_idx"], r["k_out"], r["v_out"], r["head_entropy"], r["scores"], out]
    _replays_match(g, outs, refs)
    assert np.all(np.diff(refs[0].cpu().numpy(), axis=-1) > 0)


def test_fused_scoring_split_topk_and_chunk_prune_graph_replays(api):
    """The fused scoring call, a 65,536-entry retention row (the split top-k)
    and chunk pruning with device-side chunk bounds, captured together."""
    L = api.L
    cfg = synth.small_prefill_config(n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8192,
                                     block_size=128, segment_size=2048, probe_len=64,
                                     head_types="fraction", hot_count="8", hot_dist="zipf1.2")
    inp = synth.make_prefill(cfg, 1)
    shape = prefill_shape(api, cfg)
    q, k = (dev_tensor(x, cfg.dtype) for x in (inp.q_store, inp.k_store))
    pol = api.BudgetPolicy(mode=L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.05, frac_dynamic=0.3,
                           entropy_threshold=0.5)
    import ctypes
    sc = shape.c()
    ws = torch.empty(L.LIB.egs_entropy_score_workspace(ctypes.byref(sc)), dtype=torch.uint8,
                     device=q.device)
    dc = synth.DecodeConfig("graph2", 1, 8, 2, 128, 65536, 64, 4, 256, 2048, "bf16", 0.01)
    dinp = synth.make_decode(dc, seed=4)
    dshape = api.DecodeShape(1, 8, 2, 128, 65536, 64, 4, 256, 2048)
    qo, kk, vv = (dev_tensor(x, "bf16") for x in (dinp.q_obs_store, dinp.k_store,
                                                 dinp.v_store))
    prm = api.RetainParams(entropy_kind=L.EGS_SHANNON, zeta=0.5, tau=1.0)
    dws = torch.empty(L.LIB.egs_kv_retain_workspace(ctypes.byref(dshape.c())),
                      dtype=torch.uint8, device=q.device)
    chunks = torch.from_numpy(synth.prune_chunks(65536, 64, 40, seed=4).astype(np.int32)).cuda()
    pws = torch.empty(L.LIB.egs_chunk_prune_workspace(ctypes.byref(dshape.c()), 40),
                      dtype=torch.uint8, device=q.device)
    held = {}

    def work():
        held["sel"] = api.score_select(shape, pol, q, k, 40, workspace=ws)
        held["ret"] = api.kv_retain(dshape, prm, qo, kk, vv, workspace=dws, gather=False)
        held["pr"] = api.chunk_prune(dshape, qo[0], kk[0], chunks, 0.1, 0.5, 0.1, 4, 20000,
                                     workspace=pws)

    def outputs():
        s, r, p = held["sel"], held["ret"], held["pr"]
        return [s["block_scores"], s["entropy"], s["budget"], s["block_idx"], s["block_cnt"],
                r["keep_idx"], p[0], p[1], p[2]]

    log("[graph] fused scoring + 64k retention row + chunk pruning")
    work()
    torch.cuda.synchronize()
    refs = [t.clone() for t in outputs()]
    assert int(refs[7].item()) >= 0
    g = _capture(work)
    _replays_match(g, outputs(), refs)
