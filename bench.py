#!/usr/bin/env python3
"""Benchmark of the entropy-guided sparse prefill path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  prefill layer (Llama-3-8B-shaped, 32/8 heads, d 128, 128k tokens, bf16):
      entropy_score -> allocate_budget -> select_blocks -> sparse_prefill_attn
  decode retention (batch 8, 32/8 heads, d 128, 128k-token cache, bf16):
      kv_retain -> sparse_decode_attn
Inputs are generated once and are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the executed-block attention throughput of
the prefill layer (FLOPs of every listed (head, query block, key block) tile,
4 * L_B^2 * d each) divided by the prefill layer time (all four calls).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama3-8b-128k")
    ap.add_argument("--entropy", default="shannon", choices=["shannon", "renyi2"])
    ap.add_argument("--no-decode", action="store_true", help="time the prefill layer only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other prefill workloads (32k, Qwen 64k, the other entropy)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time spent on the oracle sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB (a known-size kernel "
                         "that scales HBM byte counters taken under a profiler)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_policy(api, cfg):
    L = api.L
    if cfg.name == "tiny-2k-f32":
        return api.BudgetPolicy(mode=L.EGS_BUDGET_FIXED, frac=0.25, entropy_threshold=0.5)
    if cfg.name == "qwen-64k":
        return api.BudgetPolicy(mode=L.EGS_BUDGET_PROPORTIONAL, frac_min=0.02, frac_max=0.5,
                                entropy_threshold=0.5)
    return api.BudgetPolicy(mode=L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.05, frac_dynamic=0.30,
                            entropy_threshold=0.5)


def k_max_for(pol, api, CB, LB):
    L = api.L
    if pol.mode == L.EGS_BUDGET_FIXED:
        f = pol.frac
    elif pol.mode == L.EGS_BUDGET_TWO_LEVEL:
        f = max(pol.frac_rigid, pol.frac_dynamic)
    elif pol.mode == L.EGS_BUDGET_PROPORTIONAL:
        f = pol.frac_max
    else:
        return min(CB, int(math.ceil(3 * pol.base_tokens / LB)) + 1)
    return max(1, min(CB, int(math.ceil(f * CB)) + 1))


def executed_tiles(idx, cnt, CS, CB, LB, LS):
    """Listed (head, query block, key block) tiles incl. the own block, and the
    same count with the own block's causal half (for the exact-causal figure)."""
    Hq = cnt.shape[0]
    bps = LS // LB
    total = 0
    for h in range(Hq):
        for s in range(CS):
            sel = np.sort(idx[h, s, :cnt[h, s]])
            b = np.arange(s * bps, (s + 1) * bps)
            total += int(np.searchsorted(sel, b, side="left").sum()) + len(b)
    return total


def union_overlap(idx, cnt, Hkv):
    """UOR of the GQA groups' block lists ([EP] Sec. 7): per (KV group,
    segment), the blocks any head of the group selected over the most any one
    head selected (1 <= UOR <= r); and the distinct blocks of the groups over
    the heads' listed blocks (the share of block reads a group must fetch)."""
    Hq, CS = cnt.shape
    r = Hq // Hkv
    uors, uni, tot = [], 0, 0
    for g in range(Hkv):
        for s in range(CS):
            sets = [idx[h, s, :cnt[h, s]] for h in range(g * r, (g + 1) * r)]
            u = np.unique(np.concatenate(sets)).size
            uors.append(u / max(1, max(x.size for x in sets)))
            uni += u
            tot += sum(x.size for x in sets)
    return {"mean": round(float(np.mean(uors)), 3), "max": round(float(np.max(uors)), 3),
            "distinct_share": round(uni / max(1, tot), 4)}


def scoring_bytes(cfg, k_max, elt):
    Hq, Hkv, d, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len
    CS, CB = cfg.n_segments, cfg.n_blocks
    return (Hkv * N * d * elt                 # K read once
            + Hq * CS * cfg.probe_len * d * elt   # probe queries
            + Hq * CS * CB * 4                # observation rows written
            + Hq * CS * 4 * 2                 # entropy, budgets
            + Hq * CS * k_max * 4 + Hq * CS * 4)  # block lists, counts


TRAFFIC_FILE = "traffic_sparse_attn_llama3-8b-128k.txt"
ATTN_SOURCES = ("entropy_guided_sparse_amd/csrc/attn.hip", "entropy_guided_sparse_amd/csrc/egs_device.h")


def attn_source_hash():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name):
    """HBM bytes per launch of the attention kernel from the stored counter summary,
    or None if there is none or the kernel's source has changed since it was taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", TRAFFIC_FILE)
    if cfg_name != "llama3-8b-128k" or not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        m = line.strip().strip("`").split(":", 1)
        if len(m) == 2 and m[0].strip() in ("bytes_per_launch", "source_sha256_16"):
            rec[m[0].strip()] = m[1].strip()
    if rec.get("source_sha256_16") != attn_source_hash() or "bytes_per_launch" not in rec:
        return None
    return int(rec["bytes_per_launch"])


def back_to_back(torch, fn, flush, reps):
    """Median GPU time (ms) of fn() with no event inside it; a 512 MiB write
    before each repetition evicts the Infinity Cache, so K streams from HBM."""
    times = []
    for rep in range(reps + 1):
        flush.fill_(rep & 0x7F)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        times.append((ev0, ev1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in times[1:]]))


def prefill_workload(api, torch, dev, cfg, inp, kind, steps, flush, dev_qkv=None):
    """One prefill layer of `cfg` on its own: the fused scoring call and the
    attention, each timed back to back (median of `steps`, Infinity Cache
    evicted before each repetition); executed tiles from the GPU's lists."""
    L = api.L
    if dev_qkv is None:
        to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).to(dev)
        q, k, v = to(inp.q_store), to(inp.k_store), to(inp.v_store)
    else:
        q, k, v = dev_qkv
    shape = api.PrefillShape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                             cfg.block_size, cfg.segment_size, cfg.probe_len, torch.bfloat16)
    pol = prefill_policy(api, cfg)
    Hq, CS, CB, LB, LS, d = (cfg.n_q_heads, cfg.n_segments, cfg.n_blocks, cfg.block_size,
                             cfg.segment_size, cfg.head_dim)
    k_max = k_max_for(pol, api, CB, LB)
    import ctypes
    sc = shape.c()
    ws = torch.empty(L.LIB.egs_entropy_score_workspace(ctypes.byref(sc)), dtype=torch.uint8,
                     device=dev)
    aws = torch.empty(max(256, L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc))),
                      dtype=torch.uint8, device=dev)
    res = api.score_select(shape, pol, q, k, k_max, kind=kind, renyi_alpha=2.0, workspace=ws)
    out = torch.empty_like(q)

    def scoring():
        api.score_select(shape, pol, q, k, k_max, kind=kind, renyi_alpha=2.0, out=res,
                         workspace=ws)

    def attention():
        api.sparse_prefill_attn(shape, q, k, v, res["block_idx"], res["block_cnt"], out=out,
                                workspace=aws)

    scoring()
    attention()
    torch.cuda.synchronize()
    tiles = executed_tiles(res["block_idx"].cpu().numpy(), res["block_cnt"].cpu().numpy(),
                           CS, CB, LB, LS)
    t_s = back_to_back(torch, scoring, flush, steps)
    t_a = back_to_back(torch, attention, flush, steps)
    sbytes = scoring_bytes(cfg, k_max, 2)
    flops = tiles * 4.0 * LB * LB * d
    gbs = sbytes / (t_s * 1e-3) / 1e9
    tf = flops / (t_a * 1e-3) / 1e12
    del q, k, v, out, ws, aws, res
    return {"entropy": "renyi2" if kind == L.EGS_RENYI else "shannon",
            "ms_per_layer": round(t_s + t_a, 3), "scoring_us": round(t_s * 1e3, 1),
            "attention_ms": round(t_a, 3),
            "scoring_gbps": round(gbs, 1), "scoring_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "attention_tflops_executed": round(tf, 1),
            "attention_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "effective_tflops": round(flops / ((t_s + t_a) * 1e-3) / 1e12, 1),
            "tile_density": round(tiles / (Hq * CB * (CB + 1) // 2), 4)}


def calib_copy(torch, dev, mib):
    """One elementwise copy of `mib` MiB (read mib, write mib): torch.neg on fp32."""
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    log(f"calibration copy: {mib} MiB read + {mib} MiB written by one torch.neg kernel")
    del x, y


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, idx, cnt, seconds, pol=None, k_max=None, decode_cfg=None,
                 gpu_ms=None):
    """The float64 oracle on the host cores, stage by stage, on the step's
    inputs: scoring, budgets and selection on the whole prefill layer; the
    attention on a seeded sample of (head, query block) pairs; retention and
    decode attention on one (batch, KV group) slice of the decode workload.
    Sampled stages are scaled to the whole workload by their share of it."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import egs_oracle as O
    from entropy_guided_sparse_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    Hq, CB, LB, LS, d = cfg.n_q_heads, cfg.n_blocks, cfg.block_size, cfg.segment_size, cfg.head_dim
    stages = {}

    def stage(name, sec, sample, scale=1.0):
        est = sec * scale
        st = {"seconds": round(sec, 3), "sample": sample, "workload_seconds": round(est, 3)}
        if gpu_ms and gpu_ms.get(name):
            st["gpu_ms"] = round(gpu_ms[name], 4)
            st["gpu_speedup"] = round(est / (gpu_ms[name] * 1e-3), 1)
        stages[name] = st

    if pol is not None:
        t0 = time.perf_counter()
        r_scores, r_E = O.entropy_score(inp.q, inp.k, LS, LB, cfg.probe_len)
        t1 = time.perf_counter()
        pk = dict(frac=pol.frac, frac_rigid=pol.frac_rigid, frac_dynamic=pol.frac_dynamic,
                  frac_min=pol.frac_min, frac_max=pol.frac_max,
                  entropy_threshold=pol.entropy_threshold, base_tokens=pol.base_tokens,
                  alg3_alpha=pol.alg3_alpha, alg3_delta_t=pol.alg3_delta_t)
        _, r_budget = O.allocate_budget(r_E, LS, LB, pol.mode, **pk)
        t2 = time.perf_counter()
        O.select_blocks(r_scores, r_budget, LS, LB, k_max=k_max)
        t3 = time.perf_counter()
        stage("scoring", t1 - t0, "whole layer (pooling, probe rows, entropy)")
        stage("budget", t2 - t1, "whole layer")
        stage("select", t3 - t2, "whole layer")
        if gpu_ms:
            stages["scoring"]["gpu_ms_covers"] = "the fused scoring call: steps 1-8"

    # attention: seeded random (head, query block) pairs, scaled by FLOPs
    rng = np.random.default_rng(0)
    flops = 0.0
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < 512:
        h, b = int(rng.integers(Hq)), int(rng.integers(CB))
        O.sparse_prefill_attn_rows(inp.q, inp.k, inp.v, idx, cnt, h, b, LS, LB)
        nblk = len(O.qblock_list(idx, cnt, h, b, LS, LB))
        flops += 4.0 * LB * LB * d * nblk
        n += 1
    dt = time.perf_counter() - t0
    total_flops = 4.0 * LB * LB * d * executed_tiles(idx, cnt, cfg.n_segments, CB, LB, LS)
    stage("attention", dt, f"{n} seeded random (head, query-block) pairs using the GPU's "
          "block lists; scaled by executed-tile FLOPs", total_flops / flops)

    if decode_cfg is not None:
        dc = decode_cfg
        dinp = synth.make_decode(dc, seed=0, batch=1)
        r = dc.n_q_heads // dc.n_kv_heads
        t0 = time.perf_counter()
        keep, mu, H = O.kv_retain_slice(dinp.q_obs[0, :r], dinp.k[0, 0], dc.n_sink, dc.n_recent,
                                        dc.n_keep)
        t1 = time.perf_counter()
        O.sparse_decode_attn(dinp.q_new[0:1, :r], dinp.k[0:1, 0:1, keep],
                             dinp.v[0:1, 0:1, keep])
        t2 = time.perf_counter()
        slices = dc.batch * dc.n_kv_heads
        stage("kv_retain", t1 - t0, f"one (batch, KV group) slice of {slices}", slices)
        stage("decode_attn", t2 - t1, f"one (batch, KV group) slice of {slices}", slices)
        del dinp
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"float64 oracle sparse attention on {n} seeded random (head, query-block) "
                      f"pairs of the same {cfg.name} layer using the GPU's block lists, "
                      f"{dt:.1f} s; executed-block FLOPs / time",
            "stages": stages}


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of this "
              "build (the path shards by KV head group with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch
    from entropy_guided_sparse_amd import api, synth
    L = api.L
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_dev(store, dtype):
        t = torch.from_numpy(np.ascontiguousarray(store))
        return (t.view(torch.bfloat16) if dtype == "bf16" else t).to(dev)

    # ------------------------------------------------------------------ prefill
    cfg = synth.PREFILL_CONFIGS[args.config]
    t0 = time.perf_counter()
    inp = synth.make_prefill(cfg, seed=0)
    log(f"generated {cfg.name} in {time.perf_counter() - t0:.1f} s")
    q, k, v = (to_dev(x, cfg.dtype) for x in (inp.q_store, inp.k_store, inp.v_store))
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = api.PrefillShape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                             cfg.block_size, cfg.segment_size, cfg.probe_len, tdt)
    pol = prefill_policy(api, cfg)
    Hq, CS, CB, LB, LS, d = (cfg.n_q_heads, cfg.n_segments, cfg.n_blocks, cfg.block_size,
                             cfg.segment_size, cfg.head_dim)
    k_max = k_max_for(pol, api, CB, LB)
    kind = L.EGS_SHANNON if args.entropy == "shannon" else L.EGS_RENYI
    scores = torch.empty((Hq, CS, CB), dtype=torch.float32, device=dev)
    E = torch.empty((Hq, CS), dtype=torch.float32, device=dev)
    rigid = torch.empty((Hq,), dtype=torch.int8, device=dev)
    budget = torch.empty((Hq, CS), dtype=torch.int32, device=dev)
    idx = torch.empty((Hq, CS, k_max), dtype=torch.int32, device=dev)
    cnt = torch.empty((Hq, CS), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    import ctypes
    sc = shape.c()
    ws = torch.empty(L.LIB.egs_entropy_score_workspace(ctypes.byref(sc)), dtype=torch.uint8,
                     device=dev)
    attn_ws = torch.empty(max(256, L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc))),
                          dtype=torch.uint8, device=dev)

    sel_out = {"block_scores": scores, "entropy": E, "head_is_rigid": rigid, "budget": budget,
               "block_idx": idx, "block_cnt": cnt}

    def prefill(evs):
        # steps 1-8 in one call (the same outputs as entropy_score,
        # allocate_budget and select_blocks), then the sparse attention
        evs[0].record()
        api.score_select(shape, pol, q, k, k_max, kind=kind, renyi_alpha=2.0, out=sel_out,
                         workspace=ws)
        evs[1].record()
        evs[2].record()
        evs[3].record()
        api.sparse_prefill_attn(shape, q, k, v, idx, cnt, out=out, workspace=attn_ws)
        evs[4].record()

    # ------------------------------------------------------------------ decode
    decode = None
    if not args.no_decode:
        dcfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
        t0 = time.perf_counter()
        dinp = synth.make_decode(dcfg, seed=0)
        log(f"generated {dcfg.name} in {time.perf_counter() - t0:.1f} s")
        dq, dk, dv, dqn = (to_dev(x, "bf16") for x in (dinp.q_obs_store, dinp.k_store,
                                                      dinp.v_store, dinp.q_new_store))
        del dinp
        dshape = api.DecodeShape(dcfg.batch, dcfg.n_q_heads, dcfg.n_kv_heads, dcfg.head_dim,
                                 dcfg.cache_len, dcfg.n_obs, dcfg.n_sink, dcfg.n_recent,
                                 dcfg.n_keep)
        prm = api.RetainParams(entropy_kind=L.EGS_SHANNON, zeta=0.5, tau=1.0)
        dsc = dshape.c()
        dws = torch.empty(L.LIB.egs_kv_retain_workspace(ctypes.byref(dsc)), dtype=torch.uint8,
                          device=dev)
        n_total = api.kv_retain_total(dshape)
        aws = torch.empty(max(256, L.LIB.egs_sparse_decode_attn_workspace(ctypes.byref(dsc),
                                                                          n_total)),
                          dtype=torch.uint8, device=dev)
        dout = torch.empty_like(dqn)
        decode = dict(cfg=dcfg, shape=dshape, n_total=n_total)
        # page-level retention on the step's group scores: 16-token pages,
        # 256 kept pages per group beyond the sink and recent pages
        pg_S, pg_K = 16, 256
        mu_buf = torch.empty((dcfg.batch, dcfg.n_kv_heads, dcfg.cache_len), dtype=torch.float32,
                             device=dev)
        pg_ws = torch.empty(max(256, L.LIB.egs_page_retain_workspace(
            ctypes.byref(dsc), pg_S, pg_K, L.EGS_PAGE_LAYER_UNION)), dtype=torch.uint8,
            device=dev)

        def decode_step(evs):
            res = api.kv_retain(dshape, prm, dq, dk, dv, workspace=dws)
            evs[5].record()
            api.sparse_decode_attn(dshape, dqn, res["k_out"], res["v_out"], out=dout,
                                   workspace=aws)
            evs[6].record()

    def step(evs):
        prefill(evs)
        if decode is not None:
            decode_step(evs)

    new_events = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()

    # lists are deterministic: count executed tiles once
    g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    tiles = executed_tiles(g_idx, g_cnt, CS, CB, LB, LS)
    dense_tiles = Hq * CB * (CB + 1) // 2
    tile_flops = 4.0 * LB * LB * d

    all_evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(all_evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps

    def mean_ms(a, b):
        return float(np.mean([ev[a].elapsed_time(ev[b]) for ev in all_evs]))

    t_attn_median = float(np.median([ev[3].elapsed_time(ev[4]) for ev in all_evs]))
    t_score = mean_ms(0, 1)
    t_attn = mean_ms(3, 4)
    t_prefill = mean_ms(0, 4)
    kernel_us = {"score_select": 1e3 * t_score, "sparse_prefill_attn": 1e3 * t_attn}
    t_decode = None
    if decode is not None:
        kernel_us["kv_retain"] = 1e3 * mean_ms(4, 5)
        kernel_us["sparse_decode_attn"] = 1e3 * mean_ms(5, 6)
        t_decode = mean_ms(4, 6)

    elt = 2 if cfg.dtype == "bf16" else 4
    sbytes = scoring_bytes(cfg, k_max, elt)
    t_scoring = t_score
    scoring_gbs = sbytes / (t_scoring * 1e-3) / 1e9
    exec_flops = tiles * tile_flops
    attn_tflops = exec_flops / (t_attn * 1e-3) / 1e12
    eff_tflops = exec_flops / (t_prefill * 1e-3) / 1e12
    dense_equiv = dense_tiles * tile_flops / (t_prefill * 1e-3) / 1e12

    # the scoring pass on its own: entropy_score, allocate_budget and
    # select_blocks back to back with no event between them (the step's
    # per-call events add their own gaps).  A 512 MiB write before each
    # repetition evicts K from the 256 MB Infinity Cache, so K streams from
    # HBM as it does in the step, where the decode leg runs in between.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def three_calls():
        api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0, block_scores=scores,
                          entropy=E, workspace=ws)
        api.allocate_budget(shape, pol, E, head_is_rigid=rigid, budget=budget)
        api.select_blocks(shape, scores, budget, k_max, block_idx=idx, block_cnt=cnt)

    def fused_call():
        api.score_select(shape, pol, q, k, k_max, kind=kind, renyi_alpha=2.0, out=sel_out,
                         workspace=ws)

    t_scoring_solo = back_to_back(torch, fused_call, flush, args.steps)
    t_scoring_3 = back_to_back(torch, three_calls, flush, args.steps)
    scoring_solo_gbs = sbytes / (t_scoring_solo * 1e-3) / 1e9

    # the paper-literal max / min observation rows ([EI] Alg. 1-2), timed on
    # their own after the step loop (they are not part of the step)
    mm_scores = torch.empty_like(scores)
    mm_E = torch.empty_like(E)
    for _ in range(2):
        api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0, pool=L.EGS_POOL_MAXMIN,
                          block_scores=mm_scores, entropy=mm_E, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0, pool=L.EGS_POOL_MAXMIN,
                          block_scores=mm_scores, entropy=mm_E, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    t_mm = e0.elapsed_time(e1) / args.steps
    mm_bytes = (cfg.n_q_heads + cfg.n_kv_heads) * cfg.seq_len * d * elt + Hq * CS * CB * 4
    del mm_scores, mm_E

    # page-level retention ([EP] Sec. 7) on the decode workload's group scores
    page_us = {}
    if decode is not None:
        ds = decode["shape"]
        kr = api.kv_retain(ds, prm, dq, dk, dv, workspace=dws, want_scores=True, gather=False)
        mu_buf.copy_(kr["scores"])
        for name, mode in (("group", L.EGS_PAGE_GROUP), ("layer_union", L.EGS_PAGE_LAYER_UNION)):
            api.page_retain(ds, mu_buf, pg_S, pg_K, mode, workspace=pg_ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                api.page_retain(ds, mu_buf, pg_S, pg_K, mode, workspace=pg_ws)
            e1.record()
            torch.cuda.synchronize()
            page_us[name] = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)

    # latent decoding ([EI] Sec. 4.3): 32 generated tokens over the decode
    # workload's 128k cache, compressed after 16; per-token GPU time of the
    # steps before, at and after the compression
    latent = None
    if decode is not None:
        dc = decode["cfg"]
        G, ND = 32, 16
        C = dc.cache_len + G
        lshape = api.DecodeShape(dc.batch, dc.n_q_heads, dc.n_kv_heads, dc.head_dim, C,
                                 dc.n_obs, dc.n_sink, dc.n_recent, dc.n_keep)
        kc = torch.empty((dc.batch, dc.n_kv_heads, C, dc.head_dim), dtype=torch.bfloat16,
                         device=dev)
        vc = torch.empty_like(kc)
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        toks = [(torch.randn((dc.batch, dc.n_q_heads, dc.head_dim), generator=gen, device=dev),
                 torch.randn((dc.batch, dc.n_kv_heads, dc.head_dim), generator=gen, device=dev),
                 torch.randn((dc.batch, dc.n_kv_heads, dc.head_dim), generator=gen, device=dev))
                for _ in range(G)]
        toks = [tuple(t.bfloat16() for t in tk) for tk in toks]
        lws = torch.empty(L.LIB.egs_latent_decode_workspace(ctypes.byref(lshape.c())),
                          dtype=torch.uint8, device=dev)
        lout = torch.empty((dc.batch, dc.n_q_heads, dc.head_dim), dtype=torch.bfloat16,
                           device=dev)
        per_step = []
        for rep in range(2):                       # the first pass warms up
            kc[:, :, :dc.cache_len].copy_(dk)
            vc[:, :, :dc.cache_len].copy_(dv)
            win = dq.clone()
            stt = L.LatentStateC(length=dc.cache_len, generated=0, n_delay=ND, interval=0,
                                 compressed=0)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(G + 1)]
            torch.cuda.synchronize()
            evs[0].record()
            for i, (q1, k1, v1) in enumerate(toks):
                api.latent_decode_step(lshape, prm, stt, q1, k1, v1, win, kc, vc, out=lout,
                                       workspace=lws)
                evs[i + 1].record()
            torch.cuda.synchronize()
            per_step = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(G)]
        latent = {"tokens": G, "n_delay": ND, "cache_len": dc.cache_len,
                  "kept_after": int(stt.length) - (G - ND),
                  "dense_step_us": round(float(np.mean(per_step[:ND - 1])), 1),
                  "compress_step_us": round(per_step[ND - 1], 1),
                  "compressed_step_us": round(float(np.mean(per_step[ND:])), 1)}
        del kc, vc, lws

    # chunk pruning ([EP] Sec. 3-4) of one 128k prompt of the decode workload
    # (batch element 0): 64 candidate documents, removal up to half the prompt
    prune = None
    if decode is not None:
        dc = decode["cfg"]
        pshape = api.DecodeShape(1, dc.n_q_heads, dc.n_kv_heads, dc.head_dim, dc.cache_len,
                                 dc.n_obs, dc.n_sink, dc.n_recent, dc.n_keep)
        pch = synth.prune_chunks(dc.cache_len, dc.n_obs, 64, seed=11)
        pws = torch.empty(L.LIB.egs_chunk_prune_workspace(ctypes.byref(pshape.c()), len(pch)),
                          dtype=torch.uint8, device=dev)
        pargs = (pshape, dq[0], dk[0], pch, 0.1, 0.5, 0.1, 4, dc.cache_len // 2)
        for _ in range(2):
            api.chunk_prune(*pargs, workspace=pws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            prem, ptok, _, _ = api.chunk_prune(*pargs, workspace=pws)
        e1.record()
        torch.cuda.synchronize()
        prune = {"us": round(e0.elapsed_time(e1) / args.steps * 1e3, 1), "chunks": len(pch),
                 "seq_len": dc.cache_len, "n_obs": dc.n_obs, "eps": 0.1, "m0": 4,
                 "target": dc.cache_len // 2, "removed": int(prem.sum().item()),
                 "removed_tokens": int(ptok.item())}
        del pws

    # the other prefill workloads, each on its own (not part of the step)
    workloads = {}
    if not args.no_workloads:
        workloads[f"{cfg.name}-renyi2" if kind == L.EGS_SHANNON else f"{cfg.name}-shannon"] = \
            prefill_workload(api, torch, dev, cfg, None,
                             L.EGS_RENYI if kind == L.EGS_SHANNON else L.EGS_SHANNON,
                             args.steps, flush, dev_qkv=(q, k, v))
        for wname in ("llama3-8b-32k", "qwen-64k"):
            if wname == cfg.name:
                continue
            wc = synth.PREFILL_CONFIGS[wname]
            winp = synth.make_prefill(wc, seed=0)
            workloads[wname] = prefill_workload(api, torch, dev, wc, winp, L.EGS_SHANNON,
                                                args.steps, flush)
            del winp
            torch.cuda.empty_cache()
    del flush

    traffic = measured_traffic(cfg.name)
    if args.calib_copy_mib > 0:
        calib_copy(torch, dev, args.calib_copy_mib)

    res = {
        "metric": "sparse prefill ms/layer + effective TFLOP/s at 128k; scoring-pass GB/s",
        "value": round(eff_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} prefill layer"
                               + (" + decode-retain-b8-128k" if decode else ""),
                   "n_q_heads": Hq, "n_kv_heads": cfg.n_kv_heads, "head_dim": d,
                   "seq_len": cfg.seq_len, "block_size": LB, "segment_size": LS,
                   "probe_len": cfg.probe_len, "entropy": args.entropy,
                   "budget": "two-level 5%/30%, e_t 0.5" if pol.mode == L.EGS_BUDGET_TWO_LEVEL
                   else str(pol.mode),
                   "parallelism": "single GPU"},
        "prefill_ms_per_layer": round(t_prefill, 4),
        "scoring_pass_us": round(t_scoring_solo * 1e3, 2),
        "scoring_pass_gbps": round(scoring_solo_gbs, 1),
        "scoring_pass_bytes": sbytes,
        "scoring_pass_three_calls_us": round(t_scoring_3 * 1e3, 2),
        "scoring_pass_in_step_us": round(t_scoring * 1e3, 2),
        "scoring_pass_in_step_gbps": round(scoring_gbs, 1),
        "attn_ms": round(t_attn, 4),
        "attn_ms_median": round(t_attn_median, 4),
        "block_list_uor": union_overlap(g_idx, g_cnt, cfg.n_kv_heads),
        "attn_tflops_executed": round(attn_tflops, 2),
        "prefill_tflops_dense_equiv": round(dense_equiv, 2),
        "executed_tiles": tiles,
        "dense_causal_tiles": dense_tiles,
        "tile_density": round(tiles / dense_tiles, 4),
        "kernel_us": {kk: round(vv, 2) for kk, vv in kernel_us.items()},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "scoring_roofline": {"bound": "hbm", "achieved": round(scoring_solo_gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(scoring_solo_gbs / PEAK_HBM_GBS, 4)},
        "maxmin_scoring_us": round(t_mm * 1e3, 2),
        "maxmin_scoring_roofline": {"bound": "hbm",
                                    "achieved": round(mm_bytes / (t_mm * 1e-3) / 1e9, 1),
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(mm_bytes / (t_mm * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                  4)},
    }
    if decode is not None:
        dc = decode["cfg"]
        kv_bytes = dc.batch * dc.n_kv_heads * dc.cache_len * dc.head_dim * 2
        res["decode_ms"] = round(t_decode, 4)
        res["decode_kv_retain_gbps"] = round(kv_bytes / (kernel_us["kv_retain"] * 1e-6) / 1e9, 1)
        # kv_retain against both bounds: K read once (plus the observers) for
        # HBM, one pass of window logits 2 W d L Hq B for MFMA (the second,
        # recomputing pass is implementation work and not counted)
        qo_bytes = dc.batch * dc.n_q_heads * dc.n_obs * dc.head_dim * 2
        kr_flops = 2.0 * dc.n_obs * dc.head_dim * dc.cache_len * dc.n_q_heads * dc.batch
        kr_s = kernel_us["kv_retain"] * 1e-6
        res["kv_retain_roofline"] = {
            "hbm": {"achieved": round((kv_bytes + qo_bytes) / kr_s / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round((kv_bytes + qo_bytes) / kr_s / 1e9 / PEAK_HBM_GBS, 4),
                    "bytes": kv_bytes + qo_bytes},
            "mfma": {"achieved": round(kr_flops / kr_s / 1e12, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": round(kr_flops / kr_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "flops": kr_flops}}
        res["decode_n_total"] = decode["n_total"]
        res["page_retain_us"] = page_us
        res["latent_decode"] = latent
        res["chunk_prune"] = prune
        res["page_retain_config"] = {"page_size": pg_S, "n_keep_pages": pg_K,
                                     "scores": "kv_retain group scores, batch 8, 8 groups, 128k"}
    if workloads:
        res["workloads"] = workloads
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, inp, g_idx, g_cnt, args.cpu_seconds, pol=pol,
                                           k_max=k_max,
                                           decode_cfg=decode["cfg"] if decode else None,
                                           gpu_ms={"scoring": t_scoring_solo,
                                                   "attention": t_attn,
                                                   "kv_retain": kernel_us.get("kv_retain", 0) / 1e3,
                                                   "decode_attn":
                                                       kernel_us.get("sparse_decode_attn", 0) / 1e3})
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
