"""Shared helpers for GPU-vs-oracle parity tests (test infrastructure)."""
from __future__ import annotations

import math

import numpy as np
import torch

from entropy_guided_sparse_amd import synth

# Tolerances fixed for this method (entropy, selection band, attention) and the
# one derived for the observation rows themselves.
ENTROPY_ATOL = 1e-3          # |E_gpu - E_oracle|
SELECT_BAND = 1e-4           # scores this close to the cutoff may swap
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 1e-2
# Observation rows: logits carry ~2^-18 relative error from the bf16 hi/lo
# split of the pooled keys plus fp32 accumulation (|z| <= ~100 here), i.e.
# <= ~3e-4 absolute on z in the worst case and ~1e-5 typically; the probe
# average of softmax rows then moves by at most ~|dz| * a.  5e-5 absolute
# leaves margin over the typical case and stays below the selection band.
SCORE_ATOL = 5e-5


def dev_tensor(store: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(store))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def list_violations(gpu_idx, gpu_cnt, ref_scores, budget, L_S, L_B, band=SELECT_BAND):
    """Compare GPU block lists with the oracle's scores.

    Per (h, s) with k = budget: c = the oracle's k-th largest score; the GPU set
    must contain every block scoring above c + band and none scoring below
    c - band, and hold exactly k blocks.  Returns a list of (h, s, reason)."""
    bad = []
    Hq, CS = gpu_cnt.shape
    for h in range(Hq):
        for s in range(CS):
            cb = (s + 1) * L_S // L_B
            k = int(min(budget[h, s], cb))
            n = int(gpu_cnt[h, s])
            got = gpu_idx[h, s, :n]
            if n != k:
                bad.append((h, s, f"count {n} != {k}"))
                continue
            if np.any(np.diff(got) <= 0) or np.any(got < 0) or np.any(got >= cb):
                bad.append((h, s, "not ascending / out of range"))
                continue
            sc = ref_scores[h, s, :cb]
            if k == 0:
                continue
            c = np.sort(sc)[::-1][k - 1]
            sel = np.zeros(cb, dtype=bool)
            sel[got] = True
            must = sc > c + band
            mustnot = sc < c - band
            if np.any(must & ~sel) or np.any(mustnot & sel):
                bad.append((h, s, "selection differs outside the band"))
    return bad


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30))
    return max_abs, rel


def prefill_shape(api, cfg):
    return api.PrefillShape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len,
                            cfg.block_size, cfg.segment_size, cfg.probe_len,
                            torch_dtype(cfg.dtype))


def log(msg: str):
    print(msg, flush=True)
