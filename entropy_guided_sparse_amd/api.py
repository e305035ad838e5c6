"""Python entry points with the same names as the C ABI (include/egs.h).

Each function checks tensor placement / dtype / contiguity, allocates the
outputs and workspace with torch (device memory plumbing), and calls the
library on torch's current stream.  Nothing is computed here.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib as L

__all__ = [
    "PrefillShape", "BudgetPolicy", "DecodeShape", "RetainParams",
    "entropy_score", "allocate_budget", "select_blocks", "sparse_prefill_attn",
    "kv_retain", "sparse_decode_attn", "kv_retain_total",
]

_DT = {torch.bfloat16: L.EGS_BF16, torch.float32: L.EGS_F32}


@dataclasses.dataclass
class PrefillShape:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    block_size: int
    segment_size: int
    probe_len: int
    dtype: torch.dtype = torch.bfloat16
    sm_scale: float = 0.0

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block_size

    @property
    def n_segments(self) -> int:
        return self.seq_len // self.segment_size

    def c(self) -> L.PrefillShapeC:
        return L.PrefillShapeC(self.n_q_heads, self.n_kv_heads, self.head_dim, self.seq_len,
                               self.block_size, self.segment_size, self.probe_len,
                               _DT[self.dtype], self.sm_scale)


@dataclasses.dataclass
class BudgetPolicy:
    mode: int = L.EGS_BUDGET_FIXED
    frac: float = 0.25
    frac_rigid: float = 0.05
    frac_dynamic: float = 0.30
    frac_min: float = 0.02
    frac_max: float = 0.50
    entropy_threshold: float = 0.5
    base_tokens: float = 2048.0
    alg3_alpha: float = 0.5
    alg3_delta_t: float = 0.4

    def c(self) -> L.BudgetPolicyC:
        return L.BudgetPolicyC(self.mode, self.frac, self.frac_rigid, self.frac_dynamic,
                               self.frac_min, self.frac_max, self.entropy_threshold,
                               self.base_tokens, self.alg3_alpha, self.alg3_delta_t)


@dataclasses.dataclass
class DecodeShape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_len: int
    n_obs: int
    n_sink: int
    n_recent: int
    n_keep: int
    dtype: torch.dtype = torch.bfloat16
    sm_scale: float = 0.0

    def c(self) -> L.DecodeShapeC:
        return L.DecodeShapeC(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                              self.cache_len, self.n_obs, self.n_sink, self.n_recent,
                              self.n_keep, _DT[self.dtype], self.sm_scale)


@dataclasses.dataclass
class RetainParams:
    entropy_kind: int = L.EGS_SHANNON
    renyi_alpha: float = 2.0
    zeta: float = 0.5
    tau: float = 1.0
    raw_logit_mode: int = 0
    info_alpha: float = 1.0

    def c(self) -> L.RetainParamsC:
        return L.RetainParamsC(self.entropy_kind, self.renyi_alpha, self.zeta, self.tau,
                               self.raw_logit_mode, self.info_alpha)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns >= 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# prefill path
# ----------------------------------------------------------------------------
def entropy_score(shape: PrefillShape, q: torch.Tensor, k: torch.Tensor, kind: int = L.EGS_SHANNON,
                  renyi_alpha: float = 2.0, pool: int = L.EGS_POOL_MEAN_PROBE,
                  block_scores: Optional[torch.Tensor] = None,
                  entropy: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None):
    """Observation rows a_bar [Hq, C_S, C_B] and entropy E [Hq, C_S]."""
    s = shape
    dev = q.device
    _need(q, "q", (s.n_q_heads, s.seq_len, s.head_dim), s.dtype)
    _need(k, "k", (s.n_kv_heads, s.seq_len, s.head_dim), s.dtype, dev)
    sc = s.c()
    if block_scores is None:
        block_scores = _empty((s.n_q_heads, s.n_segments, s.n_blocks), torch.float32, dev)
    if entropy is None:
        entropy = _empty((s.n_q_heads, s.n_segments), torch.float32, dev)
    _need(block_scores, "block_scores", (s.n_q_heads, s.n_segments, s.n_blocks), torch.float32, dev)
    _need(entropy, "entropy", (s.n_q_heads, s.n_segments), torch.float32, dev)
    wsb = L.LIB.egs_entropy_score_workspace(ctypes.byref(sc))
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_entropy_score(ctypes.byref(sc), pool, kind, renyi_alpha, _ptr(q), _ptr(k),
                                    _ptr(block_scores), _ptr(entropy), _ptr(workspace),
                                    workspace.numel(), _stream(dev)))
    return block_scores, entropy


def entropy_score_static(shape: PrefillShape, q: torch.Tensor, k: torch.Tensor,
                         kind: int = L.EGS_SHANNON, renyi_alpha: float = 2.0,
                         pool: int = L.EGS_POOL_MEAN_PROBE,
                         block_scores: Optional[torch.Tensor] = None,
                         entropy: Optional[torch.Tensor] = None):
    """entropy_score on the library's static device scratch (no workspace);
    the outputs are allocated here unless passed in."""
    s = shape
    dev = q.device
    _need(q, "q", (s.n_q_heads, s.seq_len, s.head_dim), s.dtype)
    _need(k, "k", (s.n_kv_heads, s.seq_len, s.head_dim), s.dtype, dev)
    sc = s.c()
    if block_scores is None:
        block_scores = _empty((s.n_q_heads, s.n_segments, s.n_blocks), torch.float32, dev)
    if entropy is None:
        entropy = _empty((s.n_q_heads, s.n_segments), torch.float32, dev)
    _need(block_scores, "block_scores", (s.n_q_heads, s.n_segments, s.n_blocks), torch.float32, dev)
    _need(entropy, "entropy", (s.n_q_heads, s.n_segments), torch.float32, dev)
    L.check(L.LIB.egs_entropy_score_static(ctypes.byref(sc), pool, kind, renyi_alpha, _ptr(q),
                                           _ptr(k), _ptr(block_scores), _ptr(entropy),
                                           _stream(dev)))
    return block_scores, entropy


def allocate_budget(shape: PrefillShape, policy: BudgetPolicy, entropy: torch.Tensor,
                    head_is_rigid: Optional[torch.Tensor] = None,
                    budget: Optional[torch.Tensor] = None):
    """Head classes [Hq] int8 and budgets [Hq, C_S] int32 (in blocks)."""
    s = shape
    dev = entropy.device
    _need(entropy, "entropy", (s.n_q_heads, s.n_segments), torch.float32)
    if head_is_rigid is None:
        head_is_rigid = _empty((s.n_q_heads,), torch.int8, dev)
    if budget is None:
        budget = _empty((s.n_q_heads, s.n_segments), torch.int32, dev)
    _need(head_is_rigid, "head_is_rigid", (s.n_q_heads,), torch.int8, dev)
    _need(budget, "budget", (s.n_q_heads, s.n_segments), torch.int32, dev)
    sc, pc = s.c(), policy.c()
    L.check(L.LIB.egs_allocate_budget(ctypes.byref(sc), ctypes.byref(pc), _ptr(entropy),
                                      _ptr(head_is_rigid), _ptr(budget), _stream(dev)))
    return head_is_rigid, budget


def select_blocks(shape: PrefillShape, block_scores: torch.Tensor, budget: torch.Tensor,
                  k_max: int, block_idx: Optional[torch.Tensor] = None,
                  block_cnt: Optional[torch.Tensor] = None):
    """Selected block lists [Hq, C_S, k_max] (ascending, -1 padded) and counts."""
    s = shape
    dev = block_scores.device
    _need(block_scores, "block_scores", (s.n_q_heads, s.n_segments, s.n_blocks), torch.float32)
    _need(budget, "budget", (s.n_q_heads, s.n_segments), torch.int32, dev)
    if block_idx is None:
        block_idx = _empty((s.n_q_heads, s.n_segments, k_max), torch.int32, dev)
    if block_cnt is None:
        block_cnt = _empty((s.n_q_heads, s.n_segments), torch.int32, dev)
    _need(block_idx, "block_idx", (s.n_q_heads, s.n_segments, k_max), torch.int32, dev)
    _need(block_cnt, "block_cnt", (s.n_q_heads, s.n_segments), torch.int32, dev)
    sc = s.c()
    L.check(L.LIB.egs_select_blocks(ctypes.byref(sc), _ptr(block_scores), _ptr(budget), k_max,
                                    _ptr(block_idx), _ptr(block_cnt), _stream(dev)))
    return block_idx, block_cnt


def score_select(shape: PrefillShape, policy: BudgetPolicy, q: torch.Tensor, k: torch.Tensor,
                 k_max: int, kind: int = L.EGS_SHANNON, renyi_alpha: float = 2.0,
                 pool: int = L.EGS_POOL_MEAN_PROBE, out: Optional[dict] = None,
                 workspace: Optional[torch.Tensor] = None):
    """entropy_score -> allocate_budget -> select_blocks in one call.  Returns
    dict(block_scores, entropy, head_is_rigid, budget, block_idx, block_cnt);
    `out` may supply any of these tensors."""
    s = shape
    dev = q.device
    _need(q, "q", (s.n_q_heads, s.seq_len, s.head_dim), s.dtype)
    _need(k, "k", (s.n_kv_heads, s.seq_len, s.head_dim), s.dtype, dev)
    Hq, CS, CB = s.n_q_heads, s.n_segments, s.n_blocks
    want = {"block_scores": ((Hq, CS, CB), torch.float32), "entropy": ((Hq, CS), torch.float32),
            "head_is_rigid": ((Hq,), torch.int8), "budget": ((Hq, CS), torch.int32),
            "block_idx": ((Hq, CS, k_max), torch.int32), "block_cnt": ((Hq, CS), torch.int32)}
    res = dict(out or {})
    for name, (shp, dt) in want.items():
        if res.get(name) is None:
            res[name] = _empty(shp, dt, dev)
        _need(res[name], name, shp, dt, dev)
    sc, pc = s.c(), policy.c()
    wsb = L.LIB.egs_entropy_score_workspace(ctypes.byref(sc))
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_score_select(ctypes.byref(sc), pool, kind, renyi_alpha, ctypes.byref(pc),
                                   _ptr(q), _ptr(k), k_max, _ptr(res["block_scores"]),
                                   _ptr(res["entropy"]), _ptr(res["head_is_rigid"]),
                                   _ptr(res["budget"]), _ptr(res["block_idx"]),
                                   _ptr(res["block_cnt"]), _ptr(workspace), workspace.numel(),
                                   _stream(dev)))
    return res


def sparse_prefill_attn(shape: PrefillShape, q, k, v, block_idx, block_cnt,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """Block-sparse causal GQA attention output [Hq, N, d] (and lse [Hq, N])."""
    s = shape
    dev = q.device
    _need(q, "q", (s.n_q_heads, s.seq_len, s.head_dim), s.dtype)
    _need(k, "k", (s.n_kv_heads, s.seq_len, s.head_dim), s.dtype, dev)
    _need(v, "v", (s.n_kv_heads, s.seq_len, s.head_dim), s.dtype, dev)
    k_max = block_idx.shape[-1]
    _need(block_idx, "block_idx", (s.n_q_heads, s.n_segments, k_max), torch.int32, dev)
    _need(block_cnt, "block_cnt", (s.n_q_heads, s.n_segments), torch.int32, dev)
    if out is None:
        out = _empty((s.n_q_heads, s.seq_len, s.head_dim), s.dtype, dev)
    _need(out, "out", (s.n_q_heads, s.seq_len, s.head_dim), s.dtype, dev)
    if return_lse and lse is None:
        lse = _empty((s.n_q_heads, s.seq_len), torch.float32, dev)
    if lse is not None:
        _need(lse, "lse", (s.n_q_heads, s.seq_len), torch.float32, dev)
    sc = s.c()
    wsb = L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc))
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_sparse_prefill_attn(ctypes.byref(sc), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(block_idx), _ptr(block_cnt), k_max, _ptr(out),
                                          _ptr(lse), _ptr(workspace), workspace.numel(),
                                          _stream(dev)))
    return (out, lse) if (return_lse or lse is not None) else out


# ----------------------------------------------------------------------------
# decode path
# ----------------------------------------------------------------------------
def kv_retain_total(shape: DecodeShape) -> int:
    sc = shape.c()
    n = L.LIB.egs_kv_retain_total(ctypes.byref(sc))
    if n < 0:
        raise L.EgsError(L.EGS_EINVAL, L.LIB.egs_last_error().decode())
    return n


def kv_retain(shape: DecodeShape, params: RetainParams, q_obs, k_cache, v_cache,
              token_entropy: Optional[torch.Tensor] = None, gather: bool = True,
              want_head_entropy: bool = True, want_scores: bool = False,
              workspace: Optional[torch.Tensor] = None):
    """Returns dict(keep_idx, k_out, v_out, head_entropy, scores)."""
    s = shape
    dev = q_obs.device
    _need(q_obs, "q_obs", (s.batch, s.n_q_heads, s.n_obs, s.head_dim), s.dtype)
    _need(k_cache, "k_cache", (s.batch, s.n_kv_heads, s.cache_len, s.head_dim), s.dtype, dev)
    if gather:
        _need(v_cache, "v_cache", (s.batch, s.n_kv_heads, s.cache_len, s.head_dim), s.dtype, dev)
    if token_entropy is not None:
        _need(token_entropy, "token_entropy", (s.batch, s.cache_len), torch.float32, dev)
    n_total = kv_retain_total(s)
    keep = _empty((s.batch, s.n_kv_heads, n_total), torch.int32, dev)
    k_out = _empty((s.batch, s.n_kv_heads, n_total, s.head_dim), s.dtype, dev) if gather else None
    v_out = _empty((s.batch, s.n_kv_heads, n_total, s.head_dim), s.dtype, dev) if gather else None
    he = _empty((s.batch, s.n_q_heads), torch.float32, dev) if want_head_entropy else None
    sco = _empty((s.batch, s.n_kv_heads, s.cache_len), torch.float32, dev) if want_scores else None
    sc, pc = s.c(), params.c()
    wsb = L.LIB.egs_kv_retain_workspace(ctypes.byref(sc))
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_kv_retain(ctypes.byref(sc), ctypes.byref(pc), _ptr(q_obs), _ptr(k_cache),
                                _ptr(v_cache), _ptr(token_entropy), _ptr(keep), _ptr(k_out),
                                _ptr(v_out), _ptr(he), _ptr(sco), _ptr(workspace),
                                workspace.numel(), _stream(dev)))
    return {"keep_idx": keep, "k_out": k_out, "v_out": v_out, "head_entropy": he,
            "scores": sco}


def chunk_bounds_device(chunk_bounds, dev, limit: Optional[int] = None, nonempty: bool = True):
    """The chunk bounds [k, 2] int32 as a device tensor.  A device tensor is
    used as given (the library checks it on the device); host bounds are
    checked here first (ascending, disjoint and ending at or before `limit`
    when given, non-empty), with the library's error class and messages."""
    import numpy as np
    if isinstance(chunk_bounds, torch.Tensor) and chunk_bounds.device.type == "cuda":
        b = chunk_bounds
        if b.dtype != torch.int32 or not b.is_contiguous() or b.dim() != 2 or b.shape[1] != 2:
            raise ValueError("chunk_bounds must be a contiguous int32 [k, 2] tensor")
        return b
    b = np.ascontiguousarray(np.asarray(chunk_bounds, dtype=np.int32).reshape(-1, 2))
    prev = 0
    for i, (lo, hi) in enumerate(b.tolist()):
        if (limit is not None and (lo < prev or hi > limit)) or (nonempty and hi <= lo):
            raise L.EgsError(L.EGS_EINVAL, f"EGS_EINVAL: chunk {i} = [{lo}, {hi}) is not "
                             f"ascending, disjoint, non-empty and before the observers "
                             f"(T - W = {limit})")
        prev = hi
    return torch.from_numpy(b).to(dev)


def chunk_prune(shape: DecodeShape, q_obs, k, chunk_bounds, eps_s: float, lam: float,
                eps: float, m0: int, target: int, zeta: float = 0.5, tau: float = 1.0,
                want_row_mass: bool = False, workspace: Optional[torch.Tensor] = None):
    """Removal flags [k] int8, removed tokens [1] int32, priorities [k] and
    (optionally) the row-chunk masses [k, Hq*W]; chunk_bounds [k, 2] int32
    (begin, end), on the host or the device."""
    s = shape
    dev = q_obs.device
    _need(q_obs, "q_obs", (s.n_q_heads, s.n_obs, s.head_dim), s.dtype)
    _need(k, "k", (s.n_kv_heads, s.cache_len, s.head_dim), s.dtype, dev)
    b = chunk_bounds_device(chunk_bounds, dev, limit=s.cache_len - s.n_obs)
    nk = b.shape[0]
    removed = _empty((nk,), torch.int8, dev)
    tokens = _empty((1,), torch.int32, dev)
    prio = _empty((nk,), torch.float32, dev)
    row_mass = _empty((nk, s.n_q_heads * s.n_obs), torch.float32, dev) if want_row_mass else None
    sc = s.c()
    pc = L.PruneParamsC(eps_s, lam, eps, m0, target, zeta, tau)
    wsb = L.LIB.egs_chunk_prune_workspace(ctypes.byref(sc), nk)
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_chunk_prune(ctypes.byref(sc), ctypes.byref(pc), _ptr(q_obs), _ptr(k),
                                  _ptr(b), nk, _ptr(removed),
                                  _ptr(tokens), _ptr(prio), _ptr(row_mass), _ptr(workspace),
                                  workspace.numel(), _stream(dev)))
    return removed, tokens, prio, row_mass


def prune_certificate(chunk_bounds, row_mass, row_price, eps: float, m0: int, t: float,
                      workspace: Optional[torch.Tensor] = None):
    """U(y, t) of a removal as a float64 device tensor [1]; row_mass [k, R]
    and row_price [R] are float32 device tensors, chunk_bounds [k, 2] int32
    on the host or the device."""
    dev = row_mass.device
    b = chunk_bounds_device(chunk_bounds, dev)
    nk = b.shape[0]
    if row_mass.dtype != torch.float32 or not row_mass.is_contiguous() or row_mass.dim() != 2 \
            or row_mass.shape[0] != nk:
        raise ValueError(f"row_mass must be contiguous float32 [{nk}, R]")
    R = row_mass.shape[1]
    _need(row_price, "row_price", (R,), torch.float32, dev)
    out = _empty((1,), torch.float64, dev)
    if workspace is None:
        workspace = _workspace(L.LIB.egs_prune_certificate_workspace(nk), dev)
    L.check(L.LIB.egs_prune_certificate(_ptr(b), nk, R,
                                        _ptr(row_mass), _ptr(row_price), eps, m0, t, _ptr(out),
                                        _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def latent_decode_step(shape: DecodeShape, params: RetainParams, state, q_new, k_new, v_new,
                       q_window, k_cache, v_cache, out: Optional[torch.Tensor] = None,
                       keep_idx: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    """One generated token of latent decoding; `state` is an L.LatentStateC
    updated in place (shape.cache_len is the capacity of k_cache / v_cache)."""
    s = shape
    dev = q_new.device
    _need(q_new, "q_new", (s.batch, s.n_q_heads, s.head_dim), s.dtype)
    _need(k_new, "k_new", (s.batch, s.n_kv_heads, s.head_dim), s.dtype, dev)
    _need(v_new, "v_new", (s.batch, s.n_kv_heads, s.head_dim), s.dtype, dev)
    _need(q_window, "q_window", (s.batch, s.n_q_heads, s.n_obs, s.head_dim), s.dtype, dev)
    _need(k_cache, "k_cache", (s.batch, s.n_kv_heads, s.cache_len, s.head_dim), s.dtype, dev)
    _need(v_cache, "v_cache", (s.batch, s.n_kv_heads, s.cache_len, s.head_dim), s.dtype, dev)
    if out is None:
        out = _empty((s.batch, s.n_q_heads, s.head_dim), s.dtype, dev)
    _need(out, "out", (s.batch, s.n_q_heads, s.head_dim), s.dtype, dev)
    if keep_idx is not None and not (keep_idx.is_cuda and keep_idx.dtype == torch.int32
                                     and keep_idx.is_contiguous()):
        raise ValueError("keep_idx must be a contiguous int32 device tensor")
    sc, pc = s.c(), params.c()
    wsb = L.LIB.egs_latent_decode_workspace(ctypes.byref(sc))
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_latent_decode_step(ctypes.byref(sc), ctypes.byref(pc), ctypes.byref(state),
                                         _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(q_window),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(keep_idx),
                                         _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def page_retain(shape: DecodeShape, token_scores: torch.Tensor, page_size: int,
                n_keep_pages: int, mode: int = L.EGS_PAGE_GROUP,
                page_idx: Optional[torch.Tensor] = None,
                page_cnt: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None):
    """Kept pages [B, Y, cap] (ascending, -1 padded) and their counts [B, Y]."""
    s = shape
    dev = token_scores.device
    sc = s.c()
    X = s.n_q_heads if mode == L.EGS_PAGE_HEAD_UNION else s.n_kv_heads
    Y = 1 if mode == L.EGS_PAGE_LAYER_UNION else s.n_kv_heads
    _need(token_scores, "token_scores", (s.batch, X, s.cache_len), torch.float32)
    cap = L.LIB.egs_page_retain_capacity(ctypes.byref(sc), page_size, n_keep_pages, mode)
    if cap < 0:
        raise L.EgsError(L.EGS_EINVAL, L.LIB.egs_last_error().decode())
    if page_idx is None:
        page_idx = _empty((s.batch, Y, max(cap, 1)), torch.int32, dev)
    if page_cnt is None:
        page_cnt = _empty((s.batch, Y), torch.int32, dev)
    _need(page_idx, "page_idx", (s.batch, Y, max(cap, 1)), torch.int32, dev)
    _need(page_cnt, "page_cnt", (s.batch, Y), torch.int32, dev)
    wsb = L.LIB.egs_page_retain_workspace(ctypes.byref(sc), page_size, n_keep_pages, mode)
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_page_retain(ctypes.byref(sc), page_size, n_keep_pages, mode,
                                  _ptr(token_scores), _ptr(page_idx), _ptr(page_cnt),
                                  _ptr(workspace), workspace.numel(), _stream(dev)))
    return page_idx, page_cnt


def sparse_decode_attn(shape: DecodeShape, q_new, k_kept, v_kept,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    s = shape
    dev = q_new.device
    n_total = k_kept.shape[2]
    _need(q_new, "q_new", (s.batch, s.n_q_heads, s.head_dim), s.dtype)
    _need(k_kept, "k_kept", (s.batch, s.n_kv_heads, n_total, s.head_dim), s.dtype, dev)
    _need(v_kept, "v_kept", (s.batch, s.n_kv_heads, n_total, s.head_dim), s.dtype, dev)
    if out is None:
        out = _empty((s.batch, s.n_q_heads, s.head_dim), s.dtype, dev)
    _need(out, "out", (s.batch, s.n_q_heads, s.head_dim), s.dtype, dev)
    sc = s.c()
    wsb = L.LIB.egs_sparse_decode_attn_workspace(ctypes.byref(sc), n_total)
    if workspace is None:
        workspace = _workspace(wsb, dev)
    L.check(L.LIB.egs_sparse_decode_attn(ctypes.byref(sc), _ptr(q_new), _ptr(k_kept),
                                         _ptr(v_kept), n_total, _ptr(out), _ptr(workspace),
                                         workspace.numel(), _stream(dev)))
    return out
