"""Seeded synthetic inputs shaped like the workloads of the entropy-guided sparse
prefill / decode-retention method.

This module holds no step of the method itself (no pooling, scoring, entropy,
budgeting, selection or attention): it only draws Gaussian tensors, plants the
rigid / dynamic attention structure that the pages describe, and rounds the
result to the storage dtype.  Both the HIP path and the float64 oracle consume
exactly the tensors produced here.

Structure being imitated:
  * EntropyInfer (arXiv 2606.09508), Sec. 3.1 / Fig. 1: "rigid" heads whose
    attention entropy stays near zero (a sink-like key dominates) and "dynamic"
    heads whose attention spreads over a few context-dependent key blocks.
  * EntropyInfer Sec. 3.2: the head type depends on the context, so some
    workloads draw it per (head, segment).
  * Decode retention: a small fraction of cache entries carry high attention
    mass for the most recent queries (EntropyInfer Alg. 4 / InfoKV window mean).

Recipe (c = sqrt(d), directions orthonormal within a KV group):
  * Q, K, V ~ N(0, 1), drawn in that order as float32 from
    numpy.random.default_rng(seed).
  * One orthonormal bank per KV group (QR of a d x m Gaussian) supplies a
    rigid direction rho_h per head and a dynamic direction nu_{h,s} per
    (head, segment).
  * Rigid (h, s): every query of segment s gets + c * rho_h; key 0 of the KV
    group is *set* to sum_h 8 * L_B * c * rho_h over the group's heads that are
    rigid anywhere (the L_B factor makes the sink survive block-mean pooling).
  * Dynamic (h, s): every query of segment s gets + c * nu_{h,s}; every key of
    each planted hot block j in 1..C_B(s)-1 gets + 4 * c * nu_{h,s}.
  * Decode: per (batch, KV group) one unit direction; 1% of cache positions in
    [4, L-256) get + 4 * c * direction on their keys; observer and new-token
    queries of "focused" heads get + c * direction.
  * Chunk pruning (EntroPrefill Sec. 3): a prompt of T tokens is a protected
    prefix, k candidate documents separated by one protected delimiter token,
    and the protected query whose last W tokens are the observers; document
    lengths are drawn uniformly from [1/2, 3/2] of the mean and scaled to fill
    the space between prefix and query.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "PrefillConfig", "DecodeConfig", "PREFILL_CONFIGS", "DECODE_CONFIGS",
    "PrefillInputs", "DecodeInputs", "make_prefill", "make_decode",
    "round_to_bf16", "bf16_bits_to_f32", "prune_chunks",
]


# ----------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    block_size: int        # L_B
    segment_size: int      # L_S
    probe_len: int         # P: last P queries of each segment
    dtype: str             # "bf16" or "f32"
    head_types: str        # "fixed" | "fraction" | "per_segment"
    rigid_heads: tuple = ()        # used when head_types == "fixed"
    rigid_fraction: float = 0.4    # used when head_types == "fraction"
    hot_count: str = "2"           # "2", "8", or "poisson4"
    hot_dist: str = "uniform"      # "uniform" or "zipf1.2"

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block_size

    @property
    def n_segments(self) -> int:
        return self.seq_len // self.segment_size


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_len: int
    n_obs: int
    n_sink: int
    n_recent: int
    n_keep: int
    dtype: str = "bf16"
    planted_fraction: float = 0.01


PREFILL_CONFIGS = {
    # 1 layer, 4 query / 2 KV heads, d 64, 2k tokens, fp32; heads 0 and 2 rigid.
    "tiny-2k-f32": PrefillConfig("tiny-2k-f32", 4, 2, 64, 2048, 64, 512, 64, "f32",
                                 head_types="fixed", rigid_heads=(0, 2),
                                 hot_count="2"),
    # Llama-3-8B-shaped layer at 32k.
    "llama3-8b-32k": PrefillConfig("llama3-8b-32k", 32, 8, 128, 32768, 128, 4096, 64,
                                   "bf16", head_types="fraction", hot_count="2"),
    # Llama-3-8B-shaped layer at 128k, 8 hot blocks per segment, Zipf(1.2).
    "llama3-8b-128k": PrefillConfig("llama3-8b-128k", 32, 8, 128, 131072, 128, 8192,
                                    64, "bf16", head_types="fraction", hot_count="8",
                                    hot_dist="zipf1.2"),
    # Qwen-shaped layer at 64k: head type drawn per segment, Poisson(4) hot blocks.
    "qwen-64k": PrefillConfig("qwen-64k", 28, 4, 128, 65536, 128, 4096, 64, "bf16",
                              head_types="per_segment", hot_count="poisson4"),
}

DECODE_CONFIGS = {
    "decode-retain-b8-128k": DecodeConfig("decode-retain-b8-128k", 8, 32, 8, 128,
                                          131072, 64, 4, 256, 4096),
}


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) in numpy
# ----------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Return the bf16 bit patterns (int16 array) of float32 `x`, RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporary memory on very large tensors
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.size, step):
        v = flat_u[i:i + step]
        bias = ((v >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[i:i + step] = ((v + bias) >> np.uint32(16)).astype(np.uint16)
    return out.view(np.int16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (int16/uint16) to exact float32 values."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# Containers
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    seed: int
    q: np.ndarray          # storage values as float32 [Hq, N, d] (exactly representable in dtype)
    k: np.ndarray          # [Hkv, N, d]
    v: np.ndarray          # [Hkv, N, d]
    q_store: np.ndarray    # storage array: int16 bf16 bits or float32
    k_store: np.ndarray
    v_store: np.ndarray
    rigid_hs: np.ndarray   # [Hq, C_S] bool, planted head type per (head, segment)
    hot_blocks: dict       # (h, s) -> sorted np.ndarray of planted hot block ids


@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    seed: int
    q_obs: np.ndarray      # float32 values [B, Hq, W, d]
    k: np.ndarray          # [B, Hkv, L, d]
    v: np.ndarray          # [B, Hkv, L, d]
    q_new: np.ndarray      # [B, Hq, d]
    q_obs_store: np.ndarray
    k_store: np.ndarray
    v_store: np.ndarray
    q_new_store: np.ndarray
    focused: np.ndarray    # [B, Hq] bool
    planted: np.ndarray    # [B, Hkv, n_planted] int64 sorted planted positions


def _store(x: np.ndarray, dtype: str):
    if dtype == "bf16":
        bits = round_to_bf16(x)
        return bf16_bits_to_f32(bits), bits
    if dtype == "f32":
        x = np.ascontiguousarray(x, dtype=np.float32)
        return x, x
    raise ValueError(f"unknown dtype {dtype!r}")


def _orthonormal_bank(rng, d: int, m: int) -> np.ndarray:
    g = rng.standard_normal((d, m))
    qmat, _ = np.linalg.qr(g)
    return qmat[:, :m].T.copy()   # [m, d], rows orthonormal


# ----------------------------------------------------------------------------
# Prefill generator
# ----------------------------------------------------------------------------
def make_prefill(cfg: PrefillConfig, seed: int = 0) -> PrefillInputs:
    Hq, Hkv, d, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len
    LB, LS = cfg.block_size, cfg.segment_size
    if N % LS or LS % LB or Hq % Hkv:
        raise ValueError("shape does not divide")
    r = Hq // Hkv
    CS = N // LS
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((Hkv, N, d), dtype=np.float32)
    c = float(np.sqrt(d))

    m = min(d, r + r * CS)
    if r + r * CS > d:
        raise ValueError("head_dim too small for the direction bank")
    banks = [_orthonormal_bank(rng, d, m) for _ in range(Hkv)]

    # head types
    if cfg.head_types == "fixed":
        rigid_h = np.zeros(Hq, dtype=bool)
        rigid_h[list(cfg.rigid_heads)] = True
        rigid_hs = np.repeat(rigid_h[:, None], CS, axis=1)
    elif cfg.head_types == "fraction":
        n_rigid = int(round(cfg.rigid_fraction * Hq))
        rigid_h = np.zeros(Hq, dtype=bool)
        rigid_h[rng.choice(Hq, n_rigid, replace=False)] = True
        rigid_hs = np.repeat(rigid_h[:, None], CS, axis=1)
    elif cfg.head_types == "per_segment":
        rigid_hs = rng.random((Hq, CS)) < 0.5
    else:
        raise ValueError(cfg.head_types)

    # hot blocks, head-major then segment-minor
    hot_blocks = {}
    for h in range(Hq):
        for s in range(CS):
            if rigid_hs[h, s]:
                continue
            cb = (s + 1) * LS // LB
            cand = np.arange(1, cb)
            if cfg.hot_count == "poisson4":
                n_hot = int(rng.poisson(4.0))
            else:
                n_hot = int(cfg.hot_count)
            n_hot = min(n_hot, cand.size)
            if n_hot == 0:
                hot_blocks[(h, s)] = np.zeros(0, dtype=np.int64)
                continue
            if cfg.hot_dist == "uniform":
                pick = rng.choice(cand, n_hot, replace=False)
            elif cfg.hot_dist == "zipf1.2":
                w = cand.astype(np.float64) ** -1.2
                pick = rng.choice(cand, n_hot, replace=False, p=w / w.sum())
            else:
                raise ValueError(cfg.hot_dist)
            hot_blocks[(h, s)] = np.sort(pick.astype(np.int64))

    # planting (float64 directions added to float32 noise)
    sink = np.zeros((Hkv, d))
    for h in range(Hq):
        g, hl = h // r, h % r
        rho = banks[g][hl]
        if rigid_hs[h].any():
            sink[g] += 8.0 * LB * c * rho
        for s in range(CS):
            rows = slice(s * LS, (s + 1) * LS)
            if rigid_hs[h, s]:
                q[h, rows] += (c * rho).astype(np.float32)
            else:
                nu = banks[g][r + hl * CS + s]
                q[h, rows] += (c * nu).astype(np.float32)
                for j in hot_blocks[(h, s)]:
                    k[g, j * LB:(j + 1) * LB] += (4.0 * c * nu).astype(np.float32)
    for g in range(Hkv):
        if np.any(sink[g] != 0):
            k[g, 0] = sink[g].astype(np.float32)

    qv, qs = _store(q, cfg.dtype)
    del q
    kv_, ks = _store(k, cfg.dtype)
    del k
    vv, vs = _store(v, cfg.dtype)
    del v
    return PrefillInputs(cfg, seed, qv, kv_, vv, qs, ks, vs, rigid_hs, hot_blocks)


# ----------------------------------------------------------------------------
# Decode generator
# ----------------------------------------------------------------------------
def make_decode(cfg: DecodeConfig, seed: int = 0,
                batch: Optional[int] = None, cache_len: Optional[int] = None) -> DecodeInputs:
    """Decode-retention inputs.  `batch` / `cache_len` override the config to
    draw a smaller instance with the same recipe."""
    B = cfg.batch if batch is None else batch
    L = cfg.cache_len if cache_len is None else cache_len
    Hq, Hkv, d, W = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_obs
    r = Hq // Hkv
    rng = np.random.default_rng(seed)
    q_obs = rng.standard_normal((B, Hq, W, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, L, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, L, d), dtype=np.float32)
    q_new = rng.standard_normal((B, Hq, d), dtype=np.float32)
    c = float(np.sqrt(d))

    dirs = rng.standard_normal((B, Hkv, d))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    focused = rng.random((B, Hq)) < 0.5
    for b in range(B):
        for g in range(Hkv):
            if not focused[b, g * r:(g + 1) * r].any():
                focused[b, g * r + int(rng.integers(r))] = True

    lo, hi = min(4, L), max(min(4, L), L - 256)
    n_pl = min(int(round(cfg.planted_fraction * L)), hi - lo)
    planted = np.zeros((B, Hkv, n_pl), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            pos = np.sort(rng.choice(np.arange(lo, hi), n_pl, replace=False))
            planted[b, g] = pos
            k[b, g, pos] += (4.0 * c * dirs[b, g]).astype(np.float32)
    for b in range(B):
        for h in range(Hq):
            if focused[b, h]:
                add = (c * dirs[b, h // r]).astype(np.float32)
                q_obs[b, h] += add
                q_new[b, h] += add

    qo, qos = _store(q_obs, cfg.dtype)
    kk, ks = _store(k, cfg.dtype)
    del k
    vv, vs = _store(v, cfg.dtype)
    del v
    qn, qns = _store(q_new, cfg.dtype)
    return DecodeInputs(cfg, seed, qo, kk, vv, qn, qos, ks, vs, qns, focused, planted)


def prune_chunks(T: int, W: int, k: int, n_prefix: int = 64, n_query: int = 0,
                 seed: int = 0) -> np.ndarray:
    """Candidate document chunks [k, 2] int32 (begin, end) for a prompt of T
    tokens: `n_prefix` protected tokens, k documents with one protected
    delimiter after each, then the protected query of max(n_query, W) tokens."""
    q_len = max(n_query, W)
    space = T - n_prefix - q_len - k
    if k < 1 or space < k:
        raise ValueError("prompt too short for the chunks")
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.5, 1.5, k)
    n = np.maximum(1, np.floor(w / w.sum() * space).astype(np.int64))
    while n.sum() > space:
        n[int(np.argmax(n))] -= 1
    out = np.empty((k, 2), dtype=np.int32)
    pos = n_prefix
    for i in range(k):
        out[i] = (pos, pos + n[i])
        pos += int(n[i]) + 1
    return out


def small_prefill_config(**kw) -> PrefillConfig:
    """A small prefill workload with the same recipe (for tests)."""
    base = dict(name="small", n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=2048,
                block_size=64, segment_size=512, probe_len=64, dtype="bf16",
                head_types="fixed", rigid_heads=(0, 2), hot_count="2")
    base.update(kw)
    return PrefillConfig(**base)
