"""Float64 CPU oracle for entropy-guided, head-adaptive sparse prefill attention
and decode-time KV retention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The library's HIP path
never calls it, and this module shares no code, table or helper with the HIP
path: it is plain numpy in float64, written step by step from the pages.

Sources (cited by page title and section / equation / algorithm):
  [EI]  "From Rigid to Dynamic: Entropy-Guided Adaptive Inference for
        Long-Context LLMs" (EntropyInfer), arXiv 2606.09508.
  [KV]  Blog notes "attention-kv-cache-mechanics", section on InfoKV
        (eq. 4 window-mean attention score, eq. 8 fused score).
  [EP]  "EntroPrefill: Renyi-Guided Context Pruning with Conditional Stability
        Guarantees for Retrieval-Augmented Generation", Sec. 2.1 (GQA attention,
        observer-pooled measure), Sec. 3.1 (sink-isolated Renyi pooling,
        regularized head weights), Sec. 8.1 (online softmax / compaction).

Readings taken where the pages are silent or garbled are listed in each
function's docstring (R-numbers match the design notes).

Parity status: every function here is pinned by the not-gpu tests
(closed forms, worked example, library special cases, brute force) except the
tie-free part of selection beyond brute force, which is pinned only by
sorting-library brute force and planted recall.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "causal_blocks", "pool_mean", "pool_maxmin", "observation_rows",
    "observation_rows_maxmin", "shannon", "renyi", "entropy_of_rows",
    "entropy_score", "classify", "kclamp", "allocate_budget", "select_topk",
    "select_blocks", "qblock_list", "sparse_prefill_attn",
    "sparse_prefill_attn_rows", "window_mean", "head_weights", "kv_retain",
    "kv_retain_slice", "sparse_decode_attn", "softmax", "page_scores", "forced_pages",
    "page_select", "page_retain", "PAGE_GROUP", "PAGE_LAYER_UNION", "PAGE_HEAD_UNION",
    "latent_due", "latent_decode", "prune_pooled_measure", "prune_row_chunk_mass",
    "prune_priorities", "prune_greedy", "prune_certificate", "chunk_prune",
]

MODE_FIXED, MODE_TWO_LEVEL, MODE_PROPORTIONAL, MODE_ALG3 = 0, 1, 2, 3
SHANNON, RENYI = 0, 1


# ----------------------------------------------------------------------------
# helpers (plain definitions)
# ----------------------------------------------------------------------------
def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(z - max) / sum exp(z - max) along `axis`; -inf entries get 0."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_blocks(s: int, L_S: int, L_B: int) -> int:
    """C_B(s) = (s+1) * L_S / L_B: key blocks visible to segment s.
    [EI] Sec. 4.1 notation (C_{B_i} per segment); block-causal reading R3."""
    return (s + 1) * L_S // L_B


def _sm_scale(d: int, sm_scale: Optional[float]) -> float:
    # [EI] Sec. 2 / Sec. 3.1: softmax(Q K^T / sqrt(d)); applied everywhere (R2).
    return 1.0 / math.sqrt(d) if not sm_scale else float(sm_scale)


# ----------------------------------------------------------------------------
# Step 1: pooling
# ----------------------------------------------------------------------------
def pool_mean(K: np.ndarray, L_B: int) -> np.ndarray:
    """Mean of the keys of every L_B-token block: K [Hkv, N, d] -> [Hkv, N/L_B, d].
    The block partition follows [EI] Sec. 4.2 (observation matrix built from
    blocks, after CritiPrefill) and App. A eq. (1) (C_S x C_B entries).  Mean
    pooling with a query probe is the reading R1."""
    K = np.asarray(K, dtype=np.float64)
    H, N, d = K.shape
    return K.reshape(H, N // L_B, L_B, d).mean(axis=2)


def pool_maxmin(X: np.ndarray, L: int):
    """Element-wise max and min over every chunk of L rows ([EI] Sec. 4.2,
    Alg. 1: Q_Max / Q_Min by reshape(N_S, L_S, d) then max / min over dim 1;
    K_Rep "follows a similar process", taken per key block)."""
    X = np.asarray(X, dtype=np.float64)
    H, N, d = X.shape
    r = X.reshape(H, N // L, L, d)
    return r.max(axis=2), r.min(axis=2)


# ----------------------------------------------------------------------------
# Steps 2-4: observation rows
# ----------------------------------------------------------------------------
def observation_rows(Q, K, L_S: int, L_B: int, P: int, sm_scale=None) -> np.ndarray:
    """Probe observation rows a_bar [Hq, C_S, C_B] (mean-probe mode).

    For head h (KV group g = h // r, reading R12) and segment s:
      probe rows u = last P queries of segment s         (R1; CateKV rebuttal:
                                                            last queries observe best)
      z_{u,j} = sigma * q_{h,u} . kbar_{g,j},  j < C_B(s) (R3: block-causal)
      a_{u,.} = softmax_j(z_{u,.})
      a_bar_{h,s,j} = (1/P) sum_u a_{u,j}                 ([KV] eq. 4 window mean;
                                                            [EP] Sec. 2.1 observer pool)
    Entries j >= C_B(s) hold the sentinel -1."""
    Q = np.asarray(Q, dtype=np.float64)
    Hq, N, d = Q.shape
    Hkv = K.shape[0]
    r = Hq // Hkv
    C_S, C_B = N // L_S, N // L_B
    sc = _sm_scale(d, sm_scale)
    kbar = pool_mean(K, L_B)
    abar = np.full((Hq, C_S, C_B), -1.0)
    for h in range(Hq):
        g = h // r
        for s in range(C_S):
            cb = causal_blocks(s, L_S, L_B)
            probe = Q[h, (s + 1) * L_S - P:(s + 1) * L_S]
            z = sc * (probe @ kbar[g, :cb].T)
            abar[h, s, :cb] = softmax(z, axis=1).mean(axis=0)
    return abar


def observation_rows_maxmin(Q, K, L_S: int, L_B: int, sm_scale=None) -> np.ndarray:
    """Paper-literal observation rows ([EI] Sec. 4.2, Alg. 1 and Alg. 2).

    Q_max/Q_min per segment, K_max/K_min per key block;
    S1..S4 = softmax over the causal blocks of sigma * (Q_x . K_y);
    A_obs = elementwise max((S1+S2)/2, (S3+S4)/2), renormalised to sum 1 (R5).
    sigma = 1/sqrt(d) is applied although Alg. 2 omits it (R2)."""
    Q = np.asarray(Q, dtype=np.float64)
    Hq, N, d = Q.shape
    Hkv = K.shape[0]
    r = Hq // Hkv
    C_S, C_B = N // L_S, N // L_B
    sc = _sm_scale(d, sm_scale)
    qmax, qmin = pool_maxmin(Q, L_S)
    kmax, kmin = pool_maxmin(K, L_B)
    abar = np.full((Hq, C_S, C_B), -1.0)
    for h in range(Hq):
        g = h // r
        for s in range(C_S):
            cb = causal_blocks(s, L_S, L_B)
            s1 = softmax(sc * kmax[g, :cb] @ qmax[h, s])
            s2 = softmax(sc * kmin[g, :cb] @ qmax[h, s])
            s3 = softmax(sc * kmax[g, :cb] @ qmin[h, s])
            s4 = softmax(sc * kmin[g, :cb] @ qmin[h, s])
            a = np.maximum((s1 + s2) / 2.0, (s3 + s4) / 2.0)
            abar[h, s, :cb] = a / a.sum()
    return abar


# ----------------------------------------------------------------------------
# Step 5: entropy
# ----------------------------------------------------------------------------
def shannon(p) -> float:
    """H(p) = -sum_j p_j ln p_j with 0 ln 0 = 0 (natural log).
    [EI] Sec. 2 and Sec. 3.1 (row-wise attention entropy); [EP] Sec. 2.2
    (natural logarithms)."""
    p = np.asarray(p, dtype=np.float64)
    p = p[p > 0]
    return float(-np.sum(p * np.log(p)))


def renyi(p, alpha: float) -> float:
    """Renyi entropy of order alpha: ln(sum_j p_j^alpha) / (1 - alpha).
    alpha = 1 is Shannon.  [EP] Sec. 3.1 (order two: -ln of the collision sum),
    Sec. 3.2 (the Renyi family, monotone in alpha).  alpha <= 0 is rejected
    (reading R18)."""
    if not alpha > 0 or not math.isfinite(alpha):
        raise ValueError("renyi order must be finite and > 0")
    if alpha == 1.0:
        return shannon(p)
    p = np.asarray(p, dtype=np.float64)
    p = p[p > 0]
    return float(np.log(np.sum(p ** alpha)) / (1.0 - alpha))


def entropy_of_rows(abar: np.ndarray, L_S: int, L_B: int, kind: int = SHANNON,
                    alpha: float = 2.0) -> np.ndarray:
    """E[h, s] = entropy of the observation row over its causal blocks
    ([EI] Sec. 4.2: entropy of every row of A_obs; reading R4)."""
    Hq, C_S, _ = abar.shape
    E = np.zeros((Hq, C_S))
    for h in range(Hq):
        for s in range(C_S):
            row = abar[h, s, :causal_blocks(s, L_S, L_B)]
            E[h, s] = shannon(row) if kind == SHANNON else renyi(row, alpha)
    return E


def entropy_score(Q, K, L_S, L_B, P, kind=SHANNON, alpha=2.0, sm_scale=None,
                  pool="mean"):
    """Steps 1-5 together: (a_bar [Hq, C_S, C_B], E [Hq, C_S])."""
    if pool == "mean":
        abar = observation_rows(Q, K, L_S, L_B, P, sm_scale)
    elif pool == "maxmin":
        abar = observation_rows_maxmin(Q, K, L_S, L_B, sm_scale)
    else:
        raise ValueError(pool)
    return abar, entropy_of_rows(abar, L_S, L_B, kind, alpha)


# ----------------------------------------------------------------------------
# Steps 6-7: classification and budgets
# ----------------------------------------------------------------------------
def classify(E: np.ndarray, threshold: float) -> np.ndarray:
    """Rigid(h) <=> max over segments of E[h, s] < e_t.
    [EI] Sec. 4.2, Alg. 3 (the head test on the maximum segment entropy)."""
    return np.max(np.asarray(E, dtype=np.float64), axis=1) < threshold


def kclamp(x: float, cb: int) -> int:
    """Budget in blocks: min(C_B(s), max(1, ceil(x - 1e-9))) (reading R9:
    a product that lands on an integer up to rounding stays that integer)."""
    return int(min(cb, max(1, math.ceil(x - 1e-9))))


def allocate_budget(E, L_S: int, L_B: int, mode: int, frac=0.25, frac_rigid=0.05,
                    frac_dynamic=0.30, frac_min=0.02, frac_max=0.50,
                    entropy_threshold=0.5, base_tokens=2048.0, alg3_alpha=0.5,
                    alg3_delta_t=0.4):
    """Per-(head, segment) key-block budgets k [Hq, C_S] and rigid flags [Hq].

    FIXED(f):           k = kclamp(f * C_B(s))
    TWO_LEVEL(fr, fd):  f = fr for rigid heads, fd otherwise ([EI] Sec. 1:
                        rigid heads get a fixed minimal budget, dynamic more)
    PROPORTIONAL:       f = min(fmax, max(fmin, fmax * E / ln C_B(s)))  (R14)
    ALG3(B_h tokens):   [EI] Sec. 4.2, Alg. 3.  Rigid: B_s = B_h.  Dynamic:
                        B_0 = B_h; B_s = clamp(B_{s-1} + alpha * B_h *
                        (|e_s - e_{s-1}| / max(e_{s-1}, e_t) - Delta_t), B_h, 3 B_h)
                        (R6: garbled clamp read as [B_h, 3 B_h]; R7: guarded
                        divisor; R8: segments 0..C_S-1);  k = kclamp(B_s / L_B)."""
    E = np.asarray(E, dtype=np.float64)
    Hq, C_S = E.shape
    rigid = classify(E, entropy_threshold)
    k = np.zeros((Hq, C_S), dtype=np.int64)
    for h in range(Hq):
        if mode == MODE_ALG3:
            Bs = float(base_tokens)
            for s in range(C_S):
                if s > 0 and not rigid[h]:
                    prev = E[h, s - 1]
                    fluct = abs(E[h, s] - prev) / max(prev, entropy_threshold)
                    Bs = Bs + alg3_alpha * base_tokens * (fluct - alg3_delta_t)
                    Bs = min(max(Bs, base_tokens), 3.0 * base_tokens)
                k[h, s] = kclamp(Bs / L_B, causal_blocks(s, L_S, L_B))
            continue
        for s in range(C_S):
            cb = causal_blocks(s, L_S, L_B)
            if mode == MODE_FIXED:
                f = frac
            elif mode == MODE_TWO_LEVEL:
                f = frac_rigid if rigid[h] else frac_dynamic
            elif mode == MODE_PROPORTIONAL:
                ehat = E[h, s] / math.log(cb) if cb > 1 else 0.0
                f = min(frac_max, max(frac_min, frac_max * ehat))
            else:
                raise ValueError(mode)
            k[h, s] = kclamp(f * cb, cb)
    return rigid, k


# ----------------------------------------------------------------------------
# Step 8: top-k selection
# ----------------------------------------------------------------------------
def select_topk(scores: Sequence[float], k: int) -> list:
    """Indices of the k best entries under the order (score descending, index
    ascending), returned ascending.  Top-k keep rule: [EI] App. A eq. (2)
    (top-k blocks) and Alg. 4 step 3 (TopK); tie-break to the lower index."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def select_blocks(abar, budget, L_S: int, L_B: int, k_max: Optional[int] = None):
    """Sel(h, s) for every (head, segment): block_idx [Hq, C_S, k_max]
    ascending and padded with -1, block_cnt [Hq, C_S]."""
    Hq, C_S, _ = abar.shape
    budget = np.asarray(budget)
    if k_max is None:
        k_max = int(budget.max())
    idx = np.full((Hq, C_S, k_max), -1, dtype=np.int64)
    cnt = np.zeros((Hq, C_S), dtype=np.int64)
    for h in range(Hq):
        for s in range(C_S):
            cb = causal_blocks(s, L_S, L_B)
            kk = int(min(budget[h, s], cb, k_max))
            sel = select_topk(abar[h, s, :cb], kk)
            idx[h, s, :len(sel)] = sel
            cnt[h, s] = len(sel)
    return idx, cnt


# ----------------------------------------------------------------------------
# Steps 9-10: block-sparse causal GQA attention
# ----------------------------------------------------------------------------
def qblock_list(block_idx, block_cnt, h: int, b: int, L_S: int, L_B: int) -> list:
    """L(h, b) = {j in Sel(h, s) : j < b} union {b}, s = segment of q-block b.
    Reading R10: the own (diagonal) block is always attended, causally masked;
    selected blocks at or after b are not attended."""
    s = (b * L_B) // L_S
    sel = [int(j) for j in block_idx[h, s, :int(block_cnt[h, s])]]
    return sorted({j for j in sel if 0 <= j < b}) + [b]


def sparse_prefill_attn_rows(Q, K, V, block_idx, block_cnt, h: int, b: int,
                             L_S: int, L_B: int, sm_scale=None):
    """Output rows of q-block b of head h: (O [L_B, d], lse [L_B]).

    Causal GQA attention ([EP] Sec. 2.1: A_{u,j} = exp z_uj / sum_{v<=u} exp z_uv,
    z = q_u . k_{g(h), j} / sqrt(d)) restricted to the keys of the blocks in
    L(h, b) ([EI] App. A eq. (3): attention over the selected blocks only)."""
    Q = np.asarray(Q); K = np.asarray(K); V = np.asarray(V)
    Hq, N, d = Q.shape
    r = Hq // K.shape[0]
    g = h // r
    sc = _sm_scale(d, sm_scale)
    blocks = qblock_list(block_idx, block_cnt, h, b, L_S, L_B)
    keys = np.concatenate([np.arange(j * L_B, (j + 1) * L_B) for j in blocks])
    rows = np.arange(b * L_B, (b + 1) * L_B)
    q = Q[h, rows].astype(np.float64)
    kk = K[g, keys].astype(np.float64)
    vv = V[g, keys].astype(np.float64)
    z = sc * (q @ kk.T)
    z[keys[None, :] > rows[:, None]] = -np.inf
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    O = (p @ vv) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def sparse_prefill_attn(Q, K, V, block_idx, block_cnt, L_S: int, L_B: int,
                        sm_scale=None):
    """Whole output O [Hq, N, d] and lse [Hq, N] (natural log)."""
    Hq, N, d = Q.shape
    O = np.zeros((Hq, N, d))
    lse = np.zeros((Hq, N))
    for h in range(Hq):
        for b in range(N // L_B):
            o, l = sparse_prefill_attn_rows(Q, K, V, block_idx, block_cnt, h, b,
                                            L_S, L_B, sm_scale)
            O[h, b * L_B:(b + 1) * L_B] = o
            lse[h, b * L_B:(b + 1) * L_B] = l
    return O, lse


# ----------------------------------------------------------------------------
# Step 11: decode-time KV retention
# ----------------------------------------------------------------------------
def window_mean(A_rows) -> np.ndarray:
    """a_t = (1/W) sum_u A_{u,t}: [KV] eq. 4 window-mean attention score;
    [EP] Sec. 2.1 observer-pooled measure a^h_j."""
    A_rows = np.asarray(A_rows, dtype=np.float64)
    return A_rows.sum(axis=0) / A_rows.shape[0]


def sink_isolated_entropy(a, n_sink: int, kind: int = SHANNON, alpha: float = 2.0):
    """[EP] Sec. 3.1: a~_j = a_j / z_h over non-sink positions, then the entropy
    of a~ (order 2: -ln sum a~^2).  Shannon is the alpha = 1 member."""
    a = np.asarray(a, dtype=np.float64)[n_sink:]
    z = a.sum()
    if not z > 0:
        return 0.0
    at = a / z
    return shannon(at) if kind == SHANNON else renyi(at, alpha)


def head_weights(H, zeta: float, tau: float) -> np.ndarray:
    """w_h = zeta / r + (1 - zeta) * v_h, v_h = softmax_h(-H_h / tau) within the
    GQA group ([EP] Sec. 3.1: regularized head weighting with group floor zeta
    and entropy temperature tau; reading R15)."""
    H = np.asarray(H, dtype=np.float64)
    r = H.size
    v = softmax(-H / tau)
    return zeta / r + (1.0 - zeta) * v


def kv_retain_slice(q_obs, k, n_sink: int, n_recent: int, n_keep: int,
                    kind: int = SHANNON, alpha: float = 2.0, zeta: float = 0.5,
                    tau: float = 1.0, raw: bool = False, info_alpha: float = 1.0,
                    token_entropy=None, sm_scale=None):
    """Retention for one (batch, KV group) slice.

    q_obs [r, W, d] observer queries of the group's heads; k [L, d].
    Returns (keep [n_total] ascending, mu [L], H [r]).

    Observer u sits at position L - W + u and sees keys t <= L - W + u (R16).
      A^h_{u,t} = causal softmax          ([EP] Sec. 2.1)
      a^h_t     = window mean              ([KV] eq. 4)
      H_h       = sink-isolated entropy    ([EP] Sec. 3.1)
      w_h       = regularized weights      ([EP] Sec. 3.1)
      mu_t      = sum_h w_h a^h_t          ([EP] Sec. 3.1 group mixture)
      optional InfoKV fusion mu <- alpha_I mu + (1 - alpha_I) softmax_t(E_tok)
                                           ([KV] eq. 8)
    RAW mode (the literal score of [EI] Alg. 4): mu_t = sum_h sum_u
    sigma q_{h,u} . k_t with no mask and no softmax.
    keep = sinks U top-n_keep of [n_sink, L - n_recent) under (-mu, t) U recent
    (R17), or everything when n_sink + n_recent + n_keep >= L."""
    q_obs = np.asarray(q_obs, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    r, W, d = q_obs.shape
    L = k.shape[0]
    sc = _sm_scale(d, sm_scale)
    H = np.zeros(r)
    if raw:
        mu = np.zeros(L)
        for h in range(r):
            mu += (sc * (q_obs[h] @ k.T)).sum(axis=0)
    else:
        a = np.zeros((r, L))
        pos = L - W + np.arange(W)
        for h in range(r):
            z = sc * (q_obs[h] @ k.T)
            z[np.arange(L)[None, :] > pos[:, None]] = -np.inf
            a[h] = window_mean(softmax(z, axis=1))
            H[h] = sink_isolated_entropy(a[h], n_sink, kind, alpha)
        w = head_weights(H, zeta, tau)
        mu = (w[:, None] * a).sum(axis=0)
        if token_entropy is not None and info_alpha < 1.0:
            mu = info_alpha * mu + (1.0 - info_alpha) * softmax(
                np.asarray(token_entropy, dtype=np.float64))
    if n_sink + n_recent + n_keep >= L:
        return np.arange(L), mu, H
    cand_lo, cand_hi = n_sink, L - n_recent
    top = select_topk(mu[cand_lo:cand_hi], n_keep)
    keep = list(range(n_sink)) + [cand_lo + t for t in top] + list(range(cand_hi, L))
    return np.asarray(sorted(keep), dtype=np.int64), mu, H


def kv_retain(q_obs, k, v, n_sink, n_recent, n_keep, kind=SHANNON, alpha=2.0,
              zeta=0.5, tau=1.0, raw=False, info_alpha=1.0, token_entropy=None,
              sm_scale=None, slices=None):
    """All (batch, KV group) slices, or only those listed in `slices`.
    Returns dict (b, g) -> (keep, k_kept, v_kept, mu, H).  Compaction keeps
    token order ([EP] Sec. 8.1: gather of retained entries, original order;
    [EI] Alg. 4 step 4)."""
    B, Hq, W, d = q_obs.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    out = {}
    todo = slices if slices is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for (b, g) in todo:
        te = None if token_entropy is None else token_entropy[b]
        keep, mu, H = kv_retain_slice(q_obs[b, g * r:(g + 1) * r], k[b, g], n_sink,
                                      n_recent, n_keep, kind, alpha, zeta, tau, raw,
                                      info_alpha, te, sm_scale)
        out[(b, g)] = (keep, np.asarray(k[b, g], dtype=np.float64)[keep],
                       np.asarray(v[b, g], dtype=np.float64)[keep], mu, H)
    return out


# ----------------------------------------------------------------------------
# Step 12: decode attention over the kept entries
# ----------------------------------------------------------------------------
def sparse_decode_attn(q_new, k_kept, v_kept, sm_scale=None):
    """o_h = sum_t softmax_t(sigma q_h . k_{g,t}) v_{g,t} over the kept entries
    (all of them precede the new token, so there is no mask).
    q_new [B, Hq, d]; k_kept / v_kept [B, Hkv, n_total, d] -> o [B, Hq, d]."""
    q_new = np.asarray(q_new, dtype=np.float64)
    B, Hq, d = q_new.shape
    Hkv = k_kept.shape[1]
    r = Hq // Hkv
    sc = _sm_scale(d, sm_scale)
    o = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            kk = np.asarray(k_kept[b, h // r], dtype=np.float64)
            vv = np.asarray(v_kept[b, h // r], dtype=np.float64)
            p = softmax(sc * (kk @ q_new[b, h]))
            o[b, h] = p @ vv
    return o


# ----------------------------------------------------------------------------
# Page-level retention ([EP] Sec. 7, GQA unions and physical page budgets)
# ----------------------------------------------------------------------------
PAGE_GROUP, PAGE_LAYER_UNION, PAGE_HEAD_UNION = 0, 1, 2


def page_scores(p, page_size: int) -> np.ndarray:
    """I(P_i) = max over the tokens j of page P_i of p(j), pages
    P_i = [i S, (i + 1) S) clipped to [0, L) ([EP] Sec. 7: a page's importance
    is the largest token mass it holds)."""
    p = np.asarray(p, dtype=np.float64)
    L = p.size
    n_pages = -(-L // page_size)
    return np.array([p[i * page_size:min(L, (i + 1) * page_size)].max()
                     for i in range(n_pages)])


def forced_pages(L: int, page_size: int, n_sink: int, n_recent: int) -> set:
    """Pages that hold a sink (t < n_sink) or a recent position
    (t >= L - n_recent): always kept, as the token-level rule keeps those
    positions (reading R21)."""
    n_pages = -(-L // page_size)
    out = set()
    for i in range(n_pages):
        lo, hi = i * page_size, min(L, (i + 1) * page_size) - 1
        if lo < n_sink or hi >= L - n_recent:
            out.add(i)
    return out


def page_select(p, page_size: int, n_sink: int, n_recent: int, n_keep_pages: int) -> list:
    """The forced pages plus the n_keep_pages best other pages under the order
    (I(P) descending, page index ascending), returned ascending ([EP] Sec. 7:
    a page set K chosen by page maxima; tie-break as for tokens, R11)."""
    I = page_scores(p, page_size)
    forced = forced_pages(len(p), page_size, n_sink, n_recent)
    cand = [i for i in range(I.size) if i not in forced]
    top = select_topk([I[i] for i in cand], n_keep_pages)
    return sorted(forced | {cand[t] for t in top})


def page_retain(scores, page_size: int, n_sink: int, n_recent: int, n_keep_pages: int,
                mode: int = PAGE_GROUP, r: int = 1) -> list:
    """Kept page lists for every batch element ([EP] Sec. 7).

    scores [B, X, L]: per KV group (X = H_kv) for PAGE_GROUP and
    PAGE_LAYER_UNION, per query head (X = H_q, r heads per group) for
    PAGE_HEAD_UNION.
      PAGE_GROUP        K_{b,g} = page_select(scores[b, g])
      PAGE_HEAD_UNION   U_{b,g} = union over the r heads h of group g of
                        page_select(scores[b, h])   (UOR_g = |U_{b,g}| / |K_h|)
      PAGE_LAYER_UNION  U_b = union over the groups g of page_select(scores[b, g])
                        (one physical block holds every group)
    Returns out[b][y] = ascending page indices, y over groups (PAGE_GROUP,
    PAGE_HEAD_UNION) or the single layer set (PAGE_LAYER_UNION)."""
    scores = np.asarray(scores, dtype=np.float64)
    B, X, _ = scores.shape
    out = []
    for b in range(B):
        sets = [page_select(scores[b, x], page_size, n_sink, n_recent, n_keep_pages)
                for x in range(X)]
        if mode == PAGE_GROUP:
            out.append(sets)
        elif mode == PAGE_HEAD_UNION:
            out.append([sorted(set().union(*sets[g * r:(g + 1) * r])) for g in range(X // r)])
        elif mode == PAGE_LAYER_UNION:
            out.append([sorted(set().union(*sets))])
        else:
            raise ValueError(mode)
    return out


# ----------------------------------------------------------------------------
# Latent decoding ([EI] Sec. 4.3 and App. B; [KV] InfoKV: compress every fixed
# number of generated tokens)
# ----------------------------------------------------------------------------
def latent_due(step: int, n_delay: int, interval: int) -> bool:
    """Compression after the step-th generated token: once n_delay tokens have
    been generated ([EI] Sec. 4.3, N_d), then every `interval` tokens (0 = once)."""
    return step == n_delay or (interval > 0 and step > n_delay
                               and (step - n_delay) % interval == 0)


def latent_decode(k0, v0, q_win0, steps, n_sink: int, n_recent: int, n_keep: int,
                  n_delay: int, interval: int, keep_fn=None, sm_scale=None, **retain_kw):
    """Decode loop with latent compression.

    k0, v0 [B, Hkv, L0, d]: the prompt's cache; q_win0 [B, Hq, W, d]: the
    queries of its last W positions; steps: (q [B, Hq, d], k [B, Hkv, d],
    v [B, Hkv, d]) per generated token.  Each step appends (k, v), moves the
    query window by one, attends q over every cache entry (the new one
    included), and when latent_due() compresses every (b, g) cache with
    kv_retain_slice using the window as observers (so the generated queries
    take part in the ranking, [EI] Sec. 4.3); kept entries stay in order
    ([EI] Alg. 4 step 4).  keep_fn(step, b, g, keep, mu) may replace a keep set
    (tests use it to follow another implementation's equal-score choices).
    Returns (outputs [T, B, Hq, d], events [(step, {(b, g): (keep, mu)})])."""
    k0 = np.asarray(k0, dtype=np.float64)
    v0 = np.asarray(v0, dtype=np.float64)
    win = np.array(q_win0, dtype=np.float64)
    B, Hkv, _, d = k0.shape
    Hq = win.shape[1]
    r = Hq // Hkv
    Kc = [[k0[b, g] for g in range(Hkv)] for b in range(B)]
    Vc = [[v0[b, g] for g in range(Hkv)] for b in range(B)]
    outs, events = [], []
    for step, (q, k, v) in enumerate(steps, 1):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        for b in range(B):
            for g in range(Hkv):
                Kc[b][g] = np.vstack([Kc[b][g], k[b, g][None]])
                Vc[b][g] = np.vstack([Vc[b][g], v[b, g][None]])
        win = np.concatenate([win[:, :, 1:], q[:, :, None]], axis=2)
        o = np.zeros((B, Hq, d))
        for b in range(B):
            for h in range(Hq):
                g = h // r
                o[b, h] = sparse_decode_attn(q[b:b + 1, h:h + 1], Kc[b][g][None, None],
                                             Vc[b][g][None, None], sm_scale)[0, 0]
        outs.append(o)
        if latent_due(step, n_delay, interval):
            ev = {}
            for b in range(B):
                for g in range(Hkv):
                    keep, mu, _ = kv_retain_slice(win[b, g * r:(g + 1) * r], Kc[b][g], n_sink,
                                                  n_recent, n_keep, sm_scale=sm_scale,
                                                  **retain_kw)
                    if keep_fn is not None:
                        keep = np.asarray(keep_fn(step, b, g, keep, mu))
                    Kc[b][g] = Kc[b][g][keep]
                    Vc[b][g] = Vc[b][g][keep]
                    ev[(b, g)] = (keep, mu)
            events.append((step, ev))
    return np.stack(outs), events


# ----------------------------------------------------------------------------
# Chunk pruning ([EP] Sec. 2.1, Sec. 3.1-3.2, Sec. 4.1-4.2)
# ----------------------------------------------------------------------------
def _obs_rows(q_obs_h, k_g, T, sc):
    """Causal attention rows of the observers u (positions T - W + u) over all
    T positions ([EP] Sec. 2.1): A [W, T]."""
    W = q_obs_h.shape[0]
    z = sc * (q_obs_h @ k_g.T)
    pos = T - W + np.arange(W)
    z[np.arange(T)[None, :] > pos[:, None]] = -np.inf
    return softmax(z, axis=1)


def prune_pooled_measure(q_obs, k, n_sink: int, zeta: float = 0.5, tau: float = 1.0,
                         sm_scale=None, rows: bool = True):
    """mu^l_j = (1/G) sum_g sum_{h in g} w_h a^h_j with the window means a^h,
    Renyi-2 sink-isolated head entropies and the regularized weights
    ([EP] Sec. 3.1); q_obs [Hq, W, d], k [Hkv, T, d].  Returns (mu [T],
    A [Hq, W, T]); with rows=False, A is not kept (None) and the heads'
    rows are formed one head at a time."""
    Hq, W, d = np.shape(q_obs)
    Hkv, T, _ = np.shape(k)
    r = Hq // Hkv
    sc = _sm_scale(d, sm_scale)
    A = np.empty((Hq, W, T)) if rows else None
    mu = np.zeros(T)
    for g in range(Hkv):
        kg = np.asarray(k[g], dtype=np.float64)
        a = np.empty((r, T))
        for i in range(r):
            h = g * r + i
            Ah = _obs_rows(np.asarray(q_obs[h], dtype=np.float64), kg, T, sc)
            a[i] = Ah.mean(axis=0)
            if rows:
                A[h] = Ah
        H = np.array([sink_isolated_entropy(a[i], n_sink, RENYI, 2.0) for i in range(r)])
        w = head_weights(H, zeta, tau)
        mu += (w[:, None] * a).sum(axis=0)
    return mu / Hkv, A


def prune_head_rows(q_obs, k, h: int, sm_scale=None) -> np.ndarray:
    """A[h] alone, the observer rows [W, T] of query head h over its group's
    keys ([EP] Sec. 2.1), for checking single heads at sizes where all of A
    does not fit."""
    Hq, W, d = np.shape(q_obs)
    Hkv, T, _ = np.shape(k)
    g = h // (Hq // Hkv)
    return _obs_rows(np.asarray(q_obs[h], dtype=np.float64), np.asarray(k[g], dtype=np.float64),
                     T, _sm_scale(d, sm_scale))


def prune_row_chunk_mass(A, chunks) -> np.ndarray:
    """m[a, i] = sum over j in chunk i of A_{a, j}, rows a = (h, u) in
    head-major order ([EP] Sec. 4.2, the row constraints)."""
    A = np.asarray(A, dtype=np.float64)
    rows = A.reshape(-1, A.shape[-1])
    return np.stack([rows[:, b:e].sum(axis=1) for (b, e) in chunks], axis=1)


def prune_priorities(mu, chunks, eps_s: float, lam: float):
    """Null-calibrated chunk priorities ([EP] Sec. 3.2), reading R23:
    p = mu restricted to the candidate tokens and renormalised; pi_i = n_i / N
    (uniform null); M_i = sum_{j in c_i} p_j;
    p_hat_ij = (p_j + eps_s pi_i / n_i) / (M_i + eps_s pi_i);
    l_i = (M_i + eps_s pi_i) / ((1 + eps_s) pi_i);
    kappa_i = -H_2(p_hat_i) / ln n_i in [-1, 0] (0 for a one-token chunk);
    S_i = ln l_i + lam kappa_i.  Returns (S, l, kappa, M)."""
    mu = np.asarray(mu, dtype=np.float64)
    n = np.array([e - b for (b, e) in chunks], dtype=np.float64)
    N = n.sum()
    Z = sum(mu[b:e].sum() for (b, e) in chunks)
    S, ell, kap, M = [], [], [], []
    for i, (b, e) in enumerate(chunks):
        p = mu[b:e] / Z
        pi = n[i] / N
        Mi = p.sum()
        ph = (p + eps_s * pi / n[i]) / (Mi + eps_s * pi)
        li = (Mi + eps_s * pi) / ((1.0 + eps_s) * pi)
        ki = 0.0 if n[i] < 2 else -(-math.log(float((ph ** 2).sum()))) / math.log(n[i])
        S.append(math.log(li) + lam * ki)
        ell.append(li)
        kap.append(ki)
        M.append(Mi)
    return np.array(S), np.array(ell), np.array(kap), np.array(M)


def prune_greedy(S, n, m, eps: float, m0: int, target: int, dtype=np.float64):
    """The reference proposer of [EP] Sec. 4.2: chunks in increasing S_i, ties
    by larger n_i, then lower index; one scan; chunk i joins the removal set
    only if every row keeps sum_{i in E} m[a, i] <= eps and |E| <= k - m0; the
    scan stops once the removed tokens reach `target`.  The running row sums
    are kept in `dtype` (float32 when following a float32 implementation).
    Returns (removed flags [k] bool, removed tokens)."""
    k = len(S)
    order = sorted(range(k), key=lambda i: (float(S[i]), -int(n[i]), i))
    cur = np.zeros(m.shape[0], dtype=dtype)
    m = np.asarray(m, dtype=dtype)
    removed = np.zeros(k, dtype=bool)
    tokens, count = 0, 0
    for i in order:
        if tokens >= target:
            break
        if count + 1 > k - m0:
            break
        nxt = cur + m[:, i]
        if np.all(nxt <= dtype(eps)):
            cur = nxt
            removed[i] = True
            tokens += int(n[i])
            count += 1
    return removed, tokens


def prune_certificate(n, m, eps: float, m0: int, y, t: float) -> float:
    """U(y, t) = sum_a y_a eps + t (k - m0) + sum_i [n_i - sum_a y_a m[a, i] - t]_+
    with prices y_a >= 0 (one per row; a scalar prices every row alike) and
    t >= 0 ([EP] Sec. 4.2): an upper bound on the most tokens any feasible
    removal set can remove."""
    n = np.asarray(n, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    R, k = m.shape
    ya = np.broadcast_to(np.asarray(y, dtype=np.float64), (R,))
    return (float(ya.sum()) * eps + t * (k - m0)
            + float(np.maximum(n - ya @ m - t, 0.0).sum()))


def chunk_prune(q_obs, k, chunks, n_sink: int, eps_s: float, lam: float, eps: float,
                m0: int, target: int, zeta: float = 0.5, tau: float = 1.0, sm_scale=None):
    """Steps together: pooled measure, row-chunk masses, priorities, greedy
    removal.  Returns dict(mu, m, S, removed, tokens)."""
    mu, A = prune_pooled_measure(q_obs, k, n_sink, zeta, tau, sm_scale)
    m = prune_row_chunk_mass(A, chunks)
    S, ell, kap, M = prune_priorities(mu, chunks, eps_s, lam)
    n = np.array([e - b for (b, e) in chunks])
    removed, tokens = prune_greedy(S, n, m, eps, m0, target)
    return dict(mu=mu, m=m, S=S, ell=ell, kappa=kap, M=M, removed=removed, tokens=tokens)
