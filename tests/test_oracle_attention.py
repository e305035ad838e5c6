"""Pins for the block-sparse causal GQA attention oracle against torch's
float64 scaled_dot_product_attention on the CPU (a library routine)."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import egs_oracle as O

HQ, HKV, D, N, LB, LS = 4, 2, 16, 256, 16, 64
R = HQ // HKV


def _qkv(seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((HQ, N, D)), rng.standard_normal((HKV, N, D)),
            rng.standard_normal((HKV, N, D)))


def _sdpa(Q, K, V, mask=None, causal=False):
    q = torch.from_numpy(Q)[None]
    k = torch.from_numpy(np.repeat(K, R, axis=0))[None]
    v = torch.from_numpy(np.repeat(V, R, axis=0))[None]
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal)
    return out[0].numpy()


def _random_lists(seed, full=False, empty=False):
    rng = np.random.default_rng(seed)
    CS, CB = N // LS, N // LB
    abar = np.full((HQ, CS, CB), -1.0)
    budget = np.zeros((HQ, CS), dtype=np.int64)
    for h in range(HQ):
        for s in range(CS):
            cb = (s + 1) * LS // LB
            abar[h, s, :cb] = rng.dirichlet(np.ones(cb))
            budget[h, s] = cb if full else (0 if empty else rng.integers(1, cb + 1))
    return O.select_blocks(abar, budget, LS, LB, k_max=CB)


def test_full_budget_equals_dense_causal_sdpa():
    Q, K, V = _qkv(0)
    idx, cnt = _random_lists(0, full=True)
    out, lse = O.sparse_prefill_attn(Q, K, V, idx, cnt, LS, LB)
    ref = _sdpa(Q, K, V, causal=True)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # log-sum-exp of the causal scaled logits
    z = torch.from_numpy(Q) @ torch.from_numpy(np.repeat(K, R, axis=0)).transpose(1, 2)
    z = z / math.sqrt(D)
    z = z.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=-1).numpy(), atol=1e-12)


def _explicit_mask(idx, cnt):
    """N x N boolean mask per head built straight from the selected-block lists."""
    mask = np.zeros((HQ, N, N), dtype=bool)
    for h in range(HQ):
        for i in range(N):
            b, s = i // LB, i // LS
            sel = set(idx[h, s, :cnt[h, s]].tolist())
            for t in range(i + 1):
                j = t // LB
                mask[h, i, t] = (j == b) or (j in sel and j < b)
    return mask


def test_random_lists_equal_explicit_mask_sdpa():
    for seed in (1, 2):
        Q, K, V = _qkv(seed)
        idx, cnt = _random_lists(seed)
        out, _ = O.sparse_prefill_attn(Q, K, V, idx, cnt, LS, LB)
        mask = torch.from_numpy(_explicit_mask(idx, cnt))[None]
        np.testing.assert_allclose(out, _sdpa(Q, K, V, mask=mask), atol=1e-12)


def test_empty_selection_attends_own_block_only():
    Q, K, V = _qkv(3)
    idx, cnt = _random_lists(3, empty=True)
    out, _ = O.sparse_prefill_attn(Q, K, V, idx, cnt, LS, LB)
    for b in range(N // LB):
        sl = slice(b * LB, (b + 1) * LB)
        ref = _sdpa(Q[:, sl].copy(), K[:, sl].copy(), V[:, sl].copy(), causal=True)
        np.testing.assert_allclose(out[:, sl], ref, atol=1e-12)


def test_output_perturbation_bound():
    # EntroPrefill Sec. 4.1: ||o - o_R|| <= 2 V eta, eta = dense mass on the
    # excluded keys, V = max value norm.
    Q, K, V = _qkv(4)
    idx, cnt = _random_lists(4)
    out, _ = O.sparse_prefill_attn(Q, K, V, idx, cnt, LS, LB)
    dense = _sdpa(Q, K, V, causal=True)
    probs = _sdpa(Q, K.copy(), np.tile(np.eye(N), (HKV, 1, 1)), causal=True)  # rows of A
    keep = _explicit_mask(idx, cnt)
    vmax = np.linalg.norm(V, axis=-1).max()
    for h in range(HQ):
        eta = (probs[h] * (~keep[h])).sum(axis=1)
        gap = np.linalg.norm(dense[h] - out[h], axis=1)
        assert np.all(gap <= 2 * vmax * eta + 1e-10)
