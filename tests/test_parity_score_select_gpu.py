"""egs_score_select (steps 1-8 in one call) against egs_entropy_score +
egs_allocate_budget + egs_select_blocks through the C ABI: the same kernels'
arithmetic, so scores, entropies, classes, budgets and block lists must be
bit-identical, for every budget policy, both entropy kinds, both pooling
kinds, the fp32 generic path and the full-size workloads' launch shapes."""
import numpy as np
import pytest
import torch

from _parity import dev_tensor, log, prefill_shape
from bench import k_max_for, prefill_policy
from entropy_guided_sparse_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _compare(api, cfg, pol, k_max, kind=0, pool=0, seed=0):
    log(f"[score_select] {cfg.name} N={cfg.seq_len} mode={pol.mode} kind={kind} pool={pool}")
    inp = synth.make_prefill(cfg, seed=seed)
    shape = prefill_shape(api, cfg)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    scores, E = api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0, pool=pool)
    rigid, budget = api.allocate_budget(shape, pol, E)
    idx, cnt = api.select_blocks(shape, scores, budget, k_max)
    fused = api.score_select(shape, pol, q, k, k_max, kind=kind, renyi_alpha=2.0, pool=pool)
    torch.cuda.synchronize()
    for name, want in (("block_scores", scores), ("entropy", E), ("head_is_rigid", rigid),
                       ("budget", budget), ("block_idx", idx), ("block_cnt", cnt)):
        got = fused[name]
        assert torch.equal(got.view(torch.int32) if got.dtype == torch.float32 else got,
                           want.view(torch.int32) if want.dtype == torch.float32 else want), name
    log(f"  bit-identical; budgets {int(budget.min())}..{int(budget.max())}, "
        f"rigid heads {int(rigid.sum())}")


def test_tiny_fp32_fixed_and_alg3(api):
    cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    _compare(api, cfg, api.BudgetPolicy(mode=api.L.EGS_BUDGET_FIXED, frac=0.25), cfg.n_blocks)
    _compare(api, cfg, api.BudgetPolicy(mode=api.L.EGS_BUDGET_ALG3, base_tokens=512.0,
                                        entropy_threshold=1e-5), cfg.n_blocks)


def test_small_bf16_renyi_two_level_and_maxmin(api):
    cfg = synth.small_prefill_config(name="ss", n_q_heads=8, n_kv_heads=2, head_dim=128,
                                     seq_len=8192, block_size=64, segment_size=1024)
    pol = api.BudgetPolicy(mode=api.L.EGS_BUDGET_TWO_LEVEL, frac_rigid=0.1, frac_dynamic=0.4,
                           entropy_threshold=0.5)
    _compare(api, cfg, pol, 60, kind=1, seed=2)
    _compare(api, cfg, pol, 128, kind=0, pool=1, seed=3)
    _compare(api, cfg, api.BudgetPolicy(mode=api.L.EGS_BUDGET_ALG3, base_tokens=1024.0,
                                        entropy_threshold=1e-5), 128, kind=1, pool=1, seed=4)


@pytest.mark.parametrize("name", ["llama3-8b-32k", "qwen-64k", "llama3-8b-128k"])
def test_full_workloads(api, name):
    cfg = synth.PREFILL_CONFIGS[name]
    pol = prefill_policy(api, cfg)
    _compare(api, cfg, pol, k_max_for(pol, api, cfg.n_blocks, cfg.block_size))
