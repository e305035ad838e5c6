"""egs_entropy_score_static (the workspace-free form of egs_entropy_score for
callers that cannot allocate) against egs_entropy_score through the C ABI:
the same kernels on the same inputs, so block scores and entropies must be
bit-identical.  Two calls in a row, the second on a smaller layer, so the
second runs on scratch that still holds the first call's contents."""
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


def _both(api, cfg, kind, pool, seed):
    inp = synth.make_prefill(cfg, seed=seed)
    shape = prefill_shape(api, cfg)
    q = dev_tensor(inp.q_store, cfg.dtype)
    k = dev_tensor(inp.k_store, cfg.dtype)
    s_ws, e_ws = api.entropy_score(shape, q, k, kind=kind, renyi_alpha=2.0, pool=pool)
    s_st, e_st = api.entropy_score_static(shape, q, k, kind=kind, renyi_alpha=2.0, pool=pool)
    torch.cuda.synchronize()
    return s_ws.cpu().numpy(), e_ws.cpu().numpy(), s_st.cpu().numpy(), e_st.cpu().numpy()


@pytest.mark.parametrize("pool", [0, 1])
def test_static_scratch_matches_workspace_form(api, pool):
    big = synth.PREFILL_CONFIGS["qwen-64k"]
    small = synth.small_prefill_config(name="small", n_q_heads=8, n_kv_heads=2, head_dim=128,
                                       seq_len=4096, block_size=64, segment_size=1024)
    for cfg, kind, seed in ((big, 0, 0), (small, 1, 3)):
        log(f"[static scratch] {cfg.name} pool={pool} kind={kind} N={cfg.seq_len}")
        s_ws, e_ws, s_st, e_st = _both(api, cfg, kind, pool, seed)
        np.testing.assert_array_equal(s_st, s_ws)
        np.testing.assert_array_equal(e_st, e_ws)
        assert np.isfinite(e_st).all()
