"""Generator checks: bf16 rounding, determinism and planted-structure bookkeeping."""
import numpy as np
import torch

from entropy_guided_sparse_amd import synth


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1000,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.3895e38,
                                  1e-40, -2.5, 65504.0], dtype=np.float32)])
    ours = synth.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ours),
                                  torch.from_numpy(ref).view(torch.bfloat16).float().numpy())


def test_prefill_generator_is_deterministic_and_consistent():
    cfg = synth.small_prefill_config()
    a = synth.make_prefill(cfg, seed=3)
    b = synth.make_prefill(cfg, seed=3)
    np.testing.assert_array_equal(a.q_store, b.q_store)
    np.testing.assert_array_equal(a.k_store, b.k_store)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(a.k_store), a.k)
    assert a.q.shape == (4, 2048, 64) and a.k.shape == (2, 2048, 64)
    for (h, s), hot in a.hot_blocks.items():
        cb = (s + 1) * cfg.segment_size // cfg.block_size
        assert np.all((hot >= 1) & (hot < cb))
    c = synth.make_prefill(cfg, seed=4)
    assert not np.array_equal(a.q_store, c.q_store)


def test_fp32_workload_is_exact_float32():
    cfg = synth.PREFILL_CONFIGS["tiny-2k-f32"]
    a = synth.make_prefill(cfg, seed=0)
    assert a.q_store.dtype == np.float32 and a.q_store is a.q
    assert a.rigid_hs[[0, 2]].all() and not a.rigid_hs[[1, 3]].any()


def test_decode_generator_small():
    cfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
    a = synth.make_decode(cfg, seed=0, batch=2, cache_len=4096)
    assert a.k.shape == (2, 8, 4096, 128) and a.q_obs.shape == (2, 32, 64, 128)
    assert a.planted.shape == (2, 8, 41)
    assert np.all(a.planted >= 4) and np.all(a.planted < 4096 - 256)
    for b in range(2):
        for g in range(8):
            assert a.focused[b, g * 4:(g + 1) * 4].any()
