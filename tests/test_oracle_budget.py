"""Pins for head classification and budget allocation (hand-computed tables)."""
import math

import numpy as np

from oracle import egs_oracle as O


def test_fixed_quarter_of_causal_blocks_tiny_workload():
    # 2k tokens, block 64, segment 512: C_B(s) = 8, 16, 24, 32; 25% -> 2, 4, 6, 8.
    E = np.zeros((4, 4))
    _, k = O.allocate_budget(E, 512, 64, O.MODE_FIXED, frac=0.25)
    assert k.tolist() == [[2, 4, 6, 8]] * 4


def test_two_level_table_32k():
    # 32k tokens, block 128, segment 4096: C_B(s) = 32 (s + 1).
    # rigid 5%:   ceil(1.6 (s+1)) = 2, 4, 5, 7, 8, 10, 12, 13
    # dynamic 30%: ceil(9.6 (s+1)) = 10, 20, 29, 39, 48, 58, 68, 77
    E = np.array([[0.0] * 8, [0.7] * 8, [0.49] * 8, [0.0] * 7 + [0.5]])
    rigid, k = O.allocate_budget(E, 4096, 128, O.MODE_TWO_LEVEL, frac_rigid=0.05,
                                 frac_dynamic=0.30, entropy_threshold=0.5)
    assert rigid.tolist() == [True, False, True, False]
    rig = [2, 4, 5, 7, 8, 10, 12, 13]
    dyn = [10, 20, 29, 39, 48, 58, 68, 77]
    assert k.tolist() == [rig, dyn, rig, dyn]


def test_proportional_endpoints():
    # 4 segments of 8 blocks each (C_B = 8, 16, 24, 32).
    cbs = [8, 16, 24, 32]
    E = np.array([[0.0] * 4,
                  [math.log(c) for c in cbs],
                  [0.5 * math.log(c) for c in cbs],
                  [10.0] * 4])
    _, k = O.allocate_budget(E, 512, 64, O.MODE_PROPORTIONAL, frac_min=0.02, frac_max=0.5)
    assert k[0].tolist() == [1, 1, 1, 1]          # ceil(0.02 * C_B) = 1
    assert k[1].tolist() == [4, 8, 12, 16]        # 0.5 * C_B
    assert k[2].tolist() == [2, 4, 6, 8]          # 0.25 * C_B
    assert k[3].tolist() == [4, 8, 12, 16]        # capped at f_max


def test_proportional_single_block_segment():
    # C_B(0) = 1 -> normalised entropy taken as 0, budget 1.
    E = np.array([[0.3, 0.3]])
    _, k = O.allocate_budget(E, 64, 64, O.MODE_PROPORTIONAL)
    assert k.tolist() == [[1, 1]]


def test_alg3_hand_sequence():
    # B_h = 512 tokens, L_B = 64, alpha 0.5, Delta_t 0.4, e_t = 1e-5.
    # e = 1.0, 2.0, 2.0, 0.5:
    #   B0 = 512
    #   B1 = 512 + 256 * (1/1 - 0.4)      = 665.6 -> k = ceil(10.4) = 11
    #   B2 = 665.6 + 256 * (0 - 0.4)      = 563.2 -> k = ceil(8.8)  = 9
    #   B3 = 563.2 + 256 * (1.5/2 - 0.4)  = 652.8 -> k = ceil(10.2) = 11
    E = np.array([[1.0, 2.0, 2.0, 0.5]])
    rigid, k = O.allocate_budget(E, 512, 64, O.MODE_ALG3, base_tokens=512.0,
                                 entropy_threshold=1e-5, alg3_alpha=0.5, alg3_delta_t=0.4)
    assert rigid.tolist() == [False]
    assert k.tolist() == [[8, 11, 9, 11]]


def test_alg3_clamps_and_guard():
    # L_S = 2048, L_B = 64 -> C_B(s) = 32, 64, 96.
    # e = 0.1, 1.0, 1.0: B1 = 512 + 256 (9 - 0.4) = 2713.6 -> capped at 1536 (k 24);
    # B2 = 1536 - 102.4 = 1433.6 -> k = ceil(22.4) = 23.
    E = np.array([[0.1, 1.0, 1.0],
                  [0.0, 0.3, 0.3],      # previous entropy 0 -> divisor e_t
                  [0.3, 0.3, 0.3]])     # flat: lower clamp at B_h
    _, k = O.allocate_budget(E, 2048, 64, O.MODE_ALG3, base_tokens=512.0,
                             entropy_threshold=1e-5)
    assert k[0].tolist() == [8, 24, 23]
    assert k[1].tolist() == [8, 24, 23]
    assert k[2].tolist() == [8, 8, 8]


def test_alg3_rigid_head_keeps_base_budget():
    E = np.array([[0.0, 1e-6, 5e-6, 0.0]])
    rigid, k = O.allocate_budget(E, 512, 64, O.MODE_ALG3, base_tokens=512.0,
                                 entropy_threshold=1e-5)
    assert rigid.tolist() == [True]
    assert k.tolist() == [[8, 8, 8, 8]]


def test_budget_never_exceeds_causal_blocks():
    E = np.array([[3.0, 3.0]])
    _, k = O.allocate_budget(E, 128, 64, O.MODE_FIXED, frac=5.0)
    assert k.tolist() == [[2, 4]]
    _, k = O.allocate_budget(E, 128, 64, O.MODE_ALG3, base_tokens=4096.0,
                             entropy_threshold=1e-5)
    assert k.tolist() == [[2, 4]]


def test_classify_uses_maximum_over_segments():
    E = np.array([[0.1, 0.2, 0.6], [0.49, 0.0, 0.3]])
    assert O.classify(E, 0.5).tolist() == [False, True]
