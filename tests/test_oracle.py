"""CPU tests: the float64 oracle against its pins, and the input generators."""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A
import workloads as W
from tests import oracle_pins as P


@pytest.mark.parametrize("name", list(P.ALL_PINS))
def test_pin(name):
    ok, detail = P.ALL_PINS[name]()
    assert ok, f"pin {name} failed: {detail}"


def test_bf16_generator_rounding_matches_torch():
    # torch's float32 -> bfloat16 cast rounds to nearest even; an independent routine
    x = np.random.default_rng(3).standard_normal(200_000, dtype=np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # exact ties
    mine = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = W.bf16_bits_to_f64(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_oracle_bf16_grid_rounding_matches_torch():
    x = np.random.default_rng(4).standard_normal(100_000) * 7
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 + 2 ** -7, -4.0 - 3 * 2 ** -6])
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(A.bf16_round_nearest_even(x), ref)


def test_standard_workload_recipe():
    w = W.standard_config(1)
    assert w.q.shape == (1, 256, 2, 64) and w.k.shape == (1, 256, 2, 64)
    assert math.isclose(w.softmax_scale, 1 / 8)
    # same seed, same bits
    assert np.array_equal(W.standard_config(1).q, w.q)
    w4 = W.standard_config(4)
    lens = np.diff(w4.cu_seqlens_q)
    assert len(lens) == 8 and lens.min() >= 512 and lens.max() <= 8192
    assert np.array_equal(w4.cu_seqlens_q, w4.cu_seqlens_k)
    assert w4.window_left == 1024 and w4.window_right == 0 and w4.causal
    assert w4.q.shape == (int(lens.sum()), 32, 128)


def test_bf16_inputs_look_normal():
    w = W.standard_config(1)
    x = W.bf16_bits_to_f64(w.q)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_visible_pairs_closed_forms():
    # causal Sq = Sk = S: S(S+1)/2 pairs; causal window wl: sum_i min(i+1, wl+1)
    assert A.visible_pairs(100, 100, causal=True) == 100 * 101 // 2
    L, wl = 3000, 1024
    want = sum(min(i + 1, wl + 1) for i in range(L))
    assert A.visible_pairs(L, L, causal=True, window_left=wl, window_right=0) == want
    assert want == 1025 * L - 524800  # n(L) = 1025 L - 524800 for L > 1025


def test_golden_mask_normalization():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mask_normalization.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        sq, sk = c["seqlen_q"], c["seqlen_k"]
        vis = A.visible_mask(sq, sk, c["causal"], c["window_left"], c["window_right"])
        counts = [int(x) for x in vis.sum(axis=1)]
        assert counts == c["visible_per_row"], c
