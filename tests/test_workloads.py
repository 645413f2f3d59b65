"""Seeded input generators: shapes, length recipes and bf16 rounding; CPU only."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]      # exact ties round to even
    mine = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = W.bf16_bits_to_f64(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_length_recipes():
    L2 = W.lengths_cfg2(0)
    assert len(L2) == 16 and L2.sum() == 4096 and L2.min() >= 64 * 4096 // (16 * 512) - 1
    L4 = W.lengths_cfg4(0)
    assert L4[0] == 16384 and L4.sum() == 32768 and L4[1:].max() <= 1024
    L5, used = W.lengths_cfg5(0)
    assert L5.sum() == 16384 and all(v in L5.tolist() for v in W.EDGE_VALUES)
    assert (L5 == 0).any()
    raw = W.raw_lengths_cfg3(0)
    assert raw.shape == (20000,) and raw.min() >= 8 and raw.max() == 8192


def test_small_workload_shapes_and_determinism():
    w1 = W.make(1)
    assert w1.q.shape == (12, 2, 64) and w1.q.dtype == np.uint16 and w1.do is None
    w1b = W.make(1)
    assert np.array_equal(w1.q, w1b.q) and not np.array_equal(w1.q, w1.k)
    w = W.random_small(3, [5, 0, 7], H=2, d=64)
    assert w.q.shape == (12, 2, 64) and w.do.shape == (12, 2, 64)
