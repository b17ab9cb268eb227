"""The seeded input generator: deterministic, the right shapes, and the stated value mix."""
import numpy as np

from all_reduce_residual_way_amd import synth


def test_deterministic_and_seed_dependent():
    a = synth.make_problem(4, 8, 64, seed=3)
    b = synth.make_problem(4, 8, 64, seed=3)
    c = synth.make_problem(4, 8, 64, seed=4)
    for x, y in zip(a.inputs + [a.residual, a.weight], b.inputs + [b.residual, b.weight]):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.inputs[0], c.inputs[0])


def test_shapes_and_spread():
    p = synth.make_problem(8, 64, 512, seed=0)
    assert p.n == 8 and p.m == 64 and p.hidden == 512
    assert all(x.dtype == np.uint16 and x.shape == (64, 512) for x in p.inputs)
    assert p.weight.shape == (512,)
    import torch
    vals = torch.from_numpy(p.inputs[0].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert 0.45 < vals.std() < 0.55
    w = torch.from_numpy(p.weight.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert 0.95 < w.mean() < 1.05 and 0.07 < w.std() < 0.13


def test_stress_rows():
    p = synth.make_problem(8, 2048, 64, seed=5, dist="stress")
    zero, big = p.meta["zero_rows"], p.meta["big_rows"]
    assert 5 <= len(zero) <= 45 and 5 <= len(big) <= 45
    for x in p.inputs:
        assert not x[zero].any()
        assert set(np.unique(x[big]).tolist()) <= {0x46EA, 0xC6EA}


def test_stress_row_counts():
    ms = synth.stress_m_values(0)
    assert {1, 16, 17, 2048} <= set(ms) and all(1 <= m <= 2048 for m in ms)
