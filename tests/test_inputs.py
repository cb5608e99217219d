"""The seeded input generator: determinism, layout and bf16 rounding."""
import numpy as np
import pytest
import torch

import tra_inputs as ti


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, -3.0e38], dtype=np.float32)])
    # values exactly half-way between two bf16 values (ties to even)
    ties = (np.arange(1000, dtype=np.uint32) * np.uint32(0x10000) + np.uint32(0x3F808000)).view(np.float32)
    x = np.concatenate([x, ties])
    mine = ti.bf16_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = ti.bf16_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_per_head():
    q, k, v = ti.make_inputs(3, 9, 10, 3, 32, seed=0, family=7)
    q2, k2, v2 = ti.make_inputs(3, 9, 10, 3, 32, seed=0, family=7)
    assert q.shape == (3, 3, 9, 10, 32) and q.dtype == np.uint16
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    qh, kh, vh = ti.make_inputs(3, 9, 10, 3, 32, seed=0, family=7, heads_only=[2])
    assert np.array_equal(qh[0], q[2]) and np.array_equal(kh[0], k[2]) and np.array_equal(vh[0], v[2])
    q3, _, _ = ti.make_inputs(3, 9, 10, 3, 32, seed=1, family=7)
    assert not np.array_equal(q, q3)


@pytest.mark.parametrize("kind", ["smooth", "frames20", "bimodal80"])
def test_sigma_maps(kind):
    s = ti.sigma_map(10, 12, 14, kind, seed=0, family=1)
    assert s.shape == (10, 12, 14)
    assert s.min() >= 0.1 - 1e-12 and s.max() <= 1.0 + 1e-12
    if kind == "frames20":
        hi = np.all(s == 1.0, axis=(1, 2))
        assert hi.sum() == 2 and np.all(s[~hi] == 0.1)
    if kind == "bimodal80":
        frac = (s == 1.0).mean()
        assert 0.15 < frac <= 0.2 + 1e-9


def test_config_table():
    c = ti.WORKLOADS[ti.WAN13B_81F]
    assert (c.T, c.H, c.W, c.heads, c.d, c.r_min, c.r_max) == (21, 30, 52, 12, 128, 1, 8)
    assert c.N == 32760
    assert ti.WORKLOADS[ti.HUNYUAN_129F].N == 118800
