"""Seeded input generation: rounding and the named workload shapes."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-40],
                                 np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_named_workload_shapes(num):
    c = workloads.workload(num, values=False)
    L = c.lengths
    if num == 1:
        assert list(L) == [256] and c.heads == 2 and c.d == 64 and c.dtype == "fp32"
        assert c.alpha == 0.125 and c.n == 256.0
    if num == 2:
        assert list(c.offsets) == list(range(0, 65537, 4096)) and c.heads == 4
        assert c.d == 64 and c.dtype == "bf16" and c.n == 4096.0 and c.alpha == 0.125
        assert abs(c.useful_flops() - 137.47e9) < 0.01e9
    if num == 3:
        assert len(L) == 64 and L.min() >= 16 and L.max() <= 8192 and c.d == 128
        assert c.n == float(L.max()) and c.alpha == float(np.float32(1 / np.sqrt(128)))
    if num == 4:
        assert len(L) == 8 and L.min() >= 8192 and L.max() <= 20480 and c.n == 20480.0
    if num == 5:
        assert len(L) == 4096 and L.min() >= 1 and L.max() <= 256 and c.dtype == "fp16"
        assert c.heads == 2 and c.d == 128 and c.n == 256.0


def test_workload_is_deterministic():
    a = workloads.workload(1)
    b = workloads.workload(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)


def test_rab_inputs_shapes_ranges_and_determinism():
    off = workloads.offsets_from_lengths([0, 5, 300, 1])
    a = workloads.make_rab_inputs(off, 40, 12, seed=9)
    b = workloads.make_rab_inputs(off, 40, 12, seed=9)
    assert a.timestamps.dtype == np.int32 and a.timestamps.shape == (306,)
    assert a.pos_bias.dtype == np.float32 and a.pos_bias.shape == (40,)
    assert a.time_bias.dtype == np.float32 and a.time_bias.shape == (12,)
    for x, y in ((a.timestamps, b.timestamps), (a.pos_bias, b.pos_bias),
                 (a.time_bias, b.time_bias)):
        assert np.array_equal(x, y)
    # non-decreasing inside each sequence, gaps below 2^16, starts in [0, 2^30)
    for i in range(len(off) - 1):
        t = a.timestamps[off[i]:off[i + 1]].astype(np.int64)
        if len(t):
            assert 0 <= t[0] < (1 << 30)
            g = np.diff(t)
            assert np.all(g >= 0) and np.all(g < (1 << 16))


def test_rab_workload_shape():
    case, r = workloads.rab_workload(values=False)
    assert case is None
    assert r.timestamps.shape == (16 * 4096,)
    assert r.pos_bias.shape == (4096,) and r.time_bias.shape == (16,)
