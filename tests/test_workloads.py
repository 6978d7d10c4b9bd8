"""The seeded input generator: determinism, shapes, value recipe, cache table."""
import math

import numpy as np
import pytest

from head_qk_rmsnorm_amd import workloads as W
from oracle import qknr_oracle as O


def test_same_seed_same_bytes():
    c = W.case(9, 3, 2, 128, 64, True, dtype=W.FP16, pos_dtype=W.I64, seed=4)
    a, b = W.make_workload(c), W.make_workload(c)
    for f in ("q", "k", "wq", "wk", "cache", "positions"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c2 = W.case(9, 3, 2, 128, 64, True, dtype=W.FP16, pos_dtype=W.I64, seed=5)
    assert not np.array_equal(W.make_workload(c2).q, a.q)


def test_tiny_config_recipe():
    wl = W.make_workload(W.CONFIGS["tiny"])
    c = wl.cfg
    assert wl.q.shape == (16, 4, 64) and wl.k.shape == (16, 4, 64)
    assert wl.q.dtype == np.uint16 and wl.positions.dtype == np.int32
    assert np.array_equal(wl.positions, np.arange(16))
    assert wl.cache.shape == (64, 64) and wl.cache.dtype == np.float32
    w = O.decode_bf16(wl.wq)
    assert w.min() >= 0.5 and w.max() <= 1.5
    assert c.algorithmic_bytes() == 37184


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dit", "gqa", "partial"])
def test_config_shapes_and_statistics(name):
    c = W.CONFIGS[name]
    wl = W.make_workload(c)
    assert wl.q.shape == (c.T, c.Hq, c.head_dim) and wl.k.shape == (c.T, c.Hkv, c.head_dim)
    assert wl.positions.dtype == (np.int32 if c.pos_dtype == W.I32 else np.int64)
    assert wl.positions.min() >= 0 and wl.positions.max() < c.cache_rows
    x = O.decode_io(wl.q[::7], c.dtype)
    assert abs(x.mean()) < 0.01 * c.x_std and abs(x.std() / c.x_std - 1) < 0.01
    if name == "dit":
        assert np.array_equal(np.sort(wl.positions), np.arange(c.T))
        assert not np.array_equal(wl.positions, np.arange(c.T))
    if name == "gqa":
        assert wl.qkv.shape == (c.T, (c.Hq + 2 * c.Hkv) * c.head_dim)
        # q and k are views into the fused buffer with token stride (Hq+2Hkv)*D elements
        assert wl.q.strides == (wl.qkv.strides[0], c.head_dim * 2, 2)
        assert np.shares_memory(wl.q, wl.qkv) and np.shares_memory(wl.k, wl.qkv)
        assert wl.v.shape == (c.T, c.Hkv * c.head_dim)
    if name == "partial":
        assert len(np.unique(wl.positions)) < c.T  # uniform draws repeat


def test_outlier_channels():
    c = W.case(64, 3, 2, 256, 256, False, outlier_frac=0.01, outlier_scale=50.0, seed=9)
    wl = W.make_workload(c)
    x = O.decode_bf16(wl.q).reshape(c.T, -1)
    big = np.sort(np.argsort(-np.abs(x).mean(axis=0))[: int(round(0.01 * 3 * 256))])
    ch_std = x.std(axis=0)
    assert np.all(ch_std[big] > 20) and np.median(ch_std) < 2


@pytest.mark.parametrize("R,base", [(64, 1e4), (128, 1e6), (256, 1e4), (8, 1e4)])
def test_cache_table(R, base):
    """Row 0 is [1..1 | 0..0]; cos^2 + sin^2 = 1 to fp32 rounding; column j=0
    (theta_0 = 1) is cos p, sin p."""
    rows = 300
    cache = W.rope_cache(rows, R, base)
    assert np.all(cache[0, : R // 2] == 1.0) and np.all(cache[0, R // 2:] == 0.0)
    c = cache[:, : R // 2].astype(np.float64)
    s = cache[:, R // 2:].astype(np.float64)
    assert np.max(np.abs(c * c + s * s - 1.0)) < 4 * 2.0 ** -24
    p = np.arange(rows)
    np.testing.assert_allclose(c[:, 0], [math.cos(v) for v in p], atol=2 ** -24)
    np.testing.assert_allclose(s[:, 0], [math.sin(v) for v in p], atol=2 ** -24)
    # last frequency: theta_{R/2-1} = base^(-(R-2)/R)
    th = base ** (-(R - 2) / R)
    np.testing.assert_allclose(c[:, -1], np.cos(p * th), atol=2 ** -24)


def test_sample_tokens():
    s = W.sample_tokens(1000, 50, 3)
    assert s[0] == 0 and s[-1] == 999 and len(s) == 50 and np.all(np.diff(s) > 0)
    assert np.array_equal(W.sample_tokens(10, 50, 3), np.arange(10))


def test_algorithmic_bytes_of_configs():
    want = {"tiny": 37184, "dit": 115642880, "gqa": 171999744, "partial": 272761344,
            "large": 1644299264}
    for n, b in want.items():
        assert W.CONFIGS[n].algorithmic_bytes() == b, n


@pytest.mark.parametrize("name", ["gqa_tp8", "dit_hp8", "dit_sp8"])
def test_shard_workloads(name):
    """One GPU's share of the sharded runs: the heads or tokens of one shard, with
    positions of the full sequence."""
    c = W.CONFIGS[name]
    assert name in W.SHARD_ORDER and name not in W.CONFIG_ORDER
    wl = W.make_workload(c)
    assert wl.q.shape == (c.T, c.Hq, c.head_dim) and wl.k.shape == (c.T, c.Hkv, c.head_dim)
    assert wl.positions.min() >= 0 and wl.positions.max() < c.cache_rows
    full = W.CONFIGS["gqa" if name.startswith("gqa") else "dit"]
    assert (c.head_dim, c.rope_dim, c.is_neox, c.dtype, c.pos_dtype, c.base) == \
        (full.head_dim, full.rope_dim, full.is_neox, full.dtype, full.pos_dtype, full.base)
    if name == "gqa_tp8":
        assert (c.Hq, c.Hkv, c.layout) == (full.Hq // 8, full.Hkv // 8, "qkv")
        assert wl.qkv.shape == (c.T, (c.Hq + 2 * c.Hkv) * c.head_dim)
    elif name == "dit_hp8":
        assert (c.T, c.Hq, c.Hkv) == (full.T, full.Hq // 8, full.Hkv // 8)
    else:
        assert (c.T, c.Hq, c.Hkv, c.cache_rows) == (full.T // 8, full.Hq, full.Hkv, full.T)
        assert len(set(wl.positions.tolist())) == c.T  # distinct global positions
