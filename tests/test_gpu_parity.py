"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element
by element, plus untouched bytes, determinism and error paths.

Tolerance (every Q/K element): |gpu - ref| <= 2^-7 * (|ref| + 1), where ref is
the oracle's fp64 result rounded once to the I/O type; no NaN. In addition at
least 99% of elements must equal ref bit for bit: the kernel computes in fp32
and rounds to nearest even, so it may differ from the correctly rounded value
only where the fp64 result lies within the fp32 error of a rounding boundary.
"""
import sys

import numpy as np
import pytest

from head_qk_rmsnorm_amd import workloads as W
from tests import qknr_harness as Hn

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from head_qk_rmsnorm_amd import binding as B

    B.lib()  # fail loudly if the library is missing
    yield


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

def test_config_tiny_full():
    wl = W.make_workload(W.CONFIGS["tiny"])
    _say("case tiny")
    cq, ck = Hn.run_and_check(wl)
    _say("tiny", cq, ck)


@pytest.mark.parametrize("name", ["dit", "gqa", "partial", "large"])
def test_config_full_size(name):
    """Full-size launch in the benchmark's (automatic) launch configuration:
    every Q/K element against the oracle (run in token chunks on the host's
    cores) and every byte outside Q/K against its value before the call."""
    cfg = W.CONFIGS[name]
    _say(f"case {name}: T={cfg.T} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.head_dim} R={cfg.rope_dim}")
    wl = W.make_workload(cfg)
    cq, ck = Hn.run_and_check(wl)
    _say(name, cq, ck)


@pytest.mark.parametrize("name", ["gqa_tp8", "dit_hp8", "dit_sp8"])
def test_shard_workloads_full(name):
    """One GPU's share of the sharded runs, every output element, in the launch
    configuration the benchmark times."""
    cfg = W.CONFIGS[name]
    _say("case", name)
    Hn.run_and_check(W.make_workload(cfg))


# ---------------------------------------------------------------------------
# Grid: head_dim x rope_dim x pairing x dtype x positions x T, with GQA
# ---------------------------------------------------------------------------

GRID = [(D, R, neox, dt, pdt, T)
        for D in (64, 128, 256)
        for R in (D, D // 2)
        for neox in (False, True)
        for dt, pdt in ((W.BF16, W.I32), (W.FP16, W.I64), (W.BF16, W.I64), (W.FP16, W.I32))
        for T in (1, 9, 129, 1000)]


@pytest.mark.parametrize("D,R,neox,dt,pdt,T", GRID)
def test_grid(D, R, neox, dt, pdt, T):
    # Hq=5, Hkv=3: Q/K straddle inside a wave instruction for every lane mapping
    cfg = W.case(T, 5, 3, D, R, neox, dtype=dt, pos_dtype=pdt, seed=T + D + R,
                 positions="uniform")
    _say("case", cfg.name)
    Hn.run_and_check(W.make_workload(cfg))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("neox", [False, True])
def test_every_supported_rope_dim(D, neox):
    """Every rope_dim the capability predicate accepts for the compile-time
    head_dims: all even widths (interleaved), every NeoX width whose half is a
    multiple of a lane width (including rotary-lane counts that are not powers
    of two and the widths that need half or full waves per head)."""
    from head_qk_rmsnorm_amd import binding as B

    Rs = [R for R in range(2, D + 1, 2) if B.qknr_can_use(D, R, neox)]
    assert Rs
    for R in Rs:
        cfg = W.case(7, 3, 2, D, R, neox, seed=R, positions="uniform")
        _say("case", cfg.name)
        Hn.run_and_check(W.make_workload(cfg))


ANY_DIMS = [16, 24, 40, 48, 72, 80, 96, 112, 160, 192, 200, 320, 384, 504, 512]


@pytest.mark.parametrize("D", ANY_DIMS)
@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("dt", [W.BF16, W.FP16])
def test_run_time_head_dims(D, neox, dt):
    """head_dims other than 64/128/256 (run-time instances, lane groups padded
    to a power of two): full rotation and a partial one, Q/K straddling groups."""
    from head_qk_rmsnorm_amd import binding as B

    for R in (D - (D % 16) if neox else D, 16 if neox else 6):
        assert B.qknr_can_use(D, R, neox), (D, R, neox)
        cfg = W.case(33, 5, 3, D, R, neox, dtype=dt, pos_dtype=W.I64, seed=D + R)
        _say("case", cfg.name)
        Hn.run_and_check(W.make_workload(cfg))


@pytest.mark.parametrize("layout", ["padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R,neox", [(96, 96, True), (80, 64, False), (192, 128, True)])
def test_run_time_head_dim_layouts(layout, D, R, neox):
    cfg = W.case(40, 6, 2, D, R, neox, seed=7)
    Hn.run_and_check(W.make_workload(cfg), layout=layout)


RT_LAUNCHES = [
    dict(unroll=2), dict(unroll=4), dict(unroll=1, groups_per_item=3),
    dict(unroll=4, groups_per_item=1), dict(unroll=4, groups_per_item=3),
    dict(unroll=4, groups_per_item=5, block_waves=1), dict(unroll=4, max_blocks=-1),
    dict(unroll=2, groups_per_item=4, block_waves=2), dict(unroll=4, groups_per_item=9, max_blocks=5),
]


@pytest.mark.parametrize("launch", RT_LAUNCHES, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
@pytest.mark.parametrize("D,R,neox", [(80, 80, False), (96, 40, True), (72, 72, True), (104, 52, True),
                                      (40, 40, False), (160, 64, True), (320, 320, False)])
def test_run_time_launch_variants(launch, D, R, neox):
    """Run-time head_dims at unroll 2 and 4 (1 runs as 2), with work items that
    end inside an unrolled batch of head groups and Q/K straddling items."""
    cfg = W.case(29, 7, 3, D, R, neox, dtype=W.FP16, pos_dtype=W.I32, seed=D + 3 * R)
    _say("case", cfg.name, launch)
    Hn.run_and_check(W.make_workload(cfg), launch=launch)
    dc = Hn.DeviceCase(W.make_workload(cfg))
    info = dc.run(launch=launch)
    assert info["unroll"] == (4 if launch.get("unroll") == 4 else 2), info


# NeoX halves of 8m + 2, 8m + 4 and 8m + 6 dims on 16-byte lanes: partners 2, 4
# or 6 slots over in a neighbouring lane (compile-time head_dims with a partial
# rotation, run-time head_dims with a full or partial one, halves of 2, 4 and 6
# that pair inside a lane)
SHIFTED = [(96, 24), (72, 72), (40, 40), (88, 88), (136, 136), (264, 264), (200, 200), (120, 8),
           (16, 8), (64, 24), (128, 40), (128, 8), (256, 104), (256, 24),
           (80, 20), (96, 12), (40, 12), (56, 20), (104, 52), (120, 60), (200, 100), (504, 12),
           (16, 4), (24, 12), (128, 20), (64, 12), (256, 44), (128, 4), (64, 60),
           (72, 20), (152, 44), (88, 28), (96, 20), (168, 44),
           (24, 24), (40, 24), (24, 8), (56, 56)]
SHIFTED_LAUNCHES = [None, dict(unroll=4, groups_per_item=3), dict(unroll=2, groups_per_item=1, block_waves=1)]


@pytest.mark.parametrize("launch", SHIFTED_LAUNCHES,
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()) if d else "auto")
@pytest.mark.parametrize("dt", [W.BF16, W.FP16])
@pytest.mark.parametrize("D,R", SHIFTED)
def test_neox_shifted_partners(D, R, dt, launch):
    cfg = W.case(29, 7, 3, D, R, True, dtype=dt, pos_dtype=W.I64, seed=3 * D + R)
    _say("case", cfg.name, launch)
    wl = W.make_workload(cfg)
    info = Hn.DeviceCase(wl).run(launch=launch or {})
    # head_dim 96 with a NeoX half that is a multiple of 6 takes 12-byte lanes
    twelve = D == 96 and (R // 2) % 6 == 0 and (R // 2) % 8 != 0
    assert info["generic"] == 0 and info["elems_per_lane"] == (6 if twelve else 8), info
    Hn.run_and_check(wl, launch=launch)


@pytest.mark.parametrize("layout", ["padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R", [(96, 24), (128, 40), (72, 72), (80, 20), (128, 12)])
def test_neox_shifted_partners_layouts(layout, D, R):
    cfg = W.case(23, 5, 2, D, R, True, seed=D + 7 * R)
    Hn.run_and_check(W.make_workload(cfg), layout=layout)


# ---------------------------------------------------------------------------
# Launch configurations (all must give the same, correct result)
# ---------------------------------------------------------------------------

LAUNCHES = [
    dict(),
    dict(unroll=1), dict(unroll=2),
    dict(groups_per_item=1), dict(groups_per_item=3, unroll=2), dict(groups_per_item=12, unroll=4),
    dict(block_waves=1), dict(block_waves=8),
    dict(max_blocks=1), dict(max_blocks=7, groups_per_item=2),
    dict(max_blocks=-1, groups_per_item=1), dict(max_blocks=-1),
    dict(lanes_per_head=32), dict(lanes_per_head=32, unroll=4, groups_per_item=5),
    dict(lanes_per_head=64), dict(lanes_per_head=64, unroll=2, groups_per_item=3, max_blocks=3),
]


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()) or "auto")
@pytest.mark.parametrize("D,R,neox", [(64, 64, True), (128, 128, False), (128, 64, True),
                                      (256, 256, True), (256, 128, False)])
def test_launch_variants(launch, D, R, neox):
    # for head_dim 256, 32 lanes per head is the 16-byte mapping itself
    if launch.get("lanes_per_head") == 64 and D == 64:
        pytest.skip("a full wave per head needs head_dim >= 128 (two elements per lane)")
    cfg = W.case(33, 7, 3, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + R)
    _say("case", cfg.name, launch)
    Hn.run_and_check(W.make_workload(cfg), launch=launch)


# head_dim 96 of the fused op with a NeoX half that is a multiple of 6 but not
# of 8: 12-byte lanes (16 lanes of 6 elements)
@pytest.mark.parametrize("launch", [l for l in LAUNCHES if "lanes_per_head" not in l],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()) or "auto")
@pytest.mark.parametrize("D,R,neox,dt", [(96, 24, True, W.FP16), (96, 12, True, W.BF16),
                                         (96, 72, True, W.BF16), (96, 60, True, W.FP16),
                                         (96, 84, True, W.BF16)])
def test_head_dim_96_twelve_byte_lanes(launch, D, R, neox, dt):
    cfg = W.case(33, 7, 3, D, R, neox, dtype=dt, pos_dtype=W.I64, seed=D + 5 * R)
    _say("case", cfg.name, launch)
    wl = W.make_workload(cfg)
    info = Hn.DeviceCase(wl).run(launch=launch)
    assert (info["generic"], info["elems_per_lane"], info["access_bytes"]) == (0, 6, 12), info
    Hn.run_and_check(wl, launch=launch)


@pytest.mark.parametrize("layout", ["padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R,neox", [(96, 72, True), (96, 36, True)])
def test_head_dim_96_layouts(layout, D, R, neox):
    cfg = W.case(21, 5, 3, D, R, neox, seed=D + R + 1)
    Hn.run_and_check(W.make_workload(cfg), layout=layout)


# ---------------------------------------------------------------------------
# Layouts and degenerate shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["contiguous", "padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R,neox", [(64, 32, True), (128, 128, True), (256, 256, False)])
def test_layouts(layout, D, R, neox):
    cfg = W.case(65, 6, 2, D, R, neox, dtype=W.FP16, seed=3)
    _say("case", cfg.name, layout)
    Hn.run_and_check(W.make_workload(cfg), layout=layout)


@pytest.mark.parametrize("Hq,Hkv", [(0, 4), (4, 0), (1, 1), (1, 0), (31, 1), (3, 13)])
def test_head_counts(Hq, Hkv):
    cfg = W.case(17, Hq, Hkv, 128, 128, True, seed=Hq * 10 + Hkv)
    _say("case", cfg.name)
    Hn.run_and_check(W.make_workload(cfg))


def test_zero_tokens_is_noop():
    import torch

    cfg = W.case(0, 4, 4, 128, 128, True)
    wl = W.make_workload(cfg)
    dc = Hn.DeviceCase(wl)
    dc.run()
    after = dc.fetch()
    for b, a in zip(dc.storages_host, after):
        assert np.array_equal(b, a)
    torch.cuda.synchronize()


def test_special_values():
    """eps = 0; an all-zero head (eps > 0 gives exactly 0); heads scaled by 2^20
    and 2^-20 (the norm removes the scale); position 0 (norm only)."""
    import torch
    from oracle import qknr_oracle as O

    D = R = 128
    T, Hq, Hkv = 4, 3, 1
    g = np.random.default_rng(5)
    x = g.standard_normal((T, Hq, D))
    x[1, 0] = 0.0
    x[2, 1] *= 2.0 ** 20
    x[3, 2] *= 2.0 ** -20
    for eps in (0.0, 1e-6):
        if eps == 0.0:
            x[1, 0] = 1.0  # 0/0 is NaN for eps = 0, as the formula says; keep it out
        cfg = W.case(T, Hq, Hkv, D, R, True, eps=eps, seed=1)
        wl = W.make_workload(cfg)
        wl.q[...] = O.round_to_bf16_bits(x)
        wl.positions[0] = 0
        _say("case special eps", eps)
        Hn.run_and_check(wl)
    torch.cuda.synchronize()


@pytest.mark.parametrize("generic", [0, 1])
@pytest.mark.parametrize("neox", [True, False])
def test_pass_through_signed_zeros_and_non_finite(neox, generic):
    """Dims past rope_dim keep the normalised value bit for bit on both kernels:
    signed zeros (an all-zero head with negative weights there, negative-zero
    inputs) match the oracle exactly, and an infinite input there turns only
    its own element into NaN (the sum of squares is infinite, so the scale is
    0: every other element of that head is a signed zero) without reaching
    its rotation partner slot or its neighbours."""
    import torch

    from oracle import qknr_oracle as O

    D, R = 128, 64
    T, Hq, Hkv = 3, 3, 2
    cfg = W.case(T, Hq, Hkv, D, R, neox, seed=11)
    wl = W.make_workload(cfg)
    wl.q[0, 0] = 0                                   # all-zero head
    wl.wq[R:] |= np.uint16(0x8000)                   # negative weights past rope_dim
    wl.q[2, 2, R::3] = np.uint16(0x8000)             # negative zeros past rope_dim
    launch = {"generic": 1} if generic else None
    _say("case pass-through zeros", neox, generic)
    Hn.run_and_check(wl, launch=launch)
    dc = Hn.DeviceCase(wl)
    dc.run(launch=launch)
    gq, gk = dc.outputs(dc.fetch())
    refq, refk = Hn.oracle_ref(wl)
    assert np.array_equal(gq[0, 0], refq[0, 0])      # signed zeros bit for bit
    assert np.all(gq[0, 0, R:] == 0x8000)            # +0 times a negative weight
    assert np.array_equal(gq[2, 2, R::3], refq[2, 2, R::3])

    # an infinite input past rope_dim (K head 1 of token 1)
    inf_dim = R + 5
    ref_q, ref_k = Hn.oracle_ref(wl)                 # every other head is independent of it
    wl.k[1, 1, inf_dim] = np.uint16(0x7F80)
    _say("case pass-through inf", neox, generic)
    dc = Hn.DeviceCase(wl)
    dc.run(launch=launch)
    after = dc.fetch()
    dc.check_untouched(after)
    gq, gk = dc.outputs(after)
    torch.cuda.synchronize()
    head = O.decode_io(gk[1, 1], cfg.dtype)
    assert np.isnan(head[inf_dim])
    rest = np.delete(head, inf_dim)
    assert np.all(rest == 0.0), rest[rest != 0.0]
    mask = np.ones(gk.shape, dtype=bool)
    mask[1, 1] = False
    for name, g, r in (("q", gq, ref_q), ("k", gk[mask], ref_k[mask])):
        cmp = Hn.compare_bits(g, r, cfg.dtype)
        assert cmp.bad == 0 and cmp.exact_frac >= 0.99, f"{name}: {cmp}"


def test_outlier_magnitudes_fp16():
    cfg = W.case(64, 4, 4, 256, 256, False, dtype=W.FP16, outlier_frac=0.05,
                 outlier_scale=50.0, seed=8)
    Hn.run_and_check(W.make_workload(cfg))


def test_deterministic():
    cfg = W.case(300, 8, 8, 128, 64, True, seed=2)
    wl = W.make_workload(cfg)
    outs = []
    for _ in range(2):
        dc = Hn.DeviceCase(wl)
        dc.run()
        outs.append(dc.fetch())
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_side_stream():
    import torch

    cfg = W.case(129, 6, 2, 128, 128, False, seed=4)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Hn.run_and_check(W.make_workload(cfg), stream=s)


# ---------------------------------------------------------------------------
# Error paths: rejected before any launch, q and k untouched
# ---------------------------------------------------------------------------

def test_rejections_leave_buffers_untouched():
    import torch
    from head_qk_rmsnorm_amd import binding as B

    cfg = W.case(9, 4, 4, 128, 128, True, seed=6)
    wl = W.make_workload(cfg)
    dc = Hn.DeviceCase(wl)
    rows = int(wl.positions.max()) + 1  # any dummy table covers every position
    bad = [
        dict(eps=-1.0),
        dict(eps=float("nan")),
        dict(rope_dim=99),  # odd: no pairs
    ]
    for kw in bad:
        args = dict(is_neox=True, eps=1e-6)
        args.update(kw)
        rope = args.pop("rope_dim", 0)
        with pytest.raises((RuntimeError, ValueError)):
            B.qknr_inplace(dc.q, dc.k, dc.wq, dc.wk,
                           dc.cache if not rope else torch.zeros(rows, rope, device=dc.device),
                           dc.positions, rope_dim=rope, **args)
    # q at an odd byte address (not even element aligned), through the C ABI
    import ctypes

    c = wl.cfg
    P = ctypes.c_void_p
    rc = B.lib().qknr_inplace(P(dc.q.data_ptr() + 1), P(dc.k.data_ptr()), P(dc.wq.data_ptr()),
                              P(dc.wk.data_ptr()), P(dc.cache.data_ptr()),
                              P(dc.positions.data_ptr()), c.T, c.Hq, c.Hkv, c.head_dim,
                              c.rope_dim, 1, 1e-6, dc.q.stride(0) * 2, dc.q.stride(1) * 2,
                              dc.k.stride(0) * 2, dc.k.stride(1) * 2, 0, 0, P(0))
    assert rc == B.QKNR_E_ALIGN
    torch.cuda.synchronize()
    after = dc.fetch()
    for b, a in zip(dc.storages_host, after):
        assert np.array_equal(b, a)


# ---------------------------------------------------------------------------
# Measurement aids
# ---------------------------------------------------------------------------

def test_copy_and_rmw_kernels():
    import torch
    from head_qk_rmsnorm_amd import binding as B

    n = (1 << 20) + 48
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    B.qknr_copy(dst, src, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    B.qknr_rmw(dst, n, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    B.qknr_rmw(dst, n, 0xFFFFFFFF)
    torch.cuda.synchronize()
    assert torch.equal(dst, ~src)


# ---------------------------------------------------------------------------
# The unfused baseline: norm step, rope step, and the two-launch chain
# ---------------------------------------------------------------------------

UNFUSED_GRID = [(D, R, neox, dt, pdt, T)
                for D in (64, 128, 256) for R in (D, D // 2) for neox in (False, True)
                for dt, pdt in ((W.BF16, W.I64), (W.FP16, W.I32)) for T in (1, 129)]


@pytest.mark.parametrize("which", ["norm", "rope", "unfused"])
@pytest.mark.parametrize("D,R,neox,dt,pdt,T", UNFUSED_GRID)
def test_unfused_steps_grid(which, D, R, neox, dt, pdt, T):
    cfg = W.case(T, 5, 3, D, R, neox, dtype=dt, pos_dtype=pdt, seed=T + D + R + 1)
    _say("case", which, cfg.name)
    Hn.unfused_check(W.make_workload(cfg), which)


@pytest.mark.parametrize("which", ["norm", "rope", "unfused"])
@pytest.mark.parametrize("layout", ["padded", "qkv"])
def test_unfused_steps_layouts(which, layout):
    cfg = W.case(33, 6, 2, 128, 64, True, dtype=W.FP16, seed=11)
    Hn.unfused_check(W.make_workload(cfg), which, layout=layout)


@pytest.mark.parametrize("name", ["tiny", "dit", "gqa"])
def test_unfused_chain_on_workloads(name):
    """The two-launch chain on the workloads (full outputs for Tiny; DiT and GQA
    checked in full as well: the oracle handles them in seconds)."""
    _say("case unfused", name)
    Hn.unfused_check(W.make_workload(W.CONFIGS[name]), "unfused")


def test_fused_and_unfused_agree_within_page_tolerance():
    """The page's unit test tolerance between the fused op and the unfused
    chain: bf16 atol 8e-2, rtol 1e-2 (Step 4 of its rewrite guide)."""
    import torch
    from head_qk_rmsnorm_amd import binding as B

    cfg = W.case(257, 8, 4, 128, 128, False, seed=21)
    wl = W.make_workload(cfg)
    a = Hn.DeviceCase(wl)
    b = Hn.DeviceCase(wl)
    B.qknr_inplace(a.q, a.k, a.wq, a.wk, a.cache, a.positions, is_neox=False, eps=cfg.eps)
    B.qknr_unfused_inplace(b.q, b.k, b.wq, b.wk, b.cache, b.positions, is_neox=False, eps=cfg.eps)
    torch.cuda.synchronize()
    for x, y in ((a.q, b.q), (a.k, b.k)):
        xf, yf = x.float(), y.float()
        assert torch.all((xf - yf).abs() <= 8e-2 + 1e-2 * xf.abs())
        assert not torch.equal(xf, yf)


# ---------------------------------------------------------------------------
# Sibling: per-head QK LayerNorm (+ optional rotation)
# ---------------------------------------------------------------------------

LN_GRID = [(D, R, neox, dt, bias)
           for D in (64, 128, 256, 96, 192, 80, 160)
           for R, neox in ((0, False), (D, False), (D, True), (D // 2, True), (D // 2, False))
           for dt in (W.BF16, W.FP16) for bias in (False, True)]


@pytest.mark.parametrize("D,R,neox,dt,bias", LN_GRID)
def test_layernorm_sibling(D, R, neox, dt, bias):
    cfg = W.case(65, 5, 3, D, D if R == 0 else R, neox, dtype=dt, pos_dtype=W.I64, seed=D + R,
                 x_std=2.0)
    wl = W.make_workload(cfg)
    # a non-zero mean per head exercises the centring
    from oracle import qknr_oracle as O
    wl.q[...] = O.round_to_io_bits(O.decode_io(wl.q, dt) + 1.5, dt)
    _say("case layernorm", cfg.name, R, bias)
    Hn.layernorm_check(wl, R, bias)


# the LayerNorm sibling pairs the same NeoX halves on 16-byte lanes with
# shifted partners (compile-time and run-time head_dims)
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("dt", [W.BF16, W.FP16])
@pytest.mark.parametrize("D,R", SHIFTED)
def test_layernorm_sibling_shifted_partners(D, R, dt, bias):
    from oracle import qknr_oracle as O

    cfg = W.case(29, 7, 3, D, R, True, dtype=dt, pos_dtype=W.I64, seed=5 * D + R, x_std=2.0)
    wl = W.make_workload(cfg)
    wl.q[...] = O.round_to_io_bits(O.decode_io(wl.q, dt) + 1.5, dt)
    _say("case layernorm shifted", cfg.name, bias)
    Hn.layernorm_check(wl, R, bias)


@pytest.mark.parametrize("layout", ["padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R", [(96, 24), (128, 40), (80, 20), (128, 12)])
def test_layernorm_sibling_shifted_partners_layouts(layout, D, R):
    cfg = W.case(23, 5, 2, D, R, True, seed=D + 11 * R)
    Hn.layernorm_check(W.make_workload(cfg), R, True, layout=layout)


@pytest.mark.parametrize("layout", ["padded", "qkv"])
def test_layernorm_sibling_layouts(layout):
    cfg = W.case(33, 6, 2, 128, 64, True, seed=5)
    Hn.layernorm_check(W.make_workload(cfg), 64, True, layout=layout)


def test_layernorm_sibling_on_dit_workload():
    """The DiT workload with LayerNorm instead of RMSNorm (all tokens)."""
    Hn.layernorm_check(W.make_workload(W.CONFIGS["dit"]), 128, True)


@pytest.mark.parametrize("D,R,neox,launch,want", [
    (128, 128, False, {}, dict(generic=0, lanes_per_head=16, elems_per_lane=8, heads_per_wave=4)),
    (128, 64, True, {"block_waves": 2, "groups_per_item": 3},
     dict(generic=0, block_threads=128, groups_per_item=3)),
    (80, 20, True, {}, dict(generic=0, elems_per_lane=8)),
    (100, 100, True, {}, dict(generic=1, access_bytes=8)),
    (128, 0, False, {"generic": 1}, dict(generic=1, access_bytes=16)),
])
def test_layernorm_launch_report(D, R, neox, launch, want):
    """qknr_layernorm_rope_inplace_ex reports what it launched (and honours a
    launch configuration) while the result still matches the oracle."""
    cfg = W.case(37, 6, 3, D, R or D, neox, pos_dtype=W.I64, seed=D + R + 3, x_std=2.0)
    _say("case layernorm report", cfg.name, launch)
    info = Hn.layernorm_check(W.make_workload(cfg), R, True, launch=launch)
    for k, v in want.items():
        assert info[k] == v, info
    assert info["grid_blocks"] > 0 and info["items"] > 0, info


@pytest.mark.parametrize("off", [1, 2], ids=["cache_4B", "cache_8B"])
@pytest.mark.parametrize("D,R,neox", [(128, 128, True), (128, 64, True), (64, 64, True),
                                      (128, 128, False), (128, 64, False), (256, 256, True),
                                      (96, 24, True), (80, 20, True), (40, 40, True), (136, 136, True),
                                      (72, 72, True), (128, 20, True), (100, 100, True),
                                      (130, 130, False), (40, 38, True)])
def test_cache_alignment(D, R, neox, off):
    """A cos|sin table aligned to 4 or 8 bytes only (a view one or two floats
    into its allocation, NaN in front of it) takes every cos/sin read path that
    an aligned table skips: per-lane scalar loads, the LDS staging copy in
    single floats or in pairs, the element kernel's scalar row copy."""
    cfg = W.case(37, 5, 3, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + R + off)
    _say("case cache offset", off, cfg.name)
    Hn.run_and_check(W.make_workload(cfg), cache_offset=off)


@pytest.mark.parametrize("off", [1, 2], ids=["cache_4B", "cache_8B"])
@pytest.mark.parametrize("D,R", [(128, 128), (64, 32), (80, 20), (96, 24), (40, 40)])
def test_cache_alignment_layernorm(D, R, off):
    """The LayerNorm sibling (NeoX, weight and bias) on a cos|sin table aligned
    to 4 or 8 bytes only."""
    cfg = W.case(29, 4, 2, D, R, True, dtype=W.FP16, pos_dtype=W.I32, seed=3 * D + R + off)
    _say("case layernorm cache offset", off, cfg.name)
    Hn.layernorm_check(W.make_workload(cfg), R, True, cache_offset=off)


@pytest.mark.parametrize("w_off", [1, 2, 4], ids=["w_2B", "w_4B", "w_8B"])
@pytest.mark.parametrize("D,R,neox", [(128, 128, True), (128, 64, False), (64, 64, True),
                                      (96, 24, True), (80, 20, True), (256, 256, False)])
def test_weight_alignment(D, R, neox, w_off):
    """Weight rows aligned to 2, 4 or 8 bytes only: the vectorised kernel needs
    16, so every such call runs element-granular with accesses as wide as the
    weights allow, and matches the oracle."""
    cfg = W.case(33, 6, 2, D, R, neox, dtype=W.FP16, pos_dtype=W.I64, seed=7 * D + R + w_off)
    wl = W.make_workload(cfg)
    _say("case weight offset", w_off, cfg.name)
    dc = Hn.DeviceCase(wl, w_offset=w_off)
    info = dc.run(launch={})
    assert info["generic"] == 1 and info["access_bytes"] <= 2 * w_off, info
    Hn.run_and_check(wl, w_offset=w_off)


@pytest.mark.parametrize("dt", [W.BF16, W.FP16])
@pytest.mark.parametrize("T,Hq,Hkv,D,R,neox", [(1400, 24, 24, 128, 128, False),
                                               (1400, 24, 24, 128, 128, True),
                                               (1700, 32, 8, 128, 128, True),
                                               (2100, 16, 16, 128, 64, True),
                                               (700, 24, 24, 256, 256, False),
                                               (2800, 24, 24, 64, 64, True),
                                               (2800, 24, 24, 96, 96, True),
                                               (2800, 24, 24, 80, 80, False),
                                               (1400, 24, 24, 160, 160, True),
                                               (2800, 24, 24, 112, 32, True)])
def test_tail_items(T, Hq, Hkv, D, R, neox, dt):
    """Launches long enough to end on items of half as many head groups (the
    last ceil(2048 / such items per token) tokens): the launch report counts
    them, and every Q/K element matches the oracle."""
    cfg = W.case(T, Hq, Hkv, D, R, neox, dtype=dt, pos_dtype=W.I64, seed=T + D + R)
    wl = W.make_workload(cfg)
    _say("case tail items", cfg.name)
    info = Hn.DeviceCase(wl).run(launch={})
    ng, gpi = info["groups_per_token"], info["groups_per_item"]
    tnc = -(-ng // (gpi // 2))
    tail = -(-2048 // tnc)
    assert T >= 8 * tail and info["items"] == (T - tail) * -(-ng // gpi) + tail * tnc, info
    Hn.run_and_check(wl)
