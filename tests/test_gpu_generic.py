"""GPU parity of the element-granular kernel (the cases the vectorised kernel
does not take): head_dims that are not multiples of 8, NeoX halves that no lane
width divides, element-aligned pointers and odd strides, and the same shapes in
every mode (fused, unfused steps, LayerNorm sibling). Each case is checked
against the fp64 oracle element by element, with the bytes around Q/K
untouched, and the launch report confirms which kernel ran."""
import numpy as np
import pytest

from head_qk_rmsnorm_amd import workloads as W
from tests import qknr_harness as Hn
from tests.test_abi import elem_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from head_qk_rmsnorm_amd import binding as B

    B.lib()
    yield


def _view_align(dc):
    """Common alignment (2 to 16 bytes) of q, k, the weights and the strides
    that are used (token stride with T > 1, head stride with H > 1)."""
    vals = []
    for t in (dc.q, dc.k):
        es = t.element_size()
        vals.append(t.data_ptr())
        if t.size(0) > 1:
            vals.append(t.stride(0) * es)
        if t.size(1) > 1:
            vals.append(t.stride(1) * es)
    vals += [dc.wq.data_ptr(), dc.wk.data_ptr()]
    return next(b for b in (16, 8, 4, 2) if all(v % b == 0 for v in vals))


def _check_plan(info, dc):
    """The launch report of an element-granular call follows the lane-mapping rule."""
    c = dc.cfg
    pw, S, L, G, _ = elem_plan(c.head_dim, _view_align(dc), c.Hq, c.Hkv)
    assert (info["access_bytes"], info["elems_per_lane"], info["lanes_per_head"],
            info["heads_per_wave"]) == (2 * pw, S * pw, L, G), info


def _check(wl, layout=None, launch=None, min_exact=0.99):
    """One fused call through qknr_inplace_ex; returns the launch report."""
    dc = Hn.DeviceCase(wl, layout=layout)
    info = dc.run(launch=launch or {})
    after = dc.fetch()
    dc.check_untouched(after)
    dc.check_inputs_unchanged()
    gq, gk = dc.outputs(after)
    rq, rk = Hn.oracle_ref(wl)
    for name, g, r in (("q", gq, rq), ("k", gk, rk)):
        cmp = Hn.compare_bits(g, r, wl.cfg.dtype)
        assert cmp.bad == 0, f"{wl.cfg.name} {layout} {name}: {cmp}"
        assert cmp.exact_frac >= min_exact, f"{wl.cfg.name} {layout} {name}: {cmp}"
    return info, after, dc


def _rope_dims(D):
    out = {2, D - D % 2}
    mid = (D // 3) & ~1
    if mid >= 2:
        out.add(mid)
    return sorted(r for r in out if 2 <= r <= D)


ELEM_DIMS = [2, 3, 5, 8, 17, 24, 58, 64, 72, 100, 130, 200, 255, 256, 300, 510, 512]
ELEM_GRID = [(D, R, neox) for D in ELEM_DIMS for R in _rope_dims(D) for neox in (False, True)]


def _vectorised(D, R, neox):
    """Shapes of the vectorised kernel for the fused op (include/qknr.h),
    restated: head_dim a multiple of 8 in [16, 512]; NeoX needs rope_dim/2 to be
    even (16-byte lanes; partners 2, 4 or 6 slots over when it is not a
    multiple of 8)."""
    if D % 8 or D < 16 or D > 512:
        return False
    return not neox or (R // 2) % 2 == 0


@pytest.mark.parametrize("D,R,neox", ELEM_GRID)
def test_shapes(D, R, neox):
    i = ELEM_GRID.index((D, R, neox))
    dt = W.BF16 if i % 2 == 0 else W.FP16
    pdt = W.I64 if i % 3 == 0 else W.I32
    cfg = W.case(37, 5, 3, D, R, neox, dtype=dt, pos_dtype=pdt, seed=500 + i)
    print("case", cfg.name, flush=True)
    info, _, dc = _check(W.make_workload(cfg))
    assert info["generic"] == (0 if _vectorised(D, R, neox) else 1), info
    if info["generic"]:
        _check_plan(info, dc)


@pytest.mark.parametrize("layout", ["shifted", "shifted4", "odd_pad", "padded", "head_major", "qkv"])
@pytest.mark.parametrize("D,R,neox", [(128, 128, False), (128, 64, True), (100, 100, True),
                                      (72, 72, True), (64, 2, True), (3, 2, False)])
def test_layouts(layout, D, R, neox):
    cfg = W.case(29, 6, 2, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + R + 7)
    print("case", cfg.name, layout, flush=True)
    info, _, dc = _check(W.make_workload(cfg), layout=layout)
    want = 0 if (_vectorised(D, R, neox) and layout not in ("shifted", "shifted4", "odd_pad")) else 1
    assert info["generic"] == want, (layout, info)
    if want:  # 2*pw-byte accesses need head_dim % pw == 0 and 2*pw-byte aligned views
        _check_plan(info, dc)


@pytest.mark.parametrize("D,R,neox", [(64, 64, True), (64, 32, False), (128, 128, False),
                                      (128, 64, True), (256, 256, True), (256, 96, False),
                                      (96, 96, True), (200, 120, False)])
@pytest.mark.parametrize("dt", [W.BF16, W.FP16])
def test_forced_matches_vectorised(D, R, neox, dt):
    """On shapes both kernels take, the element-granular kernel (asked for
    explicitly) meets the same bar, and the two agree bit for bit wherever the
    different order of the fp32 sums does not decide a rounding."""
    cfg = W.case(65, 7, 5, D, R, neox, dtype=dt, pos_dtype=W.I32, seed=D * 3 + R)
    wl = W.make_workload(cfg)
    vi, va, vdc = _check(wl)
    gi, ga, gdc = _check(wl, launch={"generic": 1})
    assert vi["generic"] == 0 and gi["generic"] == 1
    vq, vk = vdc.outputs(va)
    gq, gk = gdc.outputs(ga)
    same = np.mean(np.concatenate([(vq == gq).ravel(), (vk == gk).ravel()]))
    assert same >= 0.99, same


LAUNCHES = [dict(generic=1, groups_per_item=1), dict(generic=1, groups_per_item=3),
            dict(generic=1, groups_per_item=64), dict(generic=1, block_waves=1),
            dict(generic=1, block_waves=8), dict(generic=1, max_blocks=-1),
            dict(generic=1, max_blocks=1), dict(generic=1, max_blocks=7, block_waves=2),
            dict(generic=1, unroll=4)]


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
@pytest.mark.parametrize("D,R,neox", [(100, 100, True), (128, 64, False), (3, 2, True)])
def test_launch_variants(launch, D, R, neox):
    cfg = W.case(45, 9, 3, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + 91)
    info, _, _ = _check(W.make_workload(cfg), launch=launch)
    assert info["generic"] == 1
    if launch.get("groups_per_item"):
        assert info["groups_per_item"] == min(launch["groups_per_item"], info["groups_per_token"])


@pytest.mark.parametrize("D,R,neox,persistent", [(40, 38, True, True), (100, 100, True, None),
                                                  (130, 130, False, None)])
def test_grid_rule(D, R, neox, persistent):
    """The automatic grid of the element-granular kernel: one work item per wave,
    or (instances that keep few waves resident) a persistent grid of whole
    rounds of workgroups over the CUs; an explicit max_blocks overrides it.
    Every launch shape computes the same result."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cfg = W.case(6000, 24, 24, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + R + 5)
    wl = W.make_workload(cfg)
    info, _, _ = _check(wl)
    assert info["generic"] == 1
    needed = -(-info["items"] // (info["block_threads"] // 64))
    grid = info["grid_blocks"]
    assert grid == needed or (grid < needed and grid % cus == 0), (info, cus)
    if persistent is not None:
        assert (grid < needed) == persistent, (info, cus)
    one, _, _ = _check(wl, launch={"max_blocks": 1 << 30})
    assert one["grid_blocks"] == needed, one
    full, _, _ = _check(wl, launch={"max_blocks": -1})
    assert full["grid_blocks"] % cus == 0 and full["grid_blocks"] <= needed, full


@pytest.mark.parametrize("Hq,Hkv", [(0, 4), (4, 0), (1, 1), (1, 0), (31, 1), (3, 13)])
def test_head_counts(Hq, Hkv):
    cfg = W.case(23, Hq, Hkv, 100, 98, True, dtype=W.FP16, pos_dtype=W.I32, seed=Hq * 17 + Hkv)
    info, _, _ = _check(W.make_workload(cfg))
    assert info["generic"] == 1


def test_special_values():
    """Zero vectors (the output is exactly 0), a head of one repeated value, a
    head of large magnitudes (sum of squares ~3e36, still finite in fp32) and a
    tiny one (sum of squares underflows; eps dominates), on the element-granular
    kernel."""
    cfg = W.case(12, 4, 4, 100, 100, True, dtype=W.BF16, pos_dtype=W.I32, seed=77)
    wl = W.make_workload(cfg)
    q = wl.q.copy()
    q[0, 0, :] = 0
    q[1, 1, :] = W.to_io_bits(np.full(100, 3.0), W.BF16)
    q[2, 2, :] = W.to_io_bits(np.linspace(-3e17, 3e17, 100), W.BF16)
    q[3, 3, :] = W.to_io_bits(np.full(100, 1e-30), W.BF16)
    wl.q[...] = q
    info, after, dc = _check(wl)
    assert info["generic"] == 1
    gq, _ = dc.outputs(after)
    assert np.all(gq[0, 0] & 0x7FFF == 0)


def test_deterministic_and_side_stream():
    import torch

    cfg = W.case(70, 6, 2, 130, 66, True, dtype=W.BF16, pos_dtype=W.I64, seed=5)
    wl = W.make_workload(cfg)
    a = Hn.DeviceCase(wl)
    b = Hn.DeviceCase(wl)
    a.run()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    b.run(stream=s)
    s.synchronize()
    for x, y in zip(a.fetch(), b.fetch()):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("which", ["norm", "rope", "unfused"])
@pytest.mark.parametrize("D,R,neox,layout", [(100, 100, True, None), (72, 72, True, "odd_pad"),
                                             (3, 2, False, None), (130, 64, True, "shifted"),
                                             (128, 128, True, "shifted"), (512, 510, True, None),
                                             (130, 64, True, "shifted4"), (100, 26, True, "shifted4")])
def test_unfused_steps(which, D, R, neox, layout):
    cfg = W.case(33, 5, 3, D, R, neox, dtype=W.FP16, pos_dtype=W.I64, seed=D + R + 3)
    print("case", which, cfg.name, layout, flush=True)
    Hn.unfused_check(W.make_workload(cfg), which, layout=layout)


@pytest.mark.parametrize("D,R,neox,bias,layout", [
    (100, 0, False, True, None), (100, 100, True, True, None), (72, 72, True, False, "odd_pad"),
    (3, 2, True, True, None), (130, 0, False, False, "shifted"), (128, 64, True, True, "shifted"),
    (512, 510, False, True, None), (128, 64, True, True, "shifted4"), (100, 26, True, True, None)])
def test_layernorm_sibling(D, R, neox, bias, layout):
    cfg = W.case(41, 5, 3, D, R if R else D - D % 2, neox, dtype=W.BF16, pos_dtype=W.I64,
                 seed=D + R + 11, x_std=2.0)
    wl = W.make_workload(cfg)
    # a non-zero mean per head exercises the centring
    from oracle import qknr_oracle as O

    wl.q[...] = O.round_to_io_bits(O.decode_io(wl.q, W.BF16) + 1.5, W.BF16)
    print("case layernorm", cfg.name, layout, flush=True)
    Hn.layernorm_check(wl, R, bias, layout=layout)


@pytest.mark.parametrize("D,R,neox,bias", [
    (40, 38, True, True), (128, 26, True, False), (72, 70, True, True), (200, 98, True, False),
    (128, 64, False, True), (256, 256, True, True), (64, 8, True, False)])
def test_layernorm_sixteen_byte_runs(D, R, neox, bias):
    """The LayerNorm sibling on the element-granular kernel's 16-byte instance,
    which lays the token's cos and signed sin out per element in LDS: odd NeoX
    halves, partial rotations, shapes forced off the vectorised kernel, with
    and without bias; once with the automatic grid and once with 8 workgroups,
    so that every wave rebuilds the pairs for many tokens in turn."""
    cfg = W.case(300, 7, 3, D, R, neox, dtype=W.BF16, pos_dtype=W.I64, seed=D + R + 23,
                 x_std=2.0)
    wl = W.make_workload(cfg)
    from oracle import qknr_oracle as O

    wl.q[...] = O.round_to_io_bits(O.decode_io(wl.q, W.BF16) + 0.75, W.BF16)
    print("case layernorm 16-byte", cfg.name, bias, flush=True)
    for launch in ({"generic": 1}, {"generic": 1, "max_blocks": 8}):
        info = Hn.layernorm_check(wl, R, bias, launch=launch)
        assert info["generic"] == 1 and info["access_bytes"] == 16, info


@pytest.mark.parametrize("D,R,neox,launch,want", [
    (128, 128, True, None, dict(lanes_per_head=64, generic=0)),   # one head per group
    (128, 64, False, None, dict(lanes_per_head=64, generic=0)),
    (64, 64, True, None, dict(generic=1)),                        # no vectorised mapping fits
    (128, 128, False, {"generic": 1}, dict(generic=1)),
])
def test_head_strides_beyond_32_bit_lane_offsets(D, R, neox, launch, want):
    """Q heads 3 GiB apart in one device buffer: a head group of several heads
    would need lane offsets above 2^31, so the planner takes one head per wave
    instruction (or the element-granular kernel, whose head bases are 64-bit).
    Every Q/K element matches the oracle and the bytes between the heads stay
    untouched."""
    import torch
    from head_qk_rmsnorm_amd import binding as B

    T, Hq, Hkv = 33, 2, 3
    cfg = W.case(T, Hq, Hkv, D, R, neox, pos_dtype=W.I64, seed=D + R + 5)
    wl = W.make_workload(cfg)
    dev = torch.device("cuda:0")
    hs = (3 << 30) // 2                  # head stride in elements (3 GiB)
    fill = 0x5A5A
    store = torch.full((hs * (Hq - 1) + T * D + 4096,), fill, dtype=torch.int16, device=dev)
    q = torch.as_strided(store, (T, Hq, D), (D, hs, 1)).view(torch.bfloat16)
    q.view(torch.int16).copy_(torch.from_numpy(wl.q.view(np.int16)).to(dev))
    k = torch.from_numpy(wl.k.view(np.int16)).to(dev).view(torch.bfloat16)
    wq = torch.from_numpy(wl.wq.view(np.int16)).to(dev).view(torch.bfloat16)
    wk = torch.from_numpy(wl.wk.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = torch.from_numpy(wl.cache).to(dev)
    pos = torch.from_numpy(wl.positions).to(dev)
    print("case", cfg.name, launch, flush=True)
    info = B.qknr_inplace_ex(q, k, wq, wk, cache, pos, is_neox=neox, eps=cfg.eps,
                             launch=launch or {})
    torch.cuda.synchronize()
    for key, v in want.items():
        assert info[key] == v, info
    gq = q.view(torch.int16).cpu().numpy().view(np.uint16)
    gk = k.view(torch.int16).cpu().numpy().view(np.uint16)
    rq, rk = Hn.oracle_ref(wl)
    for g, r in ((gq, rq), (gk, rk)):
        cmp = Hn.compare_bits(g, r, cfg.dtype)
        assert cmp.bad == 0 and cmp.exact_frac >= 0.99, cmp
    # the gap between the two heads and the tail: untouched
    for start in (T * D, T * D + (1 << 20), hs - 4096, hs + T * D):
        seg = store[start:start + 4096].cpu().numpy().view(np.uint16)
        assert np.all(seg == fill), start
    del store
    torch.cuda.empty_cache()
