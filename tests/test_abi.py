"""The C-ABI library on the CPU: it loads, exports every declared symbol, its
capability predicate matches the page's rule, and every invalid argument is
rejected with its documented status before any HIP call (no GPU needed: a call
that reached the HIP runtime here would return QKNR_E_DEVICE instead)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from head_qk_rmsnorm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        txt = open(h).read()
        names += re.findall(r"QKNR_API\s+[\w\s\*]+?\b(qknr_\w+)\s*\(", txt)
    return names


def test_library_loads_and_exports_every_declared_symbol():
    names = _declared()
    assert {"qknr_inplace", "qknr_inplace_ex", "qknr_can_use", "qknr_status_string",
            "qknr_copy", "qknr_rmw", "qknr_unfused_inplace", "qknr_rmsnorm_inplace",
            "qknr_rope_inplace", "qknr_layernorm_rope_inplace"} <= set(names)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qknr_\w+)", out))
    assert set(names) == exported, (set(names) ^ exported)


def _page_predicate(D, R, neox):
    """The capability rule of section 5.2 of the page, restated."""
    if D not in (64, 128, 256):
        return False
    if R <= 0 or R > D:
        return False
    e = D // 32
    if R % e:
        return False
    if neox:
        rl = R // e
        if rl < 2 or (rl & (rl - 1)):
            return False
    return True


def _supported(D, R, neox):
    """The library's documented set (include/qknr.h), restated: head_dim in
    [2, 512], rope_dim even in [2, head_dim], either pairing."""
    return 2 <= D <= 512 and 2 <= R <= D and R % 2 == 0


def _vectorised(D, R, neox):
    """Shapes of the vectorised kernel for the fused op (include/qknr.h),
    restated: head_dim a multiple of 8 in [16, 512]; NeoX needs rope_dim/2 to be
    even (16-byte lanes; partners 2, 4 or 6 slots over when it is not a
    multiple of 8). An odd half fits no lane width of 2 or more elements."""
    if D % 8 or D < 16 or D > 512 or not _supported(D, R, neox):
        return False
    return not neox or (R // 2) % 2 == 0


def test_can_use_covers_page_predicate_and_matches_documented_set():
    n_page = n_more = 0
    for D in (0, 1, 2, 3, 8, 16, 24, 32, 40, 64, 80, 96, 100, 128, 192, 256, 320, 512, 513, 520,
              1024):
        for R in range(-2, max(D, 8) + 3):
            for neox in (0, 1):
                got = B.qknr_can_use(D, R, neox)
                assert got == _supported(D, R, neox), (D, R, neox)
                if _page_predicate(D, R, neox):
                    assert got, (D, R, neox)
                    n_page += 1
                elif got:
                    n_more += 1
    assert n_page > 0 and n_more > n_page
    assert not B.lib().qknr_can_use(128, 128, 1, 2, 0)
    assert not B.lib().qknr_can_use(128, 128, 1, 0, 2)
    assert B.lib().qknr_can_use(128, 128, 1, 1, 1)


def test_status_strings():
    texts = {code: B.qknr_status_string(code) for code in range(-8, 1)}
    assert len(set(texts.values())) == 9
    assert "unknown status" not in " ".join(texts.values())
    assert B.qknr_status_string(-99) == B.qknr_status_string(5) == "qknr: unknown status"


P = ctypes.c_void_p
A = 0x10000  # a 16-byte aligned fake address; never dereferenced


def _call(**kw):
    return _call_info(**kw)[0]


def _call_info(**kw):
    a = dict(q=P(A), k=P(A + 0x100000), wq=P(A), wk=P(A), cache=P(A), pos=P(A), T=5, Hq=4,
             Hkv=4, D=128, R=128, neox=1, eps=1e-6, qt=4 * 256, qh=256, kt=4 * 256, kh=256,
             dtype=0, pdt=0, stream=P(0), cfg=None)
    a.update(kw)
    cfg = a.pop("cfg")
    info = B.LaunchInfo()
    args = [a[n] for n in ("q", "k", "wq", "wk", "cache", "pos", "T", "Hq", "Hkv", "D", "R",
                           "neox", "eps", "qt", "qh", "kt", "kh", "dtype", "pdt", "stream")]
    rc = B.lib().qknr_inplace_ex(*args, ctypes.byref(cfg) if cfg else None, ctypes.byref(info))
    return rc, info.as_dict()


REJECT = [
    (dict(T=-1), B.QKNR_E_SHAPE), (dict(Hq=-1), B.QKNR_E_SHAPE), (dict(Hkv=-3), B.QKNR_E_SHAPE),
    (dict(T=1 << 31), B.QKNR_E_SHAPE), (dict(T=(1 << 28), Hq=8, Hkv=8), B.QKNR_E_SHAPE),
    (dict(dtype=2), B.QKNR_E_DTYPE), (dict(dtype=-1), B.QKNR_E_DTYPE),
    (dict(pdt=2), B.QKNR_E_DTYPE),
    (dict(D=1024, R=1024), B.QKNR_E_UNSUPPORTED), (dict(D=514, R=2), B.QKNR_E_UNSUPPORTED),
    (dict(D=1, R=0), B.QKNR_E_UNSUPPORTED), (dict(R=0), B.QKNR_E_UNSUPPORTED),
    (dict(R=130), B.QKNR_E_UNSUPPORTED), (dict(R=-2), B.QKNR_E_UNSUPPORTED),
    (dict(R=7, neox=0), B.QKNR_E_UNSUPPORTED), (dict(R=99, neox=1), B.QKNR_E_UNSUPPORTED),
    (dict(eps=-1e-6), B.QKNR_E_ARG), (dict(eps=float("nan")), B.QKNR_E_ARG),
    (dict(eps=float("inf")), B.QKNR_E_ARG),
    (dict(q=P(0)), B.QKNR_E_NULL), (dict(k=P(0)), B.QKNR_E_NULL), (dict(wq=P(0)), B.QKNR_E_NULL),
    (dict(wk=P(0)), B.QKNR_E_NULL), (dict(cache=P(0)), B.QKNR_E_NULL),
    (dict(pos=P(0)), B.QKNR_E_NULL),
    (dict(qh=128), B.QKNR_E_SHAPE),            # heads overlap (stride < 256 bytes)
    (dict(qt=3 * 256), B.QKNR_E_SHAPE),        # token rows overlap
    (dict(qh=-256), B.QKNR_E_SHAPE), (dict(kt=-1024), B.QKNR_E_SHAPE),
    (dict(qt=256, qh=256), B.QKNR_E_SHAPE),    # equal strides overlap
    (dict(q=P(A + 1)), B.QKNR_E_ALIGN), (dict(k=P(A + 3)), B.QKNR_E_ALIGN),
    (dict(wq=P(A + 1)), B.QKNR_E_ALIGN), (dict(wk=P(A + 7)), B.QKNR_E_ALIGN),
    (dict(qh=257, qt=4 * 258), B.QKNR_E_ALIGN), (dict(kt=4 * 256 + 1), B.QKNR_E_ALIGN),
    (dict(cache=P(A + 2)), B.QKNR_E_ALIGN), (dict(pos=P(A + 2)), B.QKNR_E_ALIGN),
    (dict(pos=P(A + 4), pdt=1), B.QKNR_E_ALIGN),
    (dict(cfg=B.LaunchCfg(lanes_per_head=7)), B.QKNR_E_ARG),
    (dict(D=64, R=64, cfg=B.LaunchCfg(lanes_per_head=64)), B.QKNR_E_ARG),  # 1 element per lane
    (dict(cfg=B.LaunchCfg(lanes_per_head=128)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(lanes_per_head=4)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(unroll=3)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(block_waves=9)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(block_waves=-1)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(max_blocks=-2)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(groups_per_item=-1)), B.QKNR_E_ARG),
    # NeoX with 16-byte lanes needs rope_dim/2 to be even
    (dict(D=128, R=10, cfg=B.LaunchCfg(lanes_per_head=16)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(generic=2)), B.QKNR_E_ARG),
    (dict(cfg=B.LaunchCfg(generic=1, lanes_per_head=16)), B.QKNR_E_ARG),
    # an explicit lane mapping on a case only the element-granular kernel takes
    (dict(q=P(A + 8), cfg=B.LaunchCfg(lanes_per_head=16)), B.QKNR_E_ARG),
    (dict(D=100, R=100, qt=4 * 200, qh=200, kt=4 * 200, kh=200,
          cfg=B.LaunchCfg(lanes_per_head=16)), B.QKNR_E_ARG),
]

# Accepted on the element-granular kernel: shapes, alignments and strides the
# vectorised kernel cannot take (valid otherwise, so the call reaches the HIP
# runtime, which a GPU-less host does not have).
GENERIC = [
    dict(D=100, R=100, qt=4 * 200, qh=200, kt=4 * 200, kh=200),
    dict(D=8, R=8, qt=4 * 16, qh=16, kt=4 * 16, kh=16),
    dict(D=2, R=2, neox=0, qt=4 * 4, qh=4, kt=4 * 4, kh=4),
    dict(D=3, R=2, neox=1, qt=4 * 6, qh=6, kt=4 * 6, kh=6),
    dict(R=6), dict(R=98, neox=1), dict(D=64, R=2, neox=1, qt=4 * 128, qh=128, kt=4 * 128, kh=128),
    dict(D=96, R=6, neox=1, qt=4 * 192, qh=192, kt=4 * 192, kh=192),
    dict(D=512, R=510, neox=1, qt=4 * 1024, qh=1024, kt=4 * 1024, kh=1024),
    dict(q=P(A + 8)), dict(k=P(A + 2)), dict(wq=P(A + 4)), dict(wk=P(A + 8)),
    dict(qh=264, qt=4 * 264), dict(kt=4 * 256 + 8), dict(qh=258, qt=4 * 258),
    dict(cfg=B.LaunchCfg(generic=1)),
    dict(cfg=B.LaunchCfg(generic=1, groups_per_item=3, block_waves=8, unroll=4)),
]


def _no_gpu():
    try:
        import torch

        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
@pytest.mark.parametrize("kw,code", REJECT, ids=lambda v: str(v))
def test_rejections(kw, code):
    assert _call(**kw) == code


def _elem_align(kw):
    """Common alignment (2 to 16 bytes) of q, k, the weights and the used strides."""
    a = dict(q=P(A), k=P(A + 0x100000), wq=P(A), wk=P(A), D=128, qt=4 * 256, qh=256, kt=4 * 256,
             kh=256)
    a.update({n: v for n, v in kw.items() if n in a})

    def aligned(b):
        return (all(a[n].value % b == 0 for n in ("q", "k", "wq", "wk"))
                and all(a[n] % b == 0 for n in ("qt", "qh", "kt", "kh")))

    return next(b for b in (16, 8, 4, 2) if aligned(b))


def elem_plan(D, align, Hq, Hkv, groups_fit=True):
    """The element-granular kernel's lane mapping (include/qknr.h), restated:
    runs of pw elements with pw in {8, 4, 2, 1} dividing head_dim and
    2*pw <= align; S runs per lane with S*pw <= 8; L lanes per head, the lanes
    a head needs (ceil(head_dim / (S*pw)) <= 64) either rounded up to a power
    of two or exact; G = 64 // L heads per wave instruction (1 if a group's
    lane offsets would not fit 32 bits). The plan with the fewest wave
    instructions per token, S * (ceil(Hq/G) + ceil(Hkv/G)), wins; ties go to a
    power-of-two L, then the wider run, then fewer slots.
    Returns (pw, S, L, G, exact_fit)."""
    cands = []
    for pw in (8, 4, 2, 1):
        if D % pw or align < 2 * pw:
            continue
        S = 1
        while S * pw <= 8:
            lx = -(-D // (S * pw))
            if lx <= 64:
                lp = 1
                while lp < lx:
                    lp *= 2
                shapes = [(lp, False)] + ([(lx, True)] if lx != lp and groups_fit else [])
                for L, exact in shapes:
                    G = 64 // L if groups_fit else 1
                    cost = S * (-(-Hq // G) + -(-Hkv // G))
                    cands.append(((cost, exact, -pw, S), (pw, S, L, G, exact)))
            S += 1
    return min(cands)[1]


def test_element_plan_rule_examples():
    # head_dim 100 (8-byte runs): 32 lanes, 2 heads per instruction (4 before);
    # 40 with 16-byte runs: exact groups of 5 lanes, 12 heads; 130 (4-byte runs):
    # 17 lanes x 4 slots, 3 heads; odd head_dims take single elements
    assert elem_plan(100, 8, 24, 24)[:4] == (4, 1, 32, 2)
    assert elem_plan(40, 16, 24, 24) == (8, 1, 5, 12, True)
    assert elem_plan(40, 8, 24, 24) == (4, 1, 10, 6, True)
    assert elem_plan(130, 16, 24, 24) == (2, 4, 17, 3, True)
    assert elem_plan(255, 16, 24, 24)[0] == 1
    assert elem_plan(128, 16, 24, 24)[:4] == (8, 1, 16, 4)
    assert elem_plan(512, 16, 24, 24)[:4] == (8, 1, 64, 1)
    # without room for 32-bit group offsets: one head per instruction
    assert elem_plan(100, 8, 24, 24, groups_fit=False)[3] == 1
    # few heads: fewer lanes per head are no use
    assert elem_plan(40, 16, 1, 0)[3] >= 1


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
@pytest.mark.parametrize("kw", GENERIC, ids=lambda v: str(v))
def test_element_granular_cases_are_accepted(kw):
    rc, info = _call_info(**kw)
    assert rc == B.QKNR_E_DEVICE, B.qknr_status_string(rc)
    D = kw.get("D", 128)
    pw, S, L, G, _ = elem_plan(D, _elem_align(kw), 4, 4)
    assert info["generic"] == 1
    assert (info["access_bytes"], info["elems_per_lane"], info["lanes_per_head"],
            info["heads_per_wave"]) == (2 * pw, S * pw, L, G), info
    ng = 2 * -(-4 // G)
    assert info["groups_per_token"] == ng
    # 16/(S pw) groups are loaded before the first is computed, two such rounds per item
    U = 16 // (S * pw)
    cfg = kw.get("cfg")
    want = min(cfg.groups_per_item if cfg is not None and cfg.groups_per_item else 2 * U, ng)
    assert info["groups_per_item"] == want and info["unroll"] == U
    assert info["items"] == 5 * -(-ng // want)


def test_element_plan_covers_every_width():
    assert {elem_plan(kw.get("D", 128), _elem_align(kw), 4, 4)[0] for kw in GENERIC} == {1, 2, 4, 8}


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
def test_vectorised_cases_stay_vectorised():
    rc, info = _call_info()
    assert rc == B.QKNR_E_DEVICE and info["generic"] == 0 and info["lanes_per_head"] == 16


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
def test_empty_work_is_ok_without_pointers_or_device():
    z = P(0)
    assert _call(T=0, q=z, k=z, wq=z, wk=z, cache=z, pos=z) == B.QKNR_OK
    assert _call(Hq=0, Hkv=0, q=z, k=z, wq=z, wk=z, cache=z, pos=z) == B.QKNR_OK
    # with valid arguments the first HIP call is reached, which fails on a GPU-less host
    assert _call() == B.QKNR_E_DEVICE


def _plan(D, R, neox, Hq=24, Hkv=24, cfg=None):
    info = B.LaunchInfo()
    z = P(0)
    args = [z, z, z, z, z, z, 0, Hq, Hkv, D, R, int(neox), 1e-6, 0, 0, 0, 0, 0, 0, z]
    rc = B.lib().qknr_inplace_ex(*args, ctypes.byref(cfg) if cfg else None, ctypes.byref(info))
    assert rc == 0
    return info.as_dict()


@pytest.mark.parametrize("D", [64, 128, 256])
def test_plan_lane_mapping(D):
    """16-byte lanes (head_dim/8 lanes per head) whenever the pairing allows it;
    then half a wave (32 lanes), then a full wave (64 lanes) per head."""
    for neox in (0, 1):
        for R in range(2, D + 1, 2):
            if not B.qknr_can_use(D, R, neox):
                continue
            info = _plan(D, R, neox)
            if not _vectorised(D, R, neox):
                pw, S, L, G, _ = elem_plan(D, 16, 24, 24)
                assert info["generic"] == 1 and (info["lanes_per_head"], info["heads_per_wave"],
                                                 info["access_bytes"]) == (L, G, 2 * pw), (D, R, neox)
                continue
            assert info["generic"] == 0
            fits = lambda e: (not neox) or ((R // 2) % e == 0 and R // 2 >= e)
            shifted = neox and (R // 2) % 2 == 0   # 16-byte lanes, partners 2/4/6 slots over
            want_lanes = D // 8 if fits(8) or shifted else (32 if fits(D // 32) else 64)
            assert info["lanes_per_head"] == want_lanes, (D, R, neox, info)
            assert info["elems_per_lane"] * info["lanes_per_head"] == D
            assert info["heads_per_wave"] == 64 // info["lanes_per_head"]
            G = info["heads_per_wave"]
            assert info["groups_per_token"] == -(-24 // G) + -(-24 // G)
            gqa = _plan(D, R, neox, Hq=7, Hkv=3)
            assert gqa["groups_per_token"] == -(-7 // gqa["heads_per_wave"]) + -(-3 // gqa["heads_per_wave"])


def test_plan_exact_fit_groups_for_small_heads_with_partners_4_slots_over():
    """NeoX partners 4 slots over keep padded lane groups except in groups of 5
    to 8 lanes that fit at least 25% more heads (fused op): head_dim 40 takes 5
    lanes (12 heads per instruction, padded: 8); head_dim 24 (3 lanes), 56 (7
    lanes, 9 heads against 8) and 72 (9 lanes) stay padded; the LayerNorm
    sibling stays padded."""
    for D, R, lanes, G in ((40, 40, 5, 12), (40, 24, 5, 12), (24, 24, 4, 16), (24, 8, 4, 16),
                           (56, 56, 8, 8), (72, 72, 16, 4), (136, 136, 32, 2)):
        i = _plan(D, R, 1)
        assert (i["generic"], i["lanes_per_head"], i["heads_per_wave"], i["elems_per_lane"]) == \
            (0, lanes, G, 8), (D, R, i)
    info = B.LaunchInfo()
    z = P(0)
    rc = B.lib().qknr_layernorm_rope_inplace_ex(z, z, z, z, z, z, z, z, 0, 24, 24, 40, 40, 1, 1e-6,
                                                 0, 0, 0, 0, 0, 0, z, None, ctypes.byref(info))
    assert rc == 0 and info.lanes_per_head == 8, info.lanes_per_head


@pytest.mark.parametrize("D,lanes", [(16, 2), (24, 4), (40, 8), (80, 16), (112, 16),
                                     (160, 32), (192, 32), (320, 64), (512, 64)])
def test_plan_run_time_head_dims(D, lanes):
    """Other head_dims use 16-byte lanes in a lane group padded to a power of two."""
    info = _plan(D, D, 0)
    assert (info["lanes_per_head"], info["elems_per_lane"]) == (lanes, 8)
    G = 64 // lanes
    assert info["heads_per_wave"] == G
    assert info["unroll"] == (4 if G * 2 * D <= 640 else 2)   # long items: small head groups
    assert _plan(D, D - (D % 16), 1)["lanes_per_head"] == lanes


@pytest.mark.parametrize("D,R", [(96, 40), (80, 40), (112, 56), (80, 20), (72, 72), (40, 12),
                                 (120, 60), (160, 40), (96, 20), (56, 20), (104, 52), (264, 264),
                                 (200, 20), (320, 36), (504, 12), (128, 20), (64, 12), (256, 44)])
def test_plan_neox_halves_off_the_lane_width_take_shifted_partners(D, R):
    """NeoX halves that no 16-byte lane divides keep 16-byte lanes for the fused
    op: each partner sits (rope_dim/2 mod 8) slots over in a neighbouring lane
    (e.g. head_dim 96 with rope_dim 40, head_dim 80 with rope_dim 20)."""
    cap = 16
    while cap < D:
        cap *= 2
    info = _plan(D, R, 1)
    assert info["generic"] == 0 and info["elems_per_lane"] == 8, info
    assert info["lanes_per_head"] == (D // 8 if _seg(D, R) else (D if D in (64, 128, 256) else cap) // 8)


@pytest.mark.parametrize("D,R", [(200, 22), (320, 30), (96, 6), (504, 10), (72, 70), (200, 2),
                                 (128, 10), (64, 6)])
def test_plan_odd_neox_halves_use_the_element_kernel(D, R):
    info = _plan(D, R, 1)
    assert info["generic"] == 1, info


def _seg(D, R):
    """Exact-fit lane groups of head_dim/8 lanes (fused op, NeoX): partners 2 or
    6 slots over, and at least 25% more heads per wave instruction than the
    lane group padded to a power of two."""
    if D in (64, 128, 256) or D % 8 or D < 16 or (R // 2) % 8 not in (2, 6):
        return False
    lanes, cap = D // 8, 16
    while cap < D:
        cap *= 2
    return lanes <= 32 and 4 * (64 // lanes) >= 5 * (64 // (cap // 8))


@pytest.mark.parametrize("D,R,seg", [(80, 20, True), (72, 20, True), (152, 44, True), (96, 20, True),
                                     (88, 28, True), (40, 12, True), (104, 52, False),
                                     (120, 60, False), (200, 100, False), (56, 20, False),
                                     (128, 20, False), (80, 40, False), (72, 72, False),
                                     (264, 4, False)])
def test_plan_exact_fit_lane_groups(D, R, seg):
    """NeoX halves of 8m + 2 or 8m + 6 dims (partners through the LDS row) pack
    heads into exact-fit groups of head_dim/8 lanes when that fits at least 25%
    more heads into a wave instruction; otherwise the padded group stays."""
    assert _seg(D, R) == seg
    info = _plan(D, R, 1)
    cap = 16
    while cap < D:
        cap *= 2
    lanes = D // 8 if seg else (D if D in (64, 128, 256) else cap) // 8
    assert (info["generic"], info["elems_per_lane"], info["lanes_per_head"]) == (0, 8, lanes), info
    assert info["heads_per_wave"] == 64 // lanes
    G = 64 // lanes
    assert info["groups_per_token"] == -(-24 // G) * 2


def _fit96(D, R, neox):
    """head_dim 96 of the fused op on 12-byte lanes: a NeoX half that is a
    multiple of 6 but not of 8."""
    return D == 96 and bool(neox) and (R // 2) % 6 == 0 and R // 2 >= 6 and (R // 2) % 8 != 0


def test_plan_head_dim_96_takes_12_byte_lanes():
    """The fused op at head_dim 96 with a NeoX half that is a multiple of 6 but
    not of 8: 16 lanes of 6 elements (12-byte accesses, no spare lanes,
    compile-time defaults). Every other pairing keeps the padded 16-byte-lane
    mapping (shifted partners where needed), odd halves the element kernel.
    Explicit unroll 1, 2 and 4 are honoured."""
    for R in (24, 12, 72, 60, 84, 36):   # NeoX halves 12, 6, 36, 30, 42, 18
        assert _fit96(96, R, 1)
        i = _plan(96, R, 1)
        assert (i["lanes_per_head"], i["elems_per_lane"], i["access_bytes"],
                i["heads_per_wave"]) == (16, 6, 12, 4), (R, i)
        assert (i["unroll"], i["groups_per_item"], i["block_threads"]) == (2, 2, 192), i
    for R, neox in ((20, 1), (40, 1), (32, 1), (16, 1), (8, 1), (96, 1), (48, 1), (96, 0),
                    (24, 0), (30, 0)):
        assert not _fit96(96, R, neox)
        i = _plan(96, R, neox)
        lanes = 12 if neox and _seg(96, R) else 16   # 96/20: exact-fit groups of 12 lanes
        assert (i["generic"], i["lanes_per_head"], i["elems_per_lane"]) == (0, lanes, 8), (R, i)
    assert _plan(96, 6, 1)["generic"] == 1   # odd half
    for u in (1, 2, 4):
        assert _plan(96, 24, 1, cfg=B.LaunchCfg(unroll=u))["unroll"] == u
    assert _plan(96, 24, 1, cfg=B.LaunchCfg(lanes_per_head=16))["elems_per_lane"] == 6


def test_plan_defaults():
    """Automatic launch: 2 head groups per work item, both loaded up front,
    3 waves per workgroup when a head takes at most 16 lanes, 6 at head_dim 256
    on 16-byte lanes, else 4."""
    info = _plan(128, 128, 0)
    assert info["groups_per_item"] == 2 and info["unroll"] == 2
    assert info["block_threads"] == 192
    assert _plan(256, 256, 0)["block_threads"] == 384          # 32 lanes per head
    assert _plan(256, 44, 1)["block_threads"] == 384           # shifted partners, 32 lanes
    assert _plan(128, 128, 0, cfg=B.LaunchCfg(lanes_per_head=32))["block_threads"] == 256
    assert _plan(64, 64, 1)["block_threads"] == 192            # 8 lanes per head
    assert _plan(96, 96, 0)["block_threads"] == 192            # run-time head_dim, 16 lanes
    assert _plan(128, 12, 1)["lanes_per_head"] == 16            # NeoX 12: shifted partners
    # head groups never mix Q and K heads: 4 Q + 4 K heads of head_dim 64 (8 per
    # wave instruction) are two half-filled groups, one work item
    tiny = _plan(64, 64, 1, Hq=4, Hkv=4)
    assert tiny["groups_per_token"] == 2 and tiny["groups_per_item"] == 2


def _seg4_unroll2(D, R, neox):
    """Exact-fit lane groups of 5 lanes with NeoX partners 4 slots over (head_dim
    40 with rope_dim/2 = 8m + 4): the planner keeps them at unroll 2."""
    return bool(neox) and D == 40 and (R // 2) % 8 == 4


@pytest.mark.parametrize("D,R,neox,long_items", [
    (80, 80, 1, True), (96, 96, 1, True), (96, 24, 1, False), (80, 32, 1, True), (160, 160, 1, True),
    (192, 64, 1, True), (320, 320, 1, True), (48, 48, 1, True), (40, 40, 1, True),
    (40, 24, 1, True), (48, 40, 1, True), (56, 56, 1, True),
    (24, 24, 1, True), (112, 112, 1, True), (224, 224, 1, True), (72, 72, 1, True),
    (136, 136, 1, True), (104, 52, 1, True),
    (40, 40, 0, True), (80, 80, 0, True), (144, 144, 0, True), (160, 160, 0, True),
    (320, 320, 0, True), (24, 24, 0, False), (48, 48, 0, False), (56, 56, 0, False),
    (96, 96, 0, False), (112, 112, 0, False), (192, 192, 0, False), (200, 200, 0, False),
    (128, 128, 1, False), (64, 64, 1, False), (256, 256, 1, False), (128, 128, 0, False)])
def test_plan_defaults_long_items(D, R, neox, long_items):
    """Head_dims other than 64/128/256 default to long work items (unroll 4,
    4 groups per item, 2-wave workgroups) with NeoX pairing or when a head group
    holds at most 640 bytes, except that exact-fit groups of 5 lanes with
    partners 4 slots over (head_dim 40) keep unroll 2 in them; every other shape keeps
    unroll 2, 2 groups per item and 3 or 4 waves. Explicit settings are
    honoured; a run-time head_dim runs unroll 1 as 2."""
    info = _plan(D, R, neox)
    assert info["generic"] == 0, info
    G, L = info["heads_per_wave"], info["lanes_per_head"]
    assert long_items == (D not in (64, 128, 256) and not _fit96(D, R, neox)
                          and (neox == 1 or G * 2 * D <= 640))
    if long_items:
        want_u = 2 if _seg4_unroll2(D, R, neox) else 4
        assert (info["unroll"], info["groups_per_item"], info["block_threads"]) == (want_u, 4, 128), info
    else:
        assert (info["unroll"], info["groups_per_item"]) == (2, 2), info
        want = 192 if L <= 16 else 384 if (D == 256 and L == 32) else 256
        assert info["block_threads"] == want, info
    explicit = _plan(D, R, neox, cfg=B.LaunchCfg(groups_per_item=3, block_waves=5, unroll=2))
    assert (explicit["unroll"], explicit["groups_per_item"], explicit["block_threads"]) == (2, 3, 320)
    four = _plan(D, R, neox, cfg=B.LaunchCfg(unroll=4))
    assert four["unroll"] == 4
    one = _plan(D, R, neox, cfg=B.LaunchCfg(unroll=1))
    assert one["unroll"] == (1 if D in (64, 128, 256) or _fit96(D, R, neox) else 2)


@pytest.mark.parametrize("D,lanes,E", [(128, 64, 2), (256, 64, 4), (128, 32, 4), (64, 32, 2),
                                      (256, 32, 8)])
def test_plan_wave_mappings(D, lanes, E):
    info = _plan(D, D, 0, cfg=B.LaunchCfg(lanes_per_head=lanes))
    assert (info["lanes_per_head"], info["elems_per_lane"]) == (lanes, E)
    assert info["heads_per_wave"] == 64 // lanes


def test_plan_explicit_cfg():
    info = _plan(128, 128, 0, cfg=B.LaunchCfg(lanes_per_head=32, groups_per_item=5, unroll=4,
                                              block_waves=8))
    assert info == dict(lanes_per_head=32, elems_per_lane=4, heads_per_wave=2,
                        groups_per_token=24, groups_per_item=5, unroll=4, block_threads=512,
                        grid_blocks=0, items=0, generic=0, access_bytes=8)


def test_plan_element_granular():
    """head_dims the vectorised kernel does not take, NeoX halves that are not a
    multiple of a lane width, and an explicit request, plan the element-granular
    kernel: runs of 1, 2, 4 or 8 elements, several heads per wave instruction
    (expected values worked out by hand from the rule in elem_plan)."""
    info = _plan(100, 100, 1, Hq=7, Hkv=3)   # runs of 4, 32 lanes (25 used): 2 heads per group
    assert info == dict(lanes_per_head=32, elems_per_lane=4, heads_per_wave=2,
                        groups_per_token=6, groups_per_item=6, unroll=4, block_threads=256,
                        grid_blocks=0, items=0, generic=1, access_bytes=8)
    big = _plan(300, 300, 1, Hq=30, Hkv=10)  # 2 slots of 4 on a full wave: 2 groups in flight, 4 per item
    assert (big["elems_per_lane"], big["lanes_per_head"], big["unroll"], big["groups_per_item"]) == (8, 64, 2, 4)
    wide = _plan(200, 98, 1, Hq=30, Hkv=10)  # 16-byte runs, 32 lanes (25 used), 2 heads per group
    assert (wide["elems_per_lane"], wide["unroll"], wide["access_bytes"], wide["heads_per_wave"]) == (8, 2, 16, 2)
    small = _plan(40, 6, 1, Hq=30, Hkv=10)   # 16-byte runs, exact groups of 5 lanes: 12 heads
    assert (small["lanes_per_head"], small["heads_per_wave"], small["groups_per_token"],
            small["groups_per_item"]) == (5, 12, 4, 4)
    odd = _plan(45, 6, 1, Hq=30, Hkv=10)     # odd head_dim: 2-byte runs, 4 slots of 12 lanes, 5 heads
    assert (odd["elems_per_lane"], odd["lanes_per_head"], odd["heads_per_wave"], odd["unroll"],
            odd["access_bytes"]) == (4, 12, 5, 4, 2)
    assert _plan(72, 70, 1)["generic"] == 1          # NeoX half 35: no lane width divides it
    assert _plan(72, 72, 1)["elems_per_lane"] == 8   # NeoX half 36 = 8*4 + 4: 16-byte lanes
    assert _plan(72, 68, 1)["elems_per_lane"] == 8   # NeoX half 34 = 8*4 + 2: shifted partners
    assert _plan(72, 72, 0)["generic"] == 0          # interleaved: 16-byte lanes
    odd130 = _plan(130, 64, 0)                       # pairs in 4 slots of 17 lanes, 3 heads
    assert (odd130["elems_per_lane"], odd130["lanes_per_head"], odd130["heads_per_wave"]) == (8, 17, 3)
    assert _plan(132, 64, 0)["access_bytes"] == 8    # a multiple of 4: runs of 4
    forced = _plan(128, 128, 0, cfg=B.LaunchCfg(generic=1, groups_per_item=48, block_waves=2))
    assert forced["generic"] == 1 and forced["heads_per_wave"] == 4
    assert forced["groups_per_item"] == 12 and forced["block_threads"] == 128
    for D, R, neox, Hq, Hkv in ((100, 100, 1, 7, 3), (300, 300, 1, 30, 10), (200, 98, 1, 30, 10),
                                (40, 6, 1, 30, 10), (45, 6, 1, 30, 10), (130, 64, 0, 24, 24)):
        pw, S, L, G, _ = elem_plan(D, 16, Hq, Hkv)
        i = _plan(D, R, neox, Hq=Hq, Hkv=Hkv)
        assert (i["access_bytes"], i["elems_per_lane"], i["lanes_per_head"], i["heads_per_wave"]) == \
            (2 * pw, S * pw, L, G), (D, R, i)


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    c = torch.zeros(4, 64)
    p = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="HIP device"):
        B.fused_inplace_qknorm_rope(q, q, w, w, c, p, is_neox=True)


def test_harness_layouts_on_host():
    """The test harness places q/k exactly where the views say (host check)."""
    np = pytest.importorskip("numpy")
    from head_qk_rmsnorm_amd import workloads as W
    from tests import qknr_harness as Hn

    for layout in ("contiguous", "padded", "head_major", "qkv"):
        wl = W.make_workload(W.case(5, 3, 2, 64, 64, True, seed=1))
        dc = Hn.DeviceCase(wl, layout=layout, device="cpu")
        q, k = dc.outputs(dc.storages_host)
        assert np.array_equal(q, wl.q) and np.array_equal(k, wl.k), layout
        assert sum(int(m.sum()) for m in dc.masks) == wl.q.size + wl.k.size
        import torch

        assert torch.equal(dc.q.contiguous().view(torch.int16),
                           torch.from_numpy(wl.q.view(np.int16))), layout


def test_plan_falls_back_to_fewer_heads_per_group_for_huge_head_strides():
    """Lane offsets inside a head group must stay below 2^31: with head-major
    views whose head stride is ~1 GiB (or ~3 GiB) the planner takes a mapping
    with fewer heads per wave instruction, and rejects what none can address."""
    def plan(D, head_stride, Hq=8):
        info = B.LaunchInfo()
        z = P(0)
        rc = B.lib().qknr_inplace_ex(z, z, z, z, z, z, 0, Hq, 0, D, D, 0, 1e-6, 2 * D,
                                     head_stride, 2 * D, 2 * D, 0, 0, z, None,
                                     ctypes.byref(info))
        return rc, info.as_dict()

    rc, info = plan(128, 2 * 128)
    assert rc == 0 and info["lanes_per_head"] == 16
    rc, info = plan(128, 1 << 30)
    assert rc == 0 and info["lanes_per_head"] == 32
    rc, info = plan(128, 3 << 30)
    assert rc == 0 and info["lanes_per_head"] == 64
    rc, info = plan(64, 3 << 30)  # no vectorised mapping fits: element-granular, one head per group
    assert rc == 0 and info["generic"] == 1 and info["heads_per_wave"] == 1
    rc, info = plan(64, 3 << 30, Hq=1)  # one head: its stride is never used
    assert rc == 0 and info["lanes_per_head"] == 8


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
def test_unfused_entry_points_validate_before_launching():
    L = B.lib()
    z = P(0)
    a = P(A)
    # the norm step needs no cache or positions; it does need the weights
    assert L.qknr_rmsnorm_inplace(a, a, z, a, 5, 4, 4, 128, 1e-6, 1024, 256, 1024, 256, 0,
                                  z) == B.QKNR_E_NULL
    # other head_dims run on the element-granular kernel
    assert L.qknr_rmsnorm_inplace(a, a, a, a, 5, 4, 4, 96, 1e-6, 4 * 192, 192, 4 * 192, 192, 0,
                                  z) == B.QKNR_E_DEVICE
    assert L.qknr_rmsnorm_inplace(a, a, a, a, 5, 4, 4, 101, 1e-6, 4 * 208, 208, 4 * 208, 208, 0,
                                  z) == B.QKNR_E_DEVICE
    assert L.qknr_rmsnorm_inplace(a, a, a, a, 5, 4, 4, 600, 1e-6, 4 * 1200, 1200, 4 * 1200, 1200,
                                  0, z) == B.QKNR_E_UNSUPPORTED
    assert L.qknr_rmsnorm_inplace(a, a, a, a, 5, 4, 4, 128, -1.0, 1024, 256, 1024, 256, 0,
                                  z) == B.QKNR_E_ARG
    assert L.qknr_rmsnorm_inplace(a, a, a, a, 5, 4, 4, 128, 1e-6, 1024, 256, 1024, 256, 0,
                                  z) == B.QKNR_E_DEVICE  # valid: reaches the runtime
    # the rope step needs cache and positions, no weights
    assert L.qknr_rope_inplace(a, a, z, a, 5, 4, 4, 128, 128, 1, 1024, 256, 1024, 256, 0, 0,
                               z) == B.QKNR_E_NULL
    assert L.qknr_rope_inplace(a, a, a, a, 5, 4, 4, 128, 98, 1, 1024, 256, 1024, 256, 0, 0,
                               z) == B.QKNR_E_DEVICE
    assert L.qknr_rope_inplace(a, a, a, a, 5, 4, 4, 128, 97, 1, 1024, 256, 1024, 256, 0, 0,
                               z) == B.QKNR_E_UNSUPPORTED
    assert L.qknr_rope_inplace(a, a, a, P(A + 4), 5, 4, 4, 128, 128, 1, 1024, 256, 1024, 256, 0,
                               1, z) == B.QKNR_E_ALIGN
    assert L.qknr_rope_inplace(a, a, a, a, 5, 4, 4, 128, 128, 1, 1024, 256, 1024, 256, 0, 0,
                               z) == B.QKNR_E_DEVICE
    # the unfused pair validates like the fused op, before either launch
    args = [a, a, a, a, a, a, 5, 4, 4, 128, 128, 1, 1e-6, 1024, 256, 1024, 256, 0, 0, z]
    assert L.qknr_unfused_inplace(*args) == B.QKNR_E_DEVICE
    for i, bad, code in ((2, z, B.QKNR_E_NULL), (4, z, B.QKNR_E_NULL), (10, 99, B.QKNR_E_UNSUPPORTED),
                         (12, float("nan"), B.QKNR_E_ARG), (14, 128, B.QKNR_E_SHAPE)):
        bad_args = list(args)
        bad_args[i] = bad
        assert L.qknr_unfused_inplace(*bad_args) == code, i
    zero = list(args)
    zero[6] = 0
    assert L.qknr_unfused_inplace(*zero) == B.QKNR_OK


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
def test_layernorm_entry_point_validates_before_launching():
    L = B.lib()
    z = P(0)
    a = P(A)

    def call(**kw):
        d = dict(q=a, k=a, wq=a, wk=a, bq=a, bk=a, cache=a, pos=a, T=5, Hq=4, Hkv=4, D=128, R=64,
                 neox=1, eps=1e-6, qt=1024, qh=256, kt=1024, kh=256, dtype=0, pdt=0)
        d.update(kw)
        return L.qknr_layernorm_rope_inplace(*[d[n] for n in ("q", "k", "wq", "wk", "bq", "bk", "cache", "pos", "T", "Hq", "Hkv", "D", "R", "neox", "eps", "qt", "qh", "kt", "kh", "dtype", "pdt")], z)

    assert call() == B.QKNR_E_DEVICE                       # valid: reaches the runtime
    assert call(bq=z, bk=z) == B.QKNR_E_DEVICE             # no bias is fine
    assert call(bk=z) == B.QKNR_E_NULL                     # one bias without the other
    assert call(bq=P(A + 8)) == B.QKNR_E_DEVICE            # element-granular
    assert call(wq=z) == B.QKNR_E_NULL
    assert call(cache=z) == B.QKNR_E_NULL                  # rotation asked, no table
    assert call(R=0, cache=z, pos=z, neox=0) == B.QKNR_E_DEVICE  # norm alone needs no table
    assert call(R=98) == B.QKNR_E_DEVICE                   # element-granular
    assert call(R=99) == B.QKNR_E_UNSUPPORTED
    assert call(D=100, qt=800, qh=200, kt=800, kh=200, R=0) == B.QKNR_E_DEVICE
    assert call(D=600, qt=4800, qh=1200, kt=4800, kh=1200, R=0) == B.QKNR_E_UNSUPPORTED
    assert call(bq=P(A + 1)) == B.QKNR_E_ALIGN
    assert call(eps=-1.0) == B.QKNR_E_ARG
    assert call(T=0, q=z, k=z, wq=z, wk=z, bq=z, bk=z, cache=z, pos=z) == B.QKNR_OK


def test_torch_custom_ops_are_registered_with_their_mutations():
    """The ops are torch custom ops that declare q and k as mutated (what
    torch.compile needs for an in-place op), with the page's capability query."""
    torch = pytest.importorskip("torch")
    from head_qk_rmsnorm_amd import torch_ops as T

    s = str(torch.ops.qknr.fused_inplace_qknorm_rope.default._schema)
    assert "Tensor(a0!) q" in s and "Tensor(a1!) k" in s and "Tensor q_weight" in s, s
    assert "bool is_neox" in s and "-> ()" in s, s
    s = str(torch.ops.qknr.fused_inplace_qk_layernorm_rope.default._schema)
    assert "Tensor(a0!) q" in s and "Tensor(a1!) k" in s and "Tensor? q_bias" in s, s
    assert T.can_use_fused_inplace_qknorm_rope(128, 128, True, torch.bfloat16)
    assert T.can_use_fused_inplace_qknorm_rope(100, 98, True, torch.float16)
    assert not T.can_use_fused_inplace_qknorm_rope(128, 128, True, torch.float32)
    assert not T.can_use_fused_inplace_qknorm_rope(1024, 128, False, torch.bfloat16)
    # the page's accepted shapes are all accepted
    for D in (64, 128, 256):
        for R in range(D // 32, D + 1, D // 32):
            rl = R // (D // 32)
            for neox in (False, True):
                if neox and (rl < 2 or rl & (rl - 1)):
                    continue
                assert T.can_use_fused_inplace_qknorm_rope(D, R, neox, torch.bfloat16), (D, R)
    q = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        torch.ops.qknr.fused_inplace_qknorm_rope(q, q.clone(), w, w, torch.zeros(4, 64),
                                                 torch.zeros(2, dtype=torch.int32), is_neox=True)


@pytest.mark.parametrize("name", ["tiny", "dit", "gqa", "partial", "large", "gqa_tp8", "dit_hp8",
                                  "dit_sp8"])
def test_benchmark_workloads_plan_the_measured_launch(name):
    """Every benchmark and shard workload, with the strides the benchmark uses
    (contiguous or views into a fused qkv buffer), plans onto the vectorised
    kernel with 16-byte lanes, 2 head groups per item loaded together, and 3
    waves per workgroup (6 for the half-wave heads of head_dim 256)."""
    from head_qk_rmsnorm_amd import workloads as W

    c = W.CONFIGS[name]
    D = c.head_dim
    if c.layout == "qkv":
        row = (c.Hq + 2 * c.Hkv) * D * 2
        qt, qh, kt, kh = row, D * 2, row, D * 2
    else:
        qt, qh, kt, kh = c.Hq * D * 2, D * 2, c.Hkv * D * 2, D * 2
    info = B.LaunchInfo()
    z = P(0)
    rc = B.lib().qknr_inplace_ex(z, z, z, z, z, z, 0, c.Hq, c.Hkv, D, c.rope_dim, int(c.is_neox),
                                 c.eps, qt, qh, kt, kh, 0 if c.dtype == W.BF16 else 1,
                                 0 if c.pos_dtype == W.I32 else 1, z, None, ctypes.byref(info))
    assert rc == 0
    i = info.as_dict()
    assert i["generic"] == 0 and i["lanes_per_head"] == D // 8 and i["elems_per_lane"] == 8, i
    assert i["groups_per_item"] == min(2, i["groups_per_token"]) and i["unroll"] == 2, i
    assert i["block_threads"] == (384 if D // 8 > 16 else 192), i


def test_head_dim_scan_shapes_are_vectorised():
    """Every shape of bench.py's head_dim scan runs on the vectorised kernel and
    moves the DiT workload's Q/K bytes to within one token row."""
    import bench
    from head_qk_rmsnorm_amd import workloads as W

    dit = W.CONFIGS["dit"]
    for D, R, neox in bench.HEAD_DIM_SCAN:
        c = bench.head_dim_scan_case(D, R, neox)
        assert (c.head_dim, c.rope_dim, c.is_neox, c.Hq, c.Hkv) == (D, R, neox, 24, 24)
        assert abs(c.units * D - dit.units * dit.head_dim) <= 48 * D
        info = _plan(D, R, neox)
        assert info["generic"] == 0, (D, R, neox, info)


def test_every_supported_shape_plans_an_existing_instance():
    """For every head_dim 2..512, every even rope_dim and both pairings, the
    planner lands on a kernel instance that exists (with empty work a missing
    one would be QKNR_E_UNSUPPORTED before any HIP call): the fused op at each
    unroll (vectorised exactly on the documented set), the LayerNorm sibling
    with and without the rotation, and the unfused chain."""
    lib = B.lib()
    z = P(0)
    cfgs = [B.LaunchCfg(unroll=u) for u in (1, 2, 4)]
    n = 0
    for D in range(2, 513):
        assert lib.qknr_layernorm_rope_inplace(z, z, z, z, z, z, z, z, 0, 4, 4, D, 0, 0, 1e-6,
                                               0, 0, 0, 0, 0, 0, z) == 0, D
        for R in range(2, D + 1, 2):
            for neox in (0, 1):
                info = B.LaunchInfo()
                for cfg in cfgs:
                    rc = lib.qknr_inplace_ex(z, z, z, z, z, z, 0, 24, 8, D, R, neox, 1e-6, 0, 0,
                                             0, 0, 0, 0, z, ctypes.byref(cfg), ctypes.byref(info))
                    assert rc == 0, (D, R, neox, cfg.unroll, rc)
                    assert info.generic == (0 if _vectorised(D, R, neox) else 1), (D, R, neox)
                assert lib.qknr_layernorm_rope_inplace(z, z, z, z, z, z, z, z, 0, 4, 4, D, R, neox,
                                                       1e-6, 0, 0, 0, 0, 0, 0, z) == 0, (D, R, neox)
                assert lib.qknr_unfused_inplace(z, z, z, z, z, z, 0, 4, 4, D, R, neox, 1e-6, 0, 0,
                                                0, 0, 0, 0, z) == 0, (D, R, neox)
                n += 1
    assert n == 2 * sum(D // 2 for D in range(2, 513))


def test_launch_info_layout():
    """qknr_launch_info keeps its 48-byte size: access_bytes sits in what was
    the tail padding after generic, so callers built with the earlier layout
    are not written past."""
    assert ctypes.sizeof(B.LaunchInfo) == 48
    assert B.LaunchInfo.items.offset == 32 and B.LaunchInfo.generic.offset == 40
    assert B.LaunchInfo.access_bytes.offset == 44


def _tail_items(T, Hq, Hkv, D, R, neox, cfg=None):
    rc, info = _call_info(T=T, Hq=Hq, Hkv=Hkv, D=D, R=R, neox=neox, qt=Hq * D * 2, qh=D * 2,
                          kt=Hkv * D * 2, kh=D * 2, cfg=cfg)
    assert rc == B.QKNR_E_DEVICE, B.qknr_status_string(rc)
    return info


@pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run on a host without a GPU")
@pytest.mark.parametrize("T,Hq,Hkv,D,R,neox,on", [
    (4608, 24, 24, 128, 128, 0, True),    # DiT: 12 groups per token, 6 items of 2
    (8192, 32, 8, 128, 128, 1, True),     # GQA: 10 groups, 5 items
    (16384, 16, 16, 128, 64, 1, True),    # partial rotation: 8 groups, 4 items
    (8192, 24, 24, 256, 256, 0, True),    # head_dim 256: 24 groups, 12 items
    (1368, 24, 24, 128, 128, 1, True),    # just long enough: T = 8 x the 171 tail tokens
    (1367, 24, 24, 128, 128, 1, False),   # one token short: no tail
    (8192, 4, 1, 128, 128, 1, False),     # a token is one item: no tail
    (4608, 24, 24, 96, 96, 1, True),      # run-time head_dim: 3 items of 4, tail items of 2
    (4608, 24, 24, 80, 80, 0, True),      # run-time head_dim, interleaved long items
    (6144, 24, 24, 96, 24, 1, False),     # head_dim 96 on 12-byte lanes
    (14745, 24, 24, 40, 40, 1, False),    # exact-fit lane groups
    (7372, 24, 24, 80, 20, 1, False),     # exact-fit lane groups
    (4608, 24, 24, 128, 20, 1, False),    # NeoX partners 2 slots over
    (6144, 24, 24, 72, 72, 1, False),     # NeoX partners 4 slots over
])
def test_plan_tail_items(T, Hq, Hkv, D, R, neox, on):
    """The fused op on 16-byte lanes, with aligned partners outside exact-fit
    groups, with at least 3 items per token ends on ceil(2048 / tail items per token) tokens whose
    items hold half the groups of the others, when the launch is at least 8
    times that long; an explicit groups_per_item turns it off."""
    info = _tail_items(T, Hq, Hkv, D, R, neox)
    ng, gpi = info["groups_per_token"], info["groups_per_item"]
    nc = -(-ng // gpi)
    tail = 0
    if on:
        tgpi = gpi // 2
        tnc = -(-ng // tgpi)
        tail = -(-2048 // tnc)
        assert nc >= 3 and T >= 8 * tail and info["elems_per_lane"] == 8
        assert info["items"] == (T - tail) * nc + tail * tnc, info
    else:
        assert info["items"] == T * nc, info
    plain = _tail_items(T, Hq, Hkv, D, R, neox, cfg=B.LaunchCfg(groups_per_item=gpi))
    assert plain["items"] == T * nc, plain
