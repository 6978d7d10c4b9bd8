"""Pins for the fp64 oracle: each test ties it to something other than its own
formulas (hand-derived values, closed forms, invariants, library routines,
exhaustive enumeration), so that a dropped term, a wrong sign, a wrong pair
index or a transposed operand anywhere in it fails at least one test.

Formulas cited are those of the page "SGLang Diffusion fused operator
fused_inplace_qknorm_rope: in-depth technical analysis" (m.lsln.cn/news/241376),
sections 2.1 - 2.3.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import qknr_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _one_token(x, w, eps, rope_dim, cos, sin, is_neox):
    x = np.asarray(x, dtype=np.float64)[None, None, :]
    w = np.asarray(w, dtype=np.float64)
    cache = np.concatenate([np.asarray(cos, np.float32), np.asarray(sin, np.float32)])[None, :]
    pos = np.zeros(1, np.int32)
    oq, ok = O.qknorm_rope(x, x.copy(), w, w, cache, pos, is_neox=is_neox, eps=eps,
                           rope_dim=rope_dim)
    return oq[0, 0], ok[0, 0]


def _rand_heads(g, T, H, D, std=1.0):
    return g.standard_normal((T, H, D)) * std


def _cache_formula(rows, R, base=1e4):
    j = np.arange(R // 2, dtype=np.float64)
    th = base ** (-2.0 * j / R)
    ang = np.arange(rows, dtype=np.float64)[:, None] * th
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


# ---------------------------------------------------------------------------
# Hand-derived worked examples (tests/golden/hand_examples.json)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ex", _golden()["examples"], ids=lambda e: e["name"])
@pytest.mark.parametrize("neox", [False, True])
def test_golden_hand_examples(ex, neox):
    oq, ok = _one_token(ex["x"], ex["w"], ex["eps"], ex["rope_dim"], ex["cos"], ex["sin"], neox)
    want = ex["out_neox"] if neox else ex["out_interleaved"]
    # cos/sin pass through fp32 (0.6 and 0.8 are not exact), hence 1e-7 not 1e-15
    np.testing.assert_allclose(oq, want, rtol=0, atol=1e-7)
    np.testing.assert_array_equal(oq, ok)


def test_golden_bf16_rounding_cases():
    for c in _golden()["bf16_rounding"]["cases"]:
        x = c["x_value"] if "x_value" in c else float.fromhex(c["x_value_hex"])
        got = int(O.round_to_bf16_bits(np.array([x]))[0])
        assert got == int(c["bits"], 16), c


# ---------------------------------------------------------------------------
# Norm (section 2.1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_norm_matches_torch_rms_norm(eps):
    """Library routine: torch's rms_norm in float64 is an independent implementation
    of x / sqrt(mean(x^2) + eps) * w."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(11)
    for D in (4, 64, 128, 256):
        x = _rand_heads(g, 5, 3, D, std=2.0)
        w = g.uniform(0.5, 1.5, D)
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w),
                                            eps=eps).numpy()
        np.testing.assert_allclose(O.rms_norm(x, w, eps), want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("c", [-3.0, 0.5, 100.0])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_norm_constant_vector(c, eps):
    """Closed form: x = c*1 gives n = w * c / sqrt(c^2 + eps); with eps = 0 it is sign(c)*w."""
    D = 64
    w = np.linspace(0.5, 1.5, D)
    n = O.rms_norm(np.full((1, D), c), w, eps)[0]
    np.testing.assert_allclose(n, w * c / math.sqrt(c * c + eps), rtol=1e-15)
    if eps == 0.0:
        np.testing.assert_allclose(n, np.sign(c) * w, rtol=1e-15)


def test_norm_energy_identity():
    """Invariant: sum (n_i / w_i)^2 = D * m / (m + eps), m = mean square of x."""
    g = np.random.default_rng(3)
    D, eps = 128, 0.37
    x = g.standard_normal((7, D))
    w = g.uniform(0.5, 1.5, D)
    n = O.rms_norm(x, w, eps)
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sum((n / w) ** 2, axis=-1), D * m / (m + eps), rtol=1e-13)


def test_norm_divides_by_head_dim_not_rope_dim():
    """Section 2.1/2.3: the mean is over head_dim even when only part of the head rotates."""
    D, R = 8, 4
    x = np.ones((1, 1, D))
    w = np.ones(D)
    cache = np.array([[1.0] * (R // 2) + [0.0] * (R // 2)], np.float32)
    oq, _ = O.qknorm_rope(x, x, w, w, cache, np.array([0]), is_neox=True, eps=0.0, rope_dim=R)
    np.testing.assert_allclose(oq[0, 0], np.ones(D), rtol=1e-15)


# ---------------------------------------------------------------------------
# Whole op: closed forms and invariants (sections 2.2, 2.3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("D,R", [(64, 64), (128, 128), (128, 64), (256, 256), (64, 8)])
def test_position_zero_is_norm_only(neox, D, R):
    """Closed form: row 0 of the formula cache is cos = 1, sin = 0 exactly, so the
    output at position 0 is the RMSNorm result on every dim."""
    g = np.random.default_rng(D + R)
    q, k = _rand_heads(g, 3, 2, D), _rand_heads(g, 3, 1, D)
    wq, wk = g.uniform(0.5, 1.5, D), g.uniform(0.5, 1.5, D)
    cache = _cache_formula(4, R)
    assert np.all(cache[0, : R // 2] == 1.0) and np.all(cache[0, R // 2:] == 0.0)
    oq, ok = O.qknorm_rope(q, k, wq, wk, cache, np.zeros(3, np.int64), is_neox=neox, eps=1e-6)
    e = float(np.float32(1e-6))
    np.testing.assert_array_equal(oq, O.rms_norm(q, wq, e))
    np.testing.assert_array_equal(ok, O.rms_norm(k, wk, e))


@pytest.mark.parametrize("neox", [False, True])
def test_exact_quarter_half_turns(neox):
    """Textbook rotations with exact (cos, sin): 90 deg swaps and negates, 180 deg
    negates, 270 deg swaps and negates the other way."""
    D = R = 16
    g = np.random.default_rng(5)
    x = _rand_heads(g, 1, 1, D)
    w = g.uniform(0.5, 1.5, D)
    n = O.rms_norm(x, w, 0.0)[0, 0]
    if neox:
        a_idx, b_idx = np.arange(R // 2), np.arange(R // 2) + R // 2
    else:
        a_idx, b_idx = np.arange(0, R, 2), np.arange(1, R, 2)
    for (c, s, fa, fb) in [(0.0, 1.0, lambda a, b: -b, lambda a, b: a),
                           (-1.0, 0.0, lambda a, b: -a, lambda a, b: -b),
                           (0.0, -1.0, lambda a, b: b, lambda a, b: -a)]:
        cache = np.array([[c] * (R // 2) + [s] * (R // 2)], np.float32)
        o, _ = O.qknorm_rope(x, x, w, w, cache, np.array([0]), is_neox=neox, eps=0.0)
        o = o[0, 0]
        np.testing.assert_array_equal(o[a_idx], fa(n[a_idx], n[b_idx]))
        np.testing.assert_array_equal(o[b_idx], fb(n[a_idx], n[b_idx]))


@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("j0", [0, 1, 2, 3])
def test_single_pair_angle_pins_index_map(neox, j0):
    """Only angle j0 is non-zero: exactly the two dims of pair j0 change
    ((2j0, 2j0+1) interleaved, (j0, j0+R/2) NeoX)."""
    D, R = 12, 8
    g = np.random.default_rng(j0)
    x = _rand_heads(g, 1, 1, D)
    w = g.uniform(0.5, 1.5, D)
    n = O.rms_norm(x, w, 0.0)[0, 0]
    cos = np.ones(R // 2)
    sin = np.zeros(R // 2)
    cos[j0], sin[j0] = 0.0, 1.0
    cache = np.concatenate([cos, sin]).astype(np.float32)[None, :]
    o, _ = O.qknorm_rope(x, x, w, w, cache, np.array([0]), is_neox=neox, eps=0.0, rope_dim=R)
    o = o[0, 0]
    a, b = (j0, j0 + R // 2) if neox else (2 * j0, 2 * j0 + 1)
    changed = np.nonzero(o != n)[0].tolist()
    assert changed == sorted([a, b])
    assert o[a] == -n[b] and o[b] == n[a]


@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("D,R", [(64, 64), (128, 64), (256, 128)])
def test_pairs_keep_their_norm_and_tail_passes(neox, D, R):
    """Invariants: each rotated pair keeps n_a^2 + n_b^2 scaled by c^2 + s^2;
    dims R..D-1 equal the normalised input exactly."""
    g = np.random.default_rng(7)
    T = 6
    q = _rand_heads(g, T, 3, D)
    w = g.uniform(0.5, 1.5, D)
    cache = _cache_formula(50, R)
    pos = g.integers(0, 50, T)
    oq, _ = O.qknorm_rope(q, q, w, w, cache, pos, is_neox=neox, eps=1e-6)
    n = O.rms_norm(q, w, float(np.float32(1e-6)))
    c = cache[pos, : R // 2].astype(np.float64)[:, None, :]
    s = cache[pos, R // 2:].astype(np.float64)[:, None, :]
    if neox:
        ia, ib = np.arange(R // 2), np.arange(R // 2) + R // 2
    else:
        ia, ib = np.arange(0, R, 2), np.arange(1, R, 2)
    lhs = oq[..., ia] ** 2 + oq[..., ib] ** 2
    rhs = (n[..., ia] ** 2 + n[..., ib] ** 2) * (c * c + s * s)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13)
    np.testing.assert_array_equal(oq[..., R:], n[..., R:])


@pytest.mark.parametrize("R", [8, 64, 128])
def test_interleaved_equals_neox_under_permutation(R):
    """Invariant: with P taking dim 2j -> j and 2j+1 -> j+R/2 on the first R dims
    (identity beyond), interleaved(x, w) = P^-1 neox(P x, P w)."""
    D = 128
    g = np.random.default_rng(R)
    T, H = 5, 4
    x = _rand_heads(g, T, H, D)
    w = g.uniform(0.5, 1.5, D)
    cache = _cache_formula(20, R)
    pos = g.integers(0, 20, T)
    perm = np.arange(D)  # perm[new] = old
    perm[: R // 2] = np.arange(0, R, 2)
    perm[R // 2:R] = np.arange(1, R, 2)
    il, _ = O.qknorm_rope(x, x, w, w, cache, pos, is_neox=False, eps=1e-6, rope_dim=R)
    nx, _ = O.qknorm_rope(x[..., perm], x[..., perm], w[perm], w[perm], cache, pos,
                          is_neox=True, eps=1e-6, rope_dim=R)
    back = np.empty_like(nx)
    back[..., perm] = nx
    np.testing.assert_allclose(il, back, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("neox", [False, True])
def test_rotation_is_complex_multiplication(neox):
    """Library formulation: a pair (a, b) rotated by angle phi is the complex
    product (a + ib) * exp(i*phi), with numpy complex arithmetic and angles
    p * base^(-2j/R) from the definition (only the fp32 cache error remains)."""
    D, R, base = 128, 96, 1e4
    g = np.random.default_rng(17)
    T = 9
    x = _rand_heads(g, T, 2, D)
    w = g.uniform(0.5, 1.5, D)
    rows = 4096
    cache = _cache_formula(rows, R, base)
    pos = g.integers(0, rows, T)
    o, _ = O.qknorm_rope(x, x, w, w, cache, pos, is_neox=neox, eps=1e-6, rope_dim=R)
    n = O.rms_norm(x, w, float(np.float32(1e-6)))
    phi = pos[:, None, None] * base ** (-2.0 * np.arange(R // 2) / R)
    if neox:
        ia, ib = np.arange(R // 2), np.arange(R // 2) + R // 2
    else:
        ia, ib = np.arange(0, R, 2), np.arange(1, R, 2)
    z = (n[..., ia] + 1j * n[..., ib]) * np.exp(1j * phi)
    np.testing.assert_allclose(o[..., ia], z.real, atol=2e-6 * np.abs(n).max())
    np.testing.assert_allclose(o[..., ib], z.imag, atol=2e-6 * np.abs(n).max())


@pytest.mark.parametrize("neox", [False, True])
def test_relative_position_property(neox):
    """Defining property of RoPE: the dot product of rotated q at p and rotated k
    at p' depends only on p - p' (within the fp32 cache error)."""
    D = R = 64
    g = np.random.default_rng(23)
    xq = _rand_heads(g, 1, 1, D)
    xk = _rand_heads(g, 1, 1, D)
    w = np.ones(D)
    cache = _cache_formula(600, R)
    dots = []
    for p in (5, 105, 517):
        oq, _ = O.qknorm_rope(xq, xq, w, w, cache, np.array([p]), is_neox=neox, eps=0.0)
        ok, _ = O.qknorm_rope(xk, xk, w, w, cache, np.array([p - 3]), is_neox=neox, eps=0.0)
        dots.append(float(np.dot(oq[0, 0], ok[0, 0])))
    np.testing.assert_allclose(dots, dots[0], atol=1e-4)
    # and it is not trivially constant: another offset gives another value
    oq, _ = O.qknorm_rope(xq, xq, w, w, cache, np.array([5]), is_neox=neox, eps=0.0)
    ok, _ = O.qknorm_rope(xk, xk, w, w, cache, np.array([5 - 40]) + 40, is_neox=neox, eps=0.0)
    assert abs(float(np.dot(oq[0, 0], ok[0, 0])) - dots[0]) > 1e-3


def test_odd_symmetry_and_scale_invariance():
    """op(-x) = -op(x) for any eps; with eps = 0, op(a x) = op(x) for a > 0."""
    D = R = 128
    g = np.random.default_rng(29)
    x = _rand_heads(g, 4, 3, D)
    w = g.uniform(0.5, 1.5, D)
    cache = _cache_formula(10, R)
    pos = g.integers(0, 10, 4)
    for neox in (False, True):
        o, _ = O.qknorm_rope(x, x, w, w, cache, pos, is_neox=neox, eps=1e-3)
        om, _ = O.qknorm_rope(-x, -x, w, w, cache, pos, is_neox=neox, eps=1e-3)
        np.testing.assert_array_equal(om, -o)
        o0, _ = O.qknorm_rope(x, x, w, w, cache, pos, is_neox=neox, eps=0.0)
        o7, _ = O.qknorm_rope(7.5 * x, 7.5 * x, w, w, cache, pos, is_neox=neox, eps=0.0)
        np.testing.assert_allclose(o7, o0, rtol=1e-13, atol=1e-15)


def test_q_and_k_use_their_own_weights_and_positions_per_token():
    """q heads take wq, k heads take wk; all heads of token t use row positions[t]."""
    D = R = 8
    T = 3
    x = np.ones((T, 2, D))
    wq = np.full(D, 2.0)
    wk = np.full(D, 3.0)
    cache = np.zeros((3, R), np.float32)
    cache[0, : R // 2] = 1.0           # row 0: identity
    cache[1, : R // 2] = -1.0          # row 1: 180 degrees
    cache[2, R // 2:] = 1.0            # row 2: 90 degrees
    pos = np.array([1, 2, 0])
    oq, ok = O.qknorm_rope(x, x[:, :1], wq, wk, cache, pos, is_neox=False, eps=0.0)
    np.testing.assert_array_equal(oq[0], -2.0)
    np.testing.assert_array_equal(ok[0], -3.0)
    np.testing.assert_array_equal(oq[1, :, 0::2], -2.0)
    np.testing.assert_array_equal(oq[1, :, 1::2], 2.0)
    np.testing.assert_array_equal(oq[2], 2.0)
    np.testing.assert_array_equal(ok[2], 3.0)


def test_zero_vector():
    """A zero head normalises to zero for eps > 0 (r = eps^-1/2 times 0)."""
    D = 64
    x = np.zeros((1, 1, D))
    w = np.ones(D)
    cache = _cache_formula(2, D)
    o, _ = O.qknorm_rope(x, x, w, w, cache, np.array([1]), is_neox=True, eps=1e-6)
    assert np.all(o == 0.0)


def test_rejects_out_of_range_positions_and_negative_eps():
    D = 8
    x = np.ones((1, 1, D))
    w = np.ones(D)
    cache = _cache_formula(2, D)
    with pytest.raises(ValueError):
        O.qknorm_rope(x, x, w, w, cache, np.array([2]), is_neox=True, eps=1e-6)
    with pytest.raises(ValueError):
        O.qknorm_rope(x, x, w, w, cache, np.array([-1]), is_neox=True, eps=1e-6)
    with pytest.raises(ValueError):
        O.rms_norm(x, w, -1.0)


# ---------------------------------------------------------------------------
# Rounding to the I/O formats
# ---------------------------------------------------------------------------

def _all_finite_bf16():
    codes = np.arange(0x10000, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals)
    return codes[ok].astype(np.uint16), vals[ok]


def test_bf16_decode_exhaustive():
    """Every finite bf16 code decodes to the fp32 whose top half it is (torch's
    bfloat16 -> float64 conversion as the independent reference)."""
    torch = pytest.importorskip("torch")
    codes, _ = _all_finite_bf16()
    want = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.decode_bf16(codes), want)


def test_bf16_rounding_exhaustive_midpoints():
    """Brute force over all 2^16 codes: each representable value rounds to itself;
    midpoints between neighbours round to the even code; midpoints nudged by one
    fp64 ulp round to the nearer neighbour (rules out double rounding)."""
    codes, vals = _all_finite_bf16()
    assert np.array_equal(O.round_to_bf16_bits(vals), codes)
    pos = vals[(vals >= 0)]
    pos = np.unique(pos)
    lo, hi = pos[:-1], pos[1:]
    lo_c = O.round_to_bf16_bits(lo).astype(np.int64)
    hi_c = O.round_to_bf16_bits(hi).astype(np.int64)
    mid = (lo + hi) / 2.0  # exact in fp64
    for sgn in (1.0, -1.0):
        got = O.round_to_bf16_bits(sgn * mid).astype(np.int64) & 0x7FFF
        even = np.where(lo_c % 2 == 0, lo_c, hi_c) & 0x7FFF
        assert np.array_equal(got, even)
        up = O.round_to_bf16_bits(sgn * np.nextafter(mid, np.inf * (hi - lo))).astype(np.int64)
        assert np.array_equal(up & 0x7FFF, hi_c & 0x7FFF)
        dn = O.round_to_bf16_bits(sgn * np.nextafter(mid, -np.inf * (hi - lo))).astype(np.int64)
        assert np.array_equal(dn & 0x7FFF, lo_c & 0x7FFF)


def test_bf16_rounding_random_vs_nearest_search():
    """Random fp64 values: the code returned is the nearest bf16 (searched in the
    sorted table of all values), ties to even."""
    codes, vals = _all_finite_bf16()
    order = np.argsort(vals, kind="stable")
    sv, sc = vals[order], codes[order]
    g = np.random.default_rng(1)
    x = g.standard_normal(200000) * np.exp2(g.integers(-20, 20, 200000))
    got = O.round_to_bf16_bits(x)
    i = np.clip(np.searchsorted(sv, x), 1, len(sv) - 1)
    dl, dh = x - sv[i - 1], sv[i] - x
    pick = np.where(dl < dh, sc[i - 1], sc[i])
    tie = dl == dh
    assert not np.any(tie)
    # -0.0 and +0.0 sit side by side in the table; compare values there
    same = (got == pick) | (O.decode_bf16(got) == O.decode_bf16(pick))
    assert np.all(same)


def test_fp16_rounding_exhaustive_midpoints():
    codes = np.arange(0x10000, dtype=np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    assert np.array_equal(O.round_to_fp16_bits(vals[fin]), codes[fin])
    pos = np.unique(vals[fin & (vals >= 0)])
    lo, hi = pos[:-1], pos[1:]
    lo_c, hi_c = O.round_to_fp16_bits(lo).astype(np.int64), O.round_to_fp16_bits(hi).astype(np.int64)
    mid = (lo + hi) / 2.0
    got = O.round_to_fp16_bits(mid).astype(np.int64)
    assert np.array_equal(got, np.where(lo_c % 2 == 0, lo_c, hi_c))
    assert np.array_equal(O.round_to_fp16_bits(np.nextafter(mid, np.inf)), hi_c)
    assert np.array_equal(O.round_to_fp16_bits(np.nextafter(mid, -np.inf)), lo_c)


def test_io_entry_decodes_computes_rounds():
    """qknorm_rope_io = decode, fp64 op, one rounding (checked against the fp64
    entry plus the rounding helper on a bf16 and an fp16 case)."""
    g = np.random.default_rng(31)
    D = R = 64
    for dt in ("bf16", "fp16"):
        qf = g.standard_normal((3, 2, D))
        wf = g.uniform(0.5, 1.5, D)
        qb = O.round_to_io_bits(qf, dt)
        wb = O.round_to_io_bits(wf, dt)
        cache = _cache_formula(8, R)
        pos = np.array([1, 7, 3])
        rq, rk, fq, fk = O.qknorm_rope_io(qb, qb[:, :1], wb, wb, cache, pos, is_neox=True,
                                          eps=1e-6, dtype=dt)
        oq, _ = O.qknorm_rope(O.decode_io(qb, dt), O.decode_io(qb, dt), O.decode_io(wb, dt),
                              O.decode_io(wb, dt), cache, pos, is_neox=True, eps=1e-6)
        np.testing.assert_array_equal(rq, O.round_to_io_bits(oq, dt))
        np.testing.assert_array_equal(rk, rq[:, :1])
        assert np.all(O.within_tolerance(fq, oq))


def test_tolerance_formula():
    """The acceptance bound is 2^-7 * (|ref| + 1) and rejects NaN."""
    ref = np.array([0.0, 1.0, -2.0, 100.0])
    tol = np.array([2 ** -7, 2 ** -6, 3 * 2 ** -7, 101 * 2 ** -7])
    np.testing.assert_array_equal(O.tolerance(ref), tol)
    assert np.all(O.within_tolerance(ref + tol, ref))
    assert not np.any(O.within_tolerance(ref + 1.01 * tol, ref))
    assert not O.within_tolerance(np.array([np.nan]), np.array([0.0]))[0]


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (scalar loops over every head and element)
# ---------------------------------------------------------------------------

def _brute(q, k, wq, wk, cache, pos, neox, eps, R):
    eps = float(np.float32(eps))

    def one(x, w, p):
        D = len(x)
        s = 0.0
        for v in x:
            s += v * v
        r = 1.0 / math.sqrt(s / D + eps)
        n = [x[i] * r * w[i] for i in range(D)]
        out = list(n)
        half = R // 2
        for j in range(half):
            c, sn = float(cache[p][j]), float(cache[p][half + j])
            a, b = (j, j + half) if neox else (2 * j, 2 * j + 1)
            out[a] = n[a] * c - n[b] * sn
            out[b] = n[b] * c + n[a] * sn
        return out

    oq = np.array([[one(q[t, h], wq, int(pos[t])) for h in range(q.shape[1])]
                   for t in range(q.shape[0])]).reshape(q.shape)
    ok = np.array([[one(k[t, h], wk, int(pos[t])) for h in range(k.shape[1])]
                   for t in range(k.shape[0])]).reshape(k.shape)
    return oq, ok


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    g = np.random.default_rng(100 + seed)
    D = int(g.choice([64, 128, 256]))
    R = int(g.choice([D, D // 2, 16, 2 * int(g.integers(1, D // 2 + 1))]))
    neox = bool(seed % 2)
    T = int(g.integers(1, 10))
    Hq, Hkv = int(g.integers(1, 4)), int(g.integers(1, 3))
    q, k = _rand_heads(g, T, Hq, D), _rand_heads(g, T, Hkv, D)
    wq, wk = g.uniform(0.5, 1.5, D), g.uniform(0.5, 1.5, D)
    cache = _cache_formula(32, R)
    pos = g.integers(0, 32, T)
    oq, ok = O.qknorm_rope(q, k, wq, wk, cache, pos, is_neox=neox, eps=1e-6, rope_dim=R)
    bq, bk = _brute(q, k, wq, wk, cache, pos, neox, 1e-6, R)
    np.testing.assert_allclose(oq, bq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ok, bk, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_any_head_dim(seed):
    """Head_dims that are not multiples of 8 (odd ones included), any even
    rope_dim, both pairings: the vectorised oracle equals the scalar loops."""
    g = np.random.default_rng(300 + seed)
    D = int(g.integers(2, 41))
    R = 2 * int(g.integers(1, D // 2 + 1))
    neox = bool(seed % 2)
    T = int(g.integers(1, 8))
    Hq, Hkv = int(g.integers(1, 4)), int(g.integers(1, 3))
    q, k = _rand_heads(g, T, Hq, D), _rand_heads(g, T, Hkv, D)
    wq, wk = g.uniform(0.5, 1.5, D), g.uniform(0.5, 1.5, D)
    cache = _cache_formula(16, R)
    pos = g.integers(0, 16, T)
    oq, ok = O.qknorm_rope(q, k, wq, wk, cache, pos, is_neox=neox, eps=1e-6, rope_dim=R)
    bq, bk = _brute(q, k, wq, wk, cache, pos, neox, 1e-6, R)
    np.testing.assert_allclose(oq, bq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ok, bk, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# The unfused chain (norm step, intermediate rounded to the I/O type, rope step)
# ---------------------------------------------------------------------------

def test_rms_norm_io_matches_torch_bf16_rms_norm():
    """Library routine: torch's CPU rms_norm on bf16 tensors computes in fp32 and
    rounds once to bf16; it must agree with the oracle's correctly rounded norm
    to within one bf16 ulp everywhere and bit for bit almost everywhere."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(41)
    D = 128
    x = O.round_to_bf16_bits(g.standard_normal((64, 6, D)) * 2.0)
    w = O.round_to_bf16_bits(g.uniform(0.5, 1.5, D))
    ours = O.rms_norm_io(x, w, eps=1e-6, dtype="bf16")
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tw = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    theirs = torch.nn.functional.rms_norm(tx, (D,), tw, eps=1e-6).view(torch.int16).numpy().view(np.uint16)
    ulps = np.abs(ours.astype(np.int64) - theirs.astype(np.int64))
    assert ulps.max() <= 1
    assert np.mean(ours == theirs) > 0.99


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_rms_norm_io_constant_vector_is_exact(dt):
    """eps = 0, w = 1, x = c*1 gives exactly sign(c)."""
    D = 64
    for c in (-3.0, 0.25, 7.0):
        x = O.round_to_io_bits(np.full((2, 1, D), c), dt)
        w = O.round_to_io_bits(np.ones(D), dt)
        n = O.decode_io(O.rms_norm_io(x, w, eps=0.0, dtype=dt), dt)
        assert np.all(n == np.sign(c))


@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_rope_io_identity_and_quarter_turn_are_exact(neox, dt):
    """With exact (cos, sin) the rotation of representable values is
    representable: row (1, 0) returns the input bits, row (0, 1) swaps the pair
    and negates the first member."""
    D = R = 32
    g = np.random.default_rng(5)
    x = O.round_to_io_bits(g.standard_normal((3, 2, D)), dt)
    cache = np.array([[1.0] * (R // 2) + [0.0] * (R // 2), [0.0] * (R // 2) + [1.0] * (R // 2)],
                     np.float32)
    same = O.rope_io(x, cache, np.zeros(3, np.int32), is_neox=neox, dtype=dt)
    assert np.array_equal(same, x)
    turned = O.decode_io(O.rope_io(x, cache, np.ones(3, np.int32), is_neox=neox, dtype=dt), dt)
    xv = O.decode_io(x, dt)
    a, b = (np.arange(R // 2), np.arange(R // 2) + R // 2) if neox else (np.arange(0, R, 2), np.arange(1, R, 2))
    assert np.array_equal(turned[..., a], -xv[..., b])
    assert np.array_equal(turned[..., b], xv[..., a])


@pytest.mark.parametrize("neox", [False, True])
def test_unfused_chain_agrees_with_fused_within_page_tolerance(neox):
    """The page's unit test compares the fused op with the unfused chain at
    bf16 atol 8e-2, rtol 1e-2 (Step 4 of its rewrite guide). The oracle's two
    versions must satisfy that, differ somewhere (the intermediate rounding is
    real), and differ by no more than the rounding analysis allows: rounding the
    normalised pair (a, b) moves a rotated output by at most 2^-8 (|a| + |b|),
    and each side's final rounding by at most 2^-8 of its own magnitude."""
    g = np.random.default_rng(77)
    D, R = 128, 64
    q = O.round_to_bf16_bits(g.standard_normal((50, 4, D)))
    k = O.round_to_bf16_bits(g.standard_normal((50, 2, D)))
    wq = O.round_to_bf16_bits(g.uniform(0.5, 1.5, D))
    wk = O.round_to_bf16_bits(g.uniform(0.5, 1.5, D))
    cache = _cache_formula(100, R)
    pos = g.integers(0, 100, 50)
    fq, fk, fqv, fkv = O.qknorm_rope_io(q, k, wq, wk, cache, pos, is_neox=neox, eps=1e-6,
                                        dtype="bf16", rope_dim=R)
    uq, uk = O.qknorm_rope_unfused_io(q, k, wq, wk, cache, pos, is_neox=neox, eps=1e-6,
                                      dtype="bf16", rope_dim=R)
    e = float(np.float32(1e-6))
    for x, w, f, u in ((q, wq, fqv, uq), (k, wk, fkv, uk)):
        uv = O.decode_bf16(u)
        assert np.all(np.abs(uv - f) <= 8e-2 + 1e-2 * np.abs(f))
        assert np.any(uv != f)
        n = np.abs(O.rms_norm(O.decode_bf16(x), O.decode_bf16(w), e))
        pair = n.copy()
        if neox:
            pair[..., :R // 2] += n[..., R // 2:R]
            pair[..., R // 2:R] += n[..., :R // 2]
        else:
            pair[..., 0:R:2] += n[..., 1:R:2]
            pair[..., 1:R:2] += n[..., 0:R:2]
        bound = 2.0 ** -8 * (pair + np.abs(uv) + np.abs(f)) * (1 + 1e-6)
        assert np.all(np.abs(uv - f) <= bound)
    # pass-through dims see only the norm step: there the two agree exactly
    assert np.array_equal(uq[..., R:], fq[..., R:])


# ---------------------------------------------------------------------------
# Sibling: per-head QK LayerNorm (+ optional rotation)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
@pytest.mark.parametrize("bias", [False, True])
def test_layer_norm_matches_torch_layer_norm(eps, bias):
    """Library routine: torch's layer_norm in float64 (biased variance, weight, bias)."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(13)
    for D in (2, 3, 8, 17, 64, 96, 100, 128, 256):
        x = g.standard_normal((5, 3, D)) * 3.0 + 1.5
        w = g.uniform(0.5, 1.5, D)
        b = g.standard_normal(D) if bias else None
        want = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), torch.from_numpy(w),
                                              None if b is None else torch.from_numpy(b),
                                              eps=eps).numpy()
        np.testing.assert_allclose(O.layer_norm(x, w, b, eps), want, rtol=1e-12, atol=1e-12)


def test_layer_norm_closed_forms():
    """A constant head normalises to the bias; x = m + s*(+1,-1,...) normalises to
    (+-1) * s/sqrt(s^2+eps) * w + b; a shift of x changes nothing."""
    D = 16
    w = np.linspace(0.5, 1.5, D)
    b = np.linspace(-1.0, 1.0, D)
    np.testing.assert_array_equal(O.layer_norm(np.full((1, D), 7.0), w, b, 1e-6)[0], b)
    s, eps = 3.0, 0.5
    sign = np.tile([1.0, -1.0], D // 2)
    x = 10.0 + s * sign
    np.testing.assert_allclose(O.layer_norm(x[None], w, b, eps)[0], sign * s / np.sqrt(s * s + eps) * w + b,
                               rtol=1e-14)
    g = np.random.default_rng(2)
    y = g.standard_normal((4, D))
    np.testing.assert_allclose(O.layer_norm(y + 123.0, w, None, 1e-6), O.layer_norm(y, w, None, 1e-6),
                               rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("neox", [False, True])
def test_qk_layernorm_rope_composes_norm_and_rotation(neox):
    """rope_dim 0 is the norm alone; position 0 of the formula cache is the
    norm alone too; otherwise it is the rotation of the normalised heads
    (numpy complex product with angles from the definition)."""
    D, R = 64, 32
    g = np.random.default_rng(9)
    q, k = g.standard_normal((6, 3, D)), g.standard_normal((6, 2, D))
    wq, wk = g.uniform(0.5, 1.5, D), g.uniform(0.5, 1.5, D)
    bq, bk = g.standard_normal(D), None
    cache = _cache_formula(50, R)
    e = float(np.float32(1e-6))
    nq, nk = O.qk_layernorm_rope(q, k, wq, wk, bq, bk, cache, np.zeros(6, np.int64), is_neox=neox,
                                 eps=1e-6, rope_dim=0)
    np.testing.assert_array_equal(nq, O.layer_norm(q, wq, bq, e))
    np.testing.assert_array_equal(nk, O.layer_norm(k, wk, None, e))
    z, _ = O.qk_layernorm_rope(q, k, wq, wk, bq, bk, cache, np.zeros(6, np.int64), is_neox=neox,
                               eps=1e-6, rope_dim=R)
    np.testing.assert_array_equal(z, nq)
    pos = g.integers(0, 50, 6)
    oq, _ = O.qk_layernorm_rope(q, k, wq, wk, bq, bk, cache, pos, is_neox=neox, eps=1e-6, rope_dim=R)
    phi = pos[:, None, None] * 1e4 ** (-2.0 * np.arange(R // 2) / R)
    ia, ib = (np.arange(R // 2), np.arange(R // 2) + R // 2) if neox else (np.arange(0, R, 2), np.arange(1, R, 2))
    zc = (nq[..., ia] + 1j * nq[..., ib]) * np.exp(1j * phi)
    np.testing.assert_allclose(oq[..., ia], zc.real, atol=2e-6 * np.abs(nq).max())
    np.testing.assert_allclose(oq[..., ib], zc.imag, atol=2e-6 * np.abs(nq).max())
    np.testing.assert_array_equal(oq[..., R:], nq[..., R:])


def _io_bits(vals, dtype):
    """Exact values -> I/O bit patterns, encoded by torch (not by the oracle)."""
    torch = pytest.importorskip("torch")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = torch.tensor(vals, dtype=torch.float64).to(tdt)
    assert torch.equal(t.double(), torch.tensor(vals, dtype=torch.float64)), "value not exact"
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("neox", [False, True])
@pytest.mark.parametrize("bias", [True, False])
def test_golden_layernorm_io_entry(dtype, neox, bias):
    """The LayerNorm sibling's I/O entry on the hand-derived example
    (tests/golden/hand_examples.json, layernorm_examples): distinct q/k inputs,
    weights and biases, a quarter turn picked by position 1, with and without
    the bias rows. Outputs are decoded by torch and compared as values."""
    torch = pytest.importorskip("torch")
    ex = _golden()["layernorm_examples"]["cases"][0]
    D = len(ex["q"])
    bits = lambda v: _io_bits(v, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    dec = lambda b: torch.from_numpy(b.view(np.int16)).view(tdt).double().numpy()
    q = bits(ex["q"]).reshape(1, 1, D)
    k = bits(ex["k"]).reshape(1, 1, D)
    cache = np.asarray(ex["cache"], dtype=np.float32)
    pos = np.asarray(ex["positions"], dtype=np.int64)
    rq, rk = O.qk_layernorm_rope_io(q, k, bits(ex["wq"]), bits(ex["wk"]),
                                    bits(ex["bq"]) if bias else None,
                                    bits(ex["bk"]) if bias else None, cache, pos,
                                    is_neox=neox, eps=ex["eps"], dtype=dtype,
                                    rope_dim=ex["rope_dim"])
    key = ("neox" if neox else "interleaved") + ("" if bias else "_no_bias")
    np.testing.assert_array_equal(dec(rq).reshape(D), ex[f"out_q_{key}"])
    np.testing.assert_array_equal(dec(rk).reshape(D), ex[f"out_k_{key}"])


def test_layernorm_io_entry_rounds_once_and_routes_rows():
    """The I/O entry against the fp64 composition on random heads: Q rows get
    wq and bq, K rows wk and bk, one correct rounding (bf16 by torch's
    round-to-nearest-even from a float64 that is exact in float32)."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(31)
    T, Hq, Hkv, D, R = 7, 3, 2, 32, 16
    enc = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    dec = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    q, k = enc(g.standard_normal((T, Hq, D))), enc(g.standard_normal((T, Hkv, D)))
    wq, wk = enc(g.uniform(0.5, 1.5, D)), enc(g.uniform(-1.5, -0.5, D))
    bq, bk = enc(g.standard_normal(D)), enc(g.standard_normal(D) + 4.0)
    cache = _cache_formula(20, R)
    pos = g.integers(0, 20, T)
    for neox in (False, True):
        rq, rk = O.qk_layernorm_rope_io(q, k, wq, wk, bq, bk, cache, pos, is_neox=neox,
                                        eps=1e-5, dtype="bf16", rope_dim=R)
        fq, fk = O.qk_layernorm_rope(dec(q), dec(k), dec(wq), dec(wk), dec(bq), dec(bk), cache,
                                     pos, is_neox=neox, eps=1e-5, rope_dim=R)
        for got, f in ((rq, fq), (rk, fk)):
            # float64 -> float32 is exact for all but a few values; where it is not,
            # allow the one-ulp difference of a double rounding
            f32 = f.astype(np.float32)
            want = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            exact = f32.astype(np.float64) == f
            np.testing.assert_array_equal(got[exact], want[exact])
            assert np.all(np.abs(dec(got) - f) <= np.abs(f) * 2.0 ** -8 + 1e-30)
