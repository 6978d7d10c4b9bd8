"""fp64 CPU oracle for the fused in-place QK RMSNorm + rotary position embedding.

TEST INFRASTRUCTURE. Only the tests, the smoke check of ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run this module. The
product path (the HIP library and its Python binding) never calls it and
shares no code with it: this file imports numpy only.

What it computes follows the page "SGLang Diffusion fused operator
fused_inplace_qknorm_rope: in-depth technical analysis" (m.lsln.cn/news/241376).
Its formulas lost their ``=``, ``+`` and ``<`` signs in extraction; the readings
taken are the only ones consistent with the page's kernel walk-through:

* section 2.1 (QK RMSNorm): ``rms(x) = sqrt(mean_i x_i^2 + eps)``, the mean
  taken over all ``head_dim`` entries, and ``out_i = x_i / rms(x) * w_i`` with a
  learned per-channel weight ``w`` of length ``head_dim`` (plain ``w``, not ``1+w``);
* section 2.2 (RoPE): a cache row for position p is
  ``[cos(p*theta_0) .. cos(p*theta_{R/2-1}) | sin(p*theta_0) .. sin(p*theta_{R/2-1})]``;
  interleaved (GPT-J) pairing rotates ``(2j, 2j+1)``, NeoX pairing rotates
  ``(j, j+R/2)``, each pair by the angle of index j, with
  ``a' = a*cos_j - b*sin_j`` and ``b' = b*cos_j + a*sin_j``; partial RoPE rotates
  only the first R = rope_dim dims and leaves the rest as they are;
* section 2.3 (fused per-head flow): load, widen, sum of squares, scale by
  rsqrt(sum/head_dim + eps), multiply by w on every dim, rotate the first R dims,
  store in place -- no rounding between the norm and the rotation;
* section 3 (I/O contract): q ``[T, Hq, D]``, k ``[T, Hkv, D]`` (GQA allowed),
  weights ``[D]`` per Q and per K, the fp32 cache ``[rows, R]`` indexed by
  ``positions[t]``.

Everything is evaluated in float64; the only rounding to the I/O precision is
the final one (round to nearest, ties to even), done once and correctly from
the fp64 value. Parity pins for every function live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16", "decode_fp16", "decode_io", "round_to_bf16_bits", "round_to_fp16_bits",
    "round_to_io_bits", "rms_norm", "rope", "cache_cos_sin", "qknorm_rope",
    "qknorm_rope_io", "rms_norm_io", "rope_io", "qknorm_rope_unfused_io",
    "layer_norm", "qk_layernorm_rope", "qk_layernorm_rope_io",
    "within_tolerance", "tolerance",
]


# ----------------------------------------------------------------------------
# I/O formats (section 3: q/k and the weights are fp16 or bf16)
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64. Exact: a bf16 is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_io(bits: np.ndarray, dtype: str) -> np.ndarray:
    return decode_bf16(bits) if dtype == "bf16" else decode_fp16(bits)


def _f64_to_f32_round_to_odd(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 with rounding to odd: exact values stay, inexact ones
    go to whichever fp32 neighbour has an odd last mantissa bit.

    Rounding to odd into a format with at least two more bits than the final
    one makes a second round-to-nearest-even exact (Boldo and Melquiond,
    "Emulation of FMA and correctly rounded sums: proved algorithms using
    rounding to odd", IEEE Trans. Computers 57(4), 2008)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    back = f.astype(np.float64)
    inexact = back != x
    even = (f.view(np.uint32) & np.uint32(1)) == 0
    toward = np.where(back < x, np.float32(np.inf), np.float32(-np.inf))
    return np.where(inexact & even, np.nextafter(f, toward), f).astype(np.float32)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest, ties to even, from the
    fp64 value itself (one correct rounding). Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16_bits: non-finite input")
    u = _f64_to_f32_round_to_odd(x).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def round_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> fp16 bit patterns (numpy's direct double -> half conversion,
    round to nearest, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_fp16_bits: non-finite input")
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def round_to_io_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16_bits(x) if dtype == "bf16" else round_to_fp16_bits(x)


# ----------------------------------------------------------------------------
# The method (sections 2.1 - 2.3)
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Section 2.1: per head vector (last axis, length head_dim),
    x / sqrt(sum(x^2)/head_dim + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if eps < 0:
        raise ValueError("eps must be >= 0")
    head_dim = x.shape[-1]
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / head_dim
    r = 1.0 / np.sqrt(mean_sq + eps)
    return x * r * w


def rope(n: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int,
         is_neox: bool) -> np.ndarray:
    """Section 2.2: rotate the first ``rope_dim`` dims of the last axis.

    ``cos``/``sin`` hold the R/2 angle values of the pair index j and broadcast
    against ``n[..., :R/2]``. Interleaved pairs are (2j, 2j+1); NeoX pairs are
    (j, j + R/2). Dims from ``rope_dim`` on are returned unchanged."""
    n = np.asarray(n, dtype=np.float64)
    R = int(rope_dim)
    if R <= 0 or R % 2 or R > n.shape[-1]:
        raise ValueError("rope_dim must be even and in (0, head_dim]")
    half = R // 2
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    out = n.copy()
    if is_neox:
        a, b = n[..., :half], n[..., half:R]
        out[..., :half] = a * cos - b * sin
        out[..., half:R] = b * cos + a * sin
    else:
        a, b = n[..., 0:R:2], n[..., 1:R:2]
        out[..., 0:R:2] = a * cos - b * sin
        out[..., 1:R:2] = b * cos + a * sin
    return out


def cache_cos_sin(cache: np.ndarray, positions: np.ndarray, rope_dim: int):
    """Section 2.2 / section 3: row ``positions[t]`` of the fp32 table; its first
    R/2 entries are cos values and the next R/2 are sin values."""
    cache = np.asarray(cache)
    if cache.ndim != 2 or cache.shape[1] < rope_dim:
        raise ValueError("cache must be [rows, >= rope_dim]")
    p = np.asarray(positions).astype(np.int64)
    if p.size and (p.min() < 0 or p.max() >= cache.shape[0]):
        raise ValueError("position outside the cache table")
    half = rope_dim // 2
    row = cache[p].astype(np.float64)
    return row[:, :half], row[:, half:rope_dim]


def qknorm_rope(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray,
                cache: np.ndarray, positions: np.ndarray, *, is_neox: bool,
                eps: float, rope_dim: int | None = None):
    """Section 2.3, applied to every (token, head) of q ``[T,Hq,D]`` and
    k ``[T,Hkv,D]`` (values already decoded to float64). Returns the two fp64
    results; the inputs are not modified."""
    R = int(cache.shape[-1] if rope_dim is None else rope_dim)
    # eps reaches the kernel as an fp32 value.
    eps64 = float(np.float32(eps))
    cos, sin = cache_cos_sin(cache, positions, R)
    cos, sin = cos[:, None, :], sin[:, None, :]
    out_q = rope(rms_norm(q, wq, eps64), cos, sin, R, is_neox)
    out_k = rope(rms_norm(k, wk, eps64), cos, sin, R, is_neox)
    return out_q, out_k


def qknorm_rope_io(q_bits, k_bits, wq_bits, wk_bits, cache, positions, *, is_neox,
                   eps, dtype, rope_dim=None):
    """The op on I/O bit patterns: decode exactly, compute in fp64, round once
    to the I/O format. Returns (q_ref_bits, k_ref_bits, q_ref_f64, k_ref_f64)
    where the fp64 arrays are the decoded rounded values."""
    q = decode_io(q_bits, dtype)
    k = decode_io(k_bits, dtype)
    oq, ok = qknorm_rope(q, k, decode_io(wq_bits, dtype), decode_io(wk_bits, dtype),
                         cache, positions, is_neox=is_neox, eps=eps, rope_dim=rope_dim)
    rq, rk = round_to_io_bits(oq, dtype), round_to_io_bits(ok, dtype)
    return rq, rk, decode_io(rq, dtype), decode_io(rk, dtype)


# ----------------------------------------------------------------------------
# The unfused chain the fused op replaces (section 2.4 table, section 6
# fallback): an RMSNorm step that writes its result to memory in the I/O
# type, then a RoPE step that reads it back, rotates and writes it again.
# Each step rounds its own output once.
# ----------------------------------------------------------------------------

def rms_norm_io(x_bits, w_bits, *, eps, dtype):
    """Section 2.1 alone on I/O bit patterns [..., D]: decode, fp64 norm with
    eps as an fp32 value, one rounding to the I/O type."""
    n = rms_norm(decode_io(x_bits, dtype), decode_io(w_bits, dtype), float(np.float32(eps)))
    return round_to_io_bits(n, dtype)


def rope_io(x_bits, cache, positions, *, is_neox, dtype, rope_dim=None):
    """Section 2.2 alone on I/O bit patterns [T, H, D]: decode, rotate the first
    rope_dim dims with row positions[t] of the cache, one rounding."""
    R = int(cache.shape[-1] if rope_dim is None else rope_dim)
    cos, sin = cache_cos_sin(cache, positions, R)
    out = rope(decode_io(x_bits, dtype), cos[:, None, :], sin[:, None, :], R, is_neox)
    return round_to_io_bits(out, dtype)


def qknorm_rope_unfused_io(q_bits, k_bits, wq_bits, wk_bits, cache, positions, *, is_neox,
                           eps, dtype, rope_dim=None):
    """RMSNorm step then RoPE step, the intermediate rounded to the I/O type.
    Returns (q_bits, k_bits)."""
    nq = rms_norm_io(q_bits, wq_bits, eps=eps, dtype=dtype)
    nk = rms_norm_io(k_bits, wk_bits, eps=eps, dtype=dtype)
    return (rope_io(nq, cache, positions, is_neox=is_neox, dtype=dtype, rope_dim=rope_dim),
            rope_io(nk, cache, positions, is_neox=is_neox, dtype=dtype, rope_dim=rope_dim))


# ----------------------------------------------------------------------------
# Sibling: per-head QK LayerNorm (the SGLang "Kernel Design Agent (KDA)"
# kernel-directory article, FLUX.2 fused producers: a per-head LayerNorm of Q
# and K that reproduces torch's layer_norm). Read here as
# (x - mean) / sqrt(var + eps) * w + b over head_dim, biased variance, bias
# optional, optionally followed by the same rotation as the fused op.
# ----------------------------------------------------------------------------

def layer_norm(x: np.ndarray, w: np.ndarray, b, eps: float) -> np.ndarray:
    """Per head vector (last axis): (x - mean) / sqrt(mean((x - mean)^2) + eps) * w + b."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if eps < 0:
        raise ValueError("eps must be >= 0")
    head_dim = x.shape[-1]
    mean = np.sum(x, axis=-1, keepdims=True) / head_dim
    c = x - mean
    var = np.sum(c * c, axis=-1, keepdims=True) / head_dim
    out = c / np.sqrt(var + eps) * w
    if b is not None:
        out = out + np.asarray(b, dtype=np.float64)
    return out


def qk_layernorm_rope(q, k, wq, wk, bq, bk, cache, positions, *, is_neox, eps, rope_dim):
    """Per-head LayerNorm of q [T,Hq,D] and k [T,Hkv,D], then (rope_dim > 0)
    the rotation of the first rope_dim dims by row positions[t]."""
    eps64 = float(np.float32(eps))
    nq = layer_norm(q, wq, bq, eps64)
    nk = layer_norm(k, wk, bk, eps64)
    if not rope_dim:
        return nq, nk
    cos, sin = cache_cos_sin(cache, positions, rope_dim)
    cos, sin = cos[:, None, :], sin[:, None, :]
    return rope(nq, cos, sin, rope_dim, is_neox), rope(nk, cos, sin, rope_dim, is_neox)


def qk_layernorm_rope_io(q_bits, k_bits, wq_bits, wk_bits, bq_bits, bk_bits, cache, positions,
                         *, is_neox, eps, dtype, rope_dim):
    """The LayerNorm sibling on I/O bit patterns (bias bits may be None): decode,
    fp64, one rounding. Returns (q_bits, k_bits)."""
    dec = lambda b: None if b is None else decode_io(b, dtype)
    oq, ok = qk_layernorm_rope(decode_io(q_bits, dtype), decode_io(k_bits, dtype),
                               dec(wq_bits), dec(wk_bits), dec(bq_bits), dec(bk_bits), cache,
                               positions, is_neox=is_neox, eps=eps, rope_dim=rope_dim)
    return round_to_io_bits(oq, dtype), round_to_io_bits(ok, dtype)


# ----------------------------------------------------------------------------
# Acceptance: |gpu - ref| <= 2^-7 * (|ref| + 1), elementwise, no NaN
# ----------------------------------------------------------------------------

def tolerance(ref: np.ndarray) -> np.ndarray:
    return np.ldexp(1.0, -7) * (np.abs(ref) + 1.0)


def within_tolerance(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.isfinite(got) & (np.abs(got - ref) <= tolerance(ref))
