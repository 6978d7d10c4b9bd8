"""Seeded synthetic workloads for the fused in-place QK RMSNorm + RoPE op.

This module only *draws inputs*: Q/K activations, RMSNorm weights, the fp32
cos|sin cache table and the per-token positions. It holds none of the op's
arithmetic (no normalisation, no rotation, no output rounding), so the fp64
CPU oracle and the HIP path can both consume what it produces without sharing
any code with each other.

Shapes follow the tensor contract of the page "SGLang Diffusion fused operator
fused_inplace_qknorm_rope: in-depth technical analysis" (m.lsln.cn/news/241376),
section 3 (I/O contract):

* q ``[T, Hq, D]`` and k ``[T, Hkv, D]`` in fp16 or bf16, innermost stride 1;
* q_weight / k_weight ``[D]`` in the same dtype;
* cos_sin_cache ``[rows, R]`` fp32, each row ``[cos(p*theta_0..) | sin(p*theta_0..)]``
  with ``theta_j = base^(-2j/R)`` (section 2.2);
* positions ``[T]`` int32 or int64.

Half-precision values are carried on the host as ``uint16`` bit patterns
(numpy has no bfloat16). Values are drawn in fp64 from a PCG64 stream per
tensor and narrowed with torch's CPU cast, which is deterministic.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
I32 = "i32"
I64 = "i64"

# Stream ids of the per-tensor random streams.
_S_Q, _S_K, _S_WQ, _S_WK, _S_POS, _S_OUT_Q, _S_OUT_K, _S_QKV = range(8)


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shapes, pairing, dtypes and the value recipe."""

    name: str
    T: int
    Hq: int
    Hkv: int
    head_dim: int
    rope_dim: int
    is_neox: bool
    dtype: str  # BF16 | FP16
    pos_dtype: str  # I32 | I64
    eps: float
    cache_rows: int
    base: float
    x_std: float = 1.0
    positions: str = "arange"  # arange | perm | uniform | rows
    layout: str = "contiguous"  # contiguous | qkv (q,k strided views into [T,(Hq+2Hkv)*D])
    outlier_frac: float = 0.0  # fraction of (head, dim) channels scaled by outlier_scale
    outlier_scale: float = 1.0
    seed: int = 0

    @property
    def heads(self) -> int:
        return self.Hq + self.Hkv

    @property
    def units(self) -> int:
        """(token, head) vectors processed per launch."""
        return self.T * self.heads

    @property
    def io_bytes(self) -> int:
        return 2

    @property
    def pos_bytes(self) -> int:
        return 4 if self.pos_dtype == I32 else 8

    def algorithmic_bytes(self) -> int:
        """Bytes one launch must move: read+write every Q/K element once,
        one positions entry and one cos|sin row per token, both weight rows."""
        D, R = self.head_dim, self.rope_dim
        return (2 * self.units * D * self.io_bytes + self.T * self.pos_bytes
                + self.T * R * 4 + 2 * D * self.io_bytes)


# The five workloads: DiT image+text sequences (FLUX / Qwen-Image style,
# interleaved pairing) and LLaMA-style GQA prefill (NeoX pairing), plus a tiny
# case and the partial-rotary and large-head variants.
CONFIGS = {
    "tiny": Config("tiny", T=16, Hq=4, Hkv=4, head_dim=64, rope_dim=64, is_neox=True,
                   dtype=BF16, pos_dtype=I32, eps=1e-6, cache_rows=64, base=1e4,
                   positions="arange", seed=1),
    "dit": Config("dit", T=4608, Hq=24, Hkv=24, head_dim=128, rope_dim=128, is_neox=False,
                  dtype=BF16, pos_dtype=I64, eps=1e-6, cache_rows=4608, base=1e4,
                  x_std=2.0, positions="perm", seed=2),
    "gqa": Config("gqa", T=8192, Hq=32, Hkv=8, head_dim=128, rope_dim=128, is_neox=True,
                  dtype=BF16, pos_dtype=I32, eps=1e-6, cache_rows=8192, base=1e6,
                  positions="arange", layout="qkv", seed=3),
    "partial": Config("partial", T=16384, Hq=16, Hkv=16, head_dim=128, rope_dim=64,
                      is_neox=True, dtype=FP16, pos_dtype=I64, eps=1e-5, cache_rows=32768,
                      base=1e4, positions="uniform", seed=4),
    "large": Config("large", T=32768, Hq=24, Hkv=24, head_dim=256, rope_dim=256,
                    is_neox=False, dtype=BF16, pos_dtype=I32, eps=1e-6, cache_rows=32768,
                    base=1e4, positions="arange", outlier_frac=0.01, outlier_scale=50.0,
                    seed=5),
}
CONFIG_ORDER = ["tiny", "dit", "gqa", "partial", "large"]

# One GPU's share of a sharded run, at its real shape (every (token, head) is
# independent, so a shard is the same op on fewer tokens or fewer heads):
#   gqa_tp8  the GQA workload under 8-way tensor (head) parallelism: each GPU
#            holds 4 of the 32 Q heads and 1 of the 8 K heads, in its own qkv
#            shard [T, (4 + 2*1) * 128];
#   dit_hp8  the DiT workload after an 8-way head scatter (all tokens, 3 + 3 heads);
#   dit_sp8  the DiT workload under 8-way sequence parallelism: 576 of the 4608
#            tokens with their global positions (distinct rows of the full table).
CONFIGS.update({
    "gqa_tp8": Config("gqa_tp8", T=8192, Hq=4, Hkv=1, head_dim=128, rope_dim=128, is_neox=True,
                      dtype=BF16, pos_dtype=I32, eps=1e-6, cache_rows=8192, base=1e6,
                      positions="arange", layout="qkv", seed=13),
    "dit_hp8": Config("dit_hp8", T=4608, Hq=3, Hkv=3, head_dim=128, rope_dim=128,
                      is_neox=False, dtype=BF16, pos_dtype=I64, eps=1e-6, cache_rows=4608,
                      base=1e4, x_std=2.0, positions="perm", seed=12),
    "dit_sp8": Config("dit_sp8", T=576, Hq=24, Hkv=24, head_dim=128, rope_dim=128,
                      is_neox=False, dtype=BF16, pos_dtype=I64, eps=1e-6, cache_rows=4608,
                      base=1e4, x_std=2.0, positions="rows", seed=12),
})
SHARD_ORDER = ["gqa_tp8", "dit_hp8", "dit_sp8"]


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def to_io_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Narrow fp64 draws to fp16/bf16 bit patterns (uint16) with torch's CPU cast."""
    import torch

    tdt = torch.bfloat16 if dtype == BF16 else torch.float16
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64)).to(tdt)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rope_cache(rows: int, rope_dim: int, base: float) -> np.ndarray:
    """fp32 cos|sin table ``[rows, R]``: angles p*theta_j in fp64, one rounding to fp32."""
    if rope_dim % 2:
        raise ValueError("rope_dim must be even")
    half = rope_dim // 2
    ang = np.arange(rows, dtype=np.float64)[:, None] * theta(rope_dim, base)[None, :]
    out = np.empty((rows, rope_dim), dtype=np.float32)
    out[:, :half] = np.cos(ang)
    out[:, half:] = np.sin(ang)
    return out


@dataclasses.dataclass
class Workload:
    """Host-side inputs for one launch. q/k are [T,H,D] uint16 views; for the qkv
    layout they are strided views into ``qkv`` and ``v`` names the untouched slice."""

    cfg: Config
    q: np.ndarray
    k: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    cache: np.ndarray
    positions: np.ndarray
    qkv: Optional[np.ndarray] = None

    @property
    def v(self) -> Optional[np.ndarray]:
        if self.qkv is None:
            return None
        c = self.cfg
        return self.qkv[:, (c.Hq + c.Hkv) * c.head_dim:]


def _positions(cfg: Config, g: np.random.Generator) -> np.ndarray:
    npdt = np.int32 if cfg.pos_dtype == I32 else np.int64
    if cfg.positions == "arange":
        p = np.arange(cfg.T, dtype=np.int64)
    elif cfg.positions == "perm":
        p = g.permutation(cfg.T).astype(np.int64)
    elif cfg.positions == "uniform":
        p = g.integers(0, cfg.cache_rows, size=cfg.T, dtype=np.int64)
    elif cfg.positions == "rows":  # T distinct rows of the table (a shard of a permutation)
        p = g.permutation(cfg.cache_rows)[:cfg.T].astype(np.int64)
    else:
        raise ValueError(cfg.positions)
    if cfg.T and (p.min() < 0 or p.max() >= cfg.cache_rows):
        raise ValueError("positions outside the cache table")
    return p.astype(npdt)


def _activations(cfg: Config, stream: int, H: int) -> np.ndarray:
    g = rng(cfg.seed, stream)
    x = g.standard_normal((cfg.T, H, cfg.head_dim)) * cfg.x_std
    if cfg.outlier_frac > 0.0 and H > 0:
        n_ch = int(round(cfg.outlier_frac * H * cfg.head_dim))
        ch = g.choice(H * cfg.head_dim, size=n_ch, replace=False)
        x.reshape(cfg.T, H * cfg.head_dim)[:, ch] *= cfg.outlier_scale
    return to_io_bits(x, cfg.dtype)


def make_workload(cfg: Config) -> Workload:
    D = cfg.head_dim
    wq = to_io_bits(rng(cfg.seed, _S_WQ).uniform(0.5, 1.5, D), cfg.dtype)
    wk = to_io_bits(rng(cfg.seed, _S_WK).uniform(0.5, 1.5, D), cfg.dtype)
    cache = rope_cache(cfg.cache_rows, cfg.rope_dim, cfg.base)
    pos = _positions(cfg, rng(cfg.seed, _S_POS))
    if cfg.layout == "qkv":
        width = (cfg.Hq + 2 * cfg.Hkv) * D
        g = rng(cfg.seed, _S_QKV)
        qkv = to_io_bits(g.standard_normal((cfg.T, width)) * cfg.x_std, cfg.dtype)
        q = qkv[:, : cfg.Hq * D].reshape(cfg.T, cfg.Hq, D)
        k = qkv[:, cfg.Hq * D:(cfg.Hq + cfg.Hkv) * D].reshape(cfg.T, cfg.Hkv, D)
        return Workload(cfg, q, k, wq, wk, cache, pos, qkv=qkv)
    if cfg.layout != "contiguous":
        raise ValueError(cfg.layout)
    q = _activations(cfg, _S_Q, cfg.Hq)
    k = _activations(cfg, _S_K, cfg.Hkv)
    return Workload(cfg, q, k, wq, wk, cache, pos)


def case(T: int, Hq: int, Hkv: int, head_dim: int, rope_dim: int, is_neox: bool,
         dtype: str = BF16, pos_dtype: str = I32, eps: float = 1e-6, seed: int = 0,
         cache_rows: Optional[int] = None, base: float = 1e4, x_std: float = 1.0,
         positions: str = "uniform", layout: str = "contiguous",
         outlier_frac: float = 0.0, outlier_scale: float = 1.0) -> Config:
    """A small ad-hoc configuration (parity grids, edge cases)."""
    rows = cache_rows if cache_rows is not None else max(T, 1) * 2 + 7
    name = (f"T{T}_q{Hq}_k{Hkv}_D{head_dim}_R{rope_dim}_{'neox' if is_neox else 'il'}"
            f"_{dtype}_{pos_dtype}_{layout}")
    return Config(name, T=T, Hq=Hq, Hkv=Hkv, head_dim=head_dim, rope_dim=rope_dim,
                  is_neox=is_neox, dtype=dtype, pos_dtype=pos_dtype, eps=eps,
                  cache_rows=rows, base=base, x_std=x_std, positions=positions,
                  layout=layout, outlier_frac=outlier_frac, outlier_scale=outlier_scale,
                  seed=seed)


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    """Sorted distinct token indices for sampled checks at full size (always
    includes the first and the last token)."""
    if T <= n:
        return np.arange(T)
    g = rng(seed, 1000)
    pick = g.choice(T - 2, size=n - 2, replace=False) + 1
    return np.unique(np.concatenate([[0, T - 1], pick]))


def describe(cfg: Config) -> dict:
    d = dataclasses.asdict(cfg)
    d["units"] = cfg.units
    d["algorithmic_bytes"] = cfg.algorithmic_bytes()
    return d


def theta(rope_dim: int, base: float) -> np.ndarray:
    """Rotary frequencies theta_j = base^(-2j/R), j < R/2 (section 2.2)."""
    j = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / rope_dim)


__all__ = [
    "BF16", "FP16", "I32", "I64", "Config", "CONFIGS", "CONFIG_ORDER", "SHARD_ORDER", "Workload",
    "make_workload", "case", "rope_cache", "to_io_bits", "rng", "sample_tokens",
    "describe", "theta",
]
