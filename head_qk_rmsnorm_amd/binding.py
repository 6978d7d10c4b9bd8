"""Python binding of libqknr.so: argument marshalling only.

Every step of the op runs in the HIP kernels behind the C ABI declared in
``include/qknr.h``; this module turns torch tensors into pointers, sizes,
byte strides, dtype codes and the current HIP stream, and raises on a non-zero
status. torch provides device memory and streams, nothing else. There is no
fallback: if the library is missing or rejects the call, an exception is raised.

Names mirror the C entry points (``qknr_inplace``, ``qknr_inplace_ex``,
``qknr_can_use``, ``qknr_status_string``, the unfused baseline
``qknr_rmsnorm_inplace`` / ``qknr_rope_inplace`` / ``qknr_unfused_inplace``, the
LayerNorm sibling ``qknr_layernorm_rope_inplace`` / ``qknr_layernorm_rope_inplace_ex``,
and the measurement aids ``qknr_copy`` / ``qknr_rmw``), plus ``fused_inplace_qknorm_rope``
with the signature of the op on the page "SGLang Diffusion fused operator
fused_inplace_qknorm_rope: in-depth technical analysis" (m.lsln.cn/news/241376),
section 5.3: q and k are modified in place and nothing is returned.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqknr.so")

QKNR_OK = 0
QKNR_E_NULL = -1
QKNR_E_SHAPE = -2
QKNR_E_UNSUPPORTED = -3
QKNR_E_ALIGN = -4
QKNR_E_DTYPE = -5
QKNR_E_ARG = -6
QKNR_E_LAUNCH = -7
QKNR_E_DEVICE = -8
QKNR_BF16, QKNR_FP16 = 0, 1
QKNR_I32, QKNR_I64 = 0, 1


class LaunchCfg(ctypes.Structure):
    """qknr_launch_cfg: zero fields mean automatic."""

    _fields_ = [("lanes_per_head", ctypes.c_int32), ("groups_per_item", ctypes.c_int32),
                ("unroll", ctypes.c_int32), ("block_waves", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("generic", ctypes.c_int32)]


class LaunchInfo(ctypes.Structure):
    """qknr_launch_info: what a call launched."""

    _fields_ = [("lanes_per_head", ctypes.c_int32), ("elems_per_lane", ctypes.c_int32),
                ("heads_per_wave", ctypes.c_int32), ("groups_per_token", ctypes.c_int32),
                ("groups_per_item", ctypes.c_int32), ("unroll", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("grid_blocks", ctypes.c_int32),
                ("items", ctypes.c_int64), ("generic", ctypes.c_int32),
                ("access_bytes", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
INPLACE_ARGTYPES = [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                    _I64, _I64, _I64, _I64, _I32, _I32, _P]

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libqknr.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m head_qk_rmsnorm_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            L.qknr_inplace.argtypes = INPLACE_ARGTYPES
            L.qknr_inplace.restype = _I32
            L.qknr_inplace_ex.argtypes = INPLACE_ARGTYPES + [ctypes.POINTER(LaunchCfg),
                                                             ctypes.POINTER(LaunchInfo)]
            L.qknr_inplace_ex.restype = _I32
            L.qknr_can_use.argtypes = [_I32, _I32, _I32, _I32, _I32]
            L.qknr_can_use.restype = _I32
            L.qknr_status_string.argtypes = [_I32]
            L.qknr_status_string.restype = ctypes.c_char_p
            L.qknr_unfused_inplace.argtypes = INPLACE_ARGTYPES
            L.qknr_unfused_inplace.restype = _I32
            L.qknr_rmsnorm_inplace.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _I32,
                                               ctypes.c_float, _I64, _I64, _I64, _I64, _I32, _P]
            L.qknr_rmsnorm_inplace.restype = _I32
            L.qknr_rope_inplace.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32,
                                            _I64, _I64, _I64, _I64, _I32, _I32, _P]
            L.qknr_rope_inplace.restype = _I32
            L.qknr_layernorm_rope_inplace.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32,
                                                      _I32, _I32, _I32, _I32, ctypes.c_float,
                                                      _I64, _I64, _I64, _I64, _I32, _I32, _P]
            L.qknr_layernorm_rope_inplace.restype = _I32
            L.qknr_layernorm_rope_inplace_ex.argtypes = (
                L.qknr_layernorm_rope_inplace.argtypes
                + [ctypes.POINTER(LaunchCfg), ctypes.POINTER(LaunchInfo)])
            L.qknr_layernorm_rope_inplace_ex.restype = _I32
            L.qknr_copy.argtypes = [_P, _P, _I64, _P]
            L.qknr_copy.restype = _I32
            L.qknr_rmw.argtypes = [_P, _I64, ctypes.c_uint32, _P]
            L.qknr_rmw.restype = _I32
            _lib = L
    return _lib


def qknr_status_string(status: int) -> str:
    return lib().qknr_status_string(int(status)).decode()


def qknr_can_use(head_dim: int, rope_dim: int, is_neox: bool, dtype=None, pos_dtype=None) -> bool:
    """The capability predicate; dtype / pos_dtype accept torch dtypes or codes
    (default bf16 / int32)."""
    return bool(lib().qknr_can_use(int(head_dim), int(rope_dim), int(bool(is_neox)),
                                   _dtype_code(dtype) if dtype is not None else QKNR_BF16,
                                   _pos_code(pos_dtype) if pos_dtype is not None else QKNR_I32))


def _dtype_code(dt) -> int:
    import torch

    if isinstance(dt, int):
        return dt
    if dt == torch.bfloat16:
        return QKNR_BF16
    if dt == torch.float16:
        return QKNR_FP16
    raise TypeError(f"q/k dtype must be bfloat16 or float16, got {dt}")


def _pos_code(dt) -> int:
    import torch

    if isinstance(dt, int):
        return dt
    if dt == torch.int32:
        return QKNR_I32
    if dt == torch.int64:
        return QKNR_I64
    raise TypeError(f"positions dtype must be int32 or int64, got {dt}")


def _check(rc: int) -> None:
    if rc != QKNR_OK:
        raise RuntimeError(qknr_status_string(rc))


def _on_device(ref, **named):
    """Every named tensor is a torch tensor on ref's HIP device."""
    import torch

    for name, t in named.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, q on {ref.device}")


def _qk(q, k, head_dim):
    """q [T,Hq,D], k [T,Hkv,D] -> pointers, sizes, byte strides, dtype code."""
    _on_device(q, q=q, k=k)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [T, Hq, D] and k [T, Hkv, D]")
    D = int(head_dim) or int(q.size(-1))
    T = int(q.size(0))
    if q.size(-1) != D or k.size(-1) != D or k.size(0) != T:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree with head_dim={D}")
    if (q.numel() and q.stride(2) != 1) or (k.numel() and k.stride(2) != 1):
        raise ValueError("the innermost (head_dim) stride of q and k must be 1")
    if k.dtype != q.dtype:
        raise TypeError("q and k must share one dtype")
    es = q.element_size()
    return dict(q=ctypes.c_void_p(q.data_ptr()), k=ctypes.c_void_p(k.data_ptr()), T=T,
                Hq=int(q.size(1)), Hkv=int(k.size(1)), D=D, qt=int(q.stride(0)) * es,
                qh=int(q.stride(1)) * es, kt=int(k.stride(0)) * es, kh=int(k.stride(1)) * es,
                dtype=_dtype_code(q.dtype))


def _weights(q, q_weight, k_weight, D):
    _on_device(q, q_weight=q_weight, k_weight=k_weight)
    if q_weight.dtype != q.dtype or k_weight.dtype != q.dtype:
        raise TypeError("q_weight and k_weight must have the dtype of q and k")
    if tuple(q_weight.shape) != (D,) or tuple(k_weight.shape) != (D,) \
            or not q_weight.is_contiguous() or not k_weight.is_contiguous():
        raise ValueError(f"weights must be contiguous [{D}]")
    return ctypes.c_void_p(q_weight.data_ptr()), ctypes.c_void_p(k_weight.data_ptr())


def _rotation(q, cos_sin_cache, positions, T, rope_dim):
    import torch

    _on_device(q, cos_sin_cache=cos_sin_cache, positions=positions)
    R = int(rope_dim) or int(cos_sin_cache.size(-1))
    if cos_sin_cache.dtype != torch.float32 or cos_sin_cache.dim() != 2 \
            or cos_sin_cache.size(1) != R or not cos_sin_cache.is_contiguous():
        raise ValueError(f"cos_sin_cache must be a contiguous float32 [rows, {R}] table")
    if positions.dim() != 1 or positions.size(0) != T or not positions.is_contiguous():
        raise ValueError(f"positions must be a contiguous [{T}] vector")
    return (ctypes.c_void_p(cos_sin_cache.data_ptr()), ctypes.c_void_p(positions.data_ptr()), R,
            _pos_code(positions.dtype))


def _marshal(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox, eps, head_dim,
             rope_dim):
    """All arguments of qknr_inplace except the stream, in ABI order."""
    v = _qk(q, k, head_dim)
    wq, wk = _weights(q, q_weight, k_weight, v["D"])
    cache, pos, R, pcode = _rotation(q, cos_sin_cache, positions, v["T"], rope_dim)
    return (v["q"], v["k"], wq, wk, cache, pos, v["T"], v["Hq"], v["Hkv"], v["D"], R,
            int(bool(is_neox)), float(eps), v["qt"], v["qh"], v["kt"], v["kh"], v["dtype"], pcode)


def _stream_of(q, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def qknr_inplace(q, k, q_weight, k_weight, cos_sin_cache, positions, *, is_neox: bool,
                 eps: float = 1e-6, head_dim: int = 0, rope_dim: int = 0, stream=None) -> None:
    """Fused QK RMSNorm + RoPE, in place on q [T,Hq,D] and k [T,Hkv,D] (any
    strides with a unit innermost stride), enqueued on ``stream`` (default: the
    current torch stream of q's device)."""
    import torch

    args = _marshal(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox, eps,
                    head_dim, rope_dim)
    with torch.cuda.device(q.device):
        _check(lib().qknr_inplace(*args, _stream_of(q, stream)))


def qknr_inplace_ex(q, k, q_weight, k_weight, cos_sin_cache, positions, *, is_neox: bool,
                    eps: float = 1e-6, head_dim: int = 0, rope_dim: int = 0, stream=None,
                    launch: Optional[dict] = None) -> dict:
    """qknr_inplace with an explicit launch configuration (keys of LaunchCfg);
    returns what was launched (LaunchInfo as a dict)."""
    import torch

    args = _marshal(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox, eps,
                    head_dim, rope_dim)
    cfg = LaunchCfg(**(launch or {}))
    info = LaunchInfo()
    with torch.cuda.device(q.device):
        _check(lib().qknr_inplace_ex(*args, _stream_of(q, stream), ctypes.byref(cfg),
                                     ctypes.byref(info)))
    return info.as_dict()


def qknr_unfused_inplace(q, k, q_weight, k_weight, cos_sin_cache, positions, *,
                         is_neox: bool, eps: float = 1e-6, head_dim: int = 0, rope_dim: int = 0,
                         stream=None) -> None:
    """The two-launch baseline (RMSNorm step, intermediate rounded to the I/O
    type, then RoPE step); same arguments and result layout as qknr_inplace."""
    import torch

    args = _marshal(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox, eps,
                    head_dim, rope_dim)
    with torch.cuda.device(q.device):
        _check(lib().qknr_unfused_inplace(*args, _stream_of(q, stream)))


def qknr_rmsnorm_inplace(q, k, q_weight, k_weight, *, eps: float = 1e-6, stream=None) -> None:
    """The norm step alone, in place on q [T,Hq,D] and k [T,Hkv,D]."""
    import torch

    v = _qk(q, k, 0)
    wq, wk = _weights(q, q_weight, k_weight, v["D"])
    with torch.cuda.device(q.device):
        _check(lib().qknr_rmsnorm_inplace(v["q"], v["k"], wq, wk, v["T"], v["Hq"], v["Hkv"], v["D"],
                                          float(eps), v["qt"], v["qh"], v["kt"], v["kh"],
                                          v["dtype"], _stream_of(q, stream)))


def qknr_rope_inplace(q, k, cos_sin_cache, positions, *, is_neox: bool, rope_dim: int = 0,
                      stream=None) -> None:
    """The rotation step alone (no norm), in place on q and k."""
    import torch

    v = _qk(q, k, 0)
    cache, pos, R, pcode = _rotation(q, cos_sin_cache, positions, v["T"], rope_dim)
    with torch.cuda.device(q.device):
        _check(lib().qknr_rope_inplace(v["q"], v["k"], cache, pos, v["T"], v["Hq"], v["Hkv"], v["D"],
                                       R, int(bool(is_neox)), v["qt"], v["qh"], v["kt"], v["kh"],
                                       v["dtype"], pcode, _stream_of(q, stream)))


def qknr_layernorm_rope_inplace(q, k, q_weight, k_weight, q_bias=None, k_bias=None,
                                cos_sin_cache=None, positions=None, *, is_neox: bool = False,
                                eps: float = 1e-6, rope_dim: int = 0, stream=None) -> None:
    """Per-head QK LayerNorm (weight, optional bias) of q and k in place, then the
    rotation of the first rope_dim dims when a cos|sin cache is given."""
    import torch

    v = _qk(q, k, 0)
    wq, wk = _weights(q, q_weight, k_weight, v["D"])
    bq = bk = ctypes.c_void_p(0)
    if (q_bias is None) != (k_bias is None):
        raise ValueError("give both biases or neither")
    if q_bias is not None:
        bq, bk = _weights(q, q_bias, k_bias, v["D"])
    cache = pos = ctypes.c_void_p(0)
    R, pcode = 0, QKNR_I32
    if cos_sin_cache is not None:
        cache, pos, R, pcode = _rotation(q, cos_sin_cache, positions, v["T"], rope_dim)
    with torch.cuda.device(q.device):
        _check(lib().qknr_layernorm_rope_inplace(
            v["q"], v["k"], wq, wk, bq, bk, cache, pos, v["T"], v["Hq"], v["Hkv"], v["D"], R,
            int(bool(is_neox)), float(eps), v["qt"], v["qh"], v["kt"], v["kh"], v["dtype"], pcode,
            _stream_of(q, stream)))


def qknr_layernorm_rope_inplace_ex(q, k, q_weight, k_weight, q_bias=None, k_bias=None,
                                   cos_sin_cache=None, positions=None, *, is_neox: bool = False,
                                   eps: float = 1e-6, rope_dim: int = 0, stream=None,
                                   launch: Optional[dict] = None) -> dict:
    """qknr_layernorm_rope_inplace with an explicit launch configuration (keys of
    LaunchCfg); returns what was launched (LaunchInfo as a dict)."""
    import torch

    v = _qk(q, k, 0)
    wq, wk = _weights(q, q_weight, k_weight, v["D"])
    bq = bk = ctypes.c_void_p(0)
    if (q_bias is None) != (k_bias is None):
        raise ValueError("give both biases or neither")
    if q_bias is not None:
        bq, bk = _weights(q, q_bias, k_bias, v["D"])
    cache = pos = ctypes.c_void_p(0)
    R, pcode = 0, QKNR_I32
    if cos_sin_cache is not None:
        cache, pos, R, pcode = _rotation(q, cos_sin_cache, positions, v["T"], rope_dim)
    cfg = LaunchCfg(**(launch or {}))
    info = LaunchInfo()
    with torch.cuda.device(q.device):
        _check(lib().qknr_layernorm_rope_inplace_ex(
            v["q"], v["k"], wq, wk, bq, bk, cache, pos, v["T"], v["Hq"], v["Hkv"], v["D"], R,
            int(bool(is_neox)), float(eps), v["qt"], v["qh"], v["kt"], v["kh"], v["dtype"], pcode,
            _stream_of(q, stream), ctypes.byref(cfg), ctypes.byref(info)))
    return info.as_dict()


def fused_inplace_qknorm_rope(q, k, q_weight, k_weight, cos_sin_cache, positions, *,
                              is_neox: bool, eps: float = 1e-6, head_dim: int = 0,
                              rope_dim: int = 0) -> None:
    """The op under the name and signature the page gives it (section 5.3):
    head_dim defaults to q.size(-1), rope_dim to cos_sin_cache.size(-1)."""
    qknr_inplace(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox=is_neox, eps=eps,
                 head_dim=head_dim, rope_dim=rope_dim)


def qknr_copy(dst, src, nbytes: int, stream=None) -> None:
    """Measurement aid: copy nbytes from src to dst (tensors) on the stream."""
    import torch

    with torch.cuda.device(dst.device):
        _check(lib().qknr_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                               int(nbytes), _stream_of(dst, stream)))


def qknr_rmw(buf, nbytes: int, key: int = 0, stream=None) -> None:
    """Measurement aid: in-place read, XOR with key, write back (key 0 keeps data)."""
    import torch

    with torch.cuda.device(buf.device):
        _check(lib().qknr_rmw(ctypes.c_void_p(buf.data_ptr()), int(nbytes), int(key) & 0xFFFFFFFF,
                              _stream_of(buf, stream)))


class PreparedCall:
    """A qknr_inplace call with its arguments marshalled once (pointers, sizes,
    strides, stream). Calling it re-enqueues the same launch; it is meant for
    loops that launch on the same tensors many times (benchmarks), where the
    per-call Python checks would otherwise cost more than the kernel. q's
    device must be the current device when it is called."""

    def __init__(self, q, k, q_weight, k_weight, cos_sin_cache, positions, *, is_neox: bool,
                 eps: float = 1e-6, head_dim: int = 0, rope_dim: int = 0, stream=None,
                 launch: Optional[dict] = None, unfused: bool = False,
                 layernorm_bias: Optional[tuple] = None):
        """``unfused=True`` prepares the two-launch baseline; ``layernorm_bias=(bq, bk)``
        prepares the LayerNorm sibling (with rotation) instead of the fused op."""
        self._keep = (q, k, q_weight, k_weight, cos_sin_cache, positions, layernorm_bias)
        self._device = q.device
        args = _marshal(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox, eps,
                        head_dim, rope_dim)
        self._cfg = LaunchCfg(**(launch or {}))
        self.info = LaunchInfo()
        if unfused and launch:
            raise ValueError("the unfused pair takes no launch configuration")
        if unfused:
            self._args = args + (_stream_of(q, stream),)
            self._fn = lib().qknr_unfused_inplace
        elif layernorm_bias is not None:
            bq, bk = _weights(q, layernorm_bias[0], layernorm_bias[1], int(args[9]))
            self._args = args[:4] + (bq, bk) + args[4:] + (_stream_of(q, stream),
                                                          ctypes.byref(self._cfg),
                                                          ctypes.byref(self.info))
            self._fn = lib().qknr_layernorm_rope_inplace_ex
        else:
            self._args = args + (_stream_of(q, stream), ctypes.byref(self._cfg),
                                 ctypes.byref(self.info))
            self._fn = lib().qknr_inplace_ex

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != QKNR_OK:
            raise RuntimeError(qknr_status_string(rc))
