"""Shared helpers of the GPU parity tests: put a workload on the device inside
storage with canary bands and padding, run the HIP op through the binding,
compare every Q/K element with the fp64 oracle and every other byte with its
value before the call."""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from head_qk_rmsnorm_amd import workloads as W
from oracle import qknr_oracle as O

CANARY = 4096  # bytes of 0xA5 before and after every storage buffer
CANARY_ELEMS = CANARY // 2


@dataclasses.dataclass
class View:
    """A [T, H, D] view into a storage buffer, strides in elements."""

    offset: int
    strides: Tuple[int, int, int]
    shape: Tuple[int, int, int]


def layout_views(T: int, Hq: int, Hkv: int, D: int, layout: str):
    """Storage size (elements, without canaries) and the q and k views of a layout.

    contiguous: q and k in two storages, [T, H, D] row-major (returned as two entries)
    padded:     [T, H, D] with 8 spare elements after each head and 16 after each token
    head_major: storage [H, T, D] seen as [T, H, D]
    qkv:        one storage [T, (Hq + 2*Hkv) * D]; q, k side by side, v untouched after them
    shifted:    contiguous [T, H, D] starting 3 elements (6 bytes) past a 16-byte boundary
    shifted4:   contiguous [T, H, D] starting 2 elements (4 bytes) past a 16-byte boundary
    odd_pad:    [T, H, D] with 1 spare element after each head and 1 after each token
                (strides of an odd number of elements)
    """
    if layout == "qkv":
        width = (Hq + 2 * Hkv) * D
        return [(T * width, [View(0, (width, D, 1), (T, Hq, D)),
                             View(Hq * D, (width, D, 1), (T, Hkv, D))])]
    out = []
    for H in (Hq, Hkv):
        if layout == "contiguous":
            out.append((T * H * D, [View(0, (H * D, D, 1), (T, H, D))]))
        elif layout == "padded":
            hs = D + 8
            ts = H * hs + 16
            out.append((T * ts, [View(0, (ts, hs, 1), (T, H, D))]))
        elif layout == "head_major":
            out.append((T * H * D, [View(0, (D, T * D, 1), (T, H, D))]))
        elif layout == "shifted":
            out.append((T * H * D + 3, [View(3, (H * D, D, 1), (T, H, D))]))
        elif layout == "shifted4":
            out.append((T * H * D + 2, [View(2, (H * D, D, 1), (T, H, D))]))
        elif layout == "odd_pad":
            hs = D + 1
            ts = H * hs + 1
            out.append((T * ts, [View(0, (ts, hs, 1), (T, H, D))]))
        else:
            raise ValueError(layout)
    return out


class DeviceCase:
    """Inputs of one call placed on the device, with host copies of everything."""

    def __init__(self, wl: W.Workload, layout: Optional[str] = None, device: str = "cuda:0",
                 fill_seed: int = 0, cache_offset: int = 0, w_offset: int = 0):
        import torch

        self.wl = wl
        c = wl.cfg
        self.cfg = c
        self.layout = layout or c.layout
        self.device = torch.device(device)
        tdt = torch.bfloat16 if c.dtype == W.BF16 else torch.float16
        self.tdt = tdt
        g = np.random.default_rng(fill_seed + 77)
        specs = layout_views(c.T, c.Hq, c.Hkv, c.head_dim, self.layout)
        self.storages_host: List[np.ndarray] = []
        self.masks: List[np.ndarray] = []
        self.views_dev = []
        src = [wl.q, wl.k]
        si = 0
        for n_elems, views in specs:
            host = np.full(n_elems + 2 * CANARY_ELEMS, 0xA5A5, dtype=np.uint16)
            # padding / untouched regions get random bits (NaN patterns included)
            host[CANARY_ELEMS:CANARY_ELEMS + n_elems] = g.integers(0, 1 << 16, n_elems,
                                                                   dtype=np.uint16)
            mask = np.zeros_like(host, dtype=bool)
            if self.layout == "qkv" and wl.qkv is not None:
                self._strided_full(host, c)[...] = wl.qkv  # v slice keeps the workload's values
            dev_views = []
            for v in views:
                hv = self._strided(host, v)
                mv = self._strided(mask, v)
                hv[...] = src[si]
                mv[...] = True
                si += 1
                dev_views.append(v)
            self.storages_host.append(host)
            self.masks.append(mask)
            self.views_dev.append(dev_views)
        self.storages_dev = [torch.from_numpy(h.view(np.int16)).to(self.device).view(tdt)
                             for h in self.storages_host]
        tensors = []
        for sd, views in zip(self.storages_dev, self.views_dev):
            for v in views:
                tensors.append(torch.as_strided(sd, v.shape, v.strides, CANARY_ELEMS + v.offset))
        self.q, self.k = tensors
        self.wq = torch.from_numpy(wl.wq.view(np.int16)).to(self.device).view(tdt)
        self.wk = torch.from_numpy(wl.wk.view(np.int16)).to(self.device).view(tdt)
        if w_offset:
            # each weight row as a view w_offset elements into its allocation
            # (aligned to 2 * w_offset bytes at most)
            def shifted(w):
                buf = torch.zeros(w.numel() + w_offset, dtype=tdt, device=self.device)
                view = buf[w_offset:]
                view.copy_(w)
                return view
            self.wq, self.wk = shifted(self.wq), shifted(self.wk)
        self.cache = torch.from_numpy(wl.cache).to(self.device)
        if cache_offset:
            # the table as a view cache_offset floats into its allocation (so
            # aligned to 4 or 8 bytes only), NaN in front of it
            buf = torch.full((self.cache.numel() + cache_offset,), float("nan"),
                             dtype=torch.float32, device=self.device)
            view = buf[cache_offset:].view(self.cache.shape)
            view.copy_(self.cache)
            self.cache = view
        self.positions = torch.from_numpy(wl.positions).to(self.device)

    @staticmethod
    def _strided(arr: np.ndarray, v: View) -> np.ndarray:
        es = arr.itemsize
        return np.lib.stride_tricks.as_strided(arr[CANARY_ELEMS + v.offset:], shape=v.shape,
                                               strides=tuple(s * es for s in v.strides))

    @staticmethod
    def _strided_full(arr: np.ndarray, c: W.Config) -> np.ndarray:
        width = (c.Hq + 2 * c.Hkv) * c.head_dim
        return arr[CANARY_ELEMS:CANARY_ELEMS + c.T * width].reshape(c.T, width)

    def run(self, launch: Optional[dict] = None, stream=None):
        from head_qk_rmsnorm_amd import binding as B

        c = self.cfg
        kw = dict(is_neox=c.is_neox, eps=c.eps, stream=stream)
        if launch is None:
            B.qknr_inplace(self.q, self.k, self.wq, self.wk, self.cache, self.positions, **kw)
            return None
        return B.qknr_inplace_ex(self.q, self.k, self.wq, self.wk, self.cache, self.positions,
                                 launch=launch, **kw)

    def fetch(self) -> List[np.ndarray]:
        import torch

        torch.cuda.synchronize(self.device)
        return [s.view(torch.int16).cpu().numpy().view(np.uint16) for s in self.storages_dev]

    def outputs(self, after: List[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
        vals = []
        for host, views in zip(after, self.views_dev):
            for v in views:
                vals.append(np.array(self._strided(host, v)))
        return vals[0], vals[1]

    def check_untouched(self, after: List[np.ndarray]) -> None:
        for before, now, mask in zip(self.storages_host, after, self.masks):
            diff = (before != now) & ~mask
            if np.any(diff):
                idx = np.nonzero(diff)[0][:8]
                raise AssertionError(f"bytes outside Q/K changed at element offsets {idx.tolist()}")

    def check_inputs_unchanged(self) -> None:
        import torch

        assert np.array_equal(self.wq.view(torch.int16).cpu().numpy().view(np.uint16), self.wl.wq)
        assert np.array_equal(self.wk.view(torch.int16).cpu().numpy().view(np.uint16), self.wl.wk)
        assert np.array_equal(self.cache.cpu().numpy(), self.wl.cache)
        assert np.array_equal(self.positions.cpu().numpy(), self.wl.positions)


def oracle_ref(wl: W.Workload, tokens: Optional[np.ndarray] = None, chunk: int = 1024,
               workers: int = 0):
    """Oracle output bits for all tokens, or for the given token subset. Large
    workloads are split into chunks of whole tokens that run on a thread pool
    (NumPy releases the GIL in its array loops); every token is computed by the
    same oracle call it would get in one piece, so the result does not depend
    on the chunking."""
    import concurrent.futures as cf
    import os

    c = wl.cfg
    q, k, pos = wl.q, wl.k, wl.positions
    if tokens is not None:
        q, k, pos = q[tokens], k[tokens], pos[tokens]
    T = q.shape[0]
    rq = np.empty_like(q)
    rk = np.empty_like(k)

    def run(start):
        sl = slice(start, min(start + chunk, T))
        a, b, _, _ = O.qknorm_rope_io(q[sl], k[sl], wl.wq, wl.wk, wl.cache, pos[sl],
                                      is_neox=c.is_neox, eps=c.eps, dtype=c.dtype,
                                      rope_dim=c.rope_dim)
        rq[sl] = a
        rk[sl] = b

    starts = range(0, T, chunk)
    if len(starts) <= 1:
        for s0 in starts:
            run(s0)
    else:
        n = workers or max(1, min(16, os.cpu_count() or 1))
        with cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(run, starts))
    return rq, rk


@dataclasses.dataclass
class Compare:
    n: int
    bad: int
    exact_frac: float
    max_abs_err: float
    max_ulps: int

    def __str__(self):
        return (f"n={self.n} bad={self.bad} exact={self.exact_frac:.5f} "
                f"max_abs={self.max_abs_err:.3g} max_ulps={self.max_ulps}")


def compare_bits(got: np.ndarray, ref: np.ndarray, dtype: str) -> Compare:
    g = O.decode_io(got, dtype)
    r = O.decode_io(ref, dtype)
    ok = O.within_tolerance(g, r)
    # distance in units of the last place, on the sign-magnitude integer line
    gi = got.astype(np.int64)
    ri = ref.astype(np.int64)
    gi = np.where(gi & 0x8000, -(gi & 0x7FFF), gi)
    ri = np.where(ri & 0x8000, -(ri & 0x7FFF), ri)
    ulps = np.abs(gi - ri)
    return Compare(n=int(got.size), bad=int(np.sum(~ok)), exact_frac=float(np.mean(got == ref))
                   if got.size else 1.0,
                   max_abs_err=float(np.max(np.abs(g - r))) if got.size else 0.0,
                   max_ulps=int(ulps.max()) if got.size else 0)


def run_and_check(wl: W.Workload, layout: Optional[str] = None, launch: Optional[dict] = None,
                  tokens: Optional[np.ndarray] = None, min_exact: float = 0.99,
                  stream=None, cache_offset: int = 0, w_offset: int = 0) -> Tuple[Compare, Compare]:
    """One call on fresh device copies; asserts the oracle tolerance on every
    (sampled) Q/K element, untouched bytes everywhere else, unchanged read-only
    inputs, and that at least ``min_exact`` of the elements equal the oracle's
    correctly rounded value bit for bit. ``cache_offset`` places the cos|sin
    table that many floats into its allocation, ``w_offset`` the weight rows
    that many elements into theirs (see DeviceCase)."""
    dc = DeviceCase(wl, layout=layout, cache_offset=cache_offset, w_offset=w_offset)
    dc.run(launch=launch, stream=stream)
    after = dc.fetch()
    dc.check_untouched(after)
    dc.check_inputs_unchanged()
    gq, gk = dc.outputs(after)
    if tokens is not None:
        gq, gk = gq[tokens], gk[tokens]
    rq, rk = oracle_ref(wl, tokens)
    res = []
    for name, g, r in (("q", gq, rq), ("k", gk, rk)):
        cmp = compare_bits(g, r, wl.cfg.dtype)
        assert cmp.bad == 0, f"{wl.cfg.name} {name}: {cmp}"
        assert cmp.exact_frac >= min_exact, f"{wl.cfg.name} {name}: {cmp}"
        res.append(cmp)
    return res[0], res[1]


def unfused_check(wl, which, layout=None, tokens=None):
    """Run one unfused entry point on fresh device copies and compare with the
    matching oracle function (every Q/K element; bytes outside untouched)."""
    from head_qk_rmsnorm_amd import binding as B

    c = wl.cfg
    dc = DeviceCase(wl, layout=layout)
    if which == "norm":
        B.qknr_rmsnorm_inplace(dc.q, dc.k, dc.wq, dc.wk, eps=c.eps)
        rq = O.rms_norm_io(wl.q, wl.wq, eps=c.eps, dtype=c.dtype)
        rk = O.rms_norm_io(wl.k, wl.wk, eps=c.eps, dtype=c.dtype)
    elif which == "rope":
        B.qknr_rope_inplace(dc.q, dc.k, dc.cache, dc.positions, is_neox=c.is_neox)
        rq = O.rope_io(wl.q, wl.cache, wl.positions, is_neox=c.is_neox, dtype=c.dtype)
        rk = O.rope_io(wl.k, wl.cache, wl.positions, is_neox=c.is_neox, dtype=c.dtype)
    else:
        B.qknr_unfused_inplace(dc.q, dc.k, dc.wq, dc.wk, dc.cache, dc.positions,
                               is_neox=c.is_neox, eps=c.eps)
        rq, rk = O.qknorm_rope_unfused_io(wl.q, wl.k, wl.wq, wl.wk, wl.cache, wl.positions,
                                          is_neox=c.is_neox, eps=c.eps, dtype=c.dtype)
    after = dc.fetch()
    dc.check_untouched(after)
    dc.check_inputs_unchanged()
    gq, gk = dc.outputs(after)
    out = []
    for name, g, r in (("q", gq, rq), ("k", gk, rk)):
        cmp = compare_bits(g, r, c.dtype)
        assert cmp.bad == 0, f"{which} {c.name} {name}: {cmp}"
        # the rope step on stored values only adds one rounding of an fp32
        # rotation; the norm step is the fused op's first half
        assert cmp.exact_frac >= 0.99, f"{which} {c.name} {name}: {cmp}"
        out.append(cmp)
    return out


def layernorm_check(wl, rope_dim, bias, layout=None, bias_seed=0, launch=None, cache_offset=0):
    """The LayerNorm sibling on fresh device copies against the oracle (every
    Q/K element; bytes outside untouched). With ``launch`` (a dict, {} for the
    automatic choice) the call goes through qknr_layernorm_rope_inplace_ex and
    its launch report is returned."""
    from head_qk_rmsnorm_amd import binding as B

    c = wl.cfg
    dc = DeviceCase(wl, layout=layout, cache_offset=cache_offset)
    bq_bits = bk_bits = None
    bq = bk = None
    if bias:
        g = W.rng(c.seed + bias_seed, 77)
        bq_bits = W.to_io_bits(g.standard_normal(c.head_dim) * 0.5, c.dtype)
        bk_bits = W.to_io_bits(g.standard_normal(c.head_dim) * 0.5, c.dtype)
        bq = torch_from_bits(bq_bits, dc)
        bk = torch_from_bits(bk_bits, dc)
    info = None
    if launch is None:
        B.qknr_layernorm_rope_inplace(dc.q, dc.k, dc.wq, dc.wk, bq, bk,
                                      dc.cache if rope_dim else None,
                                      dc.positions if rope_dim else None,
                                      is_neox=c.is_neox, eps=c.eps, rope_dim=rope_dim)
    else:
        info = B.qknr_layernorm_rope_inplace_ex(dc.q, dc.k, dc.wq, dc.wk, bq, bk,
                                                dc.cache if rope_dim else None,
                                                dc.positions if rope_dim else None,
                                                is_neox=c.is_neox, eps=c.eps, rope_dim=rope_dim,
                                                launch=launch)
    rq, rk = O.qk_layernorm_rope_io(wl.q, wl.k, wl.wq, wl.wk, bq_bits, bk_bits,
                                    wl.cache[:, :rope_dim] if rope_dim else None, wl.positions,
                                    is_neox=c.is_neox, eps=c.eps, dtype=c.dtype,
                                    rope_dim=rope_dim)
    after = dc.fetch()
    dc.check_untouched(after)
    dc.check_inputs_unchanged()
    gq, gk = dc.outputs(after)
    for name, g, r in (("q", gq, rq), ("k", gk, rk)):
        cmp = compare_bits(g, r, c.dtype)
        assert cmp.bad == 0, f"layernorm {c.name} {name}: {cmp}"
        assert cmp.exact_frac >= 0.99, f"layernorm {c.name} {name}: {cmp}"
    return info


def torch_from_bits(bits, dc):
    import torch

    return torch.from_numpy(bits.view(np.int16)).to(dc.device).view(dc.tdt)
