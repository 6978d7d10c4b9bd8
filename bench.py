#!/usr/bin/env python3
"""One-GPU benchmark of the fused in-place QK RMSNorm + RoPE (HIP, gfx950).

A step is one launch of the op over one batch: every Q/K head vector of the
workload normalised and rotated in place. Default workload: the DiT-shaped
image+text sequence (T=4608 tokens, 24+24 heads, head_dim 128, interleaved
pairing, bf16, int64 positions). The metric is achieved HBM bandwidth in
algorithmic bytes (every Q/K element read and written once, one positions entry
and one fp32 cos|sin row per token, both weight rows) per second.

Inputs are resident in HBM before timing. The timed loop cycles through enough
independent copies of the mutable buffers (>= 1 GiB in total) that the 256 MB
Infinity Cache cannot serve a launch from the previous visit of its copy.

Prints ONE JSON line. Extra per-configuration / sweep lines go to --extra-out.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
ROT_BYTES = 1 << 30    # rotate through >= 1 GiB of copies
MAX_ROT = 64           # (tiny workloads: at most 64 copies; they are latency-bound anyway)
KERNEL_SRC = os.path.join(ROOT, "head_qk_rmsnorm_amd", "csrc", "qknr_device.h")
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def kernel_sha() -> str:
    """Hash of the fused kernel's device code (between its begin/end markers)."""
    with open(KERNEL_SRC, "rb") as f:
        src = f.read()
    a = src.index(b"// ==== fused-kernel device code begin")
    b = src.index(b"// ==== fused-kernel device code end")
    return hashlib.sha256(src[a:b]).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed launches before the timed ones (1000 lets the clocks settle)")
    ap.add_argument("--config", default="dit",
                    help="tiny | dit | gqa | partial | large, or a one-GPU shard: gqa_tp8 | "
                         "dit_hp8 | dit_sp8")
    ap.add_argument("--launch", default="", help="JSON launch configuration (qknr_launch_cfg fields)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle timing budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-yardstick", action="store_true")
    ap.add_argument("--no-unfused", action="store_true", help="skip timing the two-launch baseline")
    ap.add_argument("--op", default="fused", choices=["fused", "layernorm"],
                    help="time the fused RMSNorm+RoPE op (default) or the per-head LayerNorm+RoPE sibling")
    ap.add_argument("--sweep", action="store_true", help="time a short list of launch configurations")
    ap.add_argument("--sweep-grid", action="store_true",
                    help="time every (grid kind, groups per item, unroll, block waves) combination")
    ap.add_argument("--all-configs", action="store_true", help="also time every workload")
    ap.add_argument("--shards", action="store_true",
                    help="also time the one-GPU shard workloads (gqa_tp8, dit_hp8, dit_sp8)")
    ap.add_argument("--case", default="",
                    help="JSON keyword arguments of workloads.case (T, Hq, Hkv, head_dim, "
                         "rope_dim, is_neox, dtype, pos_dtype, ...): time that shape instead "
                         "of --config")
    ap.add_argument("--head-dim-scan", action="store_true",
                    help="also time head_dims other than 128 at the DiT workload's bytes per "
                         "launch (24+24 heads, int64 positions), automatic launch")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of one pass over the rotated copies instead of "
                         "launches from Python (for workloads shorter than the host's launch time)")
    ap.add_argument("--extra-out", default="", help="file for per-config / sweep JSON lines")
    return ap.parse_args()


class Rig:
    """Device copies of one workload and prepared launches over them."""

    def __init__(self, cfg, dev, launch=None, n_rot=None, graph=False):
        import numpy as np
        import torch

        from head_qk_rmsnorm_amd import workloads as W

        self.cfg = cfg
        self.dev = dev
        # graph mode: one pass over the rotated copies captured in a HIP graph
        # and replayed, so host launch overhead stays out of the timing
        self.gstream = torch.cuda.Stream(device=dev) if graph else None
        self.graph = None
        wl = W.make_workload(cfg)
        tdt = torch.bfloat16 if cfg.dtype == W.BF16 else torch.float16

        def d16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(tdt)

        self.wq, self.wk = d16(wl.wq), d16(wl.wk)
        self.cache = torch.from_numpy(wl.cache).to(dev)
        pos0 = torch.from_numpy(wl.positions).to(dev)
        base = [d16(wl.qkv)] if cfg.layout == "qkv" else [d16(wl.q), d16(wl.k)]
        del wl
        footprint = sum(t.numel() * t.element_size() for t in base) + pos0.numel() * pos0.element_size()
        self.n_rot = n_rot or min(MAX_ROT, max(2, math.ceil(ROT_BYTES / max(footprint, 1))))
        self.footprint = footprint
        self.copies = []
        for r in range(self.n_rot):
            bufs = [t.clone() for t in base] if r else base
            self.copies.append((bufs, pos0.clone() if r else pos0))
        self.prepare(launch)

    def views(self, bufs):
        import torch

        c, D = self.cfg, self.cfg.head_dim
        if c.layout == "qkv":
            qkv = bufs[0]
            q = torch.as_strided(qkv, (c.T, c.Hq, D), (qkv.stride(0), D, 1), 0)
            k = torch.as_strided(qkv, (c.T, c.Hkv, D), (qkv.stride(0), D, 1), c.Hq * D)
            return q, k
        return bufs[0], bufs[1]

    def prepare(self, launch=None, unfused=False, layernorm=False):
        import torch

        from head_qk_rmsnorm_amd import binding as B

        c = self.cfg
        bias = None
        if layernorm:
            # seeded bias rows for the LayerNorm sibling
            import numpy as np

            from head_qk_rmsnorm_amd import workloads as W

            g = W.rng(c.seed, 77)
            tdt = self.wq.dtype
            bias = tuple(torch.from_numpy(W.to_io_bits(g.standard_normal(c.head_dim) * 0.5,
                                                       c.dtype).view(np.int16)).to(self.dev).view(tdt)
                         for _ in range(2))
        self.calls = []
        for bufs, pos in self.copies:
            q, k = self.views(bufs)
            self.calls.append(B.PreparedCall(q, k, self.wq, self.wk, self.cache, pos,
                                             is_neox=c.is_neox, eps=c.eps, launch=launch,
                                             unfused=unfused, layernorm_bias=bias,
                                             stream=self.gstream))
        self.calls[0]()
        torch.cuda.synchronize(self.dev)
        self.info = self.calls[0].info.as_dict()
        self.graph = None
        if self.gstream is not None:
            for call in self.calls:  # one eager pass on the capture stream first
                call()
            torch.cuda.synchronize(self.dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.gstream):
                for call in self.calls:
                    call()
            torch.cuda.synchronize(self.dev)
            self.graph = g

    def time(self, steps, warmup):
        import torch

        n = self.n_rot
        if self.graph is not None:
            # whole passes over the copies: steps and warmup rounded up to multiples of n
            reps, wreps = max(1, -(-steps // n)), max(1, -(-warmup // n))
            for _ in range(wreps):
                self.graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            h0 = time.perf_counter()
            e0.record()
            for _ in range(reps):
                self.graph.replay()
            e1.record()
            host_s = time.perf_counter() - h0
            torch.cuda.synchronize()
            wall_s = time.perf_counter() - h0
            return e0.elapsed_time(e1) / (reps * n), host_s / (reps * n) * 1e3, wall_s
        for i in range(warmup):
            self.calls[i % n]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            self.calls[i % n]()
        e1.record()
        host_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - h0
        ms = e0.elapsed_time(e1) / steps
        return ms, host_s / steps * 1e3, wall_s


def yardstick(nbytes, steps, warmup, dev):
    """In-place read-xor(0)-write over the op's Q/K byte count, rotated copies."""
    import torch

    from head_qk_rmsnorm_amd import binding as B

    nbytes = (nbytes + 15) // 16 * 16
    n_rot = min(MAX_ROT, max(2, math.ceil(ROT_BYTES / nbytes)))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(i) for i in range(n_rot)]
    for i in range(warmup):
        B.qknr_rmw(bufs[i % n_rot], nbytes, 0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        B.qknr_rmw(bufs[i % n_rot], nbytes, 0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del bufs
    return ms, 2 * nbytes / (ms * 1e-3) / 1e9


def calibration_copy(dev, nbytes=512 << 20, reps=3):
    """A few plain copies of a known size: their FETCH_SIZE / WRITE_SIZE counters
    calibrate counter runs of this same command."""
    import torch

    from head_qk_rmsnorm_amd import binding as B

    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        B.qknr_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    del src, dst
    return {"bytes_per_copy": nbytes, "copies": reps}


def cpu_baseline(cfg, seconds):
    """The fp64 oracle as it stands, on the host's cores: worker threads (NumPy
    releases the GIL inside its array loops) each run the oracle over whole-token
    chunks of the same workload until the time budget is spent."""
    import concurrent.futures as cf
    import threading

    from head_qk_rmsnorm_amd import workloads as W
    from oracle import qknr_oracle as O

    wl = W.make_workload(cfg)
    try:
        omp = int(os.environ.get("OMP_NUM_THREADS", "16").split(",")[0])
    except ValueError:
        omp = 16
    workers = max(1, min(os.cpu_count() or 1, omp, 16))
    chunk = max(1, min(cfg.T, 16384 // max(cfg.heads, 1)))
    lock = threading.Lock()
    state = {"next": 0, "done": 0}
    t0 = time.perf_counter()

    def work():
        while time.perf_counter() - t0 < seconds:
            with lock:
                start = state["next"] % cfg.T
                state["next"] += chunk
            sl = slice(start, min(start + chunk, cfg.T))
            O.qknorm_rope_io(wl.q[sl], wl.k[sl], wl.wq, wl.wk, wl.cache, wl.positions[sl],
                             is_neox=cfg.is_neox, eps=cfg.eps, dtype=cfg.dtype,
                             rope_dim=cfg.rope_dim)
            with lock:
                state["done"] += sl.stop - sl.start

    with cf.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(work) for _ in range(workers)]:
            f.result()
    el = time.perf_counter() - t0
    done = state["done"]
    per_tok = cfg.algorithmic_bytes() / cfg.T
    return {
        "value": round(done * per_tok / el / 1e9, 6), "unit": "GB/s", "cores": workers,
        "kind": "oracle",
        "sample": f"{done} tokens ({done * cfg.heads} head vectors) of the '{cfg.name}' workload "
                  f"in chunks of {chunk} tokens, {el:.1f} s, numpy fp64 on {workers} threads",
        "host_cpu": platform.processor() or platform.machine(), "host_logical_cpus": os.cpu_count(),
        "gheads_per_s": round(done * cfg.heads / el / 1e9, 9),
    }


def counters_for(cfg_name):
    """Counter-based HBM traffic per launch, if it was measured on this kernel source."""
    if not os.path.exists(COUNTERS):
        return None, "no counter file"
    with open(COUNTERS) as f:
        data = json.load(f)
    ent = data.get(cfg_name)
    if not ent:
        return None, "workload not in counter file"
    if ent.get("kernel_sha") != kernel_sha():
        return None, "kernel changed since the counters were taken"
    return ent, None


def unfused_bytes(cfg):
    """Bytes the two-launch chain must move: Q/K read and written by each step,
    the weights by the norm step, positions and cos|sin rows by the rope step."""
    D, R = cfg.head_dim, cfg.rope_dim
    qk = 2 * cfg.units * D * cfg.io_bytes
    return 2 * qk + 2 * D * cfg.io_bytes + cfg.T * cfg.pos_bytes + cfg.T * R * 4


def measure(cfg, dev, steps, warmup, launch, want_yard=True, rig=None, want_unfused=True,
            op="fused", graph=False):
    own = rig is None
    layernorm = op == "layernorm"
    if own:
        rig = Rig(cfg, dev, launch=launch, graph=graph)
    if layernorm:
        rig.prepare(layernorm=True)
    elif not own:
        rig.prepare(launch)
    ms, host_ms, wall = rig.time(steps, warmup)
    # the LayerNorm sibling also reads the two bias rows
    B = cfg.algorithmic_bytes() + (2 * cfg.head_dim * cfg.io_bytes if layernorm else 0)
    gbs = B / (ms * 1e-3) / 1e9
    out = {
        "workload": cfg.name, "ms_per_step": ms, "GB_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
        "gheads_per_s": cfg.units / (ms * 1e-3) / 1e9, "host_ms_per_launch": host_ms,
        "algorithmic_bytes": B, "n_rot": rig.n_rot, "footprint_bytes": rig.footprint,
        "launch": rig.info, "op": op, "graph": rig.gstream is not None,
    }
    if want_unfused and not layernorm:
        rig.prepare(unfused=True)
        ums, _, _ = rig.time(steps, warmup)
        ub = unfused_bytes(cfg)
        out["unfused"] = {
            "ms_per_step": ums, "launches_per_step": 2, "bytes_per_step": ub,
            "GB_s": ub / (ums * 1e-3) / 1e9, "speedup_fused_over_unfused": ums / ms,
            "bytes_ratio_unfused_over_fused": ub / B,
        }
        rig.prepare(launch)
    if own:
        del rig
    if want_yard:
        ymsn, ygbs = yardstick(cfg.units * cfg.head_dim * 2, steps, warmup // 4 + 1, dev)
        out["yardstick_GB_s"] = ygbs
        out["frac_of_yardstick"] = gbs / ygbs
    return out


# (head_dim, rope_dim, NeoX) shapes of the head_dim scan: the compile-time 128
# for reference, run-time head_dims, small heads, and NeoX halves no 16-byte
# lane divides (partners 4 slots over: 72, 88, 136, 96 with rope_dim 24;
# 2 or 6 slots over: 80 with rope_dim 20, 128 with rope_dim 20).
HEAD_DIM_SCAN = [(128, 128, False), (128, 128, True), (96, 96, False), (96, 96, True),
                 (80, 80, False), (80, 80, True), (112, 112, False), (112, 112, True),
                 (160, 160, False), (160, 160, True), (192, 192, False), (192, 192, True),
                 (40, 40, False), (40, 40, True), (72, 72, True), (88, 88, True),
                 (136, 136, True), (96, 24, True), (80, 20, True), (128, 20, True)]


def head_dim_scan_case(D, R, neox):
    """24+24 heads and as many tokens as give the DiT workload's Q/K bytes
    (4608 tokens at head_dim 128); int64 positions drawn uniformly from a cache of
    T rows."""
    from head_qk_rmsnorm_amd import workloads as W

    T = int(4608 * 128 / D)
    return W.case(T, 24, 24, D, R, neox, pos_dtype=W.I64, seed=D + R, cache_rows=T)


SWEEP = [
    dict(), dict(unroll=1), dict(unroll=4),
    dict(groups_per_item=1), dict(groups_per_item=2), dict(groups_per_item=3), dict(groups_per_item=4),
    dict(groups_per_item=6), dict(groups_per_item=2, unroll=1), dict(groups_per_item=4, unroll=4),
    dict(block_waves=2), dict(block_waves=8), dict(max_blocks=-1), dict(max_blocks=-1, groups_per_item=2),
    dict(max_blocks=-1, groups_per_item=4), dict(lanes_per_head=32), dict(lanes_per_head=64),
]


SWEEP_GRID = ([dict(max_blocks=mb, groups_per_item=g, unroll=u, block_waves=bw)
               for mb in (0, -1) for g in (1, 2, 3, 4, 6, 8, 12) for u in (1, 2, 4)
               for bw in (1, 2, 4, 8) if u <= max(g, 1) and not (g == 3 and u == 4)]
              + [dict(lanes_per_head=lanes, groups_per_item=g, unroll=u, block_waves=bw)
                 for lanes in (32, 64) for g, u in ((1, 1), (2, 2), (4, 2), (4, 4), (8, 4))
                 for bw in (1, 2, 4)])


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this op runs on one GPU; every (token, head) vector is "
                          "independent, so N GPUs would each run the same kernel on their own "
                          "shard with no exchange step. Run with --gpus 1."}), flush=True)
        sys.exit(2)
    import torch

    from head_qk_rmsnorm_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    launch = json.loads(args.launch) if args.launch else None
    cfg = W.case(**json.loads(args.case)) if args.case else W.CONFIGS[args.config]
    extra = open(args.extra_out, "a") if args.extra_out else None

    calib = calibration_copy(dev)
    print(f"[bench] calibration copies done: {calib}", file=sys.stderr, flush=True)

    if args.sweep or args.sweep_grid:
        rig = Rig(cfg, dev, graph=args.graph)
        for lc in (SWEEP_GRID if args.sweep_grid else SWEEP):
            try:
                r = measure(cfg, dev, args.steps, args.warmup, lc, want_yard=False, rig=rig,
                            want_unfused=False)
            except RuntimeError as e:
                r = {"workload": cfg.name, "error": str(e)}
            r["sweep_launch"] = lc
            print(f"[bench] sweep {lc}: {r.get('GB_s', 0):.1f} GB/s", file=sys.stderr, flush=True)
            if extra:
                extra.write(json.dumps(r) + "\n")
                extra.flush()
        del rig
    if args.all_configs or args.shards:
        names = (W.CONFIG_ORDER if args.all_configs else []) + (W.SHARD_ORDER if args.shards else [])
        for name in names:
            r = measure(W.CONFIGS[name], dev, args.steps, args.warmup, launch,
                        want_yard=not args.no_yardstick, want_unfused=not args.no_unfused,
                        op=args.op, graph=args.graph)
            msg = (f"[bench] {name}: {r['GB_s']:.1f} GB/s ({r['frac_of_peak'] * 100:.1f}% of peak), "
                   f"{r['gheads_per_s']:.2f} Gheads/s")
            if "yardstick_GB_s" in r:
                msg += f", yardstick {r['yardstick_GB_s']:.1f} GB/s"
            if "unfused" in r:
                msg += (f", unfused pair {r['unfused']['ms_per_step'] * 1e3:.2f} us "
                        f"(fused {r['unfused']['speedup_fused_over_unfused']:.2f}x faster)")
            print(msg, file=sys.stderr, flush=True)
            if extra:
                extra.write(json.dumps(r) + "\n")
                extra.flush()

    if args.head_dim_scan:
        for D, R, neox in HEAD_DIM_SCAN:
            c = head_dim_scan_case(D, R, neox)
            r = measure(c, dev, args.steps, args.warmup, None, want_yard=False,
                        want_unfused=False, op=args.op, graph=args.graph)
            r["scan"] = {"head_dim": D, "rope_dim": R, "pairing": "neox" if neox else "interleaved"}
            print(f"[bench] scan {c.name}: {r['GB_s']:.1f} GB/s, launch {r['launch']}",
                  file=sys.stderr, flush=True)
            if extra:
                extra.write(json.dumps(r) + "\n")
                extra.flush()

    r = measure(cfg, dev, args.steps, args.warmup, launch, want_yard=not args.no_yardstick,
                want_unfused=not args.no_unfused, op=args.op, graph=args.graph)
    print(f"[bench] {cfg.name}: {r['GB_s']:.1f} GB/s, {r['ms_per_step'] * 1e3:.2f} us/launch",
          file=sys.stderr, flush=True)
    ent, why = counters_for(cfg.name) if args.op == "fused" else (None, "counters cover the fused op")
    traffic = None
    if ent:
        traffic = ent["fetch_bytes_per_launch"] + ent["write_bytes_per_launch"]
    roof = {"bound": "hbm", "achieved": round(r["GB_s"], 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["GB_s"] / HBM_PEAK_GBS, 5), "traffic": traffic}
    line = {
        "metric": "achieved HBM GB/s (and % of peak) + Gheads/s for fused QK RMSNorm+RoPE",
        "op": "fused QK RMSNorm + RoPE" if args.op == "fused" else
              "per-head QK LayerNorm (weight, bias) + RoPE (sibling op, not the headline metric)",
        "value": round(r["GB_s"], 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "head_dim": cfg.head_dim, "rope_dim": cfg.rope_dim,
                   "pairing": "neox" if cfg.is_neox else "interleaved", "io_dtype": cfg.dtype,
                   "pos_dtype": cfg.pos_dtype, "layout": cfg.layout,
                   "algorithmic_bytes_per_step": r["algorithmic_bytes"], "launch": r["launch"],
                   "rotated_copies": r["n_rot"]},
        "gheads_per_s": round(r["gheads_per_s"], 4),
        "frac_of_hbm_peak": round(r["frac_of_peak"], 5),
        "launch_mode": "hip graph replay" if args.graph else "eager launches from python",
        "roofline": roof,
    }
    if ent is None:
        line["roofline_traffic_note"] = why
    else:
        line["traffic_detail"] = ent
    if "yardstick_GB_s" in r:
        line["yardstick"] = {"kind": "in-place 16-byte read-xor-write over the same Q/K bytes",
                             "GB_s": round(r["yardstick_GB_s"], 3),
                             "frac_of_yardstick": round(r["frac_of_yardstick"], 5)}
    if "unfused" in r:
        u = r["unfused"]
        line["fusion"] = {
            "unfused_ms_per_step": round(u["ms_per_step"], 6),
            "unfused_launches_per_step": 2,
            "unfused_bytes_per_step": u["bytes_per_step"],
            "speedup_fused_over_unfused": round(u["speedup_fused_over_unfused"], 4),
            "bytes_ratio_unfused_over_fused": round(u["bytes_ratio_unfused_over_fused"], 4),
            "page_claim": "separate norm + RoPE kernels: 2 launches, Q/K read and written twice; "
                          "fused: about half the memory traffic and close to 2x faster (no "
                          "hardware or measured figure given)",
        }
    line["host_ms_per_launch"] = round(r["host_ms_per_launch"], 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    if extra:
        extra.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
