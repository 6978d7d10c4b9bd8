#!/usr/bin/env python3
"""One-GPU benchmark of the fused in-place QK RMSNorm + RoPE (HIP, gfx950).

A step is one launch of the op over one batch: every Q/K head vector of the
workload normalised and rotated in place. After a settle phase (untimed launches
for --settle seconds, so the clocks settle) and --warmup untimed launches, 5
batches of max(--steps, 50) launches are timed with HIP events on the launch
stream; the line reports their median (and min/max). The other workloads are
timed the same way in the same run (the line's "configs" object). Default workload: the DiT-shaped
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
CSRC = os.path.join(ROOT, "head_qk_rmsnorm_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, n) for n in ("qknr_device.h", "qknr_inst.hip", "qknr.hip")]
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
BATCHES = 5           # timed batches; the line reports their median
MIN_BATCH = 50        # launches per batch at least
SETTLE_S = 0.3        # seconds of launches before any timing, so the clocks settle
LAUNCH_INFO_KEYS = ("lanes_per_head", "elems_per_lane", "heads_per_wave", "groups_per_token",
                    "groups_per_item", "unroll", "block_threads", "grid_blocks", "items", "generic",
                    "access_bytes")


def source_sha() -> str:
    """Hash of the library's kernel and planner sources (device code, instance
    table, host planner): counters taken on other sources are not attached."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000,
                    help=f"launches per timed batch (at least {MIN_BATCH}); {BATCHES} batches are "
                         "timed and their median reported")
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed launches right before the timed batches")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed launches before anything is timed (clock settling)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads for the line's 'configs' object")
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

    def _launch_pass(self, n):
        """n launches (eager) or n passes over the copies (graph replay)."""
        if self.graph is not None:
            for _ in range(n):
                self.graph.replay()
        else:
            k = self.n_rot
            for i in range(n):
                self.calls[i % k]()

    def settle(self, seconds):
        """Untimed launches for about `seconds` of wall time, so the clocks have
        settled before anything is timed. Returns (launches, seconds)."""
        import torch

        per = 1 if self.graph is not None else 50
        n = 0
        t0 = time.perf_counter()
        while True:
            self._launch_pass(per)
            n += per * (self.n_rot if self.graph is not None else 1)
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n, time.perf_counter() - t0

    def time(self, steps, warmup, batches=BATCHES):
        """`warmup` untimed launches, then `batches` batches of max(steps,
        MIN_BATCH) launches on the launch stream, each between two HIP events.
        Graph replay times whole passes over the copies (rounded up). Returns
        the per-launch ms of every batch, their median, the launches per batch
        and the host's ms per launch."""
        import statistics

        import torch

        n = max(steps, MIN_BATCH)
        graph = self.graph is not None
        reps = max(1, -(-n // self.n_rot)) if graph else n
        per_batch = reps * self.n_rot if graph else n
        self._launch_pass(max(1, -(-warmup // self.n_rot)) if graph else warmup)
        torch.cuda.synchronize()
        out, host = [], []
        for _ in range(batches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            h0 = time.perf_counter()
            e0.record()
            self._launch_pass(reps)
            e1.record()
            host.append((time.perf_counter() - h0) / per_batch * 1e3)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / per_batch)
        return {"batch_ms": out, "ms": statistics.median(out), "launches_per_batch": per_batch,
                "host_ms": statistics.median(host)}


def yardstick(nbytes, steps, warmup, dev):
    """In-place read-xor(0)-write over the op's Q/K byte count, rotated copies,
    timed like the op (median of the batches)."""
    import statistics

    import torch

    from head_qk_rmsnorm_amd import binding as B

    nbytes = (nbytes + 15) // 16 * 16
    n_rot = min(MAX_ROT, max(2, math.ceil(ROT_BYTES / nbytes)))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(i) for i in range(n_rot)]
    n = max(steps, MIN_BATCH)
    for i in range(max(warmup, n)):
        B.qknr_rmw(bufs[i % n_rot], nbytes, 0)
    torch.cuda.synchronize()
    out = []
    for _ in range(BATCHES):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            B.qknr_rmw(bufs[i % n_rot], nbytes, 0)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / n)
    del bufs
    ms = statistics.median(out)
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
        "host_cpu": host_cpu_model(), "host_logical_cpus": os.cpu_count(),
        "gheads_per_s": round(done * cfg.heads / el / 1e9, 9),
    }


def counters_for(cfg_name, launch_info, forced_launch):
    """Counter-based HBM traffic per launch, if it was measured on these library
    sources and in this launch shape (never for an explicit --launch)."""
    if forced_launch:
        return None, "explicit launch configuration: counters cover the automatic launch only"
    if not os.path.exists(COUNTERS):
        return None, "no counter file"
    with open(COUNTERS) as f:
        data = json.load(f)
    ent = data.get(cfg_name)
    if not ent:
        return None, "workload not in counter file"
    if ent.get("source_sha") != source_sha():
        return None, "library sources changed since the counters were taken"
    want = {k: launch_info.get(k) for k in LAUNCH_INFO_KEYS}
    if {k: ent.get("launch", {}).get(k) for k in LAUNCH_INFO_KEYS} != want:
        return None, "launch shape differs from the one the counters were taken in"
    return ent, None


def unfused_bytes(cfg):
    """Bytes the two-launch chain must move: Q/K read and written by each step,
    the weights by the norm step, positions and cos|sin rows by the rope step."""
    D, R = cfg.head_dim, cfg.rope_dim
    qk = 2 * cfg.units * D * cfg.io_bytes
    return 2 * qk + 2 * D * cfg.io_bytes + cfg.T * cfg.pos_bytes + cfg.T * R * 4


def measure(cfg, dev, steps, warmup, launch, want_yard=True, rig=None, want_unfused=True,
            op="fused", graph=False, settle=0.0):
    own = rig is None
    layernorm = op == "layernorm"
    if own:
        rig = Rig(cfg, dev, launch=launch, graph=graph)
    if layernorm:
        rig.prepare(launch, layernorm=True)
    elif not own:
        rig.prepare(launch)
    settled = rig.settle(settle) if settle > 0 else (0, 0.0)
    tm = rig.time(steps, warmup)
    ms = tm["ms"]
    # the LayerNorm sibling also reads the two bias rows
    B = cfg.algorithmic_bytes() + (2 * cfg.head_dim * cfg.io_bytes if layernorm else 0)
    gbs = B / (ms * 1e-3) / 1e9
    out = {
        "workload": cfg.name, "ms_per_step": ms, "GB_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
        "gheads_per_s": cfg.units / (ms * 1e-3) / 1e9, "host_ms_per_launch": tm["host_ms"],
        "batch_ms": tm["batch_ms"], "launches_per_batch": tm["launches_per_batch"],
        "settle": {"launches": settled[0], "seconds": round(settled[1], 3)},
        "algorithmic_bytes": B, "n_rot": rig.n_rot, "footprint_bytes": rig.footprint,
        "launch": rig.info, "op": op, "graph": rig.gstream is not None,
    }
    if want_unfused and not layernorm:
        rig.prepare(unfused=True)
        ums = rig.time(steps, warmup)["ms"]
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
        ymsn, ygbs = yardstick(cfg.units * cfg.head_dim * 2, steps, warmup, dev)
        out["yardstick_GB_s"] = ygbs
        out["frac_of_yardstick"] = gbs / ygbs
    return out


def config_entry(r, forced_launch):
    """One workload's figures for the line's 'configs' object."""
    ms = r["ms_per_step"]
    e = {
        "ms_per_launch": round(ms, 6),
        "ms_per_launch_min_max": [round(min(r["batch_ms"]), 6), round(max(r["batch_ms"]), 6)],
        "GB_s": round(r["GB_s"], 3), "frac_of_hbm_peak": round(r["frac_of_peak"], 5),
        "gheads_per_s": round(r["gheads_per_s"], 4),
        "launch_mode": "hip graph replay" if r["graph"] else "eager launches from python",
        "launches_per_batch": r["launches_per_batch"], "algorithmic_bytes": r["algorithmic_bytes"],
        "launch": r["launch"],
    }
    if "yardstick_GB_s" in r:
        e["yardstick_GB_s"] = round(r["yardstick_GB_s"], 3)
        e["frac_of_yardstick"] = round(r["frac_of_yardstick"], 5)
    ent, why = counters_for(r["workload"], r["launch"], forced_launch)
    if ent:
        traffic = ent["fetch_bytes_per_launch"] + ent["write_bytes_per_launch"]
        e["traffic"] = traffic
        e["traffic_over_algorithmic"] = round(traffic / r["algorithmic_bytes"], 4)
    else:
        e["traffic"] = None
        e["traffic_note"] = why
    return e


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
                want_unfused=not args.no_unfused, op=args.op, graph=args.graph,
                settle=args.settle)
    print(f"[bench] {cfg.name}: {r['GB_s']:.1f} GB/s, {r['ms_per_step'] * 1e3:.2f} us/launch "
          f"(median of {BATCHES} batches of {r['launches_per_batch']}; "
          f"{min(r['batch_ms']) * 1e3:.2f}-{max(r['batch_ms']) * 1e3:.2f} us)",
          file=sys.stderr, flush=True)
    ent, why = (counters_for(cfg.name, r["launch"], launch is not None) if args.op == "fused"
                else (None, "counters cover the fused op"))
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
        "io_dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "head_dim": cfg.head_dim, "rope_dim": cfg.rope_dim,
                   "pairing": "neox" if cfg.is_neox else "interleaved", "io_dtype": cfg.dtype,
                   "pos_dtype": cfg.pos_dtype, "layout": cfg.layout,
                   "algorithmic_bytes_per_step": r["algorithmic_bytes"], "launch": r["launch"],
                   "rotated_copies": r["n_rot"]},
        "timing": {"batches": BATCHES, "launches_per_batch": r["launches_per_batch"],
                   "statistic": "median of the batches' per-launch times",
                   "ms_per_launch_min_median_max": [round(min(r["batch_ms"]), 6),
                                                    round(r["ms_per_step"], 6),
                                                    round(max(r["batch_ms"]), 6)],
                   "settle": dict(r["settle"], what="untimed launches before any timing, so "
                                                     "the clocks settle"),
                   "events": "HIP events on the launch stream around each batch"},
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
    if not (args.no_configs or args.case or args.op != "fused" or launch is not None):
        # the other workloads in the same run, timed the same way (the 16-token
        # workload is shorter than a launch from Python: HIP graph replay)
        line["configs"] = {}
        for name in W.CONFIG_ORDER:
            if name == cfg.name:
                continue
            c = W.CONFIGS[name]
            # (no yardstick for the latency-bound 16-token workload: its eager
            # launches would time the host, not the memory)
            rc = measure(c, dev, args.steps, args.warmup, None,
                         want_yard=not args.no_yardstick and name != "tiny",
                         want_unfused=False, graph=name == "tiny", settle=0.05)
            line["configs"][name] = config_entry(rc, False)
            print(f"[bench] config {name}: {rc['GB_s']:.1f} GB/s ({rc['frac_of_peak'] * 100:.1f}% of "
                  f"peak), {rc['ms_per_step'] * 1e3:.2f} us/launch", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
    line["host_ms_per_launch"] = round(r["host_ms_per_launch"], 5)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    if extra:
        extra.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
