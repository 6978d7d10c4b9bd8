"""Integration of the C ABI beyond the Python binding: a plain C caller, HIP
graph capture and concurrent callers from several host threads."""
import os
import subprocess
import tempfile
import threading

import numpy as np
import pytest

from head_qk_rmsnorm_amd import workloads as W
from tests import qknr_harness as Hn

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CAPI_BIN = os.path.join(HERE, "capi", "qknr_capi_run")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from head_qk_rmsnorm_amd import binding as B

    B.lib()
    yield


def _write_case(path, wl):
    c = wl.cfg
    hdr = np.array([c.T, c.Hq, c.Hkv, c.head_dim, c.rope_dim, int(c.is_neox),
                    0 if c.dtype == W.BF16 else 1, 0 if c.pos_dtype == W.I32 else 1,
                    c.cache_rows], dtype=np.int64)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.float32(c.eps).tobytes())
        for a in (wl.q, wl.k, wl.wq, wl.wk, wl.cache, wl.positions):
            f.write(np.ascontiguousarray(a).tobytes())


@pytest.mark.parametrize("cfg", [
    W.CONFIGS["tiny"],
    W.case(37, 6, 2, 128, 128, False, dtype=W.FP16, pos_dtype=W.I64, seed=3),
    W.case(19, 3, 5, 256, 128, True, seed=4),
    W.case(23, 4, 4, 96, 96, True, seed=5),
], ids=lambda c: c.name)
def test_plain_c_caller(cfg):
    """libqknr.so driven from C through include/qknr.h only (qknr_inplace, and
    qknr_inplace_ex with the element-granular kernel requested); both outputs
    checked against the fp64 oracle."""
    if not os.path.exists(CAPI_BIN):
        pytest.fail(f"{CAPI_BIN} missing: run __graft_entry__.build()")
    wl = W.make_workload(cfg)
    with tempfile.TemporaryDirectory() as d:
        case, out = os.path.join(d, "case.bin"), os.path.join(d, "out.bin")
        _write_case(case, wl)
        r = subprocess.run([CAPI_BIN, case, out], capture_output=True, text=True, timeout=120)
        print(r.stdout, r.stderr, flush=True)
        assert r.returncode == 0, r.stderr
        got = np.fromfile(out, dtype=np.uint16)
    from tests.test_abi import elem_plan

    lanes = elem_plan(cfg.head_dim, 16, cfg.Hq, cfg.Hkv)[2]
    assert f"launch: generic=1 lanes_per_head={lanes} " in r.stdout, r.stdout
    nq, nk = wl.q.size, wl.k.size
    assert got.size == 2 * (nq + nk)
    rq, rk = Hn.oracle_ref(wl)
    for base in (0, nq + nk):  # qknr_inplace, then qknr_inplace_ex on the element kernel
        gq = got[base:base + nq].reshape(wl.q.shape)
        gk = got[base + nq:base + nq + nk].reshape(wl.k.shape)
        for g, ref in ((gq, rq), (gk, rk)):
            cmp = Hn.compare_bits(g, ref, cfg.dtype)
            assert cmp.bad == 0 and cmp.exact_frac >= 0.99, (base, cmp)


@pytest.mark.parametrize("T,Hq,Hkv,D,R,neox", [
    (129, 8, 4, 128, 64, True),      # vectorised kernel
    (200, 8, 4, 80, 20, True),       # shifted partners through LDS
    (3000, 24, 24, 40, 38, True)])   # element-granular kernel, persistent grid
def test_hip_graph_capture_and_replay(T, Hq, Hkv, D, R, neox):
    """The op allocates nothing and never synchronises, so it can be captured
    in a HIP graph. Each replay applies it again in place: after n replays
    the tensors equal n eager applications, bit for bit, on every replay."""
    import torch
    from head_qk_rmsnorm_amd import binding as B

    cfg = W.case(T, Hq, Hkv, D, R, neox, seed=12 + D)
    wl = W.make_workload(cfg)
    g_case = Hn.DeviceCase(wl)
    e_case = Hn.DeviceCase(wl)
    kw = dict(is_neox=cfg.is_neox, eps=cfg.eps)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        # warm-up on the side stream: one application
        B.qknr_inplace(g_case.q, g_case.k, g_case.wq, g_case.wk, g_case.cache, g_case.positions,
                       stream=s, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        B.qknr_inplace(g_case.q, g_case.k, g_case.wq, g_case.wk, g_case.cache, g_case.positions,
                       stream=s, **kw)
    B.qknr_inplace(e_case.q, e_case.k, e_case.wq, e_case.wk, e_case.cache, e_case.positions, **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        B.qknr_inplace(e_case.q, e_case.k, e_case.wq, e_case.wk, e_case.cache, e_case.positions,
                       **kw)
        torch.cuda.synchronize()
        for a, b in zip(g_case.fetch(), e_case.fetch()):
            assert np.array_equal(a, b), f"replay {rep}"


def test_concurrent_callers():
    """Several host threads, each with its own stream and buffers, call the
    library at once; every result matches three applications of the oracle."""
    import torch
    from head_qk_rmsnorm_amd import binding as B
    from oracle import qknr_oracle as O

    cases = [W.case(65, 4 + i, 2 + i % 3, (64, 128, 256, 96)[i % 4], (64, 128, 128, 96)[i % 4],
                    bool(i % 2), seed=30 + i) for i in range(6)]
    wls = [W.make_workload(c) for c in cases]
    dcs = [Hn.DeviceCase(wl) for wl in wls]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            dc = dcs[i]
            for _ in range(3):  # three applications in a row on this stream
                B.qknr_inplace(dc.q, dc.k, dc.wq, dc.wk, dc.cache, dc.positions,
                               is_neox=cases[i].is_neox, eps=cases[i].eps, stream=s)
            s.synchronize()
        except Exception as e:  # collected and reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for wl, dc in zip(wls, dcs):
        c = wl.cfg
        q, k = wl.q, wl.k
        for _ in range(3):
            q, k, _, _ = O.qknorm_rope_io(q, k, wl.wq, wl.wk, wl.cache, wl.positions,
                                          is_neox=c.is_neox, eps=c.eps, dtype=c.dtype,
                                          rope_dim=c.rope_dim)
        gq, gk = dc.outputs(dc.fetch())
        for g, r in ((gq, q), (gk, k)):
            # each application may land one ulp away from the correctly rounded
            # value and the next one starts from there: check the tolerance only
            cmp = Hn.compare_bits(g, r, c.dtype)
            assert cmp.bad == 0, (c.name, cmp)


def test_torch_custom_ops_eager_and_compiled():
    """torch.ops.qknr.* called directly matches the oracle; inside a compiled
    function (aot_eager, full graph) the in-place updates of q and k survive and
    equal the eager result bit for bit, for the fused op and the LayerNorm
    sibling."""
    import torch
    from head_qk_rmsnorm_amd import torch_ops  # noqa: F401  (registers torch.ops.qknr)

    cfg = W.case(33, 6, 2, 128, 64, True, pos_dtype=W.I64, seed=21)
    wl = W.make_workload(cfg)
    a = Hn.DeviceCase(wl)
    torch.ops.qknr.fused_inplace_qknorm_rope(a.q, a.k, a.wq, a.wk, a.cache, a.positions,
                                             is_neox=True, eps=cfg.eps)
    gq, gk = a.outputs(a.fetch())
    rq, rk = Hn.oracle_ref(wl)
    for g, r in ((gq, rq), (gk, rk)):
        cmp = Hn.compare_bits(g, r, cfg.dtype)
        assert cmp.bad == 0 and cmp.exact_frac >= 0.99, cmp

    def step(q, k, wq, wk, cache, pos, bq, bk):
        torch.ops.qknr.fused_inplace_qknorm_rope(q, k, wq, wk, cache, pos, is_neox=True, eps=1e-6)
        s = q.float().sum() + k.float().sum()
        torch.ops.qknr.fused_inplace_qk_layernorm_rope(q, k, wq, wk, bq, bk, cache, pos,
                                                       is_neox=True, eps=1e-6, rope_dim=64)
        return s

    compiled = torch.compile(step, backend="aot_eager", fullgraph=True)
    e = Hn.DeviceCase(wl)
    c = Hn.DeviceCase(wl)
    bq = torch.linspace(-0.5, 0.5, 128, device=e.device).to(e.tdt)
    bk = torch.linspace(0.5, -0.5, 128, device=e.device).to(e.tdt)
    se = step(e.q, e.k, e.wq, e.wk, e.cache, e.positions, bq, bk)
    sc = compiled(c.q, c.k, c.wq, c.wk, c.cache, c.positions, bq, bk)
    torch.cuda.synchronize()
    assert torch.equal(se, sc)
    for x, y in zip(e.fetch(), c.fetch()):
        assert np.array_equal(x, y)


def test_prepared_calls_equal_direct_calls():
    """PreparedCall (arguments marshalled once, as the benchmark launches) gives
    the same bits as the direct binding calls, for the fused op, the unfused
    pair and the LayerNorm sibling."""
    import torch
    from head_qk_rmsnorm_amd import binding as B

    cfg = W.case(47, 5, 3, 128, 64, True, pos_dtype=W.I64, seed=77)
    wl = W.make_workload(cfg)
    kw = dict(is_neox=True, eps=cfg.eps)
    bias = (torch.linspace(-1, 1, 128, device="cuda").to(torch.bfloat16),
            torch.linspace(1, -1, 128, device="cuda").to(torch.bfloat16))
    cases = [
        (lambda d: B.PreparedCall(d.q, d.k, d.wq, d.wk, d.cache, d.positions, **kw),
         lambda d: B.qknr_inplace(d.q, d.k, d.wq, d.wk, d.cache, d.positions, **kw)),
        (lambda d: B.PreparedCall(d.q, d.k, d.wq, d.wk, d.cache, d.positions, unfused=True, **kw),
         lambda d: B.qknr_unfused_inplace(d.q, d.k, d.wq, d.wk, d.cache, d.positions, **kw)),
        (lambda d: B.PreparedCall(d.q, d.k, d.wq, d.wk, d.cache, d.positions, layernorm_bias=bias,
                                  **kw),
         lambda d: B.qknr_layernorm_rope_inplace(d.q, d.k, d.wq, d.wk, bias[0], bias[1], d.cache,
                                                 d.positions, **kw)),
    ]
    for make, direct in cases:
        a, b = Hn.DeviceCase(wl), Hn.DeviceCase(wl)
        call = make(a)
        call()
        call()  # twice in place
        direct(b)
        direct(b)
        torch.cuda.synchronize()
        for x, y in zip(a.fetch(), b.fetch()):
            assert np.array_equal(x, y)


def test_binding_rejects_bad_tensors_before_launching():
    """The Python binding checks shapes, dtypes and layouts before any launch;
    every rejection leaves q and k as they were."""
    import torch
    from head_qk_rmsnorm_amd import binding as B

    cfg = W.case(9, 4, 2, 128, 128, False, seed=78)
    wl = W.make_workload(cfg)
    d = Hn.DeviceCase(wl)
    q, k, wq, wk, cache, pos = d.q, d.k, d.wq, d.wk, d.cache, d.positions
    bad = [
        (ValueError, lambda: B.qknr_inplace(q[:, :, :64], k, wq, wk, cache, pos, is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q, k[:5], wq, wk, cache, pos, is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q[..., ::2], k[..., ::2], wq[::2], wk[::2],
                                            cache[:, :64].contiguous(), pos, is_neox=False)),
        (TypeError, lambda: B.qknr_inplace(q, k.half(), wq, wk, cache, pos, is_neox=False)),
        (TypeError, lambda: B.qknr_inplace(q, k, wq.half(), wk, cache, pos, is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q, k, wq[:64], wk, cache, pos, is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q, k, wq, wk, cache.double(), pos, is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q, k, wq, wk, cache, pos[:3], is_neox=False)),
        (TypeError, lambda: B.qknr_inplace(q, k, wq, wk, cache, pos.float(), is_neox=False)),
        (ValueError, lambda: B.qknr_inplace(q.reshape(9, 4 * 128), k, wq, wk, cache, pos,
                                            is_neox=False)),
        (ValueError, lambda: B.qknr_layernorm_rope_inplace(q, k, wq, wk, wq, None)),
        (ValueError, lambda: B.PreparedCall(q, k, wq, wk, cache, pos, is_neox=False, unfused=True,
                                            launch={"unroll": 1})),
    ]
    for i, (exc, fn) in enumerate(bad):
        with pytest.raises(exc):
            fn()
        torch.cuda.synchronize()
    for before, after in zip(d.storages_host, d.fetch()):
        assert np.array_equal(before, after)
