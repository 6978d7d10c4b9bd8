"""The library's host code under AddressSanitizer (CPU only).

The host part (validation, planning, launch report: csrc/qknr.hip) is compiled
with AddressSanitizer on its host pass only (device code is built as usual),
linked with the kernel table into a separate shared library in a temporary
folder, and driven by the plain-C program tests/capi/qknr_validate.c, built
with AddressSanitizer too: every rejection path of the entry points, empty
work, qknr_can_use over a grid of shapes, the status strings and, with no
device present, valid calls through every planner (they stop at the device
query). An invalid host memory access aborts the run and fails the test.
"""
import glob
import os
import subprocess

import pytest

from head_qk_rmsnorm_amd import build as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "capi", "qknr_validate.c")


def _tools():
    try:
        hipcc = Bd.hipcc()
    except RuntimeError:
        return None
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    rt = glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                "libclang_rt.asan-x86_64.a"))
    if not (os.path.exists(clang) and rt):
        return None
    return hipcc, clang, rocm


@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="a GPU is visible; this check is meant for a machine without one")
def test_host_code_under_address_sanitizer(tmp_path):
    tools = _tools()
    if tools is None:
        pytest.skip("hipcc, clang or the AddressSanitizer runtime not found")
    hipcc, clang, rocm = tools
    import concurrent.futures as cf

    objdir = str(tmp_path)
    cmds = Bd.compile_cmds(objdir)
    # the host code (last command) again with the sanitizer on its host pass
    host_obj, host_cmd = cmds[-1]
    host_cmd = [a for a in host_cmd if a != "-O3"]
    i = host_cmd.index("-c")
    host_cmd[i:i] = ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                     "-Xarch_host", "-fno-omit-frame-pointer"]
    cmds[-1] = (host_obj, host_cmd)
    jobs = min(len(cmds), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda c: subprocess.run(c[1], capture_output=True, text=True), cmds))
    for (_, cmd), r in zip(cmds, results):
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
    lib = os.path.join(objdir, "libqknr_asan.so")
    link = [hipcc, f"--offload-arch={Bd.ARCH}", "-shared", "-fPIC", "-o", lib,
            *[o for o, _ in cmds]]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(objdir, "qknr_validate")
    cc = [clang, "-O1", "-g", "-std=c99", "-fsanitize=address", "-fno-omit-frame-pointer",
          "-D__HIP_PLATFORM_AMD__", "-I", Bd.INCLUDE, "-I", os.path.join(rocm, "include"),
          "-o", exe, DRIVER, "-L", objdir, "-lqknr_asan", "-L", os.path.join(rocm, "lib"),
          "-lamdhip64", "-lm", f"-Wl,-rpath,{objdir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout, r.stdout
