"""The C ABI's host code under the address + undefined-behaviour sanitizers and under
the thread sanitizer (CPU only).

Every library source is compiled with the sanitizer on its host side only (each
``-fsanitize=`` behind ``-Xarch_host``; device code is built as usual and never runs),
and linked into ``tests/host_sanitize/driver.cpp``, which calls every entry point from
several threads with seeded edge-case arguments.  Each call must return the status
the header's contract gives; calls that would pass validation are made to fail by a
workspace or cache one byte short, so nothing is ever enqueued, and the driver hides
every GPU from itself as well.  The size arithmetic of the workspace and cache planners
runs at the largest sizes the contract admits (B*S = 2^30 tokens, 65535 heads), where
a signed overflow is a UBSan error and a wrapped size fails the driver's lower bound.
"""

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from int8_w8a8_flashattention_amd import build_lib

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_sanitize", "driver.cpp")

VARIANTS = {
    # instrumentation flags for the host compiler
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                   "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


def _tools():
    try:
        hipcc = build_lib.hipcc()
    except RuntimeError:
        return None
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    for c in (clang, "/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return hipcc, os.path.realpath(c)
    return None


TOOLS = _tools()
pytestmark = pytest.mark.skipif(TOOLS is None, reason="hipcc / clang++ not found")


def _host(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}")


def _build(variant, bdir):
    hipcc, clang = TOOLS
    san = VARIANTS[variant]
    os.makedirs(bdir, exist_ok=True)
    flags = [f for f in build_lib.FLAGS if f != "-Wall"] + ["-g"] + _host(san)
    jobs = []
    for src in build_lib.SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        jobs.append([hipcc, *flags, *build_lib.EXTRA_FLAGS.get(src, []), "-c",
                     os.path.join(build_lib.CSRC, src), "-o", obj])
    drv_obj = os.path.join(bdir, "driver.o")
    # The driver is plain C++: the host compiler alone, with the same instrumentation.
    jobs.append([clang, "-O1", "-g", "-std=c++17", *san, f"-I{build_lib.INCLUDE}", "-c",
                 DRIVER, "-o", drv_obj])
    return jobs, bdir


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    root = tmp_path_factory.mktemp("host_sanitize")
    plans = [_build(v, str(root / v)) for v in VARIANTS]
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        list(ex.map(_run, [j for jobs, _ in plans for j in jobs]))
    hipcc, _ = TOOLS
    exes = {}
    for v, (_, bdir) in zip(VARIANTS, plans):
        objs = sorted(os.path.join(bdir, f) for f in os.listdir(bdir) if f.endswith(".o"))
        exe = os.path.join(bdir, "driver")
        _run([hipcc, f"--offload-arch={build_lib.ARCH}", *_host(VARIANTS[v][:1]), *objs,
              "-o", exe])
        exes[v] = exe
    return exes


def _drive(exe, iters, threads):
    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1",
               HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe, str(iters), str(threads)], capture_output=True, text=True,
                       env=env, timeout=300)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "Sanitizer" not in log and "runtime error" not in log, log[-4000:]
    m = re.search(r"calls=(\d+) ok=(\d+) invalid_arg=(\d+) head_dim=(\d+) "
                  r"workspace_too_small=(\d+) failures=(\d+)", log)
    assert m, log[-2000:]
    calls, ok, inval, hdim, small, fails = map(int, m.groups())
    assert fails == 0
    # every outcome of the contract is reached many times
    assert min(ok, inval, hdim, small) >= 100, m.group(0)
    return calls


def test_address_and_undefined_behaviour_sanitizers(drivers):
    assert _drive(drivers["asan_ubsan"], 40000, 4) > 300000


def test_thread_sanitizer_per_thread_errors(drivers):
    assert _drive(drivers["tsan"], 20000, 8) > 300000
