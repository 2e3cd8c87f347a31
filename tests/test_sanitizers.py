"""The CPU tests again, under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; no GPU).

  - The library's argument validation (attn_api.cpp: every check that runs
    before a HIP call) is compiled with host sanitizers and linked with the
    kernel objects of the regular build; tests/test_abi.py then runs against it
    in a child process with the sanitizer runtime preloaded.
  - The fp64 oracle (oracle/attn_oracle.c) is compiled with gcc's sanitizers,
    and the oracle tests run against it the same way.

Any sanitizer report stops the child (halt_on_error) and fails the test, with
the report in the message.  Leak checking is off: the Python interpreter
itself keeps allocations alive until exit.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from exact_attention_87_amd import _build  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_build.HIPCC) or
                                not os.path.exists("/usr/bin/gcc"),
                                reason="needs hipcc and gcc")

# Each sanitizer flag goes to the host compiler only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def _run_child(tests, env_extra, logdir, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = ("detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:"
                           f"log_path={logdir}/asan")
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logdir}/ubsan"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=timeout)
    reports = ""
    for f in sorted(glob.glob(os.path.join(logdir, "*san*"))):
        with open(f) as fh:
            reports += fh.read()[:4000]
    return res, reports


def _preload(runtime):
    cur = os.environ.get("LD_PRELOAD", "")
    return runtime + (":" + cur if cur else "")


def test_argument_validation_under_sanitizers(tmp_path):
    # kernel objects of the regular build (compiled now if there are none)
    kernels = [s for s in _build.SOURCES if s != "attn_api.cpp"]
    if not all(os.path.exists(_build.object_path(s)) for s in kernels):
        _build.build()
    api_obj = str(tmp_path / "attn_api_san.o")
    lib = str(tmp_path / "libattn_san.so")
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([_build.HIPCC, *flags, *HOST_SANITIZE, "-c",
                    os.path.join(_build.CSRC, "attn_api.cpp"), "-o", api_obj],
                   check=True, capture_output=True, text=True, timeout=600)
    subprocess.run([_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZE,
                    api_obj, *[_build.object_path(s) for s in kernels], "-o", lib],
                   check=True, capture_output=True, text=True, timeout=600)
    runtime = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, check=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    logdir = tmp_path / "logs"
    logdir.mkdir()
    res, reports = _run_child(["tests/test_abi.py"],
                              {"LD_PRELOAD": _preload(runtime), "ATTN_TEST_LIB_PATH": lib},
                              str(logdir))
    assert res.returncode == 0 and not reports, (res.stdout[-3000:] + res.stderr[-2000:] + reports)


def test_oracle_under_sanitizers(tmp_path):
    src = os.path.join(ROOT, "oracle", "attn_oracle.c")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-std=c99", "-Wall", "-Wextra", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared",
                    "-fPIC", src, "-o", lib, "-lm"], check=True, capture_output=True, text=True,
                   timeout=300)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    logdir = tmp_path / "logs"
    logdir.mkdir()
    tests = sorted(os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "tests",
                                                                             "test_oracle_*.py")))
    assert tests
    res, reports = _run_child(tests, {"LD_PRELOAD": _preload(runtime),
                                      "ATTN_TEST_ORACLE_LIB_PATH": lib}, str(logdir))
    assert res.returncode == 0 and not reports, (res.stdout[-3000:] + res.stderr[-2000:] + reports)
