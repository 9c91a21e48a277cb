"""The C ABI's argument validation and workspace sizing under the host
address and undefined-behaviour sanitizers (CPU only).

Every csrc/*.hip source is compiled with the library's flags plus host-side
sanitizers (device code is compiled as usual and never runs here) and linked
with tests/host/abi_check.cpp, which calls every entry point with sizes from
INT64_MIN to INT64_MAX, bad dtypes and null pointers: each call must return a
status (or SIZE_MAX) before any device work, with no signed overflow,
out-of-bounds access or crash on the host.
"""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

from invariant_token_logprobs_lm_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def abi_check(tmp_path_factory):
    hipcc = build.HIPCC
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("abi_asan")
    flags = [f for f in build.DEVICE_FLAGS if f != "-O3"] + ["-O1", "-g", *SANITIZE]

    def compile_one(src):
        obj = str(out / (os.path.basename(src)[:-4] + ".o"))
        r = subprocess.run([hipcc, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, build.sources()))
    driver = str(out / "abi_check_main.o")
    r = subprocess.run([hipcc, *flags, "-c", os.path.join(ROOT, "tests", "host", "abi_check.cpp"), "-o", driver],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(out / "abi_check")
    r = subprocess.run([hipcc, f"--offload-arch={build.ARCH}", *SANITIZE, driver, *objs, "-o", exe,
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


def test_abi_validation_under_sanitizers(abi_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([abi_check], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.stdout + r.stderr)[-4000:]
