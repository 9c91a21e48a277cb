"""Host-side checks of the kernels' work decomposition: the C++ functions
the kernels use (itl_config.h, loss_plan.h, sampled_plan.h), compiled into
host programs with hipcc. The logprob kernels over a few thousand (n_tok,
vocab) pairs: every (token block, slice) pair computed once, slices tiling
the vocabulary, the narrow grid's coverage. The loss's token pass over
seeded response layouts. The backward's sampled term over seeded id arrays.
The programs run under the host address and undefined-behaviour sanitizers.
No GPU needed."""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# The checks are host programs (no device code); they are built with the
# address and undefined-behaviour sanitizers on the host side, so an
# out-of-range index or an overflow in the shared index arithmetic aborts.
SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


def _build_host_check(tmp_path_factory, name):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp(name) / name)
    cmd = [hipcc, "-O1", "-g", "-std=c++17", *SANITIZE, "-I", os.path.join(ROOT, "invariant_token_logprobs_lm_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", name + ".cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def grid_check(tmp_path_factory):
    return _build_host_check(tmp_path_factory, "grid_check")


def _run(exe, pairs):
    args = [str(x) for p in pairs for x in p]
    r = subprocess.run([exe, *args], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_workload_shapes(grid_check):
    pairs = [(1, 151936), (64, 151936), (65, 151936), (256, 151936), (2048, 151936), (2049, 151936),
             (133010, 151936), (294884, 151936), (308010, 129280), (1, 1), (5, 1), (64, 3), (700, 5000),
             (300, 4133), (513, 8448), (5200, 38383), (16684, 2000), (177, 1024)]
    _run(grid_check, pairs)


def test_random_shapes(grid_check):
    rng = np.random.default_rng(0)
    n = rng.integers(1, 40000, 600)
    v = rng.integers(1, 300000, 600)
    _run(grid_check, list(zip(n.tolist(), v.tolist())))
    # around the slice-count and group thresholds
    pairs = [(nt, vv) for nt in (1, 63, 64, 65, 255, 256, 257, 2048, 2304, 8192)
             for vv in (255, 256, 257, 65535, 65536, 65537, 65536 + 256, 131071, 200000)]
    _run(grid_check, pairs)


@pytest.fixture(scope="module")
def loss_plan_check(tmp_path_factory):
    return _build_host_check(tmp_path_factory, "loss_plan_check")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_loss_token_pass_decomposition(loss_plan_check, seed):
    """The loss's token pass (loss_plan.h): spans tile the batch, every token
    in exactly one response-relative segment owned by one window, at most one
    start of a response per span, every overlapping response enumerated, the
    segment-sum slots of different responses disjoint; 300 seeded layouts
    (tiny, short, around one segment, long, mixed, a single long response)."""
    r = subprocess.run([loss_plan_check, str(seed), "300"], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.fixture(scope="module")
def sampled_plan_check(tmp_path_factory):
    return _build_host_check(tmp_path_factory, "sampled_plan_check")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_sampled_term_decomposition(sampled_plan_check, seed):
    """The backward's sampled term (sampled_plan.h): the counting sort's
    per-block counts, digit-major scan and in-order placement give the
    stable sort by id over every pass; every token of a valid id in exactly
    one segment, every segment of a long run in one group; segment and group
    slots of different runs disjoint and in range; 60 seeded id arrays (flat,
    one id at 40 %, a single id, out-of-range ids, empty and tiny)."""
    r = subprocess.run([sampled_plan_check, str(seed), "60"], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
