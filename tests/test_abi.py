"""Host-side tests of the C ABI (no GPU needed, no kernel launched).

The library loads, exports every function include/itl.h declares, and
rejects invalid arguments with the documented status before touching the
device. Also static checks on the sources: no float atomics in kernels, and
the oracle and the product path never import each other.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "itl.h")
CSRC = os.path.join(ROOT, "invariant_token_logprobs_lm_amd", "csrc")
LIB = os.path.join(ROOT, "invariant_token_logprobs_lm_amd", "libitl.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(itl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libitl.so is not built (run python -m invariant_token_logprobs_lm_amd.build)")
    import invariant_token_logprobs_lm_amd as itl

    return itl.lib


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["itl_lmhead_logprob", "itl_group_advantage", "itl_reinforce_zero_loss",
              "itl_reinforce_zero_backward", "itl_check_inputs", "itl_build_info"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    import invariant_token_logprobs_lm_amd as itl

    assert sorted(itl.EXPORTS) == _declared()


def test_build_info_and_status_strings(lib):
    info = lib.itl_build_info().decode()
    assert "gfx950" in info and "max_slices=256" in info
    for s in range(6):
        assert lib.itl_status_string(s)


def _lmhead(lib, H=256, W=256, dtype=0, n=4, d=64, V=10, y=1, lp=1, ws=256, wsb=1 << 20):
    v = ctypes.c_void_p
    return lib.itl_lmhead_logprob(v(H), v(W), dtype, n, d, V, v(y), v(lp), None, v(ws), wsb, None)


def test_lmhead_argument_validation(lib):
    assert _lmhead(lib, n=-1) == INVALID
    assert _lmhead(lib, d=0) == INVALID
    assert _lmhead(lib, V=0) == INVALID
    assert _lmhead(lib, d=96) == UNSUPPORTED
    assert _lmhead(lib, dtype=7) == UNSUPPORTED
    assert _lmhead(lib, H=0) == INVALID
    assert _lmhead(lib, y=0) == INVALID
    assert _lmhead(lib, H=264) == INVALID  # H and W 16-byte aligned
    assert _lmhead(lib, W=258) == INVALID
    assert "16-byte" in lib.itl_last_error().decode()
    assert _lmhead(lib, ws=0) == WORKSPACE
    assert _lmhead(lib, wsb=16) == WORKSPACE
    assert _lmhead(lib, ws=255) == WORKSPACE
    assert "workspace" in lib.itl_last_error().decode()
    assert _lmhead(lib, n=0, H=0, W=0, y=0, lp=0, ws=0) == OK  # empty call is a no-op
    assert lib.itl_last_error().decode() == ""


def test_noalloc_argument_validation(lib):
    """Host-side checks of itl_lmhead_logprob_noalloc, all before any HIP call."""
    v = ctypes.c_void_p
    f = lib.itl_lmhead_logprob_noalloc
    assert f(v(1), v(1), 0, -1, 64, 10, v(1), v(1), None, None) == INVALID
    assert f(v(1), v(1), 0, 4, 96, 10, v(1), v(1), None, None) == UNSUPPORTED
    assert f(None, v(1), 0, 4, 64, 10, v(1), v(1), None, None) == INVALID
    assert f(None, None, 0, 0, 64, 10, None, None, None, None) == OK
    assert f(v(8), v(256), 0, 4, 64, 10, v(1), v(1), None, None) == INVALID  # H, W 16-byte aligned
    # the static scratch holds 64 MiB: 16,368 tokens at 256 slices
    assert f(v(256), v(256), 0, 16369, 64, 151936, v(1), v(1), None, None) == UNSUPPORTED
    assert "scratch" in lib.itl_last_error().decode()
    assert lib.itl_lmhead_logprob_workspace_bytes(16368, 151936) == 64 << 20


def test_workspace_sizes(lib):
    assert lib.itl_lmhead_logprob_workspace_bytes(0, 100) == 0
    # one (max, sumexp) float pair per token, slice and wavefront (2 per
    # slice), slices = min(vocabulary tiles, 256); then one float per token
    for n, V, slices in ((1000, 151936, 256), (1000, 5000, 20), (3, 1, 1)):
        want = -(-2 * slices * n * 8 // 256) * 256 + -(-n * 4 // 256) * 256
        assert lib.itl_lmhead_logprob_workspace_bytes(n, V) == want
    assert lib.itl_lmhead_logprob_workspace_bytes(-1, V) == ctypes.c_size_t(-1).value


def test_loss_workspace_sizes(lib):
    w = lib.itl_reinforce_zero_loss_workspace_bytes
    r = lambda x: -(-x // 256) * 256
    assert w(0, 0) == 0 and w(100, 0) == 0
    # fp64 per-response losses, two fp64 slots per 2048-token window (+2),
    # one fp64 partial per 1024 responses; above 512 responses, a 24-byte
    # holder per 2048-token window
    for n_tok, n_resp in ((10, 3), (294884, 32), (300000, 512), (300000, 513), (16 * 2 ** 20, 2 ** 21)):
        want = r(8 * n_resp) + r(8 * 2 * (-(-n_tok // 2048) + 1)) + r(8 * -(-n_resp // 1024))
        if n_resp > 512:
            want += r(24 * -(-n_tok // 2048))
        assert w(n_tok, n_resp) == want
    assert w(-1, 3) == ctypes.c_size_t(-1).value and w(3, -1) == ctypes.c_size_t(-1).value


def test_loss_and_advantage_validation(lib):
    v = ctypes.c_void_p
    assert lib.itl_group_advantage(v(1), v(1), -1, 4, v(1), None) == INVALID
    assert lib.itl_group_advantage(None, v(1), 2, 4, v(1), None) == INVALID
    assert lib.itl_group_advantage(None, None, 0, 0, None, None) == OK
    loss = lib.itl_reinforce_zero_loss
    assert loss(v(1), v(1), v(1), v(1), -1, 4, v(1), v(1), None, v(256), 1 << 20, None) == INVALID
    assert loss(v(1), v(1), v(1), None, 2, 4, v(1), v(1), None, v(256), 1 << 20, None) == INVALID
    assert loss(None, None, None, None, 0, 0, None, None, None, None, 0, None) == OK
    # workspace checked before anything is launched
    assert loss(v(1), v(1), v(1), v(1), 2, 4, v(1), v(1), None, None, 1 << 20, None) == WORKSPACE
    assert loss(v(1), v(1), v(1), v(1), 2, 4, v(1), v(1), None, v(256), 8, None) == WORKSPACE
    assert loss(v(1), v(1), v(1), v(1), 2, 4, v(1), v(1), None, v(257), 1 << 20, None) == WORKSPACE
    assert lib.itl_reinforce_zero_backward(v(1), v(1), 0, 4, 100, 10, v(1), v(1), v(1), v(1), v(1),
                                           v(256), 1 << 30, None) == UNSUPPORTED
    assert lib.itl_reinforce_zero_backward(v(1), None, 0, 4, 64, 10, v(1), v(1), v(1), v(1), v(1),
                                           v(256), 1 << 30, None) == INVALID
    # H, W, dH and dW 16-byte aligned (the sampled term's row loads and stores)
    assert lib.itl_reinforce_zero_backward(v(1), v(16), 0, 4, 64, 10, v(1), v(1), v(1), v(16), v(16),
                                           v(256), 1 << 40, None) == INVALID
    assert lib.itl_reinforce_zero_backward(v(16), v(16), 0, 4, 64, 10, v(1), v(1), v(1), v(16), v(8),
                                           v(256), 1 << 40, None) == INVALID
    # workspace checked before anything is launched
    assert lib.itl_reinforce_zero_backward(v(16), v(16), 0, 4, 64, 10, v(1), v(1), v(1), v(16), v(16),
                                           v(256), 16, None) == WORKSPACE
    assert lib.itl_reinforce_zero_backward(v(16), v(16), 0, 4, 64, 10, v(1), v(1), v(1), v(16), v(16),
                                           v(257), 1 << 40, None) == WORKSPACE


def test_kept_logits_argument_validation(lib):
    """The kept-logits entry points check the logits buffer before anything
    is launched: present, 16-byte aligned, a row stride >= vocab that is a
    multiple of 4 and small enough for 32-bit offsets over 128 rows."""
    v = ctypes.c_void_p

    def keep(Z=256, ld=12, n=4, V=10):
        return lib.itl_lmhead_logprob_keep_logits(v(256), v(256), 0, n, 64, V, v(256), v(256), None, v(Z), ld,
                                                  v(256), 1 << 20, None)

    assert keep(Z=0) == INVALID
    assert keep(ld=8) == INVALID          # below vocab
    assert keep(ld=14) == INVALID         # not a multiple of 4
    assert keep(Z=264) == INVALID         # not 16-byte aligned
    assert lib.itl_lmhead_logprob_keep_logits(v(256), v(260), 0, 4, 64, 10, v(256), v(256), None, v(256), 12,
                                              v(256), 1 << 20, None) == INVALID  # W not 16-byte aligned
    assert keep(ld=1 << 24) == UNSUPPORTED
    assert "ld_logits" in lib.itl_last_error().decode()
    assert keep(n=0, Z=0) == OK           # empty call is a no-op

    def bwd(Z=256, ld=12, n=4, V=10, ws=1 << 30):
        return lib.itl_reinforce_zero_backward_from_logits(v(256), v(256), 0, n, 64, V, v(256), v(256), v(256),
                                                           v(Z), ld, v(256), v(256), v(256), ws, None)

    assert bwd(Z=0) == INVALID
    assert bwd(ld=9) == INVALID
    assert bwd(ws=16) == WORKSPACE        # the rest as for itl_reinforce_zero_backward


def test_backward_workspace_sizes(lib):
    f = lib.itl_reinforce_zero_backward_workspace_bytes
    bf16 = f(1000, 256, 5000, 0)
    f32 = f(1000, 256, 5000, 1)
    assert 0 < bf16 < f32 < (1 << 40)
    assert f(-1, 256, 5000, 0) == ctypes.c_size_t(-1).value
    assert f(10, 256, 5000, 7) == ctypes.c_size_t(-1).value
    # transposed W and chunk buffers dominate: at least W^T plus two dlogit copies
    assert bf16 >= 256 * 5120 * 2 + 2 * 16384 * 5120 * 2


def test_binding_rejects_bad_tensors():
    import torch
    import invariant_token_logprobs_lm_amd as itl

    H = torch.zeros(4, 64, dtype=torch.bfloat16)
    W = torch.zeros(10, 64, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):  # CPU tensors are not device memory
        itl.lmhead_logprob(H, W, y)
    with pytest.raises(ValueError):
        itl.lmhead_logprob(H.float(), W, y)
    with pytest.raises(TypeError):
        itl.group_advantage([1.0], torch.zeros(2, dtype=torch.int32))


def _sources(folder, exts):
    for dp, _, fs in os.walk(folder):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


# The only atomics allowed: integer counters of the diagnostics' exact median
# (histogram counts and candidate slots) and of the backward's counting sort
# (digit counts in LDS), whose result cannot depend on the order the
# additions land in. Every floating-point result has a fixed order.
_INTEGER_ATOMIC_FILES = {"diagnostics.hip", "sampled.hip"}


def test_no_float_atomics_in_kernels():
    for p in _sources(CSRC, (".hip", ".h")):
        text = open(p).read()
        assert "unsafeAtomic" not in text, p
        calls = re.findall(r"\batomic\w*\s*\(([^;]*)", text)
        if os.path.basename(p) not in _INTEGER_ATOMIC_FILES:
            assert not calls, p
            continue
        for c in calls:  # unsigned counts and bounds only
            assert "1u" in c or "lh[i]" in c or c.startswith(("&pmin", "&pmax")), (p, c)
        assert not re.search(r"\batomic(?!Add|Min|Max)\w*\s*\(", text), p


def test_oracle_and_product_are_independent():
    pkg = os.path.join(ROOT, "invariant_token_logprobs_lm_amd")
    for p in _sources(pkg, (".py", ".hip", ".h", ".cpp")):
        assert not re.search(r"\boracle\b", open(p).read()), p
    for p in _sources(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = open(p).read()
        assert "invariant_token_logprobs_lm_amd" not in text and "import synth" not in text, p


def test_mismatch_stats_validation(lib):
    v = ctypes.c_void_p
    f = lib.itl_mismatch_stats
    assert f(v(1), v(1), None, -1, v(8), v(256), 1 << 20, None) == INVALID
    assert f(v(1), v(1), None, 10, None, v(256), 1 << 20, None) == INVALID
    assert f(None, v(1), None, 10, v(8), v(256), 1 << 20, None) == INVALID
    assert f(v(1), v(1), None, 1 << 31, v(8), v(256), 1 << 40, None) == UNSUPPORTED
    assert f(v(1), v(1), None, 10, v(8), v(256), 16, None) == WORKSPACE
    assert f(v(1), v(1), None, 10, v(8), v(257), 1 << 20, None) == WORKSPACE
    w = lib.itl_mismatch_stats_workspace_bytes
    assert w(0) == 0 and w(-1) == ctypes.c_size_t(-1).value and w(1 << 31) == ctypes.c_size_t(-1).value
    assert w(1000) >= 16 * 1000 and w(100000) > w(1000)


def test_mismatch_stat_fields_match_header_and_oracle():
    import invariant_token_logprobs_lm_amd as itl
    import oracle

    text = open(HEADER).read()
    enum = re.findall(r"\bITL_STAT_([A-Z0-9_]+)\b", text)
    enum = [e.lower() for e in dict.fromkeys(enum) if e != "COUNT"]
    assert tuple(enum) == itl.STAT_FIELDS == oracle.STAT_NAMES


def test_probe_library_is_separate_and_loads():
    """The benchmark's matrix-core probe lives in its own library; libitl.so
    does not export it."""
    probe = ctypes.CDLL(os.path.join(ROOT, "libitl_bench_probe.so"))
    for name in ("itl_probe_operand_bytes", "itl_probe_threads", "itl_probe_flops", "itl_probe_mfma_bf16"):
        assert hasattr(probe, name)
    probe.itl_probe_operand_bytes.restype = ctypes.c_size_t
    assert probe.itl_probe_operand_bytes() == 4096 * 16 * 16
    assert [probe.itl_probe_threads(s) for s in (0, 1, 2)] == [256, 512, 0]
    probe.itl_probe_flops.restype = ctypes.c_double
    probe.itl_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    # per round: 4 wavefronts x 16 MFMAs of 32x32x16, or 8 x 32 of 16x16x32
    assert probe.itl_probe_flops(0, 3, 5) == 3 * 5 * 4 * 16 * (2 * 32 * 32 * 16)
    assert probe.itl_probe_flops(1, 3, 5) == 3 * 5 * 8 * 32 * (2 * 16 * 16 * 32)
    probe.itl_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    # an unknown shape is refused before any launch
    assert probe.itl_probe_mfma_bf16(2, 1, 1, 1, 1, None) != 0
    import invariant_token_logprobs_lm_amd as itl

    assert not hasattr(itl.lib, "itl_probe_mfma_bf16")


def test_fp8_validation(lib):
    v = ctypes.c_void_p
    q = lib.itl_quantize_rows_fp8
    assert q(v(1), 0, -1, 128, v(4), v(4), None) == INVALID
    assert q(v(1), 0, 4, 96, v(4), v(4), None) == UNSUPPORTED
    assert q(v(1), 7, 4, 128, v(4), v(4), None) == UNSUPPORTED
    assert q(v(1), 0, 4, 128, v(5), v(4), None) == INVALID  # Xq misaligned
    assert q(None, 0, 4, 128, v(4), v(4), None) == INVALID
    assert q(None, 0, 0, 128, None, None, None) == OK
    f = lib.itl_lmhead_logprob_fp8
    args = lambda **k: [v(k.get("Hq", 16)), v(4), v(k.get("Wq", 16)), v(4), k.get("n", 4), k.get("d", 128),
                        k.get("V", 10), v(4), v(4), None, v(k.get("ws", 256)), k.get("wsb", 1 << 20), None]
    assert f(*args(d=64)) == UNSUPPORTED
    assert f(*args(n=-1)) == INVALID
    assert f(*args(Hq=8)) == INVALID       # 16-byte alignment
    assert f(*args(wsb=16)) == WORKSPACE
    assert f(*args(ws=255)) == WORKSPACE
    assert f(*args(n=0, Hq=0, Wq=0)) == OK


def test_mxfp4_validation(lib):
    v = ctypes.c_void_p
    q = lib.itl_quantize_rows_mxfp4
    assert q(v(1), 0, 4, 96, v(16), v(4), None) == UNSUPPORTED
    assert q(v(1), 0, 4, 128, v(8), v(4), None) == INVALID   # Xq must be 16-byte aligned
    assert q(None, 0, 0, 128, None, None, None) == OK
    f = lib.itl_lmhead_logprob_mxfp4
    args = lambda **k: [v(16), v(4), v(k.get("Wq", 16)), v(k.get("sc", 4)), k.get("n", 4), k.get("d", 128), 10,
                        v(4), v(4), None, v(256), 1 << 20, None]
    assert f(*args(d=64)) == UNSUPPORTED
    assert f(*args(Wq=8)) == INVALID
    assert f(*args(sc=2)) == INVALID
    assert f(*args(n=0)) == OK
