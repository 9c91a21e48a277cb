"""Properties of the compiled device code (CPU only: hipcc cross-compiles).

* The FP8 kernels fetch their row scales with loads issued from inline
  assembly and wait for them with an explicit s_waitcnt later on (the
  compiler cannot see those loads complete). Between a load and its wait
  nothing may read or write the destination register -- a spill, copy or
  reuse placed there by the register allocator would act on a value that
  has not arrived. This test finds every such load in the generated
  assembly and checks the instructions up to the next vmcnt wait.
* The logprob kernels and the backward's contractions compile without
  scratch (no register spills): a spill reload makes the compiler wait for
  every outstanding load, including the operand tiles in flight into LDS.
  So do the sampled term's row-sum kernels.
"""

import os
import re
import shutil
import subprocess

import pytest

from invariant_token_logprobs_lm_amd import build

HIPCC = build.HIPCC
needs_hipcc = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")

ASM_LOAD = re.compile(r"^\s*buffer_load_dword (v\d+), v\d+, s\[\d+:\d+\], 0 offen\s*$")
VMCNT = re.compile(r"s_waitcnt vmcnt\(\d+\)")


def _compile(src, out_dir, extra=()):
    flags = [f for f in build.DEVICE_FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, "--cuda-device-only", *extra, src]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=out_dir)
    assert r.returncode == 0, r.stderr[-3000:]
    return r


def _kernels(asm):
    """Map kernel symbol -> list of instruction lines."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_ZN3itl\S+):", line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name and line.startswith(".Lfunc_end"):
            name = None
            continue
        if name:
            out[name].append(line)
    return out


def _regs(text):
    regs = set()
    for a, b in re.findall(r"v\[(\d+):(\d+)\]", text):
        regs.update(range(int(a), int(b) + 1))
    regs.update(int(r) for r in re.findall(r"\bv(\d+)\b", text))
    return regs


@needs_hipcc
def test_asm_scale_loads_are_not_touched_before_their_wait(tmp_path):
    src = os.path.join(build.CSRC, "fp8.hip")
    out = str(tmp_path / "fp8.s")
    _compile(src, str(tmp_path), ("-S", "-o", out))
    kernels = _kernels(open(out).read())
    checked = 0
    for name, body in kernels.items():
        for i, line in enumerate(body):
            m = ASM_LOAD.match(line)
            if not m:
                continue
            reg = int(m.group(1)[1:])
            j = i + 1
            while j < len(body) and not VMCNT.search(body[j]):
                text = body[j].split(";")[0]
                if text.strip() and not ASM_LOAD.match(body[j]):
                    assert reg not in _regs(text), (name, body[i].strip(), body[j].strip())
                j += 1
            assert j < len(body), (name, "no wait after", body[i].strip())
            checked += 1
    # two loads in the wide FP8 kernel, two per path in the narrow one
    assert checked >= 4, checked


@needs_hipcc
@pytest.mark.parametrize("src,kernel", [
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi0ELb0E"),  # bf16, logits not kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi1ELb0E"),  # fp32, logits not kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi0ELb1E"),  # bf16, logits kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi1ELb1E"),  # fp32, logits kept
    ("lmhead.hip", "lmhead_lse_partial_narrow_kernelILi0ELb0E"),
    ("fp8.hip", "lmhead_fp8_partial_kernel"),
    ("fp8.hip", "lmhead_mxfp4_partial_kernel"),
    ("backward.hip", "dlogits_kernelILi0E"),  # the backward's contractions, on the eight-wavefront engine
    ("backward.hip", "dh_kernelILi0E"),
    ("backward.hip", "dw_kernelILi0E"),
    ("backward.hip", "dlogits_kernelILi1E"),
    ("backward.hip", "dh_kernelILi1E"),
    ("backward.hip", "dw_kernelILi1E"),
    ("sampled.hip", "short_rows_kernel"),  # the sampled term's row sums
    ("sampled.hip", "segment_sums_kernel"),
])
def test_wide_kernels_have_no_scratch(tmp_path, src, kernel):
    r = _compile(os.path.join(build.CSRC, src), str(tmp_path),
                 ("-c", "-o", str(tmp_path / "x.o"), "-Rpass-analysis=kernel-resource-usage"))
    seen = 0
    current = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and current and kernel in current:
            assert int(m.group(1)) == 0, (current, line)
            seen += 1
    assert seen >= 1, f"no resource report for {kernel}"
