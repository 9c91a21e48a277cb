"""Properties of the compiled device code (CPU only: hipcc cross-compiles).

* Every load issued from inline assembly writes LDS (the `lds` form of
  the buffer load), never a register: the compiler takes an asm output
  register as written when the statement ends, so a register load still in
  flight there could land on a value it has since put in that register.
  The test reads the inline-assembly blocks of the generated code of every
  kernel source.
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

ASM_MEM = re.compile(r"^\s*(buffer|global|flat|scratch|s)_(load|store|atomic)\S*")


def _compile(src, out_dir, extra=()):
    flags = [f for f in build.DEVICE_FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, "--cuda-device-only", *extra, src]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=out_dir)
    assert r.returncode == 0, r.stderr[-3000:]
    return r


@needs_hipcc
@pytest.mark.parametrize("src", ["lmhead.hip", "fp8.hip", "backward.hip"])
def test_inline_asm_loads_write_lds_only(tmp_path, src):
    out = str(tmp_path / "k.s")
    _compile(os.path.join(build.CSRC, src), str(tmp_path), ("-S", "-o", out))
    in_asm = False
    loads = 0
    for line in open(out):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        if in_asm:
            m = ASM_MEM.match(line.split(";")[0])
            if m:
                assert m.group(2) == "load" and m.group(1) == "buffer" and line.split(";")[0].rstrip().endswith(" lds"), \
                    line.strip()
                loads += 1
    assert loads > 0  # the operand loads into LDS are inline assembly


@needs_hipcc
@pytest.mark.parametrize("src,kernel", [
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi0ELb0E"),  # bf16, logits not kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi1ELb0E"),  # fp32, logits not kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi0ELb1E"),  # bf16, logits kept
    ("lmhead.hip", "lmhead_lse_partial8_kernelILi1ELb1E"),  # fp32, logits kept
    ("lmhead.hip", "lmhead_lse_partial_narrow_kernelILi0ELb0E"),
    ("fp8.hip", "lmhead_fp8_partial8_kernelILb0E"),  # FP8, on the eight-wavefront engine
    ("fp8.hip", "lmhead_fp8_partial8_kernelILb1E"),
    ("fp8.hip", "lmhead_fp8_partial_narrow_kernel"),
    ("fp8.hip", "lmhead_mxfp4_partial_kernel"),
    ("fp8.hip", "lmhead_mxfp4_partial_narrow_kernel"),
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
