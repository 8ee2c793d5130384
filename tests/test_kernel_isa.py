"""Static checks of the gfx950 code of the bf16 chain kernel (no GPU needed).

The kernel is compiled to assembly with the library's own flags. Each
instance of chain_kernel_ws must:

- use no scratch memory: a spill slows every workgroup and, at full-chip
  grids, limits how many waves can be resident;
- fit the 256 registers per lane that two waves per SIMD leave each wave;
- stay small: the chain's step list is unrolled at compile time, and a
  failed unroll leaves the step index dynamic, which shows as a tenfold
  larger instance full of dynamic register indexing;
- respect the DPP hazard of the fused forward substitution: a VALU write of
  a VGPR needs two wait states before a DPP instruction reads that VGPR as
  its (broadcast) first source. The DPP FMAs are inline assembly, so the
  compiler does not insert these wait states; the source guarantees them.
"""

import os
import re
import subprocess
import tempfile

import pytest

from chunkwise_delta_rule_amd import build

SRC = os.path.join(build.PKG, "csrc", "chain_bf16.hip")


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "chain_bf16.s")
        cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(build.ROOT, "include"), SRC, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        return open(out).read()


def kernels(asm_text):
    """(name, body lines, resource comment block) of every chain_kernel_ws instance."""
    out = []
    for m in re.finditer(r"^(_Z\S*chain_kernel_ws\S*):", asm_text, flags=re.M):
        name = m.group(1)
        end = asm_text.index(".Lfunc_end", m.end())
        body = asm_text[m.end():end].split("\n")
        tail = asm_text[end:end + 4000]
        out.append((name, body, tail))
    return out


def test_instances_present(asm):
    # dk, dv in {64, 128}, with and without output, with and without decay
    assert len(kernels(asm)) == 16


def test_no_scratch_and_register_budget(asm):
    for name, _, tail in kernels(asm):
        scratch = int(re.search(r"ScratchSize:\s*(\d+)", tail).group(1))
        vgprs = int(re.search(r"TotalNumVgprs:\s*(\d+)", tail).group(1))
        assert scratch == 0, f"{name}: {scratch} bytes of scratch"
        assert vgprs <= 256, f"{name}: {vgprs} VGPRs"


def test_code_size_and_static_indexing(asm):
    for name, body, _ in kernels(asm):
        insts = [l for l in body if re.match(r"\s+[a-z]", l)]
        assert len(insts) < 20000, f"{name}: {len(insts)} instructions"
        assert not any("s_set_gpr_idx_on" in l for l in insts), f"{name}: dynamic register indexing"


def _vgprs_written(line):
    """VGPRs written by a VALU instruction line (its first operand), or an empty set."""
    m = re.match(r"\s+(v_\S+)\s+(v\[(\d+):(\d+)\]|v(\d+))", line)
    if not m or m.group(1).startswith(("v_cmp", "v_readfirstlane", "v_readlane")):
        return set()
    if m.group(3) is not None:
        return set(range(int(m.group(3)), int(m.group(4)) + 1))
    return {int(m.group(5))}


def test_dpp_broadcast_sources_have_two_wait_states(asm):
    checked = 0
    for name, body, _ in kernels(asm):
        insts = [l for l in body if re.match(r"\s+[a-z]", l)]
        for i, line in enumerate(insts):
            m = re.match(r"\s+v_fmac_f32_dpp\s+v\d+,\s*v(\d+),", line)
            if not m:
                continue
            checked += 1
            src = int(m.group(1))
            waits = 0
            for prev in reversed(insts[max(0, i - 4):i]):
                if waits >= 2:
                    break
                nop = re.match(r"\s+s_nop\s+(\d+)", prev)
                if nop:
                    waits += int(nop.group(1)) + 1
                    continue
                if src in _vgprs_written(prev):
                    raise AssertionError(f"{name}: v{src} written {waits} wait states before a DPP read:\n"
                                         f"{prev}\n{line}")
                waits += 1
    assert checked > 0


def test_dpp_check_catches_a_planted_hazard():
    body = ("_Zchain_kernel_wsILi128EE:\n"
            "\tv_mul_f32_e32 v36, v1, v2\n"
            "\tv_fmac_f32_dpp v47, v36, v29 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
            ".Lfunc_end0:\n; ScratchSize: 0\n; TotalNumVgprs: 64\n")
    with pytest.raises(AssertionError, match="v36 written 0 wait states"):
        test_dpp_broadcast_sources_have_two_wait_states(body)
    ok = body.replace("\tv_fmac", "\ts_nop 1\n\tv_fmac")
    test_dpp_broadcast_sources_have_two_wait_states(ok)
