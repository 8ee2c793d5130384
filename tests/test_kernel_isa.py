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

Every kernel of the library (chain_bf16.hip, bwd_grad.hip and kernels.hip) must also keep
matrix-core accumulation chains to one product shape: no 16x16x16 product
may take the result of a 16x16x32 product (or the other way round) as its
accumulator. The compiler emitted such a pair back to back without the wait
states the hardware needs between the two shapes, and the sums came out
wrong; the kernels therefore accumulate each shape separately and add.
"""

import os
import re
import subprocess
import tempfile

import pytest

from chunkwise_delta_rule_amd import build

SRC = os.path.join(build.PKG, "csrc", "chain_bf16.hip")
SRC_OTHER = os.path.join(build.PKG, "csrc", "kernels.hip")
SRC_GRAD = os.path.join(build.PKG, "csrc", "bwd_grad.hip")


def _compile(src):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(build.ROOT, "include"), src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        return open(out).read()


@pytest.fixture(scope="module")
def asm():
    return _compile(SRC)


@pytest.fixture(scope="module")
def asm_other():
    return _compile(SRC_OTHER)


@pytest.fixture(scope="module")
def asm_grad():
    return _compile(SRC_GRAD)


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
    # dk, dv in {64, 128}, with and without decay: 64-row tiles with and
    # without output (12 waves for the output without decay, else 8), 32-row
    # tiles with output; 128-row tiles (15 waves) for the context-parallel
    # transitions at dk = dv = 128, with and without decay
    names = [name for name, _, _ in kernels(asm)]
    assert len(names) == 26
    assert sum("ELi32ELi8E" in n for n in names) == 8
    assert sum("ELi64ELi12E" in n for n in names) == 4 and sum("ELi64ELi8E" in n for n in names) == 12
    assert sum("ILi128ELi128ELb0ELb0ELi128ELi15E" in n for n in names) == 1
    assert sum("ILi128ELi128ELb0ELb1ELi128ELi15E" in n for n in names) == 1


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


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def mixed_shape_chains(asm_text):
    """(kernel, first opcode, second opcode, instructions between) for every
    MFMA whose accumulator input is the result of an MFMA of another opcode,
    with no other write of those registers in between."""
    found = []
    for m in re.finditer(r"^(_Z\S+):", asm_text, flags=re.M):
        end = asm_text.index(".Lfunc_end", m.end())
        insts = [l.strip() for l in asm_text[m.end():end].split("\n")]
        insts = [l for l in insts if l and not l.startswith((";", ".")) and not l.endswith(":")]
        parsed = []
        for l in insts:
            t = l.split(None, 1)
            parsed.append((t[0], [x.strip() for x in t[1].split(",")] if len(t) > 1 else []))
        for i, (op, ops) in enumerate(parsed):
            if not op.startswith("v_mfma"):
                continue
            dst = _regs(ops[0])
            for k in range(i + 1, min(i + 60, len(parsed))):
                op2, ops2 = parsed[k]
                if op2.startswith("v_mfma") and len(ops2) >= 4 and _regs(ops2[3]) & dst:
                    if op2 != op:
                        found.append((m.group(1), op, op2, k - i - 1))
                    break
                if ops2 and not op2.startswith(("s_", "ds_write", "global_store", "buffer_store")) and \
                        _regs(ops2[0]) & dst:
                    break
    return found


def test_no_mixed_shape_accumulation(asm, asm_other, asm_grad):
    n_mfma = asm.count("v_mfma") + asm_other.count("v_mfma") + asm_grad.count("v_mfma")
    assert n_mfma > 1000
    bad = mixed_shape_chains(asm) + mixed_shape_chains(asm_other) + mixed_shape_chains(asm_grad)
    assert not bad, "\n".join(f"{k}: {a} -> {b} ({gap} between)" for k, a, b, gap in bad[:10])


def test_mixed_shape_check_catches_a_planted_chain():
    body = ("_Zk:\n"
            "\tv_mfma_f32_16x16x16_bf16 a[0:3], v[56:57], v[58:59], a[0:3]\n"
            "\tds_read_b64 v[56:57], v241\n"
            "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[56:59], v[88:91], a[0:3]\n"
            ".Lfunc_end0:\n")
    assert len(mixed_shape_chains(body)) == 1
    same = body.replace("16x16x32_bf16 a[0:3], v[56:59]", "16x16x16_bf16 a[0:3], v[56:57]")
    assert mixed_shape_chains(same) == []
    rewritten = body.replace("\tds_read_b64", "\tv_accvgpr_write_b32 a0, 0\n\tds_read_b64")
    assert mixed_shape_chains(rewritten) == []


def test_gradient_kernel_two_workgroups_per_cu(asm_grad):
    # the chunk-parallel gradient kernel is sized for two workgroups of 4
    # waves per CU: at most 256 registers per lane, no scratch, at most 80 KB
    # of LDS
    found = 0
    for m in re.finditer(r"^(_Z\S*bwd_grad_kernel\S*):", asm_grad, flags=re.M):
        found += 1
        end = asm_grad.index(".Lfunc_end", m.end())
        tail = asm_grad[end:end + 4000]
        name = m.group(1)
        assert int(re.search(r"ScratchSize:\s*(\d+)", tail).group(1)) == 0, name
        assert int(re.search(r"TotalNumVgprs:\s*(\d+)", tail).group(1)) <= 256, name
        assert int(re.search(r"LDSByteSize:\s*(\d+)", tail).group(1)) <= 80 * 1024, name
    assert found == 4
