"""Checks on the gfx950 assembly of the attention kernels (CPU only: hipcc cross-compiles).

The tile copies are direct-to-LDS buffer loads issued through inline assembly,
tracked with explicit vmcnt waits.  The compiler does not count them, so a
vmcnt wait it inserts for one of its own loads (a q register, a spilled
register) would also wait for every copy in flight.  Inside a loop that stalls
each tile on a full HBM round trip; no such wait may appear in any loop body.
"""

import os
import re
import subprocess

import pytest

from attention_int8_quantized_amd import build


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "attnq8.s")
    cmd = [c for c in build.compile_command(out) if c not in ("-shared", "-fPIC")]
    cmd += ["--cuda-device-only", "-S"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _kernels(asm):
    names = re.findall(r"^(_ZN6attnq8\d+attend_\w+_kernelI\w+AttendArgsE):", asm, re.M)
    for n in names:
        start = asm.index(n + ":")
        yield n, asm[start:asm.index(".Lfunc_end", start)].split("\n")


def test_no_compiler_vmcnt_wait_inside_loops(device_asm):
    checked = 0
    for name, body in _kernels(device_asm):
        # every basic block opens with a label line that the compiler annotates
        # when the block lies in a loop ("in Loop: Header=..." or "Loop Header")
        in_loop = False
        loop_blocks = 0
        in_asm = False
        for line in body:
            if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", line):
                in_loop = "Loop" in line
                loop_blocks += in_loop
            elif line.lstrip().startswith("; =>") and "Loop Header" in line:
                in_loop = True
            if ";;#ASMSTART" in line:
                in_asm = True
            elif ";;#ASMEND" in line:
                in_asm = False
            elif not in_asm and in_loop and "s_waitcnt" in line and "vmcnt" in line:
                raise AssertionError(f"{name}: {line.strip()} in a loop")
        assert loop_blocks, f"{name}: no loop found"
        checked += 1
    assert checked >= 70


def test_no_scratch_in_attention_kernels(device_asm):
    for block in re.split(r"\n  - \.", device_asm.split("amdhsa.kernels:")[1]):
        name = re.search(r"name:\s+(\S+)", block)
        if not name or "attend" not in name.group(1):
            continue
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        assert spill and int(spill.group(1)) == 0, name.group(1)
        assert priv and int(priv.group(1)) == 0, name.group(1)


def test_m0_is_used_only_by_the_tile_copies(device_asm):
    """The direct-to-LDS copies set m0 (the LDS destination) in inline assembly,
    and the compiler warns that it may not preserve a reserved register across
    such a statement.  That is harmless as long as no compiler-generated
    instruction reads or writes m0: checked here for every kernel."""
    names = re.findall(r"^(_ZN6attnq8\w+):", device_asm, re.M)
    assert names
    for name in names:
        start = device_asm.index(name + ":")
        body = device_asm[start:device_asm.index(".Lfunc_end", start)].split("\n")
        in_asm = False
        for line in body:
            if ";;#ASMSTART" in line:
                in_asm = True
            elif ";;#ASMEND" in line:
                in_asm = False
            elif not in_asm and re.search(r"\bm0\b", line.split(";")[0]):
                raise AssertionError(f"{name}: compiler use of m0: {line.strip()}")
