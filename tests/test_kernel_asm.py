"""The packed grouped GEMM's k-loops as the compiler emits them (CPU only: hipcc
cross-compiles gfx950 assembly, nothing runs).

Each k-loop copy (one per count of live 32-row blocks) keeps a full k16-step of
activation fragment reads and PD steps of weight loads in flight, and waits
only for the oldest of them before each MFMA.  A wait for *every* outstanding
load or LDS read (`vmcnt(0)` / `lgkmcnt(0)`) inside such a loop drains the
pipeline once per iteration; it has appeared whenever the register allocator
gave a loop copy its weight ring in other registers than the prologue's, or when
the fragment reads ahead of the loop were emitted out of order.  These tests
fail if any k-loop block of either projection holds such a wait.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_mixture_experts_22_amd import build

KERNELS = {1: "packed_gemm_kernelILi1E", 2: "packed_gemm_kernelILi2E"}


def _asm(tmp_path) -> str:
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = os.path.join(str(tmp_path), "gemm_packed.s")
    cmd = [cc, *build.compile_flags(), "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "gemm_packed.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    with open(out) as fh:
        return fh.read()


def _kernel_blocks(asm: str, mangled: str):
    """Basic blocks (label -> instruction lines) of one kernel's body."""
    start = re.search(r"^_Z\S*" + mangled + r"\S*:", asm, flags=re.M)
    assert start, f"kernel {mangled} not found in the assembly"
    body = asm[start.end():]
    body = body[:body.index("s_endpgm")]
    blocks, label, cur = [], "entry", []
    for line in body.splitlines():
        if re.match(r"^\.LBB\S*:", line):
            blocks.append((label, cur))
            label, cur = line.split(":")[0], []
        elif line.strip() and not line.lstrip().startswith(";"):
            cur.append(line.strip())
    blocks.append((label, cur))
    return blocks


@pytest.fixture(scope="module")
def packed_asm(tmp_path_factory):
    return _asm(tmp_path_factory.mktemp("asm"))


@pytest.mark.parametrize("mode", [1, 2])
def test_packed_kloops_wait_only_for_the_oldest_loads(packed_asm, mode):
    blocks = _kernel_blocks(packed_asm, KERNELS[mode])
    loops = [(lbl, ins) for lbl, ins in blocks if sum(i.startswith("v_mfma") for i in ins) >= 32]
    # one k-loop copy per count of live row blocks: 3 (also taking 1 and 2) .. 8
    mfmas = sorted(sum(i.startswith("v_mfma") for i in ins) for _, ins in loops)
    assert mfmas == [48, 64, 80, 96, 112, 128], mfmas
    for lbl, ins in loops:
        waits = [i for i in ins if i.startswith("s_waitcnt")]
        full = [w for w in waits if re.search(r"\b(vmcnt|lgkmcnt)\(0\)", w)]
        assert not full, f"MODE {mode} k-loop block {lbl} drains the pipeline: {full}"
        assert sum(i.startswith("s_barrier") for i in ins) == 2, f"{lbl}: one barrier per 4 k16-steps"


@pytest.mark.parametrize("mode", [1, 2])
def test_packed_kernels_do_not_spill(packed_asm, mode):
    meta = packed_asm[packed_asm.index("amdhsa.kernels"):]
    for m in re.finditer(r"\.name:\s+(\S+)", meta):
        if KERNELS[mode] not in m.group(1):
            continue
        # the entry's fields follow its name (alphabetical order)
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", meta[m.end():])
        assert spill and int(spill.group(1)) == 0, f"{m.group(1)} spills VGPRs"
        return
    pytest.fail(f"no metadata for {KERNELS[mode]}")
