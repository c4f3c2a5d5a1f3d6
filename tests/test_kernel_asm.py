"""The packed grouped GEMM's k-loops as the compiler emits them (CPU only: hipcc
cross-compiles gfx950 assembly, nothing runs).

Each k-loop copy (one per count of live 32-row blocks) keeps a full k16-step of
activation fragment reads and PD steps of weight loads in flight, and waits
only for the oldest of them before each MFMA.  A wait for *every* outstanding
load or LDS read (`vmcnt(0)` / `lgkmcnt(0)`) inside such a loop drains the
pipeline once per iteration; it has appeared when the fragment reads ahead of
the loop were emitted out of order, in loop copies of one or two row blocks of
earlier forms of the kernel, and in a one-block copy (its single fragment read
per step is always the oldest; such tiles take the two-block copy).  These
tests fail if any k-loop block of either projection holds such a wait.
"""
import re

import pytest

from asm_util import basic_blocks

KERNELS = {1: "packed_gemm_kernelILi1E", 2: "packed_gemm_kernelILi2E"}


@pytest.mark.parametrize("mode", [1, 2])
def test_packed_kloops_wait_only_for_the_oldest_loads(packed_asm, mode):
    blocks = basic_blocks(packed_asm, KERNELS[mode])
    loops = [(lbl, ins) for lbl, ins, _ in blocks
             if sum(i.startswith("v_mfma") for i in ins) >= 32 and any(i.startswith("s_barrier") for i in ins)]
    # one k-loop copy per count of live row blocks: 2 (also taking 1) .. 8
    mfmas = sorted(sum(i.startswith("v_mfma") for i in ins) for _, ins in loops)
    assert mfmas == [32, 48, 64, 80, 96, 112, 128], mfmas
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
