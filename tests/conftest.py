import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


@pytest.fixture(scope="session")
def packed_asm(tmp_path_factory):
    """gfx950 assembly of the packed grouped GEMM source (compiled once)."""
    from asm_util import compile_asm
    from sparse_mixture_experts_22_amd import build
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    return compile_asm(os.path.join(build.CSRC, "gemm_packed.hip"), str(tmp_path_factory.mktemp("asm")))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configuration (seconds to minutes)")
