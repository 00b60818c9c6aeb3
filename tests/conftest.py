import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def mxlib():
    """The HIP library, built in-tree first if it is not there yet."""
    from grouped_gemm_mxfp8_amd import LIB_PATH, lib
    if not os.path.exists(LIB_PATH):
        from grouped_gemm_mxfp8_amd._build import build
        build()
    return lib()


@pytest.fixture(scope="session")
def dev(mxlib):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    d = torch.device("cuda:0")
    name = torch.cuda.get_device_name(d)
    print(f"[gpu] {name}", flush=True)
    return d
