import importlib.util
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests never skip silently: without a GPU they fail, so a deselection
    # (-m "not gpu") is the only way to leave them out.
    pass


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def forge_build_module():
    """optimizer_gemm_amd/build.py, loaded by path (importing the package would load the
    library)."""
    spec = importlib.util.spec_from_file_location("forge_build", os.path.join(ROOT, "optimizer_gemm_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="session")
def host_checked_build():
    """The library's host-checking variant (sanitizers on the host code, release device
    code), compiled once per session with the compiler's per-kernel resource report:
    (build module, library path, {source: compiler stderr})."""
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    b = forge_build_module()
    lib, stderr = b.build_sanitized(remarks=True)
    return b, lib, stderr
