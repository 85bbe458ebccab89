import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def fa_lib():
    """The built C-ABI library (built in-tree first if it is missing)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fa_amd_build", os.path.join(ROOT, "io_aware_attention_fa_amd", "build.py"))
    fabuild = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(fabuild)   # by path: the package import would load the library
    if not os.path.exists(fabuild.library_path()):
        fabuild.build_library()
    import io_aware_attention_fa_amd as fa
    return fa


@pytest.fixture(scope="session")
def gpu(fa_lib):
    if not _gpu_available():
        pytest.fail("GPU tests need a visible MI355X (gfx950); run them with -m gpu on a machine that has one")
    import torch
    torch.cuda.init()
    return fa_lib
