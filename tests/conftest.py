import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes on the CPU oracle side)")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def qmv():
    """The HIP library binding; skips when no GPU is visible (CPU-only runs)."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import gemm_dequant_matvec_amd as q
    return q
