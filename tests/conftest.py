import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def rocrand_probe():
    """Path of a host-only program that evaluates rocRAND's Philox4x32-10 block function."""
    if os.environ.get("NM_ROCRAND_PROBE"):
        return os.environ["NM_ROCRAND_PROBE"]
    src = os.path.join(ROOT, "tests", "rocrand_philox_probe.cpp")
    out = os.path.join(tempfile.mkdtemp(prefix="nm_rocrand_"), "probe")
    res = subprocess.run(["hipcc", "-O1", "-o", out, src], capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("cannot build the rocRAND probe: " + res.stderr[-400:])
    return out
