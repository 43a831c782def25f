import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP libraries")


def _ensure_host_builds():
    """The CPU-only pieces (oracle, CPU table generator) are cheap gcc builds;
    build them if missing so that CPU tests run from a clean checkout."""
    from oracle import build as ob
    from gen import build as gb
    if not os.path.exists(os.path.join(ROOT, "oracle", "libple_oracle.so")):
        ob.build()
    if not os.path.exists(os.path.join(ROOT, "gen", "libplegen_host.so")):
        import subprocess
        subprocess.run(gb.commands()[0], check=True)


_ensure_host_builds()


@pytest.fixture(scope="session")
def weights():
    from gen import inputs
    return inputs.weights()
