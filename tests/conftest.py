import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_host_libs():
    # The generator and the oracle are plain C; build them only if nothing is built yet.
    import oracle
    import ssmgen
    if not os.path.exists(ssmgen._SO):
        ssmgen.build()
    if not os.path.exists(oracle._SO):
        oracle.build()


_ensure_host_libs()
