import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test (full workload sizes)")


@pytest.fixture
def tuning():
    """tuning(name, value): force a kernel choice of liblca.so for this test
    (lca_set_tuning); every choice made is restored to automatic afterwards."""
    import long_context_compressed_append_amd as lca
    used = set()

    def apply(name, value):
        lca.set_tuning(name, int(value))
        used.add(name)

    yield apply
    for name in used:
        lca.set_tuning(name, None)
