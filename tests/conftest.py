import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


_CACHE = {}


def cached_unit(cfg: str, unit: int = 0):
    """Seeded tensors of one unit, generated once per test session."""
    import synth_weights as sw

    key = (cfg, unit)
    if key not in _CACHE:
        _CACHE[key] = sw.gen_unit(sw.config(cfg).units[unit])
    return _CACHE[key]


@pytest.fixture(scope="session")
def unit_tensors():
    return cached_unit
