import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests sort after the CPU ones so `-x` on a mixed run reports the
    # cheap failures first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session")
def tiny():
    import lasynth
    cfg = lasynth.get_config("tiny")
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    return cfg, w, p, win
