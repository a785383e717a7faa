import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # tests load the built library; build it only when nothing is built yet
    lib = os.path.join(ROOT, "dora_fine_tuning_amd", "libdora_hip.so")
    if not os.path.exists(lib):
        from dora_fine_tuning_amd import build as _b

        _b.build()
