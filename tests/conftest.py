import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    # largest output / lse / mass errors the GPU parity checks saw in this run
    mod = sys.modules.get("gpu_check")
    if mod is not None and any(v > 0 for v in getattr(mod, "WORST", {}).values()):
        terminalreporter.write_line(f"gpu_check worst errors: {mod.WORST}")
