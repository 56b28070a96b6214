import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where no GPU is visible, so that a
    # plain `pytest` on a CPU-only host still runs the CPU suite.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # The parity numbers of the GPU tests (every comparison against the
    # oracle), printed even under -q so that a run's log carries them.
    mod = sys.modules.get("gpu_helpers")
    if mod is None or not getattr(mod, "RECORDS", None):
        return
    terminalreporter.section("parity against the fp64 oracle (err / raw / worst 256x256 tile)")
    for line in mod.summary_lines(mod.RECORDS):
        terminalreporter.write_line(line)
