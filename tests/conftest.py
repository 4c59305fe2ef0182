"""pytest configuration: registers the ``gpu`` marker and puts the repository
root on ``sys.path`` so ``oracle`` and ``dense_mixed_precision_amd`` import."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a gfx950 GPU and the built HIP library")
