import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")
    config.addinivalue_line("markers", "slow: long CPU test")


# torch's first import on a fresh machine can take a minute or two; do it at
# collection time so it never counts against a single test's time limit
import torch  # noqa: E402,F401
