import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionfinish(session, exitstatus):
    """Write the worst parity errors seen (tests/dms_case.py ERRORS) to the file
    DMS_PARITY_LOG names, if any, and print them."""
    import json
    try:
        from dms_case import ERRORS
    except ImportError:
        return
    if not ERRORS:
        return
    path = os.environ.get("DMS_PARITY_LOG")
    if path:
        with open(path, "w") as f:
            json.dump(ERRORS, f, indent=1, sort_keys=True)
    for name in sorted(ERRORS):
        e = ERRORS[name]
        print("\n[parity] %s: max-abs %.3e, max-rel (|ref| >= 0.2) %.3e over %d elements in %d checks"
              % (name, e["max_abs"], e["max_rel"], e["elements"], e["checks"]), end="")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")
    config.addinivalue_line("markers", "slow: long CPU test")


# torch's first import on a fresh machine can take a minute or two; do it at
# collection time so it never counts against a single test's time limit
import torch  # noqa: E402,F401
