import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With MALA_PARITY_STATS=<path>, write every recorded parity comparison
    (strict and scaled errors, LSE errors, near-tie counts) as JSON."""
    path = os.environ.get("MALA_PARITY_STATS")
    if not path or "parity_util" not in sys.modules:
        return
    import json
    stats = sys.modules["parity_util"].STATS
    with open(path, "w") as f:
        json.dump(stats, f, indent=0)
