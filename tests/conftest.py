import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With MOE_PARITY_LOG set, write every parity check's error figures (what, error beyond the
    output's own rounding / rms, raw max|err| / rms) to that file as JSON lines."""
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    helpers = sys.modules.get("gpu_helpers")
    if helpers is None or not helpers.RECORDS:
        return
    import json
    with open(path, "w") as f:
        for what, err, raw in helpers.RECORDS:
            f.write(json.dumps({"check": what, "err_beyond_rounding": err, "raw": raw}) + "\n")
