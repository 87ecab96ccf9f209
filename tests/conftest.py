import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Per-tensor errors (max |gpu - oracle| / max |oracle|) of every full-size parity case that ran."""
    try:
        from rm_gpu import FULL_SIZE_REPORT
    except Exception:
        return
    if not FULL_SIZE_REPORT:
        return
    terminalreporter.write_line("full-size parity, max |gpu - oracle| / max |oracle| per tensor:")
    for label, errs in FULL_SIZE_REPORT:
        worst = max(errs, key=errs.get)
        terminalreporter.write_line(f"  {label}: worst {worst} {errs[worst]:.2e}; "
                                    + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
