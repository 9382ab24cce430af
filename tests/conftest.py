import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Largest parity error seen per kind (GPU runs), beside its bound."""
    import json
    try:
        from gpu_helpers import MAXERR
    except Exception:  # pragma: no cover
        return
    if not MAXERR:
        return
    terminalreporter.write_sep("-", "largest parity errors (kind: error / bound, case)")
    for kind in sorted(MAXERR):
        err, bound, label = MAXERR[kind]
        terminalreporter.write_line(f"{kind}: {err:.3e} / {bound:.1e}  ({label})")
    path = os.environ.get("DSA_MAXERR_JSON")
    if path:
        with open(path, "w") as fh:
            json.dump({k: {"err": v[0], "bound": v[1], "case": v[2]} for k, v in MAXERR.items()},
                      fh, indent=1, sort_keys=True)
