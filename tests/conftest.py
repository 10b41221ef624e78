"""Shared pytest set-up: repo root on sys.path, the ``gpu`` marker, helpers.

Tests marked ``gpu`` need an MI355X; everything else runs on a CPU-only host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a ``key value value ...`` fixture under tests/golden/ (``#`` = comment)."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


def pytest_sessionstart(session):
    """Build what is not built yet (never rebuilds an existing library)."""
    from modulated_deformable_convolution_dcn_amd import _lib
    if not os.path.exists(_lib.LIB_PATH) and os.path.exists("/opt/rocm/bin/hipcc"):
        from modulated_deformable_convolution_dcn_amd import build
        build.build()
    import oracle
    oracle.build(force=False)


def pytest_sessionfinish(session, exitstatus):
    """Write the parity margins of this session (tests/dcn_testlib.MARGINS)
    to the file named by DCN_PARITY_MARGINS, if set."""
    path = os.environ.get("DCN_PARITY_MARGINS")
    if not path:
        return
    import json
    mod = sys.modules.get("dcn_testlib")
    rows = list(getattr(mod, "MARGINS", [])) if mod is not None else []
    with open(path, "w") as fh:
        json.dump(rows, fh, indent=1)
