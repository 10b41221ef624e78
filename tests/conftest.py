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


def _margins_markdown(rows):
    """The margins as a markdown table: one row per comparison (the two
    output layouts of one case collapse to the worse), largest share of the
    bound first."""
    import re
    out = ["# Parity margins (worst error per comparison, MI355X)", "",
           "Command (repo root, one MI355X): `DCN_PARITY_MARGINS=gpurun_out/parity_margins.md "
           "python -u -m pytest tests -m gpu -x -v`",
           "", "Each row is one GPU-vs-oracle comparison: the elements compared, the worst "
           "|gpu - ref| / N",
           "(N = the oracle's absolute-term sum of that element), the tolerance factor on N, and "
           "the largest",
           "share of the whole per-element bound (tol * N + one fp32 ulp of |ref|) that any "
           "element used",
           "(1.0 would be at the limit).  Duplicates across layouts collapse to the worst.", "",
           "| comparison | elements | worst err / N | tol | bound used |", "|---|---|---|---|---|"]
    worst = {}
    for r in rows:
        key = re.sub(r"/(nchw|nhwc)", "", r["what"])
        if key not in worst or r["bound_used"] > worst[key]["bound_used"]:
            worst[key] = r
    for k in sorted(worst, key=lambda k: (-worst[k]["bound_used"], k)):
        r = worst[k]
        out.append("| %s | %d | %.2e | %.0e | %.3f |" % (
            k, r["elements"], r["worst_err_over_N"], r["tol"], r["bound_used"]))
    return "\n".join(out) + "\n"


def pytest_sessionfinish(session, exitstatus):
    """Write the parity margins of this session (tests/dcn_testlib.MARGINS)
    to the file named by DCN_PARITY_MARGINS, if set: a markdown table when
    the name ends in .md, else the rows as JSON."""
    path = os.environ.get("DCN_PARITY_MARGINS")
    if not path:
        return
    import json
    mod = sys.modules.get("dcn_testlib")
    rows = list(getattr(mod, "MARGINS", [])) if mod is not None else []
    with open(path, "w") as fh:
        if path.endswith(".md"):
            fh.write(_margins_markdown(rows))
        else:
            json.dump(rows, fh, indent=1)
