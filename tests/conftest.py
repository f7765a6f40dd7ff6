"""pytest configuration: the `gpu` marker and import paths for the repository root."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Observed parity figures (tests/parity.py OBSERVED) for the named workloads: the largest
    distance in ulps from the oracle's correctly rounded result and the share of outputs equal to
    it bit for bit. All labels go to $QKROPE_PARITY_REPORT as JSON when that is set."""
    parity = sys.modules.get("parity")
    if parity is None or not parity.OBSERVED:
        return
    import json
    from qk_rmsnorm_rope_amd import workloads as wl
    named = tuple(wl.WORKLOADS)
    rows = {k: v for k, v in parity.OBSERVED.items() if k.split()[0] in named}
    if rows:
        tr = terminalreporter
        tr.section("observed parity against the oracle's rounded result")
        tr.write_line(f"{'output':56s} {'elements':>10s} {'bit-equal':>9s} {'<=1 ulp':>8s} "
                      f"{'max ulp*':>8s} {'tol used':>8s}")
        for k in sorted(rows):
            v = rows[k]
            tr.write_line(f"{k:56s} {v['n']:10d} {v['bit_equal'] / v['n']:9.4%} "
                          f"{v['within_1ulp'] / v['n']:8.4%} {v['max_ulp']:8d} "
                          f"{v['max_tol_used']:8.3f}")
        tr.write_line("* among outputs where the relative part of the tolerance governs; "
                      "tol used: the largest err / bound (E4M3: codes)")
    out = os.environ.get("QKROPE_PARITY_REPORT")
    if out:
        with open(out, "w") as f:
            json.dump(parity.OBSERVED, f, indent=1, sort_keys=True)
