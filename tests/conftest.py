import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst fp32 parity figures of the session per check (the floored relative error, the
    unfloored one, the norm-wise one, the error as a fraction of the fp32-accumulation bound and
    how many elements took the floor); also written as JSON to $PARITY_REPORT when that is set."""
    try:
        from parity import REPORT
    except Exception:
        return
    if not REPORT:
        return
    tr = terminalreporter
    tr.write_sep("-", "fp32 parity (worst per check)")
    tr.write_line(f"{'check':44s} {'calls':>5s} {'max_rel':>10s} {'unfloored':>10s} {'normwise':>10s} "
                  f"{'/bound':>7s} {'floored':>12s}")
    for k in sorted(REPORT):
        r = REPORT[k]
        tr.write_line(f"{k[:44]:44s} {r['calls']:5d} {r['max_rel']:10.3e} {r['max_rel_unfloored']:10.3e} "
                      f"{r['normwise']:10.3e} {r['acc_bound_ratio']:7.3f} {r['n_floored']:>6d}/{r['n']:<6d}")
    path = os.environ.get("PARITY_REPORT")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(REPORT, f, indent=1, sort_keys=True)


def pytest_sessionstart(session):
    """Sanitizer runs (tests/test_sanitizers.py) point the binding and the oracle at instrumented
    host builds of the same sources."""
    lib = os.environ.get("TE_FP8_TEST_LIB")
    if lib:
        import fp8_linear_layer_amd as te
        te.LIB_PATH = lib
    olib = os.environ.get("ORACLE_TEST_LIB")
    if olib:
        import oracle
        oracle._LIB_PATH = olib
