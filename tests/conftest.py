import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size case (minutes of host-side oracle work)")


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load


# ----------------------------------------------------------------------------
# Floor-criterion bookkeeping: tests.parity.check_logits_row
# records every row it checks; each record is tagged with its test here and
# the session summary prints the totals per test function (and writes them
# as JSON to $DSA_FLOOR_JSON when that is set).
# ----------------------------------------------------------------------------
@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_call(item):
    mod = sys.modules.get("tests.parity")
    n0 = len(mod.FLOOR_LOG) if mod else 0
    yield
    mod = sys.modules.get("tests.parity")
    if mod:
        for rec in mod.FLOOR_LOG[n0:]:
            rec.setdefault("test", item.nodeid)


def _floor_totals(log):
    per = {}
    for r in log:
        key = r.get("test", "?")
        a = per.setdefault(key, {"rows": 0, "cols": 0, "viol": 0,
                                 "rows_with_viol": 0, "max_ratio": 0.0,
                                 "viol_cols_max_abs_over_S": 0.0,
                                 "viol_max_err_over_M": 0.0})
        a["rows"] += 1
        a["cols"] += r["cols"]
        a["viol"] += r["viol"]
        a["rows_with_viol"] += int(r["viol"] > 0)
        a["max_ratio"] = max(a["max_ratio"], r["max_ratio"])
        a["viol_cols_max_abs_over_S"] = max(a["viol_cols_max_abs_over_S"],
                                            r["viol_cols_max_abs_over_S"])
        a["viol_max_err_over_M"] = max(a["viol_max_err_over_M"],
                                       r.get("viol_max_err_over_M", 0.0))
    return per


def pytest_terminal_summary(terminalreporter):
    import json
    mod = sys.modules.get("tests.parity")
    if not mod or not mod.FLOOR_LOG:
        return
    per = _floor_totals(mod.FLOOR_LOG)
    funcs = {}
    for key, a in per.items():
        f = funcs.setdefault(key.split("[")[0], {"rows": 0, "cols": 0,
                                                 "viol": 0, "max_ratio": 0.0,
                                                 "max_abs": 0.0})
        f["rows"] += a["rows"]
        f["cols"] += a["cols"]
        f["viol"] += a["viol"]
        f["max_ratio"] = max(f["max_ratio"], a["max_ratio"])
        f["max_abs"] = max(f["max_abs"], a["viol_cols_max_abs_over_S"])
    tr = terminalreporter
    tr.write_sep("-", "logits criterion 2e-3 * max(|o|, 1e-2 S_t)")
    for name, f in sorted(funcs.items()):
        tr.write_line(f"{name}: {f['viol']} of {f['cols']} columns over "
                      f"({f['rows']} rows), max ratio {f['max_ratio']:.3g}, "
                      f"largest |o|/S_t among them {f['max_abs']:.3g}")
    path = os.environ.get("DSA_FLOOR_JSON")
    if path:
        with open(path, "w") as fh:
            json.dump({"per_test": per, "per_function": funcs}, fh, indent=1)
