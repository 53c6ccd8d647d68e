"""Parity margins of the GPU tests, collected during the session and printed at its end
by ``pytest_terminal_summary`` (``tests/conftest.py``), so that a quiet ``pytest -q``
run still reports the normwise error, 1 - cosine and the log-sum-exp error against the
fp64 oracle.  Records marked ``show`` (one per workload and the full-size cases) are
printed one per line; the rest are summarised by their count and worst margin."""
import os

RECORDS = []


def record(what, err, cos, lse_err=None, *, tol, cos_tol, show=False):
    """Log one comparison of the current test (named from PYTEST_CURRENT_TEST)."""
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" (")[0].split("::")[-1]
    RECORDS.append({"test": test, "what": what, "err": float(err), "one_minus_cos": 1.0 - float(cos),
                    "lse_err": None if lse_err is None else float(lse_err),
                    "tol": float(tol), "cos_tol": float(cos_tol), "show": show})


def _line(r):
    lse = "-" if r["lse_err"] is None else f"{r['lse_err']:.2e}"
    test = r["test"] if len(r["test"]) <= 60 else r["test"][:57] + "..."
    return (f"{test:<60} {r['what'][:10]:<10} {r['err']:>9.2e} {r['one_minus_cos']:>9.2e} {lse:>9}"
            f"  {r['tol']:.0e}/{1 - r['cos_tol']:.0e}")


def _rel(r):
    return max(r["err"] / r["tol"], r["one_minus_cos"] / max(1 - r["cos_tol"], 1e-300))


def summary_lines():
    if not RECORDS:
        return []
    lines = [f"{'case':<60} {'what':<10} {'normwise':>9} {'1-cos':>9} {'lse err':>9}  bar (err/1-cos)"]
    lines += [_line(r) for r in RECORDS if r["show"]]
    rest = [r for r in RECORDS if not r["show"]]
    if rest:
        w = max(rest, key=_rel)
        lines.append(f"{len(rest)} further comparisons; the closest to its bar:")
        lines.append(_line(w))
    w = max(RECORDS, key=_rel)
    lines.append(f"closest to its bar overall: {_rel(w):.2f} of the bar ({w['test']}, {w['what']})")
    return lines
