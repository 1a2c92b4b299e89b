"""Counts of the parity exemptions, per case.

The GPU parity tests excuse a difference from the oracle only where rounding
can explain it: a keep decision with |u - min(1, p/q)| < 1e-6, a drawn token in
the oracle's near set (oracle.verify.draw_rows), a Markov or RNN logit that
differs by rounding, and the token differences those cause. Each check records
how many it excused and how many it compared. conftest.py prints the table at
the end of the session; when SPECV_PARITY_LOG names a file, the records are
also written there as JSON.
"""
import json
import os

RECORDS = []


def record(kind: str, case: str, **counts):
    rec = dict(kind=kind, case=case)
    for k, v in counts.items():
        rec[k] = float(v) if isinstance(v, float) else int(v) if hasattr(v, "__int__") and not isinstance(v, bool) else v
    RECORDS.append(rec)
    path = os.environ.get("SPECV_PARITY_LOG")
    if path:
        with open(path, "w") as f:
            json.dump(RECORDS, f, indent=1)
    return rec


def lines():
    out = []
    for r in RECORDS:
        rest = " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                        for k, v in r.items() if k not in ("kind", "case"))
        out.append(f"{r['kind']:<9} {r['case']:<28} {rest}")
    return out
