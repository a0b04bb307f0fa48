import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle as O
    O.load()  # builds liboracle.so with gcc if it is missing
    return O


def pytest_sessionfinish(session, exitstatus):
    """With MTV_PARITY_LOG=<file.jsonl>, the GPU parity comparisons append
    their error figures there; at the end this writes <file>.md, one table
    row per comparison (the worst element's share of the tolerance included)."""
    path = os.environ.get("MTV_PARITY_LOG")
    if not path or not os.path.exists(path):
        return
    import json
    with open(path) as f:
        recs = [json.loads(line) for line in f if line.strip()]
    lines = ["| case | rows | max abs(dout) | rel. Frobenius | max abs(dlse) | max abs(out) | RMS out "
             "| worst err/tol out | worst err/tol lse |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in recs:
        lines.append("| %s | %d | %.3e | %.3e | %.3e | %.3f | %.4f | %.3f | %.3f |" % (
            r["label"], r["rows"], r["max_dout"], r["rel_fro"], r["max_dlse"], r["max_abs_out"],
            r["rms_out"], r["worst_ratio_out"], r["worst_ratio_lse"]))
    worst = max(recs, key=lambda r: max(r["worst_ratio_out"], r["worst_ratio_lse"]))
    lines.append("")
    lines.append("%d comparisons; the largest share of a tolerance used: %.3f (%s)." % (
        len(recs), max(worst["worst_ratio_out"], worst["worst_ratio_lse"]), worst["label"]))
    with open(os.path.splitext(path)[0] + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
