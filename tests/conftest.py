import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: a CPU test that takes more than a few seconds")


def _group(name: str) -> tuple:
    """(case, tensor) of a check name such as 'ref_shape dQ rows h=3' or
    'tiny chain dK[0,0]': the tensor is the first word naming an output."""
    words = name.split()
    for i, w in enumerate(words):
        base = re.split(r"[\[(]", w)[0]
        if base in ("O_hp", "lse", "delta", "dQ", "dK", "dV", "O"):
            case = " ".join(words[:i])
            if i + 1 < len(words) and words[i - 1:i] == ["chain"]:
                case = " ".join(words[:i])
            return case, base
    return name, "?"


def pytest_sessionfinish(session, exitstatus):
    """With ATTNQAT_PARITY_MARGINS=<path>, write the achieved errors of every
    floating-point parity check of this session as a markdown table."""
    path = os.environ.get("ATTNQAT_PARITY_MARGINS")
    if not path:
        return
    from tests._util import MARGINS
    if not MARGINS:
        return
    agg = {}
    for name, rf, emax, amax, rtol, etol in MARGINS:
        key = _group(name)
        el = emax / amax if amax > 0 else 0.0
        n, r0, e0 = agg.get(key, (0, 0.0, 0.0))
        agg[key] = (n + 1, max(r0, rf), max(e0, el))
    with open(path, "w") as f:
        f.write("| case | tensor | checks | max rel. Frobenius error (bar 5e-3) | "
                "max elementwise error / max|ref| (bar 2e-2) |\n|---|---|---|---|---|\n")
        for (case, t), (n, r0, e0) in sorted(agg.items()):
            f.write(f"| {case} | {t} | {n} | {r0:.2e} | {e0:.2e} |\n")
