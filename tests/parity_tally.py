"""Session-wide counts of the GPU parity comparisons, printed at the end of the
pytest run (tests/conftest.py): how many sequences matched the oracle exactly,
how many differed on a near tie the oracle recorded (per band), and which
comparisons failed.  Plain bookkeeping: no GPU or oracle code here."""
from __future__ import annotations

from collections import OrderedDict

# band name -> counters
TALLY: "OrderedDict[str, dict]" = OrderedDict()

BANDS = {
    "accept": "accept test |u - p/q| under its band (1e-5 on given logits; wider end to end)",
    "draw": "draw within its band of a CDF edge (1e-6 normalised on given logits)",
    "greedy": "greedy top-2 logit gap under 4 max|dz| (end to end)",
    "top_p": "top-p cut within 4e-6 of the target mass",
}


def record(kind: str, exact: int, excused_accept: int = 0, excused_draw: int = 0, excused_other: int = 0,
           failures: int = 0, max_dz: float | None = None) -> None:
    """kind: "sampled" (T > 0) or "greedy"; excused_other: top-p cut near ties."""
    t = TALLY.setdefault(kind, {"comparisons": 0, "sequences": 0, "exact": 0, "accept": 0, "draw": 0, "greedy": 0,
                                "top_p": 0, "failures": 0, "max_dz": 0.0})
    t["comparisons"] += 1
    t["sequences"] += exact + excused_accept + excused_draw + excused_other + failures
    t["exact"] += exact
    if kind == "greedy":
        t["greedy"] += excused_accept + excused_draw
    else:
        t["accept"] += excused_accept
        t["draw"] += excused_draw
    t["top_p"] += excused_other
    t["failures"] += failures
    if max_dz is not None:
        t["max_dz"] = max(t["max_dz"], float(max_dz))


def summary_lines() -> list:
    lines = []
    for kind, t in TALLY.items():
        lines.append(f"parity {kind}: {t['comparisons']} comparisons, {t['sequences']} sequences, "
                     f"exact {t['exact']}, near ties: accept {t['accept']}, draw {t['draw']}, greedy {t['greedy']}, "
                     f"top-p {t['top_p']}; failures {t['failures']}; largest end-to-end |dz| {t['max_dz']:.3e}")
    return lines
