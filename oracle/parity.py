"""Parity bookkeeping between the oracle's step and a step under test.

TEST INFRASTRUCTURE ONLY (like the rest of this package): used by ``tests/``
and by the CPU-baseline leg of ``bench.py``.  It compares emitted tokens
element by element and decides, from the margins the oracle recorded, whether
a sequence that differs sits on a near tie.  No arithmetic of the method is
done here.

A sampled step is a deterministic function of its uniforms, so two correct
implementations agree token for token except where a decision lies closer to
its threshold than their rounding can move it.  The oracle records, per
sequence, the distance |u - p/q| of every accept test and the normalised
distance of the draw's uniform from the nearest CDF edge (at T = 0: the top-2
logit gap of every row it checked).  A sequence that differs is excused only
if one of those margins, at or before the first differing position, is below
its band; every excuse is counted.
"""
from __future__ import annotations

import numpy as np


def compare_steps(gpu_tokens, gpu_num, ora, acc_band: float, draw_band) -> dict:
    """Element-by-element comparison of emitted tokens and counts.

    gpu_tokens [B, g+1] and gpu_num [B] from the step under test; ora the dict
    the oracle's verify returns (tokens, num_emitted, accept_margin,
    draw_margin).  acc_band: band of the accept tests (the top-2 logit gap for
    greedy steps); draw_band: band of the draw (a scalar or one value per
    sequence).  Returns {"exact", "excused", "failures" (list of sequences),
    "excused_accept", "excused_draw"}."""
    gpu_tokens = np.asarray(gpu_tokens)
    gpu_num = np.asarray(gpu_num)
    B, g1 = gpu_tokens.shape
    g = g1 - 1
    draw_band = np.broadcast_to(np.asarray(draw_band, dtype=np.float64), (B,))
    exact = excused_acc = excused_draw = 0
    failures = []
    for b in range(B):
        ot = ora["tokens"][b]
        if gpu_num[b] == ora["num_emitted"][b] and np.array_equal(gpu_tokens[b], ot):
            exact += 1
            continue
        diff = np.nonzero(gpu_tokens[b] != ot)[0]
        j = int(diff[0]) if diff.size else g1
        am = ora["accept_margin"][b][: min(j + 1, g)]
        am = am[~np.isnan(am)]
        near_acc = am.size > 0 and float(am.min()) < acc_band
        k = int(ora["num_emitted"][b]) - 1
        near_draw = j >= k and float(ora["draw_margin"][b]) < float(draw_band[b])
        if near_acc:
            excused_acc += 1
        elif near_draw:
            excused_draw += 1
        else:
            failures.append(b)
    return {"exact": exact, "excused": excused_acc + excused_draw, "failures": failures,
            "excused_accept": excused_acc, "excused_draw": excused_draw}


def end_to_end_bands(max_dz: float, T: float, draw_mass):
    """Bands of an end-to-end comparison, where the oracle scores in fp64 and the
    step under test in fp32: a logit error of at most max_dz moves p(x)/q(x)
    by about 2 max_dz / T relatively and a draw's CDF edge by about
    2 max_dz / (T S) (S the mass drawn from); twice that is allowed.  At T = 0
    the band is on the top-2 logit gap.  Returns (acc_band, draw_band)."""
    if T == 0.0:
        return 4.0 * max_dz, 4.0 * max_dz
    acc = max(1e-5, 4.0 * max_dz / T)
    draw = 4.0 * max_dz / (T * np.maximum(np.asarray(draw_mass, dtype=np.float64), 1e-12))
    return acc, draw
