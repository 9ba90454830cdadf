"""Pins that tie the oracle to what the pages and the mathematics fix.

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError when the
oracle disagrees with something that is known independently of it: a value the
pages print (fixtures under ``tests/golden/``), a closed form, an invariant, a
library routine that computes the same thing, or an exact brute-force
enumeration on tiny inputs.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_negative.py`` runs them on builds with a planted mistake
and requires every such build to fail at least one pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
from scipy import stats

import oracle as oracle_mod
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tv(counts: np.ndarray, p: np.ndarray) -> float:
    emp = counts / counts.sum()
    return 0.5 * float(np.abs(emp - np.asarray(p, dtype=np.float64)).sum())


def _dyadic_simplex(rng, V, bits=20):
    """Probability vector whose entries are multiples of 2**-bits and sum to exactly 1."""
    cuts = np.sort(rng.integers(0, 2**bits + 1, size=V - 1))
    k = np.diff(np.concatenate([[0], cuts, [2**bits]]))
    return (k / 2.0**bits).astype(np.float32)


# ---------------------------------------------------------------------------
# Losslessness identity: min(q, p) + max(0, p - q) = p, pointwise.

def pin_identity(o):
    rng = np.random.default_rng(11)
    for V in (2, 5, 32, 257):
        for _ in range(10):
            p, q = _dyadic_simplex(rng, V), _dyadic_simplex(rng, V)
            r, S = o.residual(p, q)
            mn = np.minimum(p, q).astype(np.float64)
            assert np.array_equal(mn + r.astype(np.float64), p.astype(np.float64)), "min(q,p)+(p-q)+ != p"
            assert S == 1.0 - mn.sum(), "residual mass != 1 - alpha"
            assert o.acceptance_rate(p, q) == mn.sum()
    # Arbitrary fp32 vectors: the identity holds up to the one rounding of p - q.
    p = rng.random(1000).astype(np.float32)
    q = rng.random(1000).astype(np.float32)
    r, _ = o.residual(p, q)
    lhs = np.minimum(p, q).astype(np.float64) + r.astype(np.float64)
    assert np.all(np.abs(lhs - p) <= np.spacing(np.maximum(p, q)).astype(np.float64))
    assert np.all(r >= 0)


def pin_prep_residual(o):
    g = golden("prep_demo.json")
    p = np.array(g["p"], np.float32)
    q = np.array(g["q"], np.float32)
    r, S = o.residual(p, q)
    assert np.allclose(r / S, g["residual_printed"], rtol=0, atol=1e-6)
    assert abs(o.acceptance_rate(p, q) - 0.85) < 1e-6
    assert abs(S - 0.15) < 1e-6


# ---------------------------------------------------------------------------
# Expected tokens per pass.

def pin_expected_tokens(o):
    g = golden("prep_demo.json")["expected_tokens_table"]
    for i, a in enumerate(g["alpha"]):
        for j, k in enumerate(g["k"]):
            assert abs(o.expected_tokens(a, k) - g["printed_3dp"][i][j]) <= 5e-4 + 1e-12, (a, k)
    m = golden("math_expected_tokens.json")
    assert abs(o.expected_tokens(m["beta"], m["gamma"]) - m["expected_tokens_3dp"]) <= 5e-4
    assert abs((1 - m["beta_pow_gamma_plus_1"]) / (1 - m["beta"]) - o.expected_tokens(m["beta"], m["gamma"])) < 1e-12
    s = golden("llmi_script.json")
    assert abs(o.expected_tokens(s["section2_alpha"], s["section2_gamma"]) - s["section2_expected_tokens_2dp"]) <= 5e-3
    for k in (0, 1, 4, 7):
        assert o.expected_tokens(1.0, k) == k + 1
        assert o.expected_tokens(0.0, k) == 1.0
        for a in (0.3, 0.77):
            # the truncated geometric sum written out term by term
            direct = sum((j + 1) * a**j * (1 - a) for j in range(k)) + (k + 1) * a**k
            assert abs(o.expected_tokens(a, k) - direct) < 1e-12
            assert abs(o.expected_tokens_rows([a] * k) - direct) < 1e-12
    assert abs(o.expected_tokens_rows([0.5, 0.25]) - 1.625) < 1e-15
    assert o.expected_tokens_rows([]) == 1.0


# ---------------------------------------------------------------------------
# Temperature softmax.

def pin_softmax(o):
    p = np.array([0.1, 0.2, 0.3, 0.4])
    z = np.log(p).astype(np.float32)
    for T, expect in ((1.0, p), (0.5, p**2 / (p**2).sum()), (2.0, np.sqrt(p) / np.sqrt(p).sum())):
        out, m, Z = o.softmax(z, T)
        assert np.allclose(out, expect, rtol=1e-6, atol=0), (T, out, expect)
        assert abs(m - float(z.max()) / T) < 1e-15
        assert abs(Z - np.exp(z.astype(np.float64) / T - m).sum()) < 1e-14
    big = np.array([1000.0, 999.0, 998.0], np.float32)
    out, _, _ = o.softmax(big, 1.0)
    e = np.exp([0.0, -1.0, -2.0])
    assert np.all(np.isfinite(out)) and np.allclose(out, e / e.sum(), rtol=1e-6, atol=0)
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, 500).astype(np.float32)
    out, _, _ = o.softmax(z, 0.7)
    shifted, _, _ = o.softmax(z + np.float32(0.0), 0.7)
    assert abs(float(out.astype(np.float64).sum()) - 1.0) < 1e-5
    assert np.array_equal(out, shifted)
    ref = np.exp(z.astype(np.float64) / 0.7 - (z.astype(np.float64) / 0.7).max())
    assert np.allclose(out, ref / ref.sum(), rtol=1e-6, atol=1e-30)


def pin_argmax(o):
    rng = np.random.default_rng(5)
    for V in (1, 2, 7, 1000):
        for _ in range(20):
            z = rng.integers(-3, 4, size=V).astype(np.float32)  # many ties
            idx, gap = o.argmax(z)
            assert idx == int(np.argmax(z)), (z, idx)
            if V > 1:
                rest = np.delete(z, idx)
                assert gap == float(z[idx] - rest.max())


# ---------------------------------------------------------------------------
# Inverse-CDF draw: smallest v with u*S < C_v, the textbook rule that
# numpy's searchsorted(side="right") computes on the fp64 prefix sums.

def pin_draw(o):
    rng = np.random.default_rng(7)
    for V in (1, 3, 8, 100):
        for _ in range(10):
            w = rng.random(V).astype(np.float32)
            w[rng.random(V) < 0.3] = 0.0
            w[0] = 0.0 if V > 1 else w[0]
            if not np.any(w > 0):
                w[-1] = 1.0
            C = np.cumsum(w.astype(np.float64))
            S = C[-1]
            us = np.concatenate([[0.0, 1 - 2.0**-24], synth.uniforms((50,), 9, V)]).astype(np.float32)
            for u in us:
                t = float(u) * S
                expect = int(np.searchsorted(C, t, side="right"))
                if expect == V:
                    expect = int(np.nonzero(w > 0)[0][-1])
                got, margin = o.draw(w, float(u))
                assert got == expect, (w, u, got, expect)
                assert w[got] > 0, "drew a token with zero weight"
                lo = C[got - 1] if got > 0 else 0.0
                assert abs(margin - min(t - lo, C[got] - t) / S) < 1e-12
    assert o.draw(np.zeros(5, np.float32), 0.3)[0] == -1


# ---------------------------------------------------------------------------
# Acceptance test: u < min(1, p/q), strict.

def pin_accept(o):
    assert o.accept(0.25, 0.5, 0.4999)[0]
    assert not o.accept(0.25, 0.5, 0.5)[0], "u == p/q must reject"
    assert not o.accept(0.25, 0.5, 0.5001)[0]
    assert not o.accept(0.125, 0.5, 0.25)[0]
    assert o.accept(0.125, 0.5, 0.2)[0] and o.accept(0.125, 0.5, 0.2499)[0]
    top = 1 - 2.0**-24
    assert o.accept(0.5, 0.25, top)[0] and o.accept(0.3, 0.3, top)[0]
    assert o.accept(0.3, 0.0, top)[0], "q below the floor must accept"
    assert not o.accept(0.0, 0.3, 0.0)[0], "p == 0 must reject even at u == 0"
    keep, m = o.accept(0.25, 0.5, 0.375)
    assert keep and abs(m - 0.125) < 1e-12
    # fraction of a uniform lattice accepted equals min(1, p/q) exactly when G*p/q is an integer
    G = 64
    lattice = ((np.arange(G) + 0.5) / G).astype(np.float32)
    for p_x, q_x in ((0.125, 0.5), (0.375, 0.5), (0.5, 0.5), (0.75, 0.25)):
        frac = np.mean([o.accept(p_x, q_x, float(u))[0] for u in lattice])
        assert frac == min(1.0, p_x / q_x), (p_x, q_x, frac)


# ---------------------------------------------------------------------------
# Exact brute force on tiny inputs.  Row i has its own dyadic (p_i, q_i), so the
# algorithm is piecewise constant in the uniforms with breakpoints on a grid of
# 1/G.  Enumerating every drafted-token combination (weighted by q) and every
# lattice point of the uniforms gives the exact probability of each emitted
# sequence, which the acceptance rule fixes in closed form: a step that keeps
# x_0..x_{k-1} and then emits y has probability
#   prod_{i<k} min(p_i(x_i), q_i(x_i)) * (p_k(y) - q_k(y))+   (k < gamma)
#   prod_{i<k} min(p_i(x_i), q_i(x_i)) * p_gamma(y)            (k = gamma).
# Summing over the ways to reach it, each emitted token follows the target row.

_BF_P = [[3 / 8, 3 / 8, 1 / 8, 1 / 8], [1 / 8, 1 / 4, 1 / 2, 1 / 8], [1 / 2, 1 / 4, 1 / 8, 1 / 8]]
_BF_Q = [[1 / 8, 1 / 8, 1 / 4, 1 / 2], [1 / 2, 1 / 8, 1 / 4, 1 / 8]]
_BF_G = 24  # multiple of 4 (ratios), 3 (residual CDF of row 1) and 8 (bonus CDF)


def bruteforce_distribution(o, gamma: int):
    V = 4
    p_rows = np.array(_BF_P[:gamma] + [_BF_P[2]], np.float32).reshape(gamma + 1, V)
    q_rows = np.array(_BF_Q[:gamma], np.float32).reshape(gamma, V)
    G = _BF_G
    lat = ((np.arange(G) + 0.5) / G).astype(np.float32)
    combos = np.array(list(itertools.product(range(V), repeat=gamma)), np.int32).reshape(V**gamma, gamma)
    grid = np.array(list(itertools.product(range(G), repeat=gamma + 1)), np.int64).reshape(-1, gamma + 1)
    nc, nl = len(combos), len(grid)
    B = nc * nl
    x = np.ascontiguousarray(np.repeat(combos, nl, axis=0))
    gi = np.tile(grid, (nc, 1))
    u = np.zeros((B, gamma + 1, 2), np.float32)
    u[:, :gamma, 0] = lat[gi[:, :gamma]]
    u[:, :, 1] = lat[gi[:, gamma]][:, None]
    wc = np.ones(nc)
    for i in range(gamma):
        wc *= q_rows[i][combos[:, i]].astype(np.float64)
    w = np.repeat(wc, nl) / float(G) ** (gamma + 1)
    p = np.broadcast_to(p_rows, (B, gamma + 1, V))
    q = np.broadcast_to(q_rows, (B, gamma, V))
    out = o.verify_probs(p, q, x, u)
    rows, inv = np.unique(out["tokens"], axis=0, return_inverse=True)
    mass = np.bincount(inv.ravel(), weights=w, minlength=len(rows))
    dist = {}
    for r, m in zip(rows, mass):
        n = int(np.sum(r >= 0))
        assert np.all(r[:n] >= 0) and np.all(r[n:] == -1)
        dist[tuple(int(t) for t in r[:n])] = dist.get(tuple(int(t) for t in r[:n]), 0.0) + float(m)
    # num_emitted must agree with the tokens it reports
    assert np.array_equal(out["num_emitted"], np.sum(out["tokens"] >= 0, axis=1))
    return dist, p_rows.astype(np.float64), q_rows.astype(np.float64)


def pin_bruteforce(o):
    for gamma in (0, 1, 2):
        dist, P, Q = bruteforce_distribution(o, gamma)
        expect = {}
        for k in range(gamma + 1):
            for keep in itertools.product(range(4), repeat=k):
                pre = np.prod([min(P[i][keep[i]], Q[i][keep[i]]) for i in range(k)]) if k else 1.0
                for y in range(4):
                    if k < gamma:
                        mass = pre * max(0.0, P[k][y] - Q[k][y])
                    else:
                        mass = pre * P[gamma][y]
                    if mass > 0:
                        expect[tuple(keep) + (y,)] = expect.get(tuple(keep) + (y,), 0.0) + mass
        keys = set(dist) | set(expect)
        for key in keys:
            assert abs(dist.get(key, 0.0) - expect.get(key, 0.0)) < 1e-12, (gamma, key, dist.get(key), expect.get(key))
        # the first emitted token follows target row 0 exactly
        first = np.zeros(4)
        for key, mass in dist.items():
            first[key[0]] += mass
        assert np.allclose(first, P[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Special cases with known answers.

def pin_special_cases(o):
    rng = np.random.default_rng(21)
    V, g, B = 16, 3, 2000
    # q == p: every draft is kept, so every step emits gamma + 1 tokens.
    p = _dyadic_simplex(rng, V)
    P = np.broadcast_to(p, (B, g + 1, V))
    Q = np.broadcast_to(p, (B, g, V))
    x = rng.integers(0, V, size=(B, g)).astype(np.int32)
    x = np.where(p[x] > 0, x, int(np.argmax(p)))
    u = synth.uniforms((B, g + 1, 2), 31, 0)
    out = o.verify_probs(P, Q, x, u)
    assert np.all(out["num_emitted"] == g + 1)
    assert np.array_equal(out["tokens"][:, :g], x)
    # disjoint supports: every draft is rejected and the residual is p itself.
    p = np.zeros(V, np.float32)
    p[0::2] = 1.0 / (V // 2)
    q = np.zeros(V, np.float32)
    q[1::2] = 1.0 / (V // 2)
    x = (2 * rng.integers(0, V // 2, size=(B, g)) + 1).astype(np.int32)
    out = o.verify_probs(np.broadcast_to(p, (B, g + 1, V)), np.broadcast_to(q, (B, g, V)), x, u)
    assert np.all(out["num_emitted"] == 1)
    assert np.all(out["tokens"][:, 0] % 2 == 0)
    # one-hot draft q = e_x: keep x with probability p(x); otherwise p without x, renormalised.
    p = np.array([1 / 8, 1 / 2, 1 / 4, 1 / 8], np.float32)
    q = np.array([0, 1, 0, 0], np.float32)
    G = 64
    lat = ((np.arange(G) + 0.5) / G).astype(np.float32)
    ua, us = np.meshgrid(lat, lat, indexing="ij")
    n = G * G
    u = np.zeros((n, 2, 2), np.float32)
    u[:, 0, 0] = ua.ravel()
    u[:, :, 1] = us.ravel()[:, None]
    out = o.verify_probs(np.broadcast_to(p, (n, 2, 4)), np.broadcast_to(q, (n, 1, 4)), np.ones((n, 1), np.int32), u)
    kept = out["num_emitted"] == 2
    assert abs(kept.mean() - 0.5) < 1e-12
    rej = out["tokens"][~kept, 0]
    assert np.all(rej != 1)
    freq = np.bincount(rej, minlength=4) / rej.size
    assert np.allclose(freq, [0.25, 0, 0.5, 0.25], atol=1e-12)
    # The same from logits with the one-hot draft kind (no draft array: q = e_x by construction).
    z = np.log(p.astype(np.float64)).astype(np.float32)
    out1 = o.verify(np.broadcast_to(z, (n, 2, 4)), None, np.ones((n, 1), np.int32), u, 1.0,
                    draft_kind=oracle_mod.Q_ONEHOT)
    kept1 = out1["num_emitted"] == 2
    assert abs(kept1.mean() - 0.5) < 1e-12
    freq1 = np.bincount(out1["tokens"][~kept1, 0], minlength=4) / (~kept1).sum()
    assert np.allclose(freq1, [0.25, 0, 0.5, 0.25], atol=1e-12)
    # and equals the probability kind fed an explicit one-hot q, step for step
    zz = synth.normal_f32((300, 3, V), 1.5, 51, 0)
    xx = synth.integers((300, 2), 0, V, 51, 1)
    uu = synth.uniforms((300, 3, 2), 51, 2)
    qq = np.zeros((300, 2, V), np.float32)
    np.put_along_axis(qq, xx[..., None].astype(np.int64), 1.0, axis=2)
    a1 = o.verify(zz, None, xx, uu, 0.9, draft_kind=oracle_mod.Q_ONEHOT)
    a2 = o.verify(zz, qq, xx, uu, 0.9, draft_kind=oracle_mod.Q_PROBS)
    assert np.array_equal(a1["tokens"], a2["tokens"]) and np.array_equal(a1["num_emitted"], a2["num_emitted"])
    # gamma = 0: one inverse-CDF draw from p.
    p = _dyadic_simplex(rng, V)
    us = synth.uniforms((500,), 41, 0)
    u = np.zeros((500, 1, 2), np.float32)
    u[:, 0, 1] = us
    out = o.verify_probs(np.broadcast_to(p, (500, 1, V)), np.zeros((500, 0, V), np.float32),
                         np.zeros((500, 0), np.int32), u)
    C = np.cumsum(p.astype(np.float64))
    assert np.array_equal(out["tokens"][:, 0], np.searchsorted(C, us.astype(np.float64) * C[-1], side="right"))
    assert np.all(out["num_emitted"] == 1)


# ---------------------------------------------------------------------------
# Greedy rule (T = 0).

def pin_greedy(o):
    V, g = 6, 3
    z = np.array([
        [0.1, 2.0, 0.3, -1.0, 0.0, 0.5],   # argmax 1
        [1.5, 0.0, 1.5, 0.2, 0.1, -3.0],   # tie between 0 and 2 -> 0
        [0.0, 0.0, 0.0, 0.0, 4.0, 0.0],    # argmax 4
        [0.0, 9.0, 0.0, 0.0, 0.0, 9.5],    # argmax 5 (bonus row)
    ], np.float32)
    cases = [
        ([1, 0, 4], [1, 0, 4, 5], 4),
        ([2, 0, 4], [1], 1),
        ([1, 2, 4], [1, 0], 2),
        ([1, 0, 3], [1, 0, 4], 3),
    ]
    for x, toks, n in cases:
        for draft, uni in ((None, None), (np.full((1, g, V), 7.0, np.float32), np.full((1, g + 1, 2), 0.99, np.float32))):
            out = o.verify(z[None], draft, np.array([x], np.int32), uni, 0.0)
            assert int(out["num_emitted"][0]) == n, (x, out)
            assert list(out["tokens"][0][:n]) == toks, (x, out)
            assert np.all(out["tokens"][0][n:] == -1)
    # random rows: the emitted tokens are the chain of row argmaxes along the kept prefix
    rng = np.random.default_rng(8)
    B, g, V = 300, 4, 50
    z = rng.integers(-5, 6, size=(B, g + 1, V)).astype(np.float32)
    am = np.argmax(z, axis=2)
    x = np.where(rng.random((B, g)) < 0.7, am[:, :g], rng.integers(0, V, size=(B, g))).astype(np.int32)
    out = o.verify(z, None, x, None, 0.0)
    for b in range(B):
        k = next((i for i in range(g) if x[b, i] != am[b, i]), g)
        assert out["num_emitted"][b] == k + 1
        assert list(out["tokens"][b][:k + 1]) == list(am[b, :k + 1])


# ---------------------------------------------------------------------------
# The linear layer.

def pin_linear(o):
    rng = np.random.default_rng(13)
    N, d, V = 7, 33, 19
    Xi = rng.integers(-8, 9, size=(N, d))
    Wi = rng.integers(-8, 9, size=(V, d))
    Y = o.linear(synth.bf16_bits(Xi.astype(np.float32)), synth.bf16_bits(Wi.astype(np.float32)))
    assert np.array_equal(Y, (Xi @ Wi.T).astype(np.float64))
    # one-hot rows of X pick out a column of W
    ks = rng.integers(0, d, size=N)
    X1 = np.zeros((N, d), np.float32)
    X1[np.arange(N), ks] = 1.0
    Wf = rng.normal(0, 1, size=(V, d)).astype(np.float32)
    Wb = synth.bf16_bits(Wf)
    Y1 = o.linear(synth.bf16_bits(X1), Wb)
    assert np.array_equal(Y1, synth.bf16_to_f32(Wb)[:, ks].T.astype(np.float64))
    ni = rng.integers(0, N, size=40)
    vi = rng.integers(0, V, size=40)
    Xb = synth.bf16_bits(rng.normal(0, 1, size=(N, d)).astype(np.float32))
    Yf = o.linear(Xb, Wb)
    assert np.array_equal(o.linear_entries(Xb, Wb, ni, vi), Yf[ni, vi])
    ref = synth.bf16_to_f32(Xb).astype(np.float64) @ synth.bf16_to_f32(Wb).astype(np.float64).T
    assert np.allclose(Yf, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Statistical pins (fixed seeds).  The first emitted token of every step must
# follow the target row; the number emitted must match the closed form.

def _first_token_stats(o, p, q, gamma, trials, seed):
    V = p.size
    xs = np.empty((trials, gamma), np.int32)
    du = synth.uniforms((trials, gamma), seed, synth.STREAM_DRAFT_SAMPLE)
    C = np.cumsum(q.astype(np.float64))
    xs[:] = np.searchsorted(C, du.astype(np.float64) * C[-1], side="right")
    u = synth.uniforms((trials, gamma + 1, 2), seed, synth.STREAM_STEP_UNIFORMS)
    out = o.verify_probs(np.broadcast_to(p, (trials, gamma + 1, V)), np.broadcast_to(q, (trials, gamma, V)), xs, u)
    counts = np.bincount(out["tokens"][:, 0], minlength=V).astype(np.float64)
    return counts, out


def pin_prep_tv(o):
    g = golden("prep_demo.json")
    p = np.array(g["p"], np.float32)
    q = np.array(g["q"], np.float32)
    counts, _ = _first_token_stats(o, p, q, 1, g["trials"], seed=42)
    tv = _tv(counts, p)
    assert tv < 0.005 and tv < g["tv_bound_asserted"], tv


def pin_llmi_toy(o):
    g = golden("llmi_script.json")
    p = np.array(g["p"], np.float32)
    q = np.array(g["q"], np.float32)
    trials = 200_000
    counts, out = _first_token_stats(o, p, q, g["gamma"], trials, seed=7)
    tv = _tv(counts, p)
    assert tv < 0.005, tv
    alpha = o.acceptance_rate(p, q)
    assert abs(alpha - 0.80) < 1e-6
    e = o.expected_tokens(alpha, g["gamma"])
    n = out["num_emitted"].astype(np.float64)
    assert abs(n.mean() - e) < 4 * n.std() / math.sqrt(trials), (n.mean(), e)


# ---------------------------------------------------------------------------
# Tree verification ([LLMI] section 3; [MATH] "SpecInfer and Tree-Based
# Verification").

def _tree_paths_bruteforce(parents, node_tokens, best):
    """Every root-to-node path, taken whole: a path is kept iff each of its nodes after the root carries the argmax of
    the previous node's row.  Returns (deepest kept path (lowest end index among equals), its end)."""
    M = len(parents)
    kept = []
    for end in range(M):
        path, cur, ok = [], end, True
        while True:
            path.append(cur)
            if cur == 0:
                break
            p = parents[cur]
            if not (0 <= p < cur):
                ok = False
                break
            cur = p
        if not ok:
            continue
        path = path[::-1]
        if all(node_tokens[path[j]] == best[path[j - 1]] for j in range(1, len(path))):
            kept.append(path)
    return max(kept, key=lambda pth: (len(pth), -pth[-1]))


def pin_tree(o):
    g = golden("llmi_tree_and_paged_kv.json")
    mask, depth, add = o.tree_mask(g["tree_parents"])
    assert depth.tolist() == g["tree_depths_asserted"]
    # ancestors-or-self of [-1, 0, 0, 1, 1, 2]: {0}, {0,1}, {0,2}, {0,1,3}, {0,1,4}, {0,2,5}
    assert mask.tolist() == [0b1, 0b11, 0b101, 0b1011, 0b10011, 0b100101]
    assert np.array_equal(add == 0, ((mask[:, None] >> np.arange(6, dtype=np.uint64)[None, :]) & 1) == 1)
    assert np.all(np.isneginf(add[add != 0]))
    # A worked tree: root 0; children 1 (token 7) and 2 (token 3); 3 under 2 (token 5); 4 under 1 (token 9).
    V = 16
    z = np.zeros((5, V), np.float32)
    z[0, 3] = z[1, 9] = z[2, 5] = z[3, 11] = z[4, 2] = 4.0
    tok, nodes, n = o.tree_greedy(z, [-1, 0, 0, 2, 1], [0, 7, 3, 5, 9])
    assert n == 3 and tok[:3].tolist() == [3, 5, 11] and nodes[:3].tolist() == [0, 2, 3]
    assert np.all(tok[3:] == -1) and np.all(nodes[3:] == -1)
    # Two siblings carrying the same right token: the lower index is kept.
    tok, nodes, n = o.tree_greedy(z[:3], [-1, 0, 0], [0, 3, 3])
    assert n == 2 and nodes[:2].tolist() == [0, 1] and tok[:2].tolist() == [3, 9]
    # A detached node (parent not before it) is never kept and has depth 0.
    _, dep, _ = o.tree_mask([-1, 0, 5, 1])
    assert dep.tolist() == [0, 1, 0, 2]
    tok, nodes, n = o.tree_greedy(z[:3], [-1, 7, 0], [0, 3, 3])  # node 1 detached although its token is right
    assert n == 2 and nodes[:2].tolist() == [0, 2] and tok[:2].tolist() == [3, 5]
    # A chain is the linear greedy rule: node i carries draft i-1, row i scores the position after it.
    rng = np.random.default_rng(71)
    for _ in range(20):
        M, V = int(rng.integers(2, 9)), 12
        zz = synth.normal_f32((M, V), 1.0, int(rng.integers(1 << 30)), 0)
        best = zz.argmax(axis=1)
        x = np.where(rng.random(M - 1) < 0.7, best[:-1], rng.integers(0, V, M - 1)).astype(np.int32)
        tok, nodes, n = o.tree_greedy(zz, [-1] + list(range(M - 1)), np.concatenate([[0], x]))
        lin = o.verify(zz[None], None, x[None], None, 0.0)
        assert n == lin["num_emitted"][0] and np.array_equal(tok[:n], lin["tokens"][0][:n])
        assert nodes[:n].tolist() == list(range(n))
    # Brute force over random small trees: every path checked whole.
    for trial in range(200):
        M, V = int(rng.integers(1, 12)), 4
        parents = [-1] + [int(rng.integers(-1, i + 1)) if rng.random() < 0.1 else int(rng.integers(0, i))
                          for i in range(1, M)]
        zz = synth.integers((M, V), 0, 3, trial, 9).astype(np.float32)  # many ties: lowest index wins
        best = [min(np.flatnonzero(zz[i] == zz[i].max())) for i in range(M)]
        node_tokens = [0] + [int(rng.integers(0, V)) for _ in range(1, M)]
        path = _tree_paths_bruteforce(parents, node_tokens, best)
        tok, nodes, n = o.tree_greedy(zz, parents, node_tokens)
        assert n == len(path) and nodes[:n].tolist() == path
        assert tok[:n].tolist() == [node_tokens[j] for j in path[1:]] + [best[path[-1]]]


# ---------------------------------------------------------------------------
# Paged KV cache ([LLMI] section 1; the section 5 script's rollback check).

def pin_paged_kv(o):
    g = golden("llmi_tree_and_paged_kv.json")["paged_kv"]
    kv = o.kv_cache(1, g["num_blocks"], g["block_size"], g["n_kv_heads"], g["head_dim"], max_blocks=8)
    k = synth.normal_f32((1, g["n_kv_heads"], g["appended_tokens"], g["head_dim"]), 1.0, 81, 0)
    v = synth.normal_f32(k.shape, 1.0, 81, 1)
    assert kv.append(k, v) == 0
    assert kv.tables[0, :3].tolist() == [0, 1, 2]  # the free list starts reversed, so blocks come out 0, 1, 2
    kv.rollback([g["rollback_to"]])
    kg, vg = kv.gather(0)
    n = g["gather_equals_first"]
    assert np.array_equal(kg, k[0, :, :n]) and np.array_equal(vg, v[0, :, :n])
    assert kv.lens[0] == 6 and kv.top[0] == g["num_blocks"] - 2
    # the freed block is the first one handed out again
    assert kv.append(k[:, :, :3], v[:, :, :3]) == 0 and kv.tables[0, 2] == 2
    # several trailing blocks go back last-logical-first: the earlier one is on top
    kv2 = o.kv_cache(1, 8, 4, 1, 4, max_blocks=8)
    z = synth.normal_f32((1, 1, 12, 4), 1.0, 82, 0)
    kv2.append(z, z)
    kv2.rollback([1])
    assert kv2.stack[kv2.top[0] - 1] == 1 and kv2.stack[kv2.top[0] - 2] == 2
    # not enough free blocks, or a table too short: nothing changes
    snap = (kv2.lens.copy(), kv2.top.copy(), kv2.tables.copy())
    big = synth.normal_f32((1, 1, 40, 4), 1.0, 83, 0)
    assert kv2.append(big, big) == 2
    kv3 = o.kv_cache(2, 3, 4, 1, 4, max_blocks=8)
    zz = synth.normal_f32((2, 1, 8, 4), 1.0, 84, 0)
    assert kv3.append(zz, zz) == 1 and kv3.lens.tolist() == [0, 0] and kv3.top[0] == 3
    assert np.array_equal(kv2.lens, snap[0]) and np.array_equal(kv2.top, snap[1])
    # a request asked to grow is left as it is
    assert kv2.rollback([5]) == 1 and kv2.lens[0] == 1
    # Random batches of appends and rollbacks against a plain list of tokens per request.
    rng = np.random.default_rng(85)
    R, NB, BS, H, D = 5, 64, 4, 2, 8
    kv = o.kv_cache(R, NB, BS, H, D, max_blocks=12)
    plain = [np.zeros((H, 0, D), np.float32) for _ in range(R)]
    for step in range(40):
        if rng.random() < 0.6:
            n_new = int(rng.integers(1, 6))
            kn = synth.normal_f32((R, H, n_new, D), 1.0, 900 + step, 0)
            vn = synth.normal_f32((R, H, n_new, D), 1.0, 900 + step, 1)
            if all(plain[r].shape[1] + n_new <= 12 * BS for r in range(R)) and kv.append(kn, vn) == 0:
                plain = [np.concatenate([plain[r], kn[r]], axis=1) for r in range(R)]
        else:
            keep = [int(rng.integers(0, plain[r].shape[1] + 1)) for r in range(R)]
            assert kv.rollback(keep) == 0
            plain = [plain[r][:, :keep[r]] for r in range(R)]
        used = [int(b) for r in range(R) for b in kv.tables[r, :(kv.lens[r] + BS - 1) // BS]]
        assert sorted(used + kv.stack[:kv.top[0]].tolist()) == list(range(NB))  # every block exactly once
        for r in range(R):
            kg, _ = kv.gather(r)
            assert np.array_equal(kg, plain[r])


# ---------------------------------------------------------------------------
# top-k / top-p warping before the rule ([LESS] "Why the output is exactly p";
# [PREP] "Correctness").

def pin_warp(o):
    # top-k on a worked row: ranking by logit, ties to the lower index.
    z = np.array([3.0, 1.0, 2.0, 2.0, 0.0], np.float32)
    p, n, _ = o.warp(z, 1.0, top_k=2)
    assert n == 2 and np.flatnonzero(p).tolist() == [0, 2]
    e = np.exp(np.array([3.0, 2.0]) - 3.0)
    assert np.allclose(p[[0, 2]], e / e.sum(), rtol=1e-7, atol=0)
    # top-p on dyadic probabilities [1/2, 1/4, 1/8, 1/8]: the shortest prefix reaching p; reaching it exactly counts
    z = np.log(np.array([0.5, 0.25, 0.125, 0.125])).astype(np.float32)
    for top_p, kept in ((0.7, 2), (0.75, 2), (0.76, 3), (0.5, 1), (0.1, 1), (0.999, 4)):
        p, n, _ = o.warp(z, 1.0, top_p=top_p)
        assert n == kept, (top_p, n)
        assert abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-6
    # top-p after top-k: the mass is that of the top-k survivors
    p, n, _ = o.warp(z, 1.0, top_k=2, top_p=0.7)  # survivors [2/3, 1/3]: 2/3 < 0.7
    assert n == 2
    p, n, _ = o.warp(z, 1.0, top_k=2, top_p=0.6)
    assert n == 1 and p[0] == 1.0
    # no warping reproduces the plain rule
    zz = synth.normal_f32((200, 4, 64), 1.5, 61, 0)
    dd = zz[:, :3] + synth.normal_f32((200, 3, 64), 1.0, 61, 1)
    xx = synth.integers((200, 3), 0, 64, 61, 2)
    uu = synth.uniforms((200, 4, 2), 61, 3)
    a = o.verify(zz, dd, xx, uu, 0.8)
    b = o.verify_warped(zz, dd, xx, uu, 0.8, top_k=0, top_p=1.0)
    c = o.verify_warped(zz, dd, xx, uu, 0.8, top_k=64, top_p=1.5)
    for r in (b, c):
        assert np.array_equal(a["tokens"], r["tokens"]) and np.array_equal(a["num_emitted"], r["num_emitted"])
    # the rule reproduces the warped p: exact distribution of the first emitted token over a lattice of uniforms
    V = 6
    zt = np.array([2.0, 1.5, 1.0, 0.2, -0.5, 0.1], np.float32)
    zd = np.array([0.5, 2.0, 0.0, 1.0, 0.3, -1.0], np.float32)
    for top_k, top_p in ((3, 1.0), (0, 0.8), (4, 0.9)):
        pw, _, _ = o.warp(zt, 1.0, top_k, top_p)
        qw, _, _ = o.warp(zd, 1.0, top_k, top_p)
        G = 512
        lat = ((np.arange(G) + 0.5) / G).astype(np.float32)
        tot = np.zeros(V)
        for x in np.flatnonzero(qw):  # the draft's token, weighted by q
            uu = np.zeros((G * G, 2, 2), np.float32)
            ua, us = np.meshgrid(lat, lat, indexing="ij")
            uu[:, 0, 0] = ua.ravel()
            uu[:, :, 1] = us.ravel()[:, None]
            out = o.verify_warped(np.broadcast_to(zt, (G * G, 2, V)), np.broadcast_to(zd, (G * G, 1, V)),
                                  np.full((G * G, 1), x, np.int32), uu, 1.0, top_k, top_p)
            tot += float(qw[x]) * np.bincount(out["tokens"][:, 0], minlength=V) / (G * G)
        assert np.abs(tot - pw).max() < 4.0 / G, (top_k, top_p, tot, pw)


def toy_config_inputs(o, w: synth.Workload, independent_rows: bool = False):
    """The reject-only toy workload: target logits z ~ N(0, target_std) for one row (or one per position),
    draft logits z + N(0, noise_std), replicated over B trials; drafted tokens follow q (drawn with the oracle)."""
    nrow = w.gamma + 1 if independent_rows else 1
    z = synth.normal_f32((nrow, w.V), w.target_std, w.seed, synth.STREAM_TARGET)
    dz = z[: max(1, min(nrow, w.gamma))] + synth.normal_f32((max(1, min(nrow, w.gamma)), w.V), w.noise_std, w.seed,
                                                          synth.STREAM_DRAFT_NOISE)
    zt = np.ascontiguousarray(np.broadcast_to(z if independent_rows else z[0], (w.B, w.gamma + 1, w.V)))
    zd_rows = dz if independent_rows else np.broadcast_to(dz[0], (w.gamma, w.V))
    zd = np.ascontiguousarray(np.broadcast_to(zd_rows, (w.B, w.gamma, w.V)))
    du = synth.draft_sample_uniforms(w)
    x = np.empty((w.B, w.gamma), np.int32)
    for i in range(w.gamma):
        x[:, i] = _sample_column(o, zd_rows[i], du[:, i], w.temperature)
    return zt, zd, x, synth.step_uniforms(w)


def _sample_column(o, zrow, us, T):
    p, _, _ = o.softmax(zrow, T)
    C = np.cumsum(p.astype(np.float64))
    # same inverse-CDF rule as the oracle's draw, applied to many uniforms at once
    idx = np.searchsorted(C, us.astype(np.float64) * C[-1], side="right")
    return np.minimum(idx, p.size - 1).astype(np.int32)


def pin_config_toy(o):
    w = synth.WORKLOADS["toy_v32"]
    zt, zd, x, u = toy_config_inputs(o, w)
    out = o.verify(zt, zd, x, u, w.temperature)
    p, _, _ = o.softmax(zt[0, 0], w.temperature)
    q, _, _ = o.softmax(zd[0, 0], w.temperature)
    counts = np.bincount(out["tokens"][:, 0], minlength=w.V).astype(np.float64)
    tv = _tv(counts, p)
    assert tv < 0.005, tv
    expected = w.B * p.astype(np.float64)
    keep = expected >= 5
    chi2 = float((((counts - expected) ** 2) / expected)[keep].sum()) + \
        float(((counts[~keep].sum() - expected[~keep].sum()) ** 2) / max(expected[~keep].sum(), 1e-300))
    dof = int(keep.sum()) - (0 if (~keep).any() else 1)
    assert chi2 < stats.chi2.ppf(0.95, dof), (chi2, dof)
    alpha = o.acceptance_rate(p, q)
    n = out["num_emitted"].astype(np.float64)
    assert abs(n.mean() - o.expected_tokens(alpha, w.gamma)) < 4 * n.std() / math.sqrt(w.B)
    # independent rows: E[N] follows the product form
    zt, zd, x, u = toy_config_inputs(o, w, independent_rows=True)
    out = o.verify(zt, zd, x, u, w.temperature)
    alphas = [o.acceptance_rate(o.softmax(zt[0, i], 1.0)[0], o.softmax(zd[0, i], 1.0)[0]) for i in range(w.gamma)]
    n = out["num_emitted"].astype(np.float64)
    assert abs(n.mean() - o.expected_tokens_rows(alphas)) < 4 * n.std() / math.sqrt(w.B)


ALL_PINS = [
    pin_identity, pin_prep_residual, pin_expected_tokens, pin_softmax, pin_argmax, pin_draw, pin_accept,
    pin_bruteforce, pin_special_cases, pin_greedy, pin_linear, pin_prep_tv, pin_llmi_toy, pin_config_toy, pin_tree,
    pin_paged_kv, pin_warp,
]
