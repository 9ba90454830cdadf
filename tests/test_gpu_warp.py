"""Parity of top-k / top-p warping before the rule (specdec_reject_sample_warped,
specdec_verify_step_warped) with the oracle's verify_warped.

Top-k cuts are taken on the same fp32 logits with the same ranking (logit, then
lower index), so the kept sets agree exactly.  The top-p cut compares exact
fixed-point sums of fp32 masses exp((z - max z) * fl32(1/T)) with top_p, where
the oracle adds fp64 masses rounded to fp32 probabilities.  Each device mass is
within (1 + D) * 3 * 2^-24 + 2 ulp relative of the exact one, D = (max z - z)/T,
so the cumulative fraction is within twice that (mass-weighted D <= 10 here):
WARP_BAND = 4e-6.  A sequence may differ only where the oracle's cumulative
mass at its cut is within WARP_BAND of top_p (counted, and rare).  Accept tests and draws have the near-tie bands of the unwarped
tests.  Two settings reduce the rule to the greedy one exactly (top_k = 1, and
a top_p below every row's largest probability) and are compared bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import speculative_decoding_verification_09_amd as sd
import synth
import parity_tally
from oracle.parity import compare_steps
from gpu_util import (abs_dot_bound, announce, dev, dev_bf16, first_token_tv, host, oracle_linear, reject,
                      reject_warped, weights)

pytestmark = pytest.mark.gpu

ACC_BAND = 1e-5
DRAW_BAND = 1e-6
WARP_BAND = 4e-6


def _sample_warped(orc, z, us, T, top_k, top_p):
    """Inverse-CDF draws from the oracle's warped distribution of each row of z (one uniform per row)."""
    out = np.empty(z.shape[0], np.int32)
    for r in range(z.shape[0]):
        p, _, _ = orc.warp(z[r], T, top_k, top_p)
        C = np.cumsum(p.astype(np.float64))
        out[r] = min(int(np.searchsorted(C, float(us[r]) * C[-1], side="right")), z.shape[1] - 1)
    return out


def _inputs(orc, B, g, V, std, T, top_k, top_p, kind, ties, seed):
    """Target logits ~ N(0, std), or integers in [0, 4) (ties="ties": long runs of equal logits), or uniform in
    [1, 1.125) (ties="narrow": one octave-eighth, so distinct values crowd one 12-bit key bucket), or N(0, std)
    with 16 entries per row near 60 (ties="spikes": the two octaves below the largest value hold too few of the
    row's sampled entries for the top-k threshold, so the full sample histograms run); draft = target
    + N(0, 1), or a fresh row of the same kind; drafted tokens drawn from the draft's warped distribution (logits),
    its unwarped one (probabilities) or uniformly over the vocabulary (one-hot)."""
    if ties in (True, "ties"):
        zt = synth.integers((B, g + 1, V), 0, 4, seed, synth.STREAM_TARGET).astype(np.float32)
        zd = synth.integers((B, g, V), 0, 4, seed, synth.STREAM_DRAFT_NOISE).astype(np.float32)
    elif ties == "spikes":
        zt = synth.normal_f32((B, g + 1, V), std, seed, synth.STREAM_TARGET)
        pos = synth.integers((B, g + 1, 16), 0, V, seed + 1, synth.STREAM_REPLACE)
        amp = np.float32(60.0) + synth.normal_f32((B, g + 1, 16), 1.0, seed + 1, synth.STREAM_TARGET)
        np.put_along_axis(zt, pos, amp, axis=2)
        zd = zt[:, :g] + synth.normal_f32((B, g, V), 1.0, seed, synth.STREAM_DRAFT_NOISE)
    elif ties == "narrow":
        zt = 1.0 + np.float32(0.125) * synth.uniforms((B, g + 1, V), seed, synth.STREAM_TARGET)
        zd = 1.0 + np.float32(0.125) * synth.uniforms((B, g, V), seed, synth.STREAM_DRAFT_NOISE)
        zt, zd = zt.astype(np.float32), zd.astype(np.float32)
    else:
        zt = synth.normal_f32((B, g + 1, V), std, seed, synth.STREAM_TARGET)
        zd = zt[:, :g] + synth.normal_f32((B, g, V), 1.0, seed, synth.STREAM_DRAFT_NOISE)
    du = synth.uniforms((B * g,), seed, synth.STREAM_DRAFT_SAMPLE)
    zd2 = np.ascontiguousarray(zd.reshape(B * g, V))
    if kind == sd.SPECDEC_DRAFT_LOGITS:
        x = _sample_warped(orc, zd2, du, T, top_k, top_p) if g else np.zeros(0, np.int32)
        draft = np.ascontiguousarray(zd)
    elif kind == sd.SPECDEC_DRAFT_PROBS:
        q = np.stack([orc.softmax(r, T)[0] for r in zd2]) if g else np.zeros((0, V), np.float32)
        x = orc.sample_rows(zd2, du, T) if g else np.zeros(0, np.int32)
        draft = np.ascontiguousarray(q.reshape(B, g, V))
    else:
        x = synth.integers((B * g,), 0, V, seed, synth.STREAM_REPLACE)
        draft = None
    u = synth.uniforms((B, g + 1, 2), seed, synth.STREAM_STEP_UNIFORMS)
    return np.ascontiguousarray(zt), draft, x.reshape(B, g).astype(np.int32), u


def _check(tok, num, ora, acc_band=ACC_BAND, draw_band=DRAW_BAND, warp_band=WARP_BAND, max_frac=0.02):
    res = compare_steps(tok, num, ora, acc_band, draw_band)
    fails = [b for b in res["failures"] if not ora["warp_margin"][b] < warp_band]
    excused = res["excused"] + len(res["failures"]) - len(fails)
    parity_tally.record("sampled", res["exact"], res["excused_accept"], res["excused_draw"],
                        len(res["failures"]) - len(fails), len(fails))
    print(f"  exact={res['exact']} excused={excused} failures={fails[:10]}", flush=True)
    assert not fails, f"sequences differ without a near tie: {fails[:10]}"
    assert excused <= max(1, max_frac * len(num))
    assert np.all((num >= 1) & (num <= tok.shape[1]))


# (B, gamma, V, logit std, T, top_k, top_p, draft kind, integer logits with ties, largest excused fraction)
# The broad top-p cases put entries of about 1e-6 probability at the cut, so a
# quarter of their sequences have an oracle margin under 1e-6: a few may differ.
CASES = [
    (64, 4, 32000, 2.0, 0.8, 50, 1.0, 0, False, 0.02),     # top-k only
    (64, 4, 32000, 3.0, 1.0, 0, 0.9, 0, False, 0.1),       # top-p only, broad
    (64, 4, 32000, 3.0, 0.7, 200, 0.8, 0, False, 0.02),    # both
    (40, 7, 4099, 2.0, 1.0, 1000, 0.95, 0, False, 0.1),    # V % 4 != 0, broad
    (200, 3, 37, 1.0, 1.0, 5, 0.7, 0, False, 0.02),        # a vocabulary under one chunk
    (64, 4, 32000, 2.0, 1.0, 20, 0.9, 1, False, 0.02),     # draft probabilities (used as given)
    (64, 4, 32000, 2.0, 1.0, 20, 0.9, 2, False, 0.02),     # one-hot drafts
    (100, 4, 3000, 0.0, 1.0, 7, 1.0, 0, True, 0.02),       # the top-k cut inside a run of equal logits
    (100, 4, 3000, 0.0, 1.0, 0, 0.5, 0, True, 0.05),       # the top-p cut inside a run of equal logits
    (100, 4, 3000, 0.0, 1.0, 900, 0.3, 2, True, 0.02),     # both, ties, one-hot
    (16, 0, 5000, 2.0, 1.0, 10, 0.9, 0, False, 0.02),      # gamma = 0: the bonus row alone
    (8, 7, 128256, 2.5, 0.8, 50, 0.95, 0, False, 0.02),    # a 128K vocabulary
    (8, 7, 128256, 2.5, 0.8, 0, 0.9, 0, False, 0.05),      # top-p alone over a 128K vocabulary (a window of keys)
    (6, 3, 40003, 2.0, 1.0, 40, 0.9, 0, False, 0.02),      # V % 4 != 0 with a long row
    (6, 3, 40003, 2.0, 1.0, 0, 0.9, 0, False, 0.05),       # top-p alone, V % 4 != 0: the window with element loads
    (24, 3, 32000, 2.0, 1.0, 5000, 1.0, 0, False, 0.02),   # top-k survivors beyond what LDS holds
    (24, 3, 32000, 0.0, 1.0, 100, 1.0, 0, "narrow", 0.02),  # the cut's bucket over capacity: a second level
    (24, 3, 32000, 0.0, 0.05, 0, 0.5, 0, "narrow", 0.1),   # the same for the top-p cut (broad: T over the range)
    (24, 3, 32000, 0.0, 1.0, 100, 1.0, 2, "ties", 0.02),   # runs of equal keys past capacity: index-order scan
    (24, 3, 32000, 0.0, 1.0, 0, 0.5, 2, "ties", 0.05),     # the same for top-p
    (24, 3, 32000, 0.0, 1.0, 3000, 0.9, 0, "ties", 0.05),  # both, over capacity
    (24, 3, 32000, 2.0, 1.0, 50, 0.9, 0, "spikes", 0.02),  # a few far larger logits: the sample's full histograms
    (24, 3, 32000, 2.0, 1.0, 0, 0.9, 0, "spikes", 0.05),   # top-p alone with the mass held by a few spikes
]


@pytest.mark.parametrize("B,g,V,std,T,k,p,kind,ties,frac", CASES)
def test_warped_parity(orc, B, g, V, std, T, k, p, kind, ties, frac):
    seed = 7000 + V + 13 * k
    zt, draft, x, u = _inputs(orc, B, g, V, std, T, k, p, kind, ties, seed)
    announce(f"warped B={B} gamma={g} V={V} T={T} top_k={k} top_p={p} kind={kind} ties={ties}")
    tok, num, probs = reject_warped(zt, draft, x, u, T, k, p, kind=kind)
    ora = orc.verify_warped(zt, draft, x, u, T, k, float(np.float32(p)), draft_kind=kind)
    _check(tok, num, ora, max_frac=frac)
    if g:  # reported p(x) of the warped target rows, where no near tie moved the cut
        for b in range(min(B, 8)):
            if ora["warp_margin"][b] < WARP_BAND:
                continue
            for i in range(g):
                pw, _, _ = orc.warp(zt[b, i], T, k, float(np.float32(p)))
                assert abs(float(probs[b, i, 0]) - float(pw[x[b, i]])) <= 1e-5


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("k,p", [(1, 1.0), (0, 1e-7), (1, 0.5)], ids=["top1", "tiny_top_p", "top1_and_p"])
def test_single_survivor_is_the_greedy_rule(orc, kind, k, p):
    """With one survivor per row the warped rule must emit exactly what the greedy rule does (any T > 0)."""
    B, g, V = 300, 5, 2053
    for ties in (False, True):
        zt, draft, x, u = _inputs(orc, B, g, V, 2.0, 1.0, 0, 1.0, kind, ties, 7100 + kind)
        # half the drafted tokens are the target argmax, so acceptance runs are long
        am = np.array([[orc.argmax(zt[b, i])[0] for i in range(g)] for b in range(B)], np.int32)
        x = np.where(synth.bernoulli((B, g), 0.5, 7101, 0), am, x).astype(np.int32)
        announce(f"single survivor kind={kind} top_k={k} top_p={p} ties={ties}")
        tok, num, _ = reject_warped(zt, draft, x, u, 1.3, k, p, kind=kind, probs=False)
        gtok, gnum, _ = reject(zt, None, x, None, 0.0, probs=False)
        assert np.array_equal(num, gnum) and np.array_equal(tok, gtok)
        ora = orc.verify(zt, None, x, None, 0.0)
        assert np.array_equal(num, ora["num_emitted"]) and np.array_equal(tok, ora["tokens"])


def test_output_follows_the_warped_target(orc):
    """The rule reproduces the warped p: over 200k trials of one row pair the first emitted token follows
    warp(p), and the mean number emitted follows the closed form with alpha = sum min(p_w, q_w)."""
    B, g, V, T, k, p = 200_000, 4, 32, 1.0, 10, 0.8
    z = synth.normal_f32((1, V), 2.0, 7200, synth.STREAM_TARGET)[0]
    zq = z + synth.normal_f32((1, V), 1.0, 7200, synth.STREAM_DRAFT_NOISE)[0]
    zt = np.ascontiguousarray(np.broadcast_to(z, (B, g + 1, V)))
    zd = np.ascontiguousarray(np.broadcast_to(zq, (B, g, V)))
    pw, _, _ = orc.warp(z, T, k, float(np.float32(p)))
    qw, _, _ = orc.warp(zq, T, k, float(np.float32(p)))
    du = synth.uniforms((B, g), 7200, synth.STREAM_DRAFT_SAMPLE)
    C = np.cumsum(qw.astype(np.float64))
    x = np.minimum(np.searchsorted(C, du.astype(np.float64) * C[-1], side="right"), V - 1).astype(np.int32)
    u = synth.uniforms((B, g + 1, 2), 7200, synth.STREAM_STEP_UNIFORMS)
    announce(f"warped toy B={B} V={V} top_k={k} top_p={p}")
    tok, num, _ = reject_warped(zt, zd, x, u, T, k, p, probs=False)
    tv = first_token_tv(tok[:, 0], pw)
    pf = pw.astype(np.float64)
    tv_noise = 0.5 * float(np.sum(np.sqrt(2 * pf * (1 - pf) / (math.pi * B))))
    print(f"  TV(first token, warped p) = {tv:.5f} (sampling noise ~{tv_noise:.5f})", flush=True)
    assert tv < 3 * tv_noise
    assert np.all(pw[tok[:, 0]] > 0)  # never a token the warping drops
    alpha = orc.acceptance_rate(pw, qw)
    e = orc.expected_tokens(alpha, g)
    n = num.astype(np.float64)
    print(f"  E[N] gpu {n.mean():.4f} closed form {e:.4f} (alpha {alpha:.4f})", flush=True)
    assert abs(n.mean() - e) < 4 * n.std() / math.sqrt(B)
    ora = orc.verify_warped(zt[:2000], zd[:2000], x[:2000], u[:2000], T, k, float(np.float32(p)))
    _check(tok[:2000], num[:2000], ora)


def _topk_gap(z, k):
    """Gap between the k-th and (k+1)-th largest logits of a row (inf when top-k is off)."""
    if k <= 0 or k >= z.size:
        return np.inf
    s = np.sort(z.astype(np.float64))[::-1]
    return float(s[k - 1] - s[k])


@pytest.mark.parametrize("k,p", [(50, 0.95), (0, 0.9)], ids=["topk50_topp0.95", "topp0.9"])
def test_warped_step_lmhead_b8_g7_full_size(orc, k, p):
    """The warped step at the larger LM-head workload (B=8, gamma=7, d=8192, V=128256, T=0.7), every sequence
    against the oracle on its fp64 scores: top-k with top-p (the candidate path), and top-p alone (the window
    of keys).  Drafted tokens are drawn from the draft's warped distribution."""
    w = synth.WORKLOADS["lmhead_b8_g7"]
    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    X, W = synth.lm_head_inputs(w)
    Y64 = oracle_linear(orc, X, W)
    zt = Y64.astype(np.float32).reshape(B, g + 1, V)
    zd = np.ascontiguousarray(zt[:, :g] + synth.normal_f32((B, g, V), w.noise_std, w.seed, synth.STREAM_DRAFT_NOISE))
    du = synth.uniforms((B * g,), w.seed, synth.STREAM_DRAFT_SAMPLE)
    x = _sample_warped(orc, zd.reshape(B * g, V), du, T, k, p).reshape(B, g)
    u = synth.step_uniforms(w)
    logits = torch.full((B * (g + 1), V), float("nan"), device="cuda")
    ot = torch.full((B, g + 1), -7, dtype=torch.int32, device="cuda")
    on = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((sd.step_workspace_bytes(B, g, d, V, sd.SPECDEC_WEIGHTS_PACKED),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    announce(f"warped step {w.name} full size top_k={k} top_p={p}")
    sd.specdec_verify_step_warped(dev_bf16(X), weights(W, True), dev(zd), dev(x), T, k, p, dev(u), logits, ot, on, ws)
    torch.cuda.synchronize()
    dz = np.abs(host(logits).astype(np.float64) - Y64)
    assert np.all(dz <= abs_dot_bound(X, W) + 1e-30)
    max_dz = float(dz.max())
    tok, num = host(ot), host(on)
    ora = orc.verify_warped(zt, zd, x, u, T, k, float(np.float32(p)))
    res = compare_steps(tok, num, ora, max(ACC_BAND, 4 * max_dz / T),
                        4 * max_dz / (T * np.maximum(ora["draw_mass"], 1e-12)))
    fails = []
    for b in res["failures"]:
        gap = min(_topk_gap(zt[b, i], k) for i in range(g + 1))
        if not (ora["warp_margin"][b] < max(WARP_BAND, 4 * max_dz / T) or gap < 4 * max_dz):
            fails.append(b)
    parity_tally.record("sampled", res["exact"], res["excused_accept"], res["excused_draw"],
                        len(res["failures"]) - len(fails), len(fails), max_dz=max_dz)
    print(f"  max|dz|={max_dz:.3e} exact={res['exact']} failures={fails}", flush=True)
    assert not fails
    assert res["exact"] >= B - 2


@pytest.mark.parametrize("packed", [True, False], ids=["packed", "rowmajor"])
def test_warped_step(orc, packed):
    """The whole step with warping on a GEMM; the oracle scores in fp64 (rounded to fp32).  Bands widen with the
    measured logit error: accept and draw as in the unwarped step test, top-k gap < 4 max|dz|, top-p margin
    < 4 max|dz| / T."""
    B, g, d, V, T, k, p = 6, 4, 512, 20000, 0.9, 40, 0.9
    X = synth.normal_bf16((B * (g + 1), d), 1.0, 7300, synth.STREAM_X)
    W = synth.normal_bf16((V, d), 0.1, 7300, synth.STREAM_W)
    Y64 = orc.linear(X, W)
    zt = Y64.astype(np.float32).reshape(B, g + 1, V)
    zd = np.ascontiguousarray(zt[:, :g] + synth.normal_f32((B, g, V), 1.0, 7300, synth.STREAM_DRAFT_NOISE))
    du = synth.uniforms((B * g,), 7300, synth.STREAM_DRAFT_SAMPLE)
    x = _sample_warped(orc, zd.reshape(B * g, V), du, T, k, p).reshape(B, g)
    u = synth.uniforms((B, g + 1, 2), 7300, synth.STREAM_STEP_UNIFORMS)
    layout = sd.SPECDEC_WEIGHTS_PACKED if packed else sd.SPECDEC_WEIGHTS_ROW_MAJOR
    logits = torch.full((B * (g + 1), V), float("nan"), device="cuda")
    ot = torch.full((B, g + 1), -7, dtype=torch.int32, device="cuda")
    on = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = torch.full((sd.step_workspace_bytes(B, g, d, V, layout),), 0xFF, dtype=torch.uint8, device="cuda")
    announce(f"warped step B={B} gamma={g} d={d} V={V} packed={packed}")
    sd.specdec_verify_step_warped(dev_bf16(X), weights(W, packed), dev(zd), dev(x), T, k, p, dev(u), logits, ot, on,
                                  ws)
    torch.cuda.synchronize()
    got = host(logits).astype(np.float64)
    dz = np.abs(got - Y64)
    assert np.all(dz <= abs_dot_bound(X, W) + 1e-30)
    max_dz = float(dz.max())
    tok, num = host(ot), host(on)
    ora = orc.verify_warped(zt, zd, x, u, T, k, float(np.float32(p)))
    res = compare_steps(tok, num, ora, max(ACC_BAND, 4 * max_dz / T),
                        4 * max_dz / (T * np.maximum(ora["draw_mass"], 1e-12)))
    fails = []
    for b in res["failures"]:
        gap = min(_topk_gap(zt[b, i], k) for i in range(g + 1))
        if not (ora["warp_margin"][b] < max(WARP_BAND, 4 * max_dz / T) or gap < 4 * max_dz):
            fails.append(b)
    parity_tally.record("sampled", res["exact"], res["excused_accept"], res["excused_draw"],
                        len(res["failures"]) - len(fails), len(fails), max_dz=max_dz)
    print(f"  max|dz|={max_dz:.3e} exact={res['exact']} failures={fails}", flush=True)
    assert not fails
    assert res["exact"] >= B - max(1, B // 3)
