"""Seeded random configurations of the whole step (and of the warped rule) against the oracle.

Each case draws a batch, a draft length, a hidden size, a vocabulary, a
temperature, a draft kind and a weight layout at random (from a fixed seed),
so that the dispatcher's choices meet in combinations the targeted tests do
not list:
* scoring kernels: panel shapes and the deep kernel, or the tiled kernel for
  row-major weights;
* statistics: fused or from the statistics kernel;
* rule paths: logits, probabilities or one-hot drafts, and the greedy rule.
The checks are those of the step tests: logits within the fp32 accumulation
bound, emitted tokens equal to the oracle's sequence by sequence, with the
same bands for decisions at their thresholds.
"""
import numpy as np
import pytest

import speculative_decoding_verification_09_amd as sd
import synth
from gpu_util import announce
from test_gpu_step import _draft_and_tokens, check_sequences, run_step

pytestmark = pytest.mark.gpu

KINDS = (sd.SPECDEC_DRAFT_LOGITS, sd.SPECDEC_DRAFT_PROBS, sd.SPECDEC_DRAFT_ONEHOT)


def _configs(n, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        g = int(rng.integers(0, 9))
        B = int(rng.integers(1, 49))
        if B * (g + 1) > 320:
            continue
        d = int(rng.choice([32, 64, 96, 128, 256, 384, 512]))
        V = int(np.exp(rng.uniform(np.log(2), np.log(6000))))
        T = float(rng.choice([0.0, 0.5, 0.8, 1.0, 1.7]))
        kind = int(rng.choice(KINDS))
        packed = bool(rng.random() < 0.75)
        out.append((len(out), B, g, d, V, T, kind, packed))
    return out


def _sweep_configs(n, seed=20261203):
    """Long vocabularies with at most 16 positions: the sweep kernel and its epilogues."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        g = int(rng.integers(0, 8))
        B = int(rng.integers(1, 5))
        if B * (g + 1) > 16:
            continue
        d = int(rng.choice([32, 64, 128, 256]))
        V = int(rng.integers(65536, 70001))
        T = float(rng.choice([0.0, 0.7, 1.0, 1.4]))
        kind = int(rng.choice(KINDS))
        out.append((100 + len(out), B, g, d, V, T, kind, True))
    return out


CONFIGS = _configs(48) + _sweep_configs(8)


@pytest.mark.parametrize("case,B,g,d,V,T,kind,packed", CONFIGS, ids=[f"fuzz{c[0]}" for c in CONFIGS])
def test_random_step(orc, case, B, g, d, V, T, kind, packed):
    seed = 4000 + case
    X = synth.normal_bf16((B * (g + 1), d), 1.0, seed, synth.STREAM_X)
    W = synth.normal_bf16((V, d), 2.0 / np.sqrt(d), seed, synth.STREAM_W)
    target32 = orc.linear(X, W).astype(np.float32).reshape(B, g + 1, V)
    greedy = T == 0.0
    if greedy:
        kind = sd.SPECDEC_DRAFT_LOGITS
        draft = None
        am = np.array([[orc.argmax(target32[b, i])[0] for i in range(g)] for b in range(B)], np.int32).reshape(B, g)
        rnd = synth.integers((B, g), 0, V, seed, synth.STREAM_REPLACE)
        tokens = np.where(synth.bernoulli((B, g), 0.3, seed, synth.STREAM_REPLACE + 1), rnd, am).astype(np.int32)
        u = None
    else:
        draft, tokens = _draft_and_tokens(orc, target32, g, 1.0, T, seed)
        if kind == sd.SPECDEC_DRAFT_PROBS:
            rows = [orc.softmax(draft[b, i], T)[0] for b in range(B) for i in range(g)]
            draft = np.ascontiguousarray(np.stack(rows).reshape(B, g, V) if rows else np.zeros((B, 0, V)), np.float32)
        elif kind == sd.SPECDEC_DRAFT_ONEHOT:
            draft = None
        u = synth.uniforms((B, g + 1, 2), seed, synth.STREAM_STEP_UNIFORMS)
    announce(f"step fuzz case {case}: B={B} gamma={g} d={d} V={V} T={T} kind={kind} packed={packed}")
    logits, tok, num = run_step(X, W, draft, tokens, u, T, B, g, V, packed=packed, kind=kind)
    check_sequences(orc, X, W, logits, tok, num, draft, tokens, u, T, g, V, list(range(B)), greedy=greedy, kind=kind)


def _warp_configs(n, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        B = int(rng.integers(1, 41))
        g = int(rng.integers(0, 8))
        V = int(np.exp(rng.uniform(np.log(8), np.log(40000))))
        k = int(rng.choice([0, 1, 5, 50, 300])) if rng.random() < 0.8 else int(rng.integers(1, V + 1))
        p = float(rng.choice([1.0, 0.95, 0.7, 0.3]))
        T = float(rng.choice([0.6, 1.0, 1.5]))
        kind = int(rng.choice(KINDS))
        ties = bool(rng.random() < 0.2)
        out.append((c, B, g, V, T, k, p, kind, ties))
    return out


WARP_CONFIGS = _warp_configs(24)


@pytest.mark.parametrize("case,B,g,V,T,k,p,kind,ties", WARP_CONFIGS, ids=[f"warp{c[0]}" for c in WARP_CONFIGS])
def test_random_warped_rule(orc, case, B, g, V, T, k, p, kind, ties):
    from test_gpu_warp import _check, _inputs
    from gpu_util import reject_warped
    seed = 8000 + case
    zt, draft, x, u = _inputs(orc, B, g, V, 2.0, T, k, p, kind, ties, seed)
    announce(f"warped fuzz case {case}: B={B} gamma={g} V={V} T={T} top_k={k} top_p={p} kind={kind} ties={ties}")
    tok, num, _ = reject_warped(zt, draft, x, u, T, k, p, kind=kind, probs=False)
    ora = orc.verify_warped(zt, draft, x, u, T, k, float(np.float32(p)), draft_kind=kind)
    _check(tok, num, ora, max_frac=0.1)

