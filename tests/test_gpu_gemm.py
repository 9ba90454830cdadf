"""Parity of the scoring GEMM (specdec_verify_logits) with the oracle's fp64 linear layer.

Tolerances come from the arithmetic: products of two bf16 values are exact in
fp32 and the kernel accumulates in fp32, so |y_gpu - y| <= g_d * sum_k |x_k w_k|
with g_d = d*u / (1 - d*u), u = 2**-24 (the standard bound for any order of
fp32 summation).  Integer-valued inputs whose partial sums stay below 2**24
are summed exactly in any order, so those results must be bit-identical.
The stated criterion for bf16 outputs (relative error 2e-2, with a floor of
1e-3 of the output RMS for entries near zero) is checked as well.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_09_amd as sd
import synth
from gpu_util import announce, dev_bf16, gemm, host, oracle_linear, weights

pytestmark = pytest.mark.gpu

U = 2.0**-24
# (N, d, V): every kernel shape of the dispatcher, k tails (d % chunk != 0),
# vocabulary tails (V % 128 != 0, V % 4 != 0), several token-column tiles.
SHAPES = [
    (1, 8, 1), (5, 64, 37), (16, 256, 128), (17, 264, 1000), (33, 512, 777), (64, 520, 1030),
    (100, 1024, 2053), (200, 320, 515), (320, 136, 300), (513, 96, 129), (1, 4104, 4099),
]
# Packed weights (d % 32 == 0).  Covers the sweep kernel (long vocabularies,
# N <= 16, X whole in LDS: up to 16 positions, vocabulary tails), every panel
# shape (4x1, 4x2, 4x4, 8x2, 8x4 token x vocabulary tiles per wave) and the
# deep kernel, with and without k-groups, k-step counts that leave waves idle
# or partly filled (d = 96, 5120), vocabulary tails.
PACKED_SHAPES = [
    (1, 64, 17), (5, 4096, 1000), (5, 8192, 515), (3, 5120, 513), (7, 96, 50), (16, 4096, 300),
    (16, 32, 16), (8, 28672, 40), (17, 256, 1000), (33, 512, 777), (64, 1024, 1030), (100, 512, 2053),
    (200, 320, 515), (513, 96, 129), (16, 256, 65541), (9, 4096, 65536), (12, 1024, 70001),
    (40, 1024, 66000), (8, 4128, 65536), (120, 256, 65541), (130, 128, 65536),
    # the deep kernel (N > 128, d % 128 == 0): several trips, k-groups, token passes, tails
    (96, 4096, 3000), (300, 1024, 4100), (65, 384, 1029), (512, 256, 2000), (129, 4096, 1000), (160, 8192, 700),
    # its 192-position passes (long vocabularies, fewer passes than 128): a ragged last pass and vocabulary tail
    (260, 128, 65541),
    # ... over several trips of its prefetch ring, one pass and two (the second ragged)
    (200, 1024, 65600), (330, 2048, 66000),
    # its 160-position passes: every tile full (one pass, two), and a ragged second pass
    (160, 1024, 65536), (320, 256, 65541), (300, 128, 65600),
]


def _bound(Xf, Wf, d):
    g = d * U / (1 - d * U)
    return g * (np.abs(Xf.astype(np.float64)) @ np.abs(Wf.astype(np.float64)).T)


@pytest.mark.parametrize("N,d,V", SHAPES)
def test_integer_inputs_bit_exact(orc, N, d, V):
    X = synth.integer_bf16((N, d), 8, 17, N)
    W = synth.integer_bf16((V, d), 8, 18, V)
    announce(f"gemm integer N={N} d={d} V={V}")
    Y = host(gemm(X, W))
    ref = orc.linear(X, W)
    assert np.array_equal(Y.astype(np.float64), ref), np.abs(Y - ref).max()


@pytest.mark.parametrize("N,d,V", SHAPES)
def test_normal_inputs_within_fp32_bound(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 27, N)
    W = synth.normal_bf16((V, d), 0.02, 28, V)
    announce(f"gemm normal N={N} d={d} V={V}")
    Y = host(gemm(X, W)).astype(np.float64)
    ref = orc.linear(X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    err = np.abs(Y - ref)
    assert np.all(err <= bound + 1e-30), float((err - bound).max())
    rms = float(np.sqrt(np.mean(ref**2)))
    assert np.all(err <= 2e-2 * np.maximum(np.abs(ref), 1e-3 * rms))


@pytest.mark.parametrize("N,d,V", [(5, 64, 37), (64, 520, 1030), (320, 136, 300), (513, 96, 129)])
def test_bf16_output(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 37, N)
    W = synth.normal_bf16((V, d), 0.02, 38, V)
    announce(f"gemm bf16-out N={N} d={d} V={V}")
    Y = gemm(X, W, out_bf16=True)
    Yf = host(Y.float()).astype(np.float64)
    ref = orc.linear(X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    # one rounding to bf16 (8 significant bits, nearest even) on top of the fp32 result
    assert np.all(np.abs(Yf - ref) <= 2.0**-8 * (np.abs(ref) + bound) + bound + 1e-30)
    rms = float(np.sqrt(np.mean(ref**2)))
    assert np.all(np.abs(Yf - ref) <= 2e-2 * np.maximum(np.abs(ref), 1e-3 * rms))


@pytest.mark.parametrize("N,d,V", PACKED_SHAPES)
def test_packed_integer_bit_exact(orc, N, d, V):
    X = synth.integer_bf16((N, d), 8, 71, N)
    W = synth.integer_bf16((V, d), 8, 72, V)
    announce(f"gemm packed integer N={N} d={d} V={V}")
    Y = host(gemm(X, W, packed=True))
    assert np.array_equal(Y.astype(np.float64), oracle_linear(orc, X, W))


@pytest.mark.parametrize("N,d,V", PACKED_SHAPES)
def test_packed_normal_within_fp32_bound(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 81, N)
    W = synth.normal_bf16((V, d), 0.02, 82, V)
    announce(f"gemm packed normal N={N} d={d} V={V}")
    Y = host(gemm(X, W, packed=True)).astype(np.float64)
    ref = oracle_linear(orc, X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    assert np.all(np.abs(Y - ref) <= bound + 1e-30)


@pytest.mark.parametrize("N,d,V", [(5, 4096, 1000), (64, 1024, 1030)])
def test_packed_bf16_output(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 91, N)
    W = synth.normal_bf16((V, d), 0.02, 92, V)
    announce(f"gemm packed bf16-out N={N} d={d} V={V}")
    Yf = host(gemm(X, W, out_bf16=True, packed=True).float()).astype(np.float64)
    ref = orc.linear(X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    assert np.all(np.abs(Yf - ref) <= 2.0**-8 * (np.abs(ref) + bound) + bound + 1e-30)


# Packed shapes whose k range is split into groups (fp32 partials in the
# workspace, added in group order): short vocabularies whose blocks would
# leave CUs idle, at every token count; vocabulary and k tails.
SPLIT_SHAPES = [
    (40, 2048, 300), (8, 9984, 100), (8, 9984, 5000), (17, 4096, 300), (100, 1024, 64), (3, 16384, 40),
    (5, 28672, 77), (64, 8192, 1030), (130, 2048, 500),
]


def _gemm_ws(X_bits, W_bits, out_bf16=False):
    """Packed GEMM with an explicit workspace poisoned with NaN bytes (every partial must be overwritten)."""
    X = dev_bf16(X_bits)
    W = weights(W_bits, True)
    N, V, d = X.shape[0], W_bits.shape[0], X_bits.shape[1]
    need = sd.logits_workspace_bytes(N, d, V, sd.SPECDEC_WEIGHTS_PACKED)
    assert need > 0, "shape does not split k"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    Y = torch.full((N, V), float("nan"), device="cuda", dtype=torch.bfloat16 if out_bf16 else torch.float32)
    sd.specdec_verify_logits(X, W, Y, sd.SPECDEC_OUT_BF16 if out_bf16 else sd.SPECDEC_OUT_F32, workspace=ws)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("N,d,V", SPLIT_SHAPES)
def test_split_k_integer_bit_exact(orc, N, d, V):
    X = synth.integer_bf16((N, d), 8, 61, N)
    W = synth.integer_bf16((V, d), 8, 62, V)
    announce(f"gemm split-k integer N={N} d={d} V={V}")
    Y = host(_gemm_ws(X, W))
    assert np.array_equal(Y.astype(np.float64), orc.linear(X, W))


@pytest.mark.parametrize("N,d,V", SPLIT_SHAPES)
def test_split_k_normal_within_fp32_bound(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 63, N)
    W = synth.normal_bf16((V, d), 0.02, 64, V)
    announce(f"gemm split-k normal N={N} d={d} V={V}")
    Y = host(_gemm_ws(X, W)).astype(np.float64)
    ref = orc.linear(X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    assert np.all(np.abs(Y - ref) <= bound + 1e-30)
    rms = float(np.sqrt(np.mean(ref**2)))
    assert np.all(np.abs(Y - ref) <= 2e-2 * np.maximum(np.abs(ref), 1e-3 * rms))


@pytest.mark.parametrize("N,d,V", [(64, 8192, 1030), (5, 28672, 77), (130, 2048, 500)])
def test_split_k_workspace_reused(orc, N, d, V):
    """Back-to-back launches on one workspace (zeroed first, then holding the previous launch's partials): each
    result is exact, and rounded sums come out in the same bits every time (partials added in group order)."""
    W_bits = synth.integer_bf16((V, d), 8, 67, V)
    W = weights(W_bits, True)
    need = sd.logits_workspace_bytes(N, d, V, sd.SPECDEC_WEIGHTS_PACKED)
    ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")
    announce(f"gemm split-k reused workspace N={N} d={d} V={V}")
    outs = []
    for i, seed in enumerate((68, 69, 68)):
        X_bits = synth.integer_bf16((N, d), 8, seed, N)
        Y = torch.full((N, V), float("nan"), device="cuda")
        sd.specdec_verify_logits(dev_bf16(X_bits), W, Y, sd.SPECDEC_OUT_F32, workspace=ws)
        torch.cuda.synchronize()
        outs.append(host(Y))
        assert np.array_equal(outs[-1].astype(np.float64), orc.linear(X_bits, W_bits)), i
    # normal inputs (rounded sums): the same bits from two launches
    X = dev_bf16(synth.normal_bf16((N, d), 1.0, 70, N))
    Wn = weights(synth.normal_bf16((V, d), 0.02, 71, V), True)
    Ys = []
    for _ in range(2):
        Y = torch.empty((N, V), device="cuda")
        sd.specdec_verify_logits(X, Wn, Y, sd.SPECDEC_OUT_F32, workspace=ws)
        torch.cuda.synchronize()
        Ys.append(host(Y))
    assert np.array_equal(Ys[0].view(np.uint32), Ys[1].view(np.uint32))


@pytest.mark.parametrize("N,d,V", [(8, 9984, 5000), (40, 2048, 300)])
def test_split_k_bf16_output(orc, N, d, V):
    X = synth.normal_bf16((N, d), 1.0, 65, N)
    W = synth.normal_bf16((V, d), 0.02, 66, V)
    announce(f"gemm split-k bf16-out N={N} d={d} V={V}")
    Yf = host(_gemm_ws(X, W, out_bf16=True).float()).astype(np.float64)
    ref = orc.linear(X, W)
    bound = _bound(synth.bf16_to_f32(X), synth.bf16_to_f32(W), d)
    assert np.all(np.abs(Yf - ref) <= 2.0**-8 * (np.abs(ref) + bound) + bound + 1e-30)


@pytest.mark.parametrize("V,d", [(16, 32), (37, 64), (1000, 96)])
def test_pack_layout(V, d):
    """The packed buffer holds W[16t + m][32s + 8g + e] at ((t*nsteps + s)*64 + 16g + m)*8 + e; padded rows are 0."""
    W = synth.integer_bf16((V, d), 100, 5, V)
    announce(f"pack layout V={V} d={d}")
    Wp = weights(W, packed=True)
    got = host(Wp.data).view(np.uint16)
    tiles, nsteps = (V + 15) // 16, d // 32
    Wpad = np.zeros((tiles * 16, d), np.uint16)
    Wpad[:V] = W
    expect = Wpad.reshape(tiles, 16, nsteps, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("N,d,V", [(5, 4096, 65541), (16, 256, 70001)])
def test_sweep_tile_queue_workspace(orc, N, d, V):
    """The sweep kernel takes its last tiles from a queue whose counter sits in the workspace and is reset by
    the call itself: a workspace full of 0xFF bytes, then the same workspace again (left at the previous call's
    final count), then again with other inputs, all give the exact result (integer inputs)."""
    need = sd.logits_workspace_bytes(N, d, V, sd.SPECDEC_WEIGHTS_PACKED)
    assert need == 256
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for call, seed in enumerate((61, 61, 62)):
        X_bits = synth.integer_bf16((N, d), 8, seed, N)
        W_bits = synth.integer_bf16((V, d), 8, seed + 100, V)
        X = dev_bf16(X_bits)
        W = weights(W_bits, True)
        Y = torch.full((N, V), float("nan"), device="cuda", dtype=torch.float32)
        announce(f"sweep queue call {call} N={N} d={d} V={V}")
        sd.specdec_verify_logits(X, W, Y, sd.SPECDEC_OUT_F32, workspace=ws)
        torch.cuda.synchronize()
        ref = orc.linear(X_bits, W_bits)
        assert np.array_equal(host(Y).astype(np.float64), ref), (call, np.nanmax(np.abs(host(Y) - ref)))


def test_nan_poisoned_output_fully_written(orc):
    """Every output entry is written (the buffer starts as NaN)."""
    X = synth.normal_bf16((37, 72), 1.0, 47, 0)
    W = synth.normal_bf16((997, 72), 0.02, 48, 0)
    announce("gemm coverage N=37 d=72 V=997")
    Y = host(gemm(X, W))
    assert np.all(np.isfinite(Y))


def test_deterministic():
    X = synth.normal_bf16((64, 1024), 1.0, 57, 0)
    W = synth.normal_bf16((5000, 1024), 0.02, 58, 0)
    announce("gemm determinism N=64 d=1024 V=5000")
    a = host(gemm(X, W))
    b = host(gemm(X, W))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------------------
# Full configuration sizes, in the launch configuration the benchmark times,
# checked on sampled entries that the oracle computes one by one.

FULL = [
    ("lmhead_b1_g4", 5, 4096, 128256, 0.02, False),
    ("lmhead_b8_g7", 64, 8192, 128256, 0.015, False),
    ("greedy_b64_g4", 320, 5120, 152064, 0.02, False),
    ("proj_up_n1", 1, 8192, 28672, 0.02, True),
    ("proj_up_n64", 64, 8192, 28672, 0.02, True),
    ("proj_up_n512", 512, 8192, 28672, 0.02, True),
    ("proj_down_n5", 5, 28672, 8192, 0.02, True),
    ("proj_down_n256", 256, 28672, 8192, 0.02, True),
]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("name,N,d,V,wstd,bf16", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(orc, name, N, d, V, wstd, bf16, packed):
    seed = 9000 + N
    X = synth.normal_bf16((N, d), 1.0, seed, synth.STREAM_X)
    W = synth.normal_bf16((V, d), wstd, seed, synth.STREAM_W)
    announce(f"gemm full-size {name} N={N} d={d} V={V} bf16_out={bf16} packed={packed}")
    Y = gemm(X, W, out_bf16=bf16, packed=packed)
    rng = np.random.default_rng(seed)
    n_idx = np.concatenate([rng.integers(0, N, 3000), np.full(64, N - 1)])
    v_idx = np.concatenate([rng.integers(0, V, 3000), np.arange(V - 64, V)])
    got = Y[torch.from_numpy(n_idx).cuda(), torch.from_numpy(v_idx).cuda()].float().cpu().numpy().astype(np.float64)
    ref = orc.linear_entries(X, W, n_idx, v_idx)
    Xs = np.abs(synth.bf16_to_f32(X[n_idx]))
    Ws = np.abs(synth.bf16_to_f32(W[v_idx]))
    absdot = np.einsum("ij,ij->i", Xs, Ws, dtype=np.float64)
    g = d * U / (1 - d * U)
    bound = g * absdot
    if bf16:
        bound = bound + 2.0**-8 * (np.abs(ref) + bound)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    rms = float(np.sqrt(np.mean(ref**2)))
    assert np.all(np.abs(got - ref) <= 2e-2 * np.maximum(np.abs(ref), 1e-3 * rms))
    assert bool(torch.isfinite(Y).all())
