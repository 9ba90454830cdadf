"""Seeded synthetic inputs for the verification step.

This module is the only code that both the oracle tests and the GPU path use.
It holds no arithmetic of the method itself: it draws random numbers (Philox
streams), rounds fp32 to bf16 bit patterns (round to nearest even) and
describes the workload shapes.  Composite inputs that need the method's
arithmetic -- drafted tokens sampled from q, draft logits built on top of
target logits -- are put together by the caller (the tests use the oracle for
that, the benchmark uses the library under test).

Random streams.  Every array comes from numpy's Philox bit generator keyed by
(seed, stream, chunk): the same seed always gives the same bytes, on any
machine and with any number of worker threads.  Normal values are standard
deviations times numpy's float32 standard normals.  Uniforms are
(x >> 40) * 2**-24 for a 64-bit Philox output x, so they lie in [0, 1) on the
2**-24 grid and are exact fp32 numbers.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Stream numbers inside one workload seed.
STREAM_X = 0
STREAM_W = 1
STREAM_DRAFT_NOISE = 2
STREAM_DRAFT_SAMPLE = 3
STREAM_STEP_UNIFORMS = 4
STREAM_REPLACE = 5
STREAM_TARGET = 6

_CHUNK = 1 << 22  # elements per Philox chunk for large arrays


def generator(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    key = np.array([(int(seed) << 20) ^ int(stream), int(chunk)], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def _fill_chunked(n: int, seed: int, stream: int, fill, dtype, workers: int | None = None) -> np.ndarray:
    out = np.empty(n, dtype=dtype)
    chunks = [(i, min(n, i + _CHUNK)) for i in range(0, n, _CHUNK)]

    def work(ci):
        lo, hi = chunks[ci]
        fill(generator(seed, stream, ci), out[lo:hi])

    if len(chunks) <= 1:
        for ci in range(len(chunks)):
            work(ci)
    else:
        workers = workers or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(work, range(len(chunks))))
    return out


def normal_f32(shape, std: float, seed: int, stream: int) -> np.ndarray:
    """fp32 values ~ N(0, std^2) (std is a standard deviation)."""
    n = int(np.prod(shape))

    def fill(g, dst):
        g.standard_normal(out=dst, dtype=np.float32)
        dst *= np.float32(std)

    return _fill_chunked(n, seed, stream, fill, np.float32).reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the 16-bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std: float, seed: int, stream: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, std^2) values, rounded to nearest even."""
    n = int(np.prod(shape))

    def fill(g, dst):
        tmp = g.standard_normal(size=dst.size, dtype=np.float32)
        tmp *= np.float32(std)
        dst[:] = bf16_bits(tmp)

    return _fill_chunked(n, seed, stream, fill, np.uint16).reshape(shape)


def uniforms(shape, seed: int, stream: int) -> np.ndarray:
    """fp32 uniforms in [0, 1) on the 2**-24 grid."""
    n = int(np.prod(shape))

    def fill(g, dst):
        raw = g.integers(0, 2**64 - 1, size=dst.size, dtype=np.uint64, endpoint=True)
        dst[:] = (raw >> np.uint64(40)).astype(np.float32) * np.float32(2.0**-24)

    return _fill_chunked(n, seed, stream, fill, np.float32).reshape(shape)


def integers(shape, low: int, high: int, seed: int, stream: int) -> np.ndarray:
    """int32 values uniform in [low, high)."""
    return generator(seed, stream).integers(low, high, size=shape, dtype=np.int64).astype(np.int32)


def bernoulli(shape, prob: float, seed: int, stream: int) -> np.ndarray:
    return uniforms(shape, seed, stream) < np.float32(prob)


def integer_bf16(shape, bound: int, seed: int, stream: int) -> np.ndarray:
    """bf16 bit patterns of integers uniform in [-bound, bound] (exact in bf16 for bound <= 256)."""
    vals = generator(seed, stream).integers(-bound, bound + 1, size=shape).astype(np.float32)
    return bf16_bits(vals)


# --------------------------------------------------------------------------
# Workload recipes.  Shapes and distributions follow the pages' examples: a
# Llama-3-sized vocabulary of 128,256 entries, 4-8 drafted tokens, hidden
# sizes 4096-8192.  "N(0, s)" means standard deviation s.

@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    gamma: int
    V: int
    d: int = 0                 # hidden size (0: reject/sample only)
    x_std: float = 1.0         # hidden states ~ N(0, x_std)
    w_std: float = 0.02        # LM-head weights ~ N(0, w_std)
    noise_std: float = 1.0     # draft logits = target logits + N(0, noise_std)
    temperature: float = 1.0   # 0 selects the greedy rule
    target_std: float = 0.0    # reject-only workloads: target logits ~ N(0, target_std)
    replace_prob: float = 0.0  # greedy workloads: share of drafts replaced by random ids
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.B * (self.gamma + 1)


WORKLOADS = {
    # One toy row pair replicated over 200k trials (reject/sample only).
    "toy_v32": Workload("toy_v32", seed=1000, B=200_000, gamma=4, V=32, target_std=2.0, noise_std=1.0,
                        temperature=1.0),
    # Llama-8B-shaped LM head, one sequence, 4 drafts.
    "lmhead_b1_g4": Workload("lmhead_b1_g4", seed=2000, B=1, gamma=4, V=128256, d=4096, x_std=1.0, w_std=0.02,
                             noise_std=1.0, temperature=1.0),
    # Larger head and batch, 7 drafts, high acceptance, T = 0.7.
    "lmhead_b8_g7": Workload("lmhead_b8_g7", seed=3000, B=8, gamma=7, V=128256, d=8192, x_std=1.0, w_std=0.015,
                             noise_std=0.5, temperature=0.7),
    # Large-batch greedy verify.
    "greedy_b64_g4": Workload("greedy_b64_g4", seed=5000, B=64, gamma=4, V=152064, d=5120, x_std=1.0, w_std=0.02,
                              temperature=0.0, replace_prob=0.3),
}

# Workloads of the extensions beyond the plain step, each timed on its own.
EXTENSIONS = {
    # Top-k / top-p warping of every target and draft row of the larger LM-head step.
    "warp": {"workload": "lmhead_b8_g7", "top_k": 50, "top_p": 0.95, "top_p_alone": 0.9},
    # The same step with one-hot drafts (greedy or prompt-lookup drafters): no draft array is read.
    "onehot": {"workload": "lmhead_b8_g7"},
    # Greedy verification of 8 binary trees of 16 nodes (parent of node i is (i - 1) // 2) on a Llama-8B head;
    # a node carries its parent row's argmax with probability `right`, else a random id.
    "tree": {"seed": 6000, "B": 8, "M": 16, "V": 128256, "d": 4096, "x_std": 1.0, "w_std": 0.02, "right": 0.7},
    # Paged KV cache around a verify step: 64 requests with 1000-token contexts, 8 KV heads of 128 (bf16), 16-token
    # blocks; each step appends gamma + 1 = 8 positions and rolls back to the emitted ones (uniform in 1 .. 8).
    "paged_kv": {"seed": 6100, "R": 64, "heads": 8, "head_dim": 128, "block_size": 16, "ctx": 1000, "gamma": 7},
}

# Decoder-layer projection stack in the verify pass: [N x d_in] . [d_in x d_out].
PROJECTION_SWEEP = {
    "seed": 4000,
    "shapes": [(8192, 28672), (28672, 8192)],
    "N": [1, 5, 8, 16, 32, 64, 128, 256, 512],
    "w_std": 0.02,
    "x_std": 1.0,
}


def lm_head_inputs(w: Workload):
    """X [N, d] and W [V, d] as bf16 bit patterns."""
    X = normal_bf16((w.N, w.d), w.x_std, w.seed, STREAM_X)
    W = normal_bf16((w.V, w.d), w.w_std, w.seed, STREAM_W)
    return X, W


def draft_noise(w: Workload) -> np.ndarray:
    return normal_f32((w.B, w.gamma, w.V), w.noise_std, w.seed, STREAM_DRAFT_NOISE)


def draft_sample_uniforms(w: Workload) -> np.ndarray:
    return uniforms((w.B, w.gamma), w.seed, STREAM_DRAFT_SAMPLE)


def step_uniforms(w: Workload) -> np.ndarray:
    """[B, gamma+1, 2]: slot 0 decides acceptance at a row, slot 1 drives the draw there."""
    return uniforms((w.B, w.gamma + 1, 2), w.seed, STREAM_STEP_UNIFORMS)
