"""CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It wraps the plain C
reference in ``specdec_oracle.c`` (single-threaded, fp64 except where the pages
fix fp32) and shares nothing with the GPU library.

Every function here is argument marshalling: the arithmetic lives in the C file,
which cites the passage of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "specdec_oracle.c")
LIBRARY = os.path.join(_HERE, "libspecdec_oracle.so")

Q_LOGITS = 0
Q_PROBS = 1
Q_ONEHOT = 2

# Planted mistakes compiled in with -DORACLE_PLANT=<n>; see specdec_oracle.c.
PLANTS = {
    "resample_from_p": 1,
    "residual_sign": 2,
    "no_bonus": 3,
    "temp_multiply": 4,
    "linear_transpose": 5,
    "uniform_slots": 6,
    "draw_le": 7,
    "argmax_last_tie": 8,
    "greedy_keep_draft": 9,
    "ratio_inverted": 10,
    "no_max_shift": 11,
    "row_offset": 12,
    "drop_last_term": 13,
    "accept_le": 14,
    "tree_depth": 15,
    "tree_self_argmax": 16,
    "kv_free_order": 17,
    "kv_offset": 18,
    "topk_tie_high": 19,
    "topp_strict": 20,
}


def build_library(out_path: str = LIBRARY, plant: int = 0, extra_flags=()) -> str:
    """Compile the oracle with gcc -O2 (no OpenMP, no SIMD intrinsics); extra_flags are appended (a sanitizer
    build, for instance)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           f"-DORACLE_PLANT={int(plant)}", *extra_flags, SOURCE, "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


_i64 = ctypes.c_int64
_f64 = ctypes.c_double


class Oracle:
    """Handle on one build of the oracle library (the real one by default)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built (run oracle.build_library())")
        self.path = path
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_linear.argtypes = [P, P, _i64, _i64, _i64, P]
        lib.oracle_linear_entries.argtypes = [P, P, _i64, _i64, P, P, _i64, P]
        lib.oracle_softmax.argtypes = [P, _i64, _f64, P, P, P]
        lib.oracle_argmax.argtypes = [P, _i64, P]
        lib.oracle_argmax.restype = _i64
        lib.oracle_accept.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float, P]
        lib.oracle_accept.restype = ctypes.c_int
        lib.oracle_residual.argtypes = [P, P, _i64, P]
        lib.oracle_residual.restype = _f64
        lib.oracle_draw.argtypes = [P, _i64, ctypes.c_float, P, P]
        lib.oracle_draw.restype = _i64
        lib.oracle_tree_mask.argtypes = [P, _i64, P, P, P]
        lib.oracle_tree_mask.restype = None
        lib.oracle_tree_greedy.argtypes = [P, P, P, _i64, _i64, P, P, P]
        lib.oracle_tree_greedy.restype = ctypes.c_int
        lib.oracle_kv_init.argtypes = [P, P, P, _i64, _i64]
        lib.oracle_kv_init.restype = None
        lib.oracle_kv_append.argtypes = [P, P, P, P, P, P, P, P, _i64, _i64, _i64, _i64, _i64, _i64, _i64]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_kv_rollback.argtypes = [P, P, P, P, P, _i64, _i64, _i64]
        lib.oracle_kv_rollback.restype = ctypes.c_int
        lib.oracle_kv_gather.argtypes = [P, P, P, P, _i64, _i64, _i64, _i64, _i64, _i64, P, P]
        lib.oracle_kv_gather.restype = None
        lib.oracle_warp.argtypes = [P, _i64, ctypes.c_double, _i64, ctypes.c_double, P, P, P]
        lib.oracle_warp.restype = _i64
        lib.oracle_verify_warped.argtypes = [P, P, ctypes.c_int, P, ctypes.c_double, P, _i64, _i64, _i64, _i64,
                                             ctypes.c_double, P, P, P, P, P, P, P, P]
        lib.oracle_verify_warped.restype = ctypes.c_int
        lib.oracle_verify_probs.argtypes = [P, P, P, P, _i64, _i64, _i64, P, P, P, P, P, P]
        lib.oracle_verify_probs.restype = ctypes.c_int
        lib.oracle_verify.argtypes = [P, P, ctypes.c_int, P, _f64, P, _i64, _i64, _i64, P, P, P, P, P, P]
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_sample_rows.argtypes = [P, _i64, _i64, _f64, P, P, P]
        lib.oracle_acceptance_rate.argtypes = [P, P, _i64]
        lib.oracle_acceptance_rate.restype = _f64
        lib.oracle_expected_tokens.argtypes = [_f64, _i64]
        lib.oracle_expected_tokens.restype = _f64
        lib.oracle_expected_tokens_rows.argtypes = [P, _i64]
        lib.oracle_expected_tokens_rows.restype = _f64
        lib.oracle_planted.restype = ctypes.c_int
        self.lib = lib

    @property
    def planted(self) -> int:
        return int(self.lib.oracle_planted())

    # -- scoring ---------------------------------------------------------
    def linear(self, X_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
        """Y[n, v] = sum_k X[n, k] W[v, k] in fp64; X [N, d], W [V, d] as bf16 bit patterns (uint16)."""
        X = np.ascontiguousarray(X_bits, dtype=np.uint16)
        W = np.ascontiguousarray(W_bits, dtype=np.uint16)
        N, d = X.shape
        V, d2 = W.shape
        assert d == d2
        Y = np.empty((N, V), dtype=np.float64)
        self.lib.oracle_linear(X.ctypes.data, W.ctypes.data, N, d, V, Y.ctypes.data)
        return Y

    def linear_entries(self, X_bits, W_bits, n_idx, v_idx) -> np.ndarray:
        X = np.ascontiguousarray(X_bits, dtype=np.uint16)
        W = np.ascontiguousarray(W_bits, dtype=np.uint16)
        n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
        v_idx = np.ascontiguousarray(v_idx, dtype=np.int64)
        assert n_idx.shape == v_idx.shape
        assert n_idx.size == 0 or (n_idx.min() >= 0 and n_idx.max() < X.shape[0])
        assert v_idx.size == 0 or (v_idx.min() >= 0 and v_idx.max() < W.shape[0])
        out = np.empty(n_idx.shape, dtype=np.float64)
        self.lib.oracle_linear_entries(X.ctypes.data, W.ctypes.data, X.shape[1], W.shape[0],
                                       n_idx.ctypes.data, v_idx.ctypes.data, n_idx.size, out.ctypes.data)
        return out

    # -- distributions ---------------------------------------------------
    def softmax(self, z, T: float = 1.0):
        """Returns (p fp32 [V], m fp64, Z fp64) for one row of logits."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        p = np.empty_like(z)
        m = np.zeros(1)
        Z = np.zeros(1)
        self.lib.oracle_softmax(z.ctypes.data, z.size, float(T), p.ctypes.data, m.ctypes.data, Z.ctypes.data)
        return p, float(m[0]), float(Z[0])

    def argmax(self, z):
        """Returns (index, top-2 gap) of one row; ties go to the lowest index."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        gap = np.zeros(1)
        idx = self.lib.oracle_argmax(z.ctypes.data, z.size, gap.ctypes.data)
        return int(idx), float(gap[0])

    def accept(self, p_x: float, q_x: float, u: float):
        m = np.zeros(1)
        keep = self.lib.oracle_accept(float(p_x), float(q_x), float(u), m.ctypes.data)
        return bool(keep), float(m[0])

    def residual(self, p, q):
        """Returns (r fp32 [V], S fp64) with r = max(0, p - q)."""
        p = np.ascontiguousarray(p, dtype=np.float32)
        q = np.ascontiguousarray(q, dtype=np.float32)
        r = np.empty_like(p)
        S = self.lib.oracle_residual(p.ctypes.data, q.ctypes.data, p.size, r.ctypes.data)
        return r, float(S)

    def draw(self, w, u: float):
        """Inverse-CDF draw from unnormalised weights; returns (token or -1, margin)."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        m = np.zeros(1)
        t = self.lib.oracle_draw(w.ctypes.data, w.size, float(u), m.ctypes.data, None)
        return int(t), float(m[0])

    def acceptance_rate(self, p, q) -> float:
        p = np.ascontiguousarray(p, dtype=np.float32)
        q = np.ascontiguousarray(q, dtype=np.float32)
        return float(self.lib.oracle_acceptance_rate(p.ctypes.data, q.ctypes.data, p.size))

    def expected_tokens(self, alpha: float, gamma: int) -> float:
        return float(self.lib.oracle_expected_tokens(float(alpha), int(gamma)))

    def expected_tokens_rows(self, alphas) -> float:
        a = np.ascontiguousarray(alphas, dtype=np.float64)
        return float(self.lib.oracle_expected_tokens_rows(a.ctypes.data, a.size))

    # -- the step --------------------------------------------------------
    def verify_probs(self, p, q, draft_tokens, uniforms):
        """Step on probability rows.  p [B, g+1, V], q [B, g, V] fp32, tokens [B, g], uniforms [B, g+1, 2].

        Returns dict(tokens [B, g+1] int32 (-1 padded), num_emitted [B], accept_margin [B, g],
        draw_margin [B], draw_mass [B])."""
        p = np.ascontiguousarray(p, dtype=np.float32)
        B, g1, V = p.shape
        g = g1 - 1
        q = np.ascontiguousarray(q, dtype=np.float32).reshape(B, g, V)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, g)
        u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, g1, 2)
        out = self._outputs(B, g)
        scratch = np.empty(V, dtype=np.float32)
        rc = self.lib.oracle_verify_probs(p.ctypes.data, q.ctypes.data, x.ctypes.data, u.ctypes.data, B, g, V,
                                          scratch.ctypes.data, out["tokens"].ctypes.data,
                                          out["num_emitted"].ctypes.data, out["accept_margin"].ctypes.data,
                                          out["draw_margin"].ctypes.data, out["draw_mass"].ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_verify_probs rejected its inputs (code {rc})")
        return out

    def verify(self, target_logits, draft, draft_tokens, uniforms, temperature: float, draft_kind: int = Q_LOGITS):
        """The full step from logits.  target [B, g+1, V] fp32, draft [B, g, V] fp32 (logits or probs),
        draft_tokens [B, g], uniforms [B, g+1, 2] (unused at T == 0).  Returns as verify_probs."""
        z = np.ascontiguousarray(target_logits, dtype=np.float32)
        B, g1, V = z.shape
        g = g1 - 1
        if draft is None:
            draft = np.zeros((B, g, V), dtype=np.float32)
        d = np.ascontiguousarray(draft, dtype=np.float32).reshape(B, g, V)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, g)
        if uniforms is None:
            uniforms = np.zeros((B, g1, 2), dtype=np.float32)
        u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, g1, 2)
        out = self._outputs(B, g)
        scratch = np.empty(2 * g1 * V, dtype=np.float32)
        rc = self.lib.oracle_verify(z.ctypes.data, d.ctypes.data, int(draft_kind), x.ctypes.data, float(temperature),
                                    u.ctypes.data, B, g, V, scratch.ctypes.data, out["tokens"].ctypes.data,
                                    out["num_emitted"].ctypes.data, out["accept_margin"].ctypes.data,
                                    out["draw_margin"].ctypes.data, out["draw_mass"].ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_verify rejected its inputs (code {rc})")
        return out

    # -- top-k / top-p warping -------------------------------------------
    def warp(self, z, T: float, top_k: int = 0, top_p: float = 1.0):
        """Warped probabilities of one row of logits: returns (p fp32 [V], number kept, top-p margin)."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        p = np.empty_like(z)
        order = np.empty(z.size, np.int32)
        mg = np.zeros(1)
        n = self.lib.oracle_warp(z.ctypes.data, z.size, float(T), int(top_k), float(top_p), p.ctypes.data,
                                 order.ctypes.data, mg.ctypes.data)
        return p, int(n), float(mg[0])

    def verify_warped(self, target_logits, draft, draft_tokens, uniforms, temperature: float, top_k: int = 0,
                      top_p: float = 1.0, draft_kind: int = Q_LOGITS):
        """The step with top-k/top-p warping of p (and of q given as logits).  Returns as verify, plus
        warp_margin [B]."""
        z = np.ascontiguousarray(target_logits, dtype=np.float32)
        B, g1, V = z.shape
        g = g1 - 1
        if draft is None:
            draft = np.zeros((B, g, V), dtype=np.float32)
        d = np.ascontiguousarray(draft, dtype=np.float32).reshape(B, g, V)
        x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, g)
        if uniforms is None:
            uniforms = np.zeros((B, g1, 2), dtype=np.float32)
        u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, g1, 2)
        out = self._outputs(B, g)
        out["warp_margin"] = np.empty(B, np.float64)
        scratch = np.empty(2 * g1 * V, dtype=np.float32)
        order = np.empty(V, np.int32)
        rc = self.lib.oracle_verify_warped(z.ctypes.data, d.ctypes.data, int(draft_kind), x.ctypes.data,
                                           float(temperature), u.ctypes.data, B, g, V, int(top_k), float(top_p),
                                           scratch.ctypes.data, order.ctypes.data, out["tokens"].ctypes.data,
                                           out["num_emitted"].ctypes.data, out["accept_margin"].ctypes.data,
                                           out["draw_margin"].ctypes.data, out["draw_mass"].ctypes.data,
                                           out["warp_margin"].ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle_verify_warped rejected its inputs (code {rc})")
        return out

    # -- trees -----------------------------------------------------------
    def tree_mask(self, parents):
        """Returns (ancestor bit masks uint64 [M], depths int32 [M], additive mask fp32 [M, M] of 0 / -inf)."""
        par = np.ascontiguousarray(parents, dtype=np.int32)
        M = par.size
        mask = np.empty(M, np.uint64)
        depth = np.empty(M, np.int32)
        add = np.empty((M, M), np.float32)
        self.lib.oracle_tree_mask(par.ctypes.data, M, mask.ctypes.data, depth.ctypes.data, add.ctypes.data)
        return mask, depth, add

    def tree_greedy(self, z, parents, node_tokens):
        """Greedy tree verification of one tree: z [M, V] fp32, parents [M], node_tokens [M].
        Returns (tokens [M] (-1 padded), path nodes [M] (-1 padded), number emitted)."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        M, V = z.shape
        par = np.ascontiguousarray(parents, dtype=np.int32).reshape(M)
        tok = np.ascontiguousarray(node_tokens, dtype=np.int32).reshape(M)
        out_t = np.empty(M, np.int32)
        out_n = np.empty(M, np.int32)
        scratch = np.empty(3 * M, np.int32)
        n = self.lib.oracle_tree_greedy(z.ctypes.data, par.ctypes.data, tok.ctypes.data, M, V, scratch.ctypes.data,
                                        out_t.ctypes.data, out_n.ctypes.data)
        return out_t, out_n, int(n)

    # -- paged KV cache --------------------------------------------------
    def kv_cache(self, R, num_blocks, block_size, heads, head_dim, max_blocks, dtype=np.float32):
        return OracleKV(self, R, num_blocks, block_size, heads, head_dim, max_blocks, dtype)

    def sample_rows(self, z, u, T: float = 1.0) -> np.ndarray:
        """One inverse-CDF draw per row of softmax(z / T); z [R, V], u [R]."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        R, V = z.shape
        u = np.ascontiguousarray(u, dtype=np.float32).reshape(R)
        out = np.empty(R, dtype=np.int32)
        scratch = np.empty(V, dtype=np.float32)
        self.lib.oracle_sample_rows(z.ctypes.data, R, V, float(T), u.ctypes.data, scratch.ctypes.data, out.ctypes.data)
        return out

    @staticmethod
    def _outputs(B, g):
        return {
            "tokens": np.empty((B, g + 1), dtype=np.int32),
            "num_emitted": np.empty(B, dtype=np.int32),
            "accept_margin": np.empty((B, g), dtype=np.float64),
            "draw_margin": np.empty(B, dtype=np.float64),
            "draw_mass": np.empty(B, dtype=np.float64),
        }


_DEFAULT: Oracle | None = None


class OracleKV:
    """State of the oracle's paged KV cache (numpy arrays) and its operations."""

    def __init__(self, o, R, num_blocks, block_size, heads, head_dim, max_blocks, dtype=np.float32):
        self.o, self.R, self.nb, self.bs, self.H, self.D, self.mb = o, R, num_blocks, block_size, heads, head_dim, max_blocks
        self.dtype = np.dtype(dtype)
        self.k = np.zeros((num_blocks, heads, block_size, head_dim), self.dtype)
        self.v = np.zeros_like(self.k)
        self.tables = np.full((R, max_blocks), -1, np.int32)
        self.lens = np.zeros(R, np.int32)
        self.stack = np.zeros(num_blocks, np.int32)
        self.top = np.zeros(1, np.int32)
        o.lib.oracle_kv_init(self.stack.ctypes.data, self.top.ctypes.data, self.lens.ctypes.data, R, num_blocks)

    def append(self, knew, vnew) -> int:
        """knew, vnew: [R, heads, n_new, head_dim].  Returns the status (0 ok)."""
        knew = np.ascontiguousarray(knew, self.dtype)
        vnew = np.ascontiguousarray(vnew, self.dtype)
        n_new = knew.shape[2]
        return int(self.o.lib.oracle_kv_append(self.k.ctypes.data, self.v.ctypes.data, self.tables.ctypes.data,
                                               self.lens.ctypes.data, self.stack.ctypes.data, self.top.ctypes.data,
                                               knew.ctypes.data, vnew.ctypes.data, self.R, n_new, self.H, self.bs,
                                               self.D, self.dtype.itemsize, self.mb))

    def rollback(self, keep_lens) -> int:
        keep = np.ascontiguousarray(keep_lens, np.int32)
        return int(self.o.lib.oracle_kv_rollback(self.tables.ctypes.data, self.lens.ctypes.data,
                                                 self.stack.ctypes.data, self.top.ctypes.data, keep.ctypes.data,
                                                 self.R, self.bs, self.mb))

    def gather(self, r):
        n = int(self.lens[r])
        ko = np.zeros((self.H, n, self.D), self.dtype)
        vo = np.zeros_like(ko)
        self.o.lib.oracle_kv_gather(self.k.ctypes.data, self.v.ctypes.data, self.tables.ctypes.data,
                                    self.lens.ctypes.data, r, self.H, self.bs, self.D, self.dtype.itemsize, self.mb,
                                    ko.ctypes.data, vo.ctypes.data)
        return ko, vo


def load(build_if_missing: bool = True) -> Oracle:
    """The real oracle, built on first use if no build is present."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIBRARY) and build_if_missing:
            build_library()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def load_planted(name: str, directory: str | None = None) -> Oracle:
    """A deliberately wrong build (negative controls); compiled into a temporary directory."""
    directory = directory or tempfile.mkdtemp(prefix="oracle_plant_")
    path = os.path.join(directory, f"liboracle_plant_{PLANTS[name]}.so")
    if not os.path.exists(path):
        build_library(path, PLANTS[name])
    return Oracle(path)
