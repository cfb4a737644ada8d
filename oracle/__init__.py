"""CPU oracle for Key-Key Semantic Affinity block selection.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.  The
arithmetic lives in ``kka_oracle.c`` (plain single-threaded C, fp64 sums,
one rounding to fp32 per output); this module only marshals numpy arrays
and strings the per-block functions together in the order the page
"Key-Key Semantic Affinity: Key vectors replace attention scores for
KV-cache importance" (10100.com) describes in sections 2.2, 5.1 and 5.2:
pool every block, pool the anchor, build the Grid -> Chunk -> Page vectors,
score, select.

Parity status of each function is recorded in its docstring.  Functions
pinned by the CPU tests in ``tests/test_oracle_pins.py`` say which pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kka_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so: gcc -O2, no fast-math, no threads."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _KPool(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("L", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("B", ctypes.c_int32),
        ("P", ctypes.c_int64),
        ("sL", ctypes.c_int64), ("sB", ctypes.c_int64), ("sT", ctypes.c_int64), ("sH", ctypes.c_int64),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.oracle_head_weights.argtypes = [ctypes.POINTER(_KPool), vp, i32, vp]
        L.oracle_pool_block.argtypes = [ctypes.POINTER(_KPool), i64, i32, vp, vp]
        L.oracle_pool_anchor.argtypes = [ctypes.POINTER(_KPool), vp, i32, i32, vp, vp]
        L.oracle_build_levels.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oracle_affinity.argtypes = [vp, i64, i32, vp, vp]
        L.oracle_select.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_stability.argtypes = [vp, i32, i64, i32, ctypes.c_float, vp, vp]
        L.oracle_attention_blocks.argtypes = [ctypes.POINTER(_KPool), vp, i32, i32, vp, ctypes.c_double, vp]
        for f in (L.oracle_head_weights, L.oracle_pool_block, L.oracle_pool_anchor, L.oracle_build_levels,
                  L.oracle_affinity, L.oracle_select, L.oracle_stability, L.oracle_attention_blocks):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


class KPool:
    """A paged bf16 key pool: ``k`` uint16 bit patterns, element (l, p, t, h, d)
    at ``l*sL + p*sB + t*sT + h*sH + d`` (strides default to contiguous
    [L][P][B][H][D])."""

    def __init__(self, k: np.ndarray, L: int, H: int, D: int, B: int, P: int, strides=None):
        if k.dtype != np.uint16:
            raise TypeError("k must hold bf16 bit patterns as uint16")
        self.k = k
        self.L, self.H, self.D, self.B, self.P = L, H, D, B, P
        self.strides = strides or (P * B * H * D, B * H * D, H * D, D)
        s = _KPool()
        s.k = k.ctypes.data
        s.L, s.H, s.D, s.B, s.P = L, H, D, B, P
        s.sL, s.sB, s.sT, s.sH = self.strides
        self._s = s

    @classmethod
    def of(cls, w) -> "KPool":
        """From any object with k, L, H, D, B, P (and optionally strides)."""
        return cls(w.k, w.L, w.H, w.D, w.B, w.P, getattr(w, "strides", None))


def head_weights(kp: KPool, table: np.ndarray, T: int) -> np.ndarray:
    """Variance head weights of one sequence, fp32 [L*H].  Pinned: equal
    variances -> uniform, hand example, constant-offset invariance."""
    table = np.ascontiguousarray(table, dtype=np.int32)
    out = np.empty(kp.L * kp.H, dtype=np.float32)
    _check(lib().oracle_head_weights(ctypes.byref(kp._s), _p(table), int(T), _p(out)), "head_weights")
    return out


def pool_block(kp: KPool, phys: int, n_valid: int, weights=None) -> np.ndarray:
    """v_b of one block, fp32 [D].  Pinned: constant keys, linearity,
    token-order invariance, pure-noise variance, hand example."""
    out = np.empty(kp.D, dtype=np.float32)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    _check(lib().oracle_pool_block(ctypes.byref(kp._s), int(phys), int(n_valid), _p(w), _p(out)), "pool_block")
    return out


def pool_anchor(kp: KPool, table: np.ndarray, T: int, W: int, weights=None) -> np.ndarray:
    """v_anchor of one sequence, fp32 [D].  Pinned: block-aligned window
    equals that block's v_b, hand example."""
    table = np.ascontiguousarray(table, dtype=np.int32)
    out = np.empty(kp.D, dtype=np.float32)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    _check(lib().oracle_pool_anchor(ctypes.byref(kp._s), _p(table), int(T), int(W), _p(w), _p(out)),
           "pool_anchor")
    return out


def build_levels(pages: np.ndarray, ppc: int, cpg: int):
    """(chunks [n_c][D], grids [n_g][D]) from page vectors [n_p][D].
    Pinned: full grid = mean of its pages, hand example."""
    pages = np.ascontiguousarray(pages, dtype=np.float32)
    n_p, D = pages.shape
    n_c = -(-n_p // ppc)
    n_g = -(-n_c // cpg)
    chunks = np.empty((n_c, D), dtype=np.float32)
    grids = np.empty((n_g, D), dtype=np.float32)
    _check(lib().oracle_build_levels(_p(pages), n_p, D, ppc, cpg, _p(chunks), _p(grids)), "build_levels")
    return chunks, grids


def affinity(rows: np.ndarray, anchor: np.ndarray) -> np.ndarray:
    """(1 + cos) / 2 of each row with the anchor, fp32.  Pinned: self = 1,
    opposite = 0, orthogonal = 0.5, positive-scale invariance, hand values."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    anchor = np.ascontiguousarray(anchor, dtype=np.float32)
    n = rows.shape[0]
    D = anchor.shape[0]
    out = np.empty(n, dtype=np.float32)
    _check(lib().oracle_affinity(_p(rows.reshape(n, D) if n else rows), n, D, _p(anchor), _p(out)), "affinity")
    return out


def select(aff_pages, aff_chunks=None, aff_grids=None, *, hierarchical: int, k_grid: int = 0, k_chunk: int = 0,
           k_page: int, pages_per_chunk: int = 16, chunks_per_grid: int = 16):
    """(page indices int32 [k_eff], masked scores fp32 [k_eff]).
    Pinned: brute force over all subsets on tiny inputs, hierarchy hand
    example, full-keep hierarchy == flat."""
    aff_pages = np.ascontiguousarray(aff_pages, dtype=np.float32)
    n_p = aff_pages.shape[0]
    ac = None if aff_chunks is None else np.ascontiguousarray(aff_chunks, dtype=np.float32)
    ag = None if aff_grids is None else np.ascontiguousarray(aff_grids, dtype=np.float32)
    kmax = max(0, min(k_page, n_p))
    idx = np.full(max(1, kmax), -1, dtype=np.int32)
    sc = np.zeros(max(1, kmax), dtype=np.float32)
    cnt = np.zeros(1, dtype=np.int32)
    _check(lib().oracle_select(_p(aff_pages), _p(ac), _p(ag), n_p, pages_per_chunk, chunks_per_grid,
                               int(hierarchical), k_grid, k_chunk, k_page, _p(idx), _p(sc), _p(cnt)), "select")
    c = int(cnt[0])
    return idx[:c].copy(), sc[:c].copy()


def stability(aff_hist, window: int, theta: float):
    """(score fp32 [n], window bits uint32 [n]) of n blocks from their
    affinities over the steps so far (aff_hist [n_steps][n], oldest first;
    a step before a block existed carries an affinity <= theta).
    Pinned: the page's worked values (golden W3), closed forms."""
    a = np.ascontiguousarray(aff_hist, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("aff_hist must be [n_steps][n]")
    n_steps, n = a.shape
    score = np.zeros(n, dtype=np.float32)
    bits = np.zeros(n, dtype=np.uint32) if window <= 32 else None
    _check(lib().oracle_stability(_p(a) if a.size else None, n_steps, n, window, float(theta),
                                  _p(score) if n else None, _p(bits) if (bits is not None and n) else None),
           "stability")
    return score, bits


def attention_blocks(kp: KPool, table: np.ndarray, T: int, q: np.ndarray, scale: float) -> np.ndarray:
    """Attention mass per block [ceil(T/B)] of one decode query q [L][Hq][D],
    averaged over layers and query heads (GQA: head hq reads KV head
    hq // (Hq / H)).  Pinned: uniform cases, a two-token closed form, shift
    invariance, unit total mass, the GQA head mapping."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    L, Hq, D = q.shape
    if L != kp.L or D != kp.D:
        raise ValueError("query shape does not match the pool")
    table = np.ascontiguousarray(table, dtype=np.int32)
    nb = -(-T // kp.B)
    out = np.zeros(max(1, nb), dtype=np.float32)
    _check(lib().oracle_attention_blocks(ctypes.byref(kp._s), _p(table), int(T), Hq, _p(q), float(scale), _p(out)),
           "attention_blocks")
    return out[:nb]


def overlap(a, b, k: int) -> float:
    """|top-k set a  intersect  top-k set b| / k (the overlap rate the page reports)."""
    if k <= 0:
        return 0.0
    return len(set(np.asarray(a)[:k].tolist()) & set(np.asarray(b)[:k].tolist())) / k


# --------------------------------------------------------------- pipelines

def seq_table(block_offsets, block_table, s):
    return np.ascontiguousarray(block_table[block_offsets[s]:block_offsets[s + 1]], dtype=np.int32)


def n_valid(seq_len, B, i, s):
    return int(max(0, min(B, int(seq_len[s]) - i * B)))


def weights_all(kp: KPool, seq_len, block_offsets, block_table, seqs=None) -> np.ndarray:
    """Head weights [S][L*H] for the listed sequences (rows of the others are NaN)."""
    S = len(seq_len)
    out = np.full((S, kp.L * kp.H), np.nan, dtype=np.float32)
    for s in (range(S) if seqs is None else seqs):
        out[s] = head_weights(kp, seq_table(block_offsets, block_table, s), int(seq_len[s]))
    return out


def pool_blocks(kp: KPool, seq_len, block_offsets, block_table, weights=None, blocks=None) -> dict:
    """{global logical block id: v_b} for the listed blocks (all by default).
    weights: None (uniform) or [S][L*H]."""
    S = len(seq_len)
    out = {}
    for s in range(S):
        lo, hi = int(block_offsets[s]), int(block_offsets[s + 1])
        for b in range(lo, hi):
            if blocks is not None and b not in blocks:
                continue
            w = None if weights is None else weights[s]
            out[b] = pool_block(kp, int(block_table[b]), n_valid(seq_len, kp.B, b - lo, s), w)
    return out


def score_select(level_pages, anchor, sel: dict):
    """Oracle levels + affinities + selection for one sequence.
    Returns dict(chunks, grids, aff_pages, aff_chunks, aff_grids, idx, score)."""
    level_pages = np.ascontiguousarray(level_pages, dtype=np.float32)
    out = {}
    if sel["hierarchical"]:
        chunks, grids = build_levels(level_pages, sel["pages_per_chunk"], sel["chunks_per_grid"])
        out["chunks"], out["grids"] = chunks, grids
        out["aff_chunks"] = affinity(chunks, anchor)
        out["aff_grids"] = affinity(grids, anchor)
    else:
        out["aff_chunks"] = out["aff_grids"] = None
    out["aff_pages"] = affinity(level_pages, anchor)
    out["idx"], out["score"] = select(out["aff_pages"], out["aff_chunks"], out["aff_grids"],
                                      hierarchical=sel["hierarchical"], k_grid=sel["k_grid"],
                                      k_chunk=sel["k_chunk"], k_page=sel["k_page"],
                                      pages_per_chunk=sel["pages_per_chunk"],
                                      chunks_per_grid=sel["chunks_per_grid"])
    return out
