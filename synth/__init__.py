"""Seeded synthetic workloads for Key-Key Semantic Affinity.

Input generation only: paged bf16 key pools behind block tables, planted
topics, ragged batches and fp32 block-vector tables.  Nothing here pools,
scores or selects; the oracle (``oracle/``) and the HIP library both consume
these arrays.  The heavy lifting is ``synth.c`` (counter-based SplitMix64 +
Box-Muller, multi-threaded) loaded through ctypes.

The workload recipes follow the shapes the page "Key-Key Semantic Affinity:
Key vectors replace attention scores for KV-cache importance" (10100.com)
gives in its sections 3.3 and 5.2: Qwen2.5-0.5B keys (2 KV heads, head_dim
64) and Qwen2.5-7B keys (4 KV heads, head_dim 128), paged in blocks of
16-256 tokens (section 1).  Real keys need trained weights, which are not
available; planted-topic keys stand in for them.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# stream tags (any distinct integers)
TAG_TOPIC_PERM = 11
TAG_TOPIC_DIR = 12
TAG_BIAS_DIR = 13
TAG_PHYS_PERM = 14
TAG_ANCHOR_TOPIC = 15
TAG_SEQ_LEN = 16
TAG_HEAD_VAR = 17
TAG_VB = 18
TAG_ANCHOR = 19
TAG_RUN_POS = 20
TAG_QUERY = 21
TAG_HEAD_ROLE = 22
TAG_RELEVANCE = 23
TAG_BLOCK_DIR = 24
TAG_POS_DIR = 25
TAG_NOISE = 26


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (plain C, no GPU code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, f32, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_stream.argtypes = [u64, u64]
        L.synth_stream.restype = u64
        L.synth_u64.argtypes = [u64, u64, u64]
        L.synth_u64.restype = u64
        L.synth_normal.argtypes = [u64, u64, u64]
        L.synth_normal.restype = f64
        L.synth_uniform.argtypes = [u64, u64, u64]
        L.synth_uniform.restype = f64
        L.synth_f32_to_bf16.argtypes = [vp, vp, i64]
        L.synth_uniform_int.argtypes = [u64, u64, i64, i64, i64, vp]
        L.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
        L.synth_normal_f64.argtypes = [u64, u64, i64, f64, f64, vp]
        L.synth_permutation.argtypes = [u64, u64, i64, vp]
        L.synth_unit_dirs.argtypes = [u64, u64, i64, i32, vp]
        L.synth_kpool.argtypes = [vp, vp, ctypes.c_int]
        L.synth_kpool.restype = ctypes.c_int
        L.synth_rows.argtypes = [u64, u64, i64, i32, vp, vp, i32, f32, f32, vp, ctypes.c_int]
        L.synth_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def n_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- primitives

def permutation(seed: int, tag: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, tag, n, _ptr(out))
    return out


def uniform_int(seed: int, tag: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    lib().synth_uniform_int(seed, tag, n, lo, hi, _ptr(out))
    return out


def uniform(seed: int, tag: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(seed, tag, n, _ptr(out))
    return out


def normal(seed: int, tag: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_normal_f64(seed, tag, n, mean, std, _ptr(out))
    return out


def unit_dirs(seed: int, tag: int, n_vec: int, dim: int) -> np.ndarray:
    out = np.empty((n_vec, dim), dtype=np.float32)
    lib().synth_unit_dirs(seed, tag, n_vec, dim, _ptr(out))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


class _KpoolSpec(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("B", ctypes.c_int32),
        ("P", ctypes.c_int64),
        ("sL", ctypes.c_int64), ("sB", ctypes.c_int64), ("sT", ctypes.c_int64), ("sH", ctypes.c_int64),
        ("S", ctypes.c_int32),
        ("gen_len", ctypes.c_void_p), ("block_offsets", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("block_topic", ctypes.c_void_p), ("topic_dir", ctypes.c_void_p), ("n_topics", ctypes.c_int32),
        ("amp", ctypes.c_float), ("jitter", ctypes.c_float),
        ("noise_std", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("seed", ctypes.c_uint64),
    ]


# ---------------------------------------------------------------- workloads

@dataclass
class KWorkload:
    """A batch of sequences whose keys sit in one paged bf16 pool.

    ``k`` has shape [L][P][B][H][D] (bf16 bit patterns, contiguous), so the
    element strides are (P*B*H*D, B*H*D, H*D, D, 1).  Logical block i of
    sequence s is global logical block ``block_offsets[s] + i`` and lives in
    physical block ``block_table[block_offsets[s] + i]``.
    """
    name: str
    L: int
    H: int
    D: int
    B: int
    P: int
    k: np.ndarray
    seq_len: np.ndarray
    block_offsets: np.ndarray
    block_table: np.ndarray
    window: int
    mode: str  # "uniform" or "variance"
    select: dict
    block_topic: Optional[np.ndarray] = None
    anchor_topic: Optional[np.ndarray] = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def strides(self):
        P, B, H, D = self.P, self.B, self.H, self.D
        return (P * B * H * D, B * H * D, H * D, D)

    @property
    def total_blocks(self) -> int:
        return int(self.block_offsets[-1])

    def max_pages(self) -> int:
        return int(np.max(np.diff(self.block_offsets))) if self.S else 0


@dataclass
class VbWorkload:
    """Block vectors written directly (no pooling): vb [S][n_pages][D] fp32,
    anchors [S][D], page topics [S][n_pages], anchor topic per sequence."""
    name: str
    D: int
    vb: np.ndarray
    anchors: np.ndarray
    n_pages: np.ndarray
    page_topic: np.ndarray
    anchor_topic: np.ndarray
    select: dict
    seed: int = 0


def _csr(nblocks: np.ndarray):
    off = np.zeros(len(nblocks) + 1, dtype=np.int32)
    off[1:] = np.cumsum(nblocks)
    return off


def _gen_kpool(L, H, D, B, P, gen_len, block_offsets, block_table, block_topic, topic_dir, amp, jitter,
               noise_std, bias, seed) -> np.ndarray:
    k = np.zeros((L, P, B, H, D), dtype=np.uint16)
    spec = _KpoolSpec()
    spec.L, spec.H, spec.D, spec.B, spec.P = L, H, D, B, P
    spec.sL, spec.sB, spec.sT, spec.sH = P * B * H * D, B * H * D, H * D, D
    spec.S = len(gen_len)
    gen_len = np.ascontiguousarray(gen_len, dtype=np.int32)
    block_offsets = np.ascontiguousarray(block_offsets, dtype=np.int32)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    keep = [gen_len, block_offsets, block_table]
    spec.gen_len = gen_len.ctypes.data
    spec.block_offsets = block_offsets.ctypes.data
    spec.block_table = block_table.ctypes.data
    if block_topic is not None:
        block_topic = np.ascontiguousarray(block_topic, dtype=np.int32)
        keep.append(block_topic)
        spec.block_topic = block_topic.ctypes.data
        topic_dir = np.ascontiguousarray(topic_dir, dtype=np.float32)
        keep.append(topic_dir)
        spec.topic_dir = topic_dir.ctypes.data
        spec.n_topics = topic_dir.shape[0]
    spec.amp = amp
    spec.jitter = jitter
    noise_std = np.ascontiguousarray(noise_std, dtype=np.float32).reshape(L * H)
    keep.append(noise_std)
    spec.noise_std = noise_std.ctypes.data
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32).reshape(L, H, D)
        keep.append(bias)
        spec.bias = bias.ctypes.data
    spec.seed = seed
    rc = lib().synth_kpool(ctypes.byref(spec), _ptr(k), n_threads())
    if rc != 0:
        raise RuntimeError("synth_kpool failed")
    return k


def planted_kpool(name: str, *, L: int, H: int, D: int, B: int, n_blocks: int, n_topics: int, seed: int,
                  amp: float, jitter: float, noise: float, bias_heads=(), bias_amp: float = 0.0,
                  topic_layout: str = "balanced", run_len: int = 1, permute_phys: bool = False,
                  tail_tokens: Optional[int] = None, window: int = 16, select: Optional[dict] = None,
                  mode: str = "uniform") -> KWorkload:
    """One sequence of n_blocks blocks with planted topics.

    topic_layout "balanced": block b gets topic perm[b] % n_topics, so every
    topic owns n_blocks / n_topics blocks at random positions; the anchor
    topic is the last block's topic.
    topic_layout "runs": blocks form aligned runs of run_len; run r gets topic
    perm[r]; the anchor topic is the topic of a run drawn in the first half,
    and the last block is overwritten to it.
    Keys: amp * g * u[topic][l][h] + bias + noise * N(0,1) per element,
    g ~ N(1, jitter); u unit directions; bias = bias_amp * unit direction per
    (l, h) on the heads in bias_heads (constant over tokens).
    """
    T = n_blocks * B if tail_tokens is None else (n_blocks - 1) * B + tail_tokens
    if topic_layout == "balanced":
        perm = permutation(seed, TAG_TOPIC_PERM, n_blocks)
        topic = (perm % n_topics).astype(np.int32)
        anchor_run = None
    elif topic_layout == "runs":
        n_runs = n_blocks // run_len
        perm = permutation(seed, TAG_TOPIC_PERM, n_runs)
        topic = np.repeat(perm % n_topics, run_len).astype(np.int32)
        anchor_run = int(uniform_int(seed, TAG_RUN_POS, 1, 0, max(0, n_runs // 2 - 1))[0])
        topic[-1] = topic[anchor_run * run_len]
    else:
        raise ValueError(topic_layout)
    dirs = unit_dirs(seed, TAG_TOPIC_DIR, n_topics * L * H, D).reshape(n_topics, L, H, D)
    bias = None
    if bias_heads:
        bdir = unit_dirs(seed, TAG_BIAS_DIR, L * H, D).reshape(L, H, D)
        bias = np.zeros((L, H, D), dtype=np.float32)
        for h in bias_heads:
            bias[:, h, :] = bias_amp * bdir[:, h, :]
    table = permutation(seed, TAG_PHYS_PERM, n_blocks) if permute_phys else np.arange(n_blocks, dtype=np.int32)
    off = np.array([0, n_blocks], dtype=np.int32)
    seq_len = np.array([T], dtype=np.int32)
    noise_std = np.full(L * H, noise, dtype=np.float32)
    k = _gen_kpool(L, H, D, B, n_blocks, seq_len, off, table, topic, dirs, amp, jitter, noise_std, bias, seed)
    sel = select or {"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 16,
                     "pages_per_chunk": 16, "chunks_per_grid": 16}
    w = KWorkload(name=name, L=L, H=H, D=D, B=B, P=n_blocks, k=k, seq_len=seq_len, block_offsets=off,
                  block_table=table.astype(np.int32), window=window, mode=mode, select=sel,
                  block_topic=topic[None, :].copy(), anchor_topic=np.array([topic[-1]], dtype=np.int32),
                  seed=seed)
    w.extra["anchor_run"] = anchor_run
    w.extra["run_len"] = run_len
    w.extra["n_topics"] = n_topics
    return w


def planted_queries(w: KWorkload, n_q_heads: int, amp: float, noise: float, seed: int = 0,
                    topic: Optional[int] = None) -> np.ndarray:
    """Decode-step queries [L][n_q_heads][D] (fp32) for a planted workload:
    query head hq of layer l points along the planted direction of `topic`
    (default: the anchor topic) for KV head hq // (n_q_heads / H), scaled by
    amp, plus N(0, noise) per element.  Grouped query heads share their KV
    head's direction.  Only random numbers and the workload's own planted
    directions; no attention arithmetic."""
    L, H, D = w.L, w.H, w.D
    if n_q_heads % H:
        raise ValueError("n_q_heads must be a multiple of the KV heads")
    G = n_q_heads // H
    n_topics = w.extra["n_topics"]
    t = int(w.anchor_topic[0]) if topic is None else int(topic)
    dirs = unit_dirs(w.seed, TAG_TOPIC_DIR, n_topics * L * H, D).reshape(n_topics, L, H, D)
    q = amp * np.repeat(dirs[t], G, axis=1)  # [L][Hq][D]
    q = q + normal(seed, TAG_QUERY, L * n_q_heads * D, 0.0, noise).reshape(L, n_q_heads, D)
    return np.ascontiguousarray(q, dtype=np.float32)


def config1(seed: int = 0) -> KWorkload:
    """Qwen2.5-0.5B shape: 24 layers x 2 KV heads x head_dim 64, 4096 tokens in
    blocks of 16 (256 blocks); 8 balanced planted topics; unit directions
    scaled by N(1, 0.1) plus N(0, 0.5) noise; anchor = last 8 tokens; flat
    top-16."""
    return planted_kpool("c1_qwen05b_4k_b16", L=24, H=2, D=64, B=16, n_blocks=256, n_topics=8, seed=seed,
                         amp=1.0, jitter=0.1, noise=0.5, topic_layout="balanced", window=8,
                         select={"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 16,
                                 "pages_per_chunk": 16, "chunks_per_grid": 16})


def config2(seed: int = 0, n_blocks: int = 256) -> KWorkload:
    """Qwen2.5-7B shape: 28 x 4 x 128, 32768 tokens in blocks of 128 (256
    blocks); 32 balanced topics with per-element signal RMS 1.0 and noise
    sigma 1.0, plus a constant positional-bias offset on KV heads 2 and 3;
    anchor = last 16 tokens; uniform pooling; flat top-32."""
    D = 128
    return planted_kpool("c2_qwen7b_32k_b128", L=28, H=4, D=D, B=128, n_blocks=n_blocks, n_topics=32, seed=seed,
                         amp=math.sqrt(D), jitter=0.0, noise=1.0, bias_heads=(2, 3), bias_amp=math.sqrt(D),
                         topic_layout="balanced", window=16,
                         select={"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 32,
                                 "pages_per_chunk": 16, "chunks_per_grid": 16})


def config3(seed: int = 0, n_blocks: int = 8192, L: int = 28) -> KWorkload:
    """Qwen2.5-7B shape at 131072 tokens in blocks of 16 (8192 blocks), 256
    topics in aligned runs of 32 blocks, physical blocks permuted behind the
    table; 16 pages per chunk, 16 chunks per grid; top-4 grids, top-16
    chunks, top-64 pages; anchor = last 16 tokens."""
    D = 128
    n_topics = max(1, n_blocks // 32)
    return planted_kpool("c3_qwen7b_128k_b16", L=L, H=4, D=D, B=16, n_blocks=n_blocks, n_topics=n_topics,
                         seed=seed, amp=math.sqrt(D), jitter=0.0, noise=1.0, bias_heads=(2, 3),
                         bias_amp=math.sqrt(D), topic_layout="runs", run_len=32, permute_phys=True, window=16,
                         select={"hierarchical": 1, "k_grid": 4, "k_chunk": 16, "k_page": 64,
                                 "pages_per_chunk": 16, "chunks_per_grid": 16})


def config4(seed: int = 0, n_seqs: int = 64, n_pages: int = 8192, D: int = 128, n_topics: int = 64,
            run_len: int = 128) -> VbWorkload:
    """Serving-scale decode step: n_seqs sequences of n_pages fp32 block
    vectors (D = 128) drawn as sqrt(D) * u_topic + N(0, 0.3) per element,
    topics in aligned runs of 128 pages (a seeded permutation of the 64 topic
    directions per sequence); per-sequence anchor sqrt(D) * u_t* + N(0, 0.3)
    with a seeded t*; Grid->Chunk->Page 16/16 with k = 4/16/64."""
    dirs = unit_dirs(seed, TAG_TOPIC_DIR, n_topics, D)
    n_runs = n_pages // run_len
    page_topic = np.empty((n_seqs, n_pages), dtype=np.int32)
    for s in range(n_seqs):
        perm = permutation(seed, TAG_TOPIC_PERM * 1000003 + s, n_runs)
        page_topic[s] = np.repeat(perm % n_topics, run_len)
    anchor_topic = uniform_int(seed, TAG_ANCHOR_TOPIC, n_seqs, 0, n_topics - 1).astype(np.int32)
    amp = math.sqrt(D)
    vb = np.empty((n_seqs, n_pages, D), dtype=np.float32)
    lib().synth_rows(seed, TAG_VB, n_seqs * n_pages, D, _ptr(page_topic), _ptr(dirs), n_topics, amp, 0.3,
                     _ptr(vb), n_threads())
    anchors = np.empty((n_seqs, D), dtype=np.float32)
    lib().synth_rows(seed, TAG_ANCHOR, n_seqs, D, _ptr(anchor_topic), _ptr(dirs), n_topics, amp, 0.3,
                     _ptr(anchors), n_threads())
    return VbWorkload(name="c4_serving_64x8192", D=D, vb=vb, anchors=anchors,
                      n_pages=np.full(n_seqs, n_pages, dtype=np.int32), page_topic=page_topic,
                      anchor_topic=anchor_topic,
                      select={"hierarchical": 1, "k_grid": 4, "k_chunk": 16, "k_page": 64,
                              "pages_per_chunk": 16, "chunks_per_grid": 16}, seed=seed)


def config5(seed: int = 0, n_seqs: int = 32, len_lo: int = 4096, len_hi: int = 65536, L: int = 28, H: int = 4,
            D: int = 128, B: int = 64) -> KWorkload:
    """Ragged batch: n_seqs sequences with lengths uniform in [len_lo,
    len_hi], 7B shape, blocks of 64, one shared physical pool in a seeded
    permutation.  Keys N(0, v_lh) per element with v_lh = exp(U[ln 0.1,
    ln 4]) per (layer, head).  Head-variance-weighted pooling, anchor = last
    16 tokens, flat top-48.  The pool also holds one appended token per
    sequence (position seq_len[s]) so a decode step can be replayed:
    ``extra['after']`` holds the CSR state after that append."""
    T = uniform_int(seed, TAG_SEQ_LEN, n_seqs, len_lo, len_hi).astype(np.int32)
    nb_after = (T + 1 + B - 1) // B
    nb_before = (T + B - 1) // B
    P = int(nb_after.sum())
    phys = permutation(seed, TAG_PHYS_PERM, P)
    off_after = _csr(nb_after)
    table_after = phys.astype(np.int32)
    off_before = _csr(nb_before)
    table_before = np.concatenate([table_after[off_after[s]:off_after[s] + nb_before[s]]
                                   for s in range(n_seqs)]).astype(np.int32)
    u = uniform(seed, TAG_HEAD_VAR, L * H)
    var = np.exp(math.log(0.1) + u * (math.log(4.0) - math.log(0.1)))
    noise_std = np.sqrt(var).astype(np.float32)
    k = _gen_kpool(L, H, D, B, P, T + 1, off_after, table_after, None, None, 0.0, 0.0, noise_std, None, seed)
    w = KWorkload(name="c5_ragged32_b64_weighted", L=L, H=H, D=D, B=B, P=P, k=k, seq_len=T.copy(),
                  block_offsets=off_before, block_table=table_before, window=16, mode="variance",
                  select={"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 48,
                          "pages_per_chunk": 16, "chunks_per_grid": 16}, seed=seed)
    w.extra["after"] = {"seq_len": (T + 1).astype(np.int32), "block_offsets": off_after,
                        "block_table": table_after}
    w.extra["head_var"] = var.reshape(L, H)
    return w


def positional_heads_workload(seed: int = 0, n_topic_heads: int = 16, amp_topic: float = 1.0,
                              amp_pos: float = 0.3, noise: float = 0.2, query_amp: float = 8.0):
    """0.5B key shape (24 layers x 2 KV heads x head_dim 64, 4096 tokens in
    blocks of 16, identity table, anchor = last 8 tokens, flat top-16) with
    two kinds of heads, for the overlap of key-key selection with attention
    (the page's section 3.3 and 6.1 experiment):

    * n_topic_heads "topic" heads (a seeded choice among the 48): every block
      b has a relevance r_b ~ U(0, 1) (the last block, which holds the
      anchor, has r = 1), and its keys are amp_topic * sqrt(D) * (r_b * u_h +
      sqrt(1 - r_b^2) * w_bh) with u_h the head's anchor direction and w_bh a
      per-block direction orthogonal to it: a large spread over the context.
    * the other heads are "positional": amp_pos * sqrt(D) * (cos(th_t) e1 +
      sin(th_t) e2), th_t = pi * t / T, the same two directions for every
      such head -- a component that drifts with position, not with content,
      and a small spread over the context.
    * every element also carries N(0, noise).

    Queries [L][14][D] (7 query heads per KV head): amp along u_h for the
    query heads of topic heads, zero for the others, so attention follows
    the graded relevance and the positional heads attend uniformly.
    Returns (KWorkload, queries, relevance[256], topic_head_mask[L][H])."""
    L, H, D, B, nb, Hq = 24, 2, 64, 16, 256, 14
    T = nb * B
    LH = L * H
    role = np.zeros(LH, dtype=bool)
    role[permutation(seed, TAG_HEAD_ROLE, LH)[:n_topic_heads]] = True
    rel = uniform(seed, TAG_RELEVANCE, nb).astype(np.float64)
    rel[-1] = 1.0
    u = unit_dirs(seed, TAG_TOPIC_DIR, LH, D).astype(np.float64)             # [LH][D]
    wdir = unit_dirs(seed, TAG_BLOCK_DIR, nb * LH, D).astype(np.float64).reshape(nb, LH, D)
    wdir -= np.einsum("bhd,hd->bh", wdir, u)[..., None] * u[None]            # orthogonal to u_h
    wdir /= np.linalg.norm(wdir, axis=-1, keepdims=True)
    e = unit_dirs(seed, TAG_POS_DIR, 2, D).astype(np.float64)
    e[1] -= (e[1] @ e[0]) * e[0]
    e[1] /= np.linalg.norm(e[1])
    th = np.pi * np.arange(T) / T
    pos = amp_pos * math.sqrt(D) * (np.cos(th)[:, None] * e[0] + np.sin(th)[:, None] * e[1])   # [T][D]
    topic = amp_topic * math.sqrt(D) * (rel[:, None, None] * u[None] +
                                        np.sqrt(1.0 - rel ** 2)[:, None, None] * wdir)        # [nb][LH][D]
    keys = np.empty((T, LH, D), dtype=np.float64)
    keys[:, role] = np.repeat(topic[:, role], B, axis=0)
    keys[:, ~role] = pos[:, None, :]
    keys += normal(seed, TAG_NOISE, T * LH * D, 0.0, noise).reshape(T, LH, D)
    # [T][L][H][D] -> [L][P=nb][B][H][D]
    k = keys.reshape(nb, B, L, H, D).transpose(2, 0, 1, 3, 4)
    w = kpool_from_f32("quality_0.5b_positional_heads", k.astype(np.float32), [T], [0, nb],
                       np.arange(nb, dtype=np.int32), window=8, mode="uniform",
                       select={"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 16,
                               "pages_per_chunk": 16, "chunks_per_grid": 16})
    w.seed = seed
    q = np.zeros((L, Hq, D), dtype=np.float32)
    G = Hq // H
    for l in range(L):
        for h in range(H):
            if role[l * H + h]:
                q[l, h * G:(h + 1) * G] = (query_amp * u[l * H + h]).astype(np.float32)
    return w, q, rel, role.reshape(L, H)


def kpool_from_f32(name: str, keys: np.ndarray, seq_len, block_offsets, block_table, window: int = 16,
                   mode: str = "uniform", select: Optional[dict] = None) -> KWorkload:
    """Wrap explicit fp32 keys [L][P][B][H][D] (rounded to bf16) as a workload."""
    keys = np.asarray(keys, dtype=np.float32)
    L, P, B, H, D = keys.shape
    sel = select or {"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 4,
                     "pages_per_chunk": 2, "chunks_per_grid": 2}
    return KWorkload(name=name, L=L, H=H, D=D, B=B, P=P, k=to_bf16_bits(keys),
                     seq_len=np.asarray(seq_len, dtype=np.int32),
                     block_offsets=np.asarray(block_offsets, dtype=np.int32),
                     block_table=np.asarray(block_table, dtype=np.int32), window=window, mode=mode, select=sel)
