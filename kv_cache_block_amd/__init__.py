"""Key-Key Semantic Affinity block selection for paged KV caches on MI355X.

Thin ctypes binding of ``libkka.so`` (C ABI in ``include/kka.h``).  PyTorch
only supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  The binding checks that
tensors live on the GPU and are large enough for what the kernels will
touch, builds the C structs and raises :class:`KkaError` on a non-zero
status.  There is no CPU fallback: without the built library every call
raises.

Entry points keep the C names: :func:`kka_pool_blocks`,
:func:`kka_pool_anchor`, :func:`kka_pool_on_write`, :func:`kka_build_levels`, :func:`kka_score_topk`,
:func:`kka_score_topk_lazy`, :func:`kka_score_topk_stable` (through
:func:`kka_score_topk` with ``history=``), :func:`kka_device_error` (plus the
``*_workspace`` size queries).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkka.so")

WEIGHT_UNIFORM = 0
WEIGHT_VARIANCE = 1
WEIGHT_GIVEN = 2

DEVERR_BLOCK_TABLE = 1
DEVERR_SEQ_LEN = 2
DEVERR_ROW = 4
DEVERR_PAGES = 8
DEVERR_OFFSETS = 16
DEVERR_WORKSPACE = 32

_STATUS = {0: "ok", 1: "KKA_ERR_NULL", 2: "KKA_ERR_SHAPE", 3: "KKA_ERR_ALIGN", 4: "KKA_ERR_WORKSPACE",
           5: "KKA_ERR_DEVICE", 6: "KKA_ERR_SCRATCH"}

ENTRY_POINTS = (
    "kka_pool_blocks", "kka_pool_blocks_workspace", "kka_pool_anchor", "kka_pool_anchor_workspace", "kka_pool_on_write",
    "kka_level_rows", "kka_build_levels", "kka_score_topk", "kka_score_topk_workspace", "kka_score_topk_lazy",
    "kka_score_topk_stable", "kka_attention_topk", "kka_attention_topk_workspace", "kka_device_error",
    "kka_status_string", "kka_version", "kka_pool_anchor_noalloc", "kka_pool_anchor_noalloc_scratch",
)


class KkaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({status_string(status)})")


class c_kpool(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_phys_blocks", ctypes.c_int64),
        ("stride_layer", ctypes.c_int64), ("stride_block", ctypes.c_int64), ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
    ]


class c_seqs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_blocks", ctypes.c_int32), ("seq_len", ctypes.c_void_p),
        ("block_offsets", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
    ]


class c_level_layout(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("hierarchical", ctypes.c_int32), ("pages_per_chunk", ctypes.c_int32),
        ("chunks_per_grid", ctypes.c_int32),
    ]


class c_select(ctypes.Structure):
    _fields_ = [("k_grid", ctypes.c_int32), ("k_chunk", ctypes.c_int32), ("k_page", ctypes.c_int32)]


class c_stability(ctypes.Structure):
    _fields_ = [("history", ctypes.c_void_p), ("score_out", ctypes.c_void_p), ("window", ctypes.c_int32),
                ("theta", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkka.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_block_amd._build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.kka_pool_blocks.argtypes = [P(c_kpool), P(c_seqs), vp, i32, i32, vp, vp, i64, vp, sz, vp]
        L.kka_pool_blocks_workspace.argtypes = [P(c_kpool), P(c_seqs), vp, i32, i32]
        L.kka_pool_anchor.argtypes = [P(c_kpool), P(c_seqs), i32, vp, vp, vp, sz, vp]
        L.kka_pool_anchor_workspace.argtypes = [P(c_kpool), P(c_seqs), i32]
        L.kka_pool_anchor_noalloc.argtypes = [P(c_kpool), P(c_seqs), i32, vp, vp, vp]
        L.kka_pool_anchor_noalloc_scratch.argtypes = [P(c_kpool), P(c_seqs)]
        L.kka_pool_on_write.argtypes = [P(c_kpool), P(c_seqs), vp, i32, vp, vp, i32, vp, i64, vp]
        L.kka_attention_topk.argtypes = [P(c_kpool), P(c_seqs), vp, i32, ctypes.c_float, i32, vp, i64, vp, vp, vp,
                                         vp, sz, vp]
        L.kka_attention_topk_workspace.argtypes = [P(c_kpool), P(c_seqs), i32]
        L.kka_level_rows.argtypes = [P(c_level_layout)]
        L.kka_build_levels.argtypes = [P(c_level_layout), vp, vp, vp, vp]
        L.kka_score_topk.argtypes = [P(c_level_layout), vp, vp, vp, P(c_select), vp, vp, vp, vp, vp, sz, vp]
        L.kka_score_topk_workspace.argtypes = [P(c_level_layout), P(c_select), i32]
        L.kka_score_topk_lazy.argtypes = [P(c_level_layout), vp, vp, vp, P(c_select), vp, vp, vp, vp, vp, sz, vp]
        L.kka_score_topk_stable.argtypes = [P(c_level_layout), vp, vp, vp, P(c_select), P(c_stability), vp, vp, vp,
                                            vp, vp, sz, vp]
        L.kka_device_error.argtypes = [vp]
        L.kka_status_string.argtypes = [ctypes.c_int]
        for f in ("kka_pool_blocks", "kka_pool_anchor", "kka_build_levels", "kka_score_topk", "kka_score_topk_lazy",
                  "kka_score_topk_stable", "kka_pool_on_write", "kka_attention_topk", "kka_pool_anchor_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        for f in ("kka_pool_blocks_workspace", "kka_pool_anchor_workspace", "kka_score_topk_workspace",
                  "kka_attention_topk_workspace", "kka_pool_anchor_noalloc_scratch"):
            getattr(L, f).restype = sz
        L.kka_level_rows.restype = i64
        L.kka_device_error.restype = i32
        L.kka_status_string.restype = ctypes.c_char_p
        L.kka_version.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().kka_status_string(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


# ---------------------------------------------------------------- marshalling

def _dev(t: Optional[torch.Tensor], name: str, dtype=None, min_numel: int = 0, allow_none: bool = False):
    """Device pointer of `t` after checking device, dtype and size."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int, what: str):
    if rc != 0:
        raise KkaError(rc, what)


_KEY_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)


class KPool:
    """A paged key pool on the GPU: bf16 bit patterns in `k` (bfloat16, int16
    or uint16 tensor), element (l, p, t, h, d) at
    l*stride_layer + p*stride_block + t*stride_token + h*stride_head + d.
    Strides default to a contiguous [L][P][B][H][D] tensor."""

    def __init__(self, k: torch.Tensor, num_layers: int, num_kv_heads: int, head_dim: int, block_size: int,
                 num_phys_blocks: int, strides: Optional[Sequence[int]] = None):
        L, H, D, B, P = num_layers, num_kv_heads, head_dim, block_size, num_phys_blocks
        if strides is None:
            strides = (P * B * H * D, B * H * D, H * D, D)
        sL, sB, sT, sH = (int(x) for x in strides)
        last = (L - 1) * sL + (P - 1) * sB + (B - 1) * sT + (H - 1) * sH + D
        ptr = _dev(k, "k", _KEY_DTYPES, min_numel=last)
        self.k = k
        self.c = c_kpool(ptr.value, L, H, D, B, P, sL, sB, sT, sH)
        self.num_layers, self.num_kv_heads, self.head_dim, self.block_size, self.num_phys_blocks = L, H, D, B, P


class Seqs:
    """CSR batch: int32 GPU tensors seq_len [S], block_offsets [S+1] and
    block_table [total_blocks]; total_blocks is the host copy of
    block_offsets[S]."""

    def __init__(self, seq_len: torch.Tensor, block_offsets: torch.Tensor, block_table: torch.Tensor,
                 total_blocks: int):
        S = int(seq_len.numel())
        self.tensors = (seq_len, block_offsets, block_table)
        self.c = c_seqs(S, int(total_blocks),
                        _dev(seq_len, "seq_len", torch.int32).value,
                        _dev(block_offsets, "block_offsets", torch.int32, min_numel=S + 1).value,
                        _dev(block_table, "block_table", torch.int32, min_numel=int(total_blocks)).value
                        if total_blocks > 0 else None)
        self.num_seqs, self.total_blocks = S, int(total_blocks)


class LevelLayout:
    """Geometry of a level buffer: per sequence, rows_per_seq rows of head_dim
    fp32 holding pages, then chunks, then grids."""

    def __init__(self, num_seqs: int, max_pages: int, head_dim: int, hierarchical: bool,
                 pages_per_chunk: int = 16, chunks_per_grid: int = 16):
        self.c = c_level_layout(num_seqs, max_pages, head_dim, 1 if hierarchical else 0, pages_per_chunk,
                                chunks_per_grid)
        self.num_seqs, self.max_pages, self.head_dim = num_seqs, max_pages, head_dim
        self.hierarchical = bool(hierarchical)
        self.pages_per_chunk, self.chunks_per_grid = pages_per_chunk, chunks_per_grid
        rows = lib().kka_level_rows(ctypes.byref(self.c))
        if rows < 0:
            raise KkaError(2, "kka_level_rows")
        self.rows_per_seq = int(rows)

    @property
    def chunk_row0(self) -> int:
        return self.max_pages

    @property
    def grid_row0(self) -> int:
        return self.max_pages + -(-self.max_pages // self.pages_per_chunk)

    def new_buffer(self, device="cuda", zero: bool = True) -> torch.Tensor:
        shape = (self.num_seqs, self.rows_per_seq, self.head_dim)
        f = torch.zeros if zero else torch.empty
        return f(shape, dtype=torch.float32, device=device)


def new_workspace(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled byte tensor of at least nbytes (None for 0)."""
    if nbytes <= 0:
        return None
    return torch.zeros(int(nbytes), dtype=torch.uint8, device=device)


def _torch_stream(stream, device) -> Optional[torch.cuda.Stream]:
    """`stream` as a torch stream object when it is not torch's current stream
    on `device` (None when it is, or when stream is None)."""
    if stream is None:
        return None
    cur = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        st = stream
    else:
        st = torch.cuda.ExternalStream(int(stream), device=device)
    return None if st.cuda_stream == cur.cuda_stream else st


def order_after_current(stream, device, *tensors):
    """Makes work enqueued on `stream` start after everything already queued
    on torch's current stream (zero fills, uploads), and tells torch's
    allocator that `tensors` are in use on `stream`, so their memory is not
    handed out again before that work ends.  No-op on the current stream."""
    st = _torch_stream(stream, device)
    if st is None:
        return
    st.wait_stream(torch.cuda.current_stream(device))
    for t in tensors:
        if t is not None:
            t.record_stream(st)


def _ws(ws: Optional[torch.Tensor], need: int, device, stream=None) -> tuple:
    if need <= 0 and ws is None:
        return None, 0, None
    if ws is None:
        # zero-filled on torch's current stream; the call may run on another
        ws = new_workspace(need, device)
        order_after_current(stream, ws.device, ws)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")
    return _dev(ws, "workspace"), ws.numel() * ws.element_size(), ws


# ---------------------------------------------------------------- entry points

def kka_pool_blocks_workspace(kp: KPool, seqs: Seqs, mode: int = WEIGHT_UNIFORM,
                              blocks: Optional[torch.Tensor] = None) -> int:
    nb = 0 if blocks is None else int(blocks.numel())
    bp = None if blocks is None else ctypes.c_void_p(blocks.data_ptr())
    return int(lib().kka_pool_blocks_workspace(ctypes.byref(kp.c), ctypes.byref(seqs.c), bp, nb, int(mode)))


def kka_pool_blocks(kp: KPool, seqs: Seqs, vb_out: torch.Tensor, mode: int = WEIGHT_UNIFORM,
                    head_weight: Optional[torch.Tensor] = None, blocks: Optional[torch.Tensor] = None,
                    vb_seq_stride: int = 0, workspace: Optional[torch.Tensor] = None, stream=None):
    """Block vectors v_b into vb_out (fp32 rows of head_dim)."""
    D, S = kp.head_dim, seqs.num_seqs
    nb = seqs.total_blocks if blocks is None else int(blocks.numel())
    rows = S * vb_seq_stride if vb_seq_stride > 0 else seqs.total_blocks
    outp = _dev(vb_out, "vb_out", torch.float32, min_numel=rows * D, allow_none=nb == 0)
    bp = _dev(blocks, "blocks", torch.int32, allow_none=True)
    hw = _dev(head_weight, "head_weight", torch.float32, min_numel=S * kp.num_layers * kp.num_kv_heads,
              allow_none=mode == WEIGHT_UNIFORM)
    need = kka_pool_blocks_workspace(kp, seqs, mode, blocks)
    wp, wbytes, keep = _ws(workspace, need, vb_out.device if vb_out is not None else "cuda", stream)
    _check(lib().kka_pool_blocks(ctypes.byref(kp.c), ctypes.byref(seqs.c), bp, nb, int(mode), hw, outp,
                                 int(vb_seq_stride), wp, wbytes, _stream(stream)), "kka_pool_blocks")
    return keep


def kka_pool_anchor_workspace(kp: KPool, seqs: Seqs, window: int) -> int:
    return int(lib().kka_pool_anchor_workspace(ctypes.byref(kp.c), ctypes.byref(seqs.c), int(window)))


def kka_pool_anchor(kp: KPool, seqs: Seqs, window: int, anchor_out: torch.Tensor,
                    head_weight: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None):
    """Anchors [S][head_dim] from the last `window` tokens of each sequence."""
    S, D = seqs.num_seqs, kp.head_dim
    ap = _dev(anchor_out, "anchor_out", torch.float32, min_numel=S * D)
    hw = _dev(head_weight, "head_weight", torch.float32, min_numel=S * kp.num_layers * kp.num_kv_heads,
              allow_none=True)
    need = kka_pool_anchor_workspace(kp, seqs, window)
    wp, wbytes, keep = _ws(workspace, need, anchor_out.device, stream)
    _check(lib().kka_pool_anchor(ctypes.byref(kp.c), ctypes.byref(seqs.c), int(window), hw, ap, wp, wbytes,
                                 _stream(stream)), "kka_pool_anchor")
    return keep


def kka_pool_anchor_noalloc_scratch(kp: KPool, seqs: Seqs) -> int:
    return int(lib().kka_pool_anchor_noalloc_scratch(ctypes.byref(kp.c), ctypes.byref(seqs.c)))


def kka_pool_anchor_noalloc(kp: KPool, seqs: Seqs, window: int, anchor_out: torch.Tensor,
                            head_weight: Optional[torch.Tensor] = None, stream=None):
    """kka_pool_anchor without a workspace and without any device allocation
    (the library's fixed per-device scratch array holds the partial sums)."""
    S, D = seqs.num_seqs, kp.head_dim
    ap = _dev(anchor_out, "anchor_out", torch.float32, min_numel=S * D)
    hw = _dev(head_weight, "head_weight", torch.float32, min_numel=S * kp.num_layers * kp.num_kv_heads,
              allow_none=True)
    _check(lib().kka_pool_anchor_noalloc(ctypes.byref(kp.c), ctypes.byref(seqs.c), int(window), hw, ap,
                                         _stream(stream)), "kka_pool_anchor_noalloc")


def kka_pool_on_write(kp: KPool, seqs: Seqs, vb_out: torch.Tensor, running: torch.Tensor, *,
                      new_k: Optional[torch.Tensor] = None, mode: int = WEIGHT_UNIFORM,
                      head_weight: Optional[torch.Tensor] = None, seed: bool = False, vb_seq_stride: int = 0,
                      stream=None):
    """One decode step of pool-on-write: each sequence's newest token
    (seq_len[s] - 1) is stored from new_k [S][L][H][D] (bf16 bits) into the
    pool, or read from it when new_k is None, and its block's vector is
    brought up to date from the running sums [S][D] (seed=True rebuilds
    them from the pool)."""
    S, D, LH = seqs.num_seqs, kp.head_dim, kp.num_layers * kp.num_kv_heads
    nk = _dev(new_k, "new_k", _KEY_DTYPES, min_numel=S * LH * D, allow_none=True)
    hw = _dev(head_weight, "head_weight", torch.float32, min_numel=S * LH, allow_none=mode != WEIGHT_GIVEN)
    rp = _dev(running, "running", torch.float32, min_numel=S * D)
    rows = S * vb_seq_stride if vb_seq_stride else seqs.total_blocks
    vp_ = _dev(vb_out, "vb_out", torch.float32, min_numel=rows * D)
    _check(lib().kka_pool_on_write(ctypes.byref(kp.c), ctypes.byref(seqs.c), nk, int(mode), hw, rp,
                                   1 if seed else 0, vp_, int(vb_seq_stride), _stream(stream)), "kka_pool_on_write")


def kka_attention_topk_workspace(kp: KPool, seqs: Seqs, num_q_heads: int) -> int:
    return int(lib().kka_attention_topk_workspace(ctypes.byref(kp.c), ctypes.byref(seqs.c), int(num_q_heads)))


def kka_attention_topk(kp: KPool, seqs: Seqs, queries: torch.Tensor, num_q_heads: int, block_score_out: torch.Tensor,
                       out_seq_stride: int, *, scale: Optional[float] = None, k: int = 0,
                       idx_out: Optional[torch.Tensor] = None, score_out: Optional[torch.Tensor] = None,
                       n_selected_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None):
    """Attention mass per block for one decode query per sequence
    (queries [S][L][Hq][D] fp32), averaged over layers and query heads, and
    the top-k blocks by it (the page's reference selection)."""
    S, L, D = seqs.num_seqs, kp.num_layers, kp.head_dim
    qp = _dev(queries, "queries", torch.float32, min_numel=S * L * num_q_heads * D)
    op = _dev(block_score_out, "block_score_out", torch.float32, min_numel=S * out_seq_stride)
    ip = _dev(idx_out, "idx_out", torch.int32, min_numel=S * k, allow_none=k == 0)
    sp = _dev(score_out, "score_out", torch.float32, min_numel=S * k, allow_none=True)
    cp = _dev(n_selected_out, "n_selected_out", torch.int32, min_numel=S, allow_none=True)
    need = kka_attention_topk_workspace(kp, seqs, num_q_heads)
    wp, wbytes, keep = _ws(workspace, need, block_score_out.device, stream)
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    _check(lib().kka_attention_topk(ctypes.byref(kp.c), ctypes.byref(seqs.c), qp, int(num_q_heads), sc, int(k), op,
                                    int(out_seq_stride), ip, sp, cp, wp, wbytes, _stream(stream)),
           "kka_attention_topk")
    return keep


def kka_build_levels(lay: LevelLayout, level_buf: torch.Tensor, n_pages: torch.Tensor,
                     first_dirty_page: Optional[torch.Tensor] = None, stream=None):
    """Chunk and grid rows of a hierarchical level buffer (no-op when flat)."""
    S = lay.num_seqs
    lp = _dev(level_buf, "level_buf", torch.float32, min_numel=S * lay.rows_per_seq * lay.head_dim)
    npp = _dev(n_pages, "n_pages", torch.int32, min_numel=S)
    fd = _dev(first_dirty_page, "first_dirty_page", torch.int32, min_numel=S, allow_none=True)
    _check(lib().kka_build_levels(ctypes.byref(lay.c), lp, npp, fd, _stream(stream)), "kka_build_levels")


def kka_score_topk_workspace(lay: LevelLayout, with_affinity_out: bool, k_page: int = 0, k_grid: int = 0,
                             k_chunk: int = 0) -> int:
    """Workspace bytes of a kka_score_topk call (tile counters, plus scratch
    affinities when affinity_out is not given)."""
    sel = c_select(int(k_grid), int(k_chunk), int(k_page))
    return int(lib().kka_score_topk_workspace(ctypes.byref(lay.c), ctypes.byref(sel), 1 if with_affinity_out else 0))


def kka_score_topk(lay: LevelLayout, level_buf: torch.Tensor, n_pages: torch.Tensor, anchors: torch.Tensor, *,
                   k_page: int, k_grid: int = 0, k_chunk: int = 0, page_idx_out: torch.Tensor,
                   page_score_out: Optional[torch.Tensor] = None, n_selected_out: Optional[torch.Tensor] = None,
                   affinity_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None, lazy: bool = False, history: Optional[torch.Tensor] = None,
                   stability_out: Optional[torch.Tensor] = None, window: int = 20, theta: float = 0.5):
    """Affinities of every level row and the top-k pages of each sequence.
    lazy=True: kka_score_topk_lazy (scores only children of kept parents).
    history given: kka_score_topk_stable (uint32 [S][max_pages] window words
    updated in place; stability scores into stability_out when given)."""
    S, D = lay.num_seqs, lay.head_dim
    lp = _dev(level_buf, "level_buf", torch.float32, min_numel=S * lay.rows_per_seq * D)
    npp = _dev(n_pages, "n_pages", torch.int32, min_numel=S)
    anc = _dev(anchors, "anchors", torch.float32, min_numel=S * D)
    idx = _dev(page_idx_out, "page_idx_out", torch.int32, min_numel=S * k_page, allow_none=k_page == 0)
    sc = _dev(page_score_out, "page_score_out", torch.float32, min_numel=S * k_page, allow_none=True)
    cnt = _dev(n_selected_out, "n_selected_out", torch.int32, min_numel=S, allow_none=True)
    aff = _dev(affinity_out, "affinity_out", torch.float32, min_numel=S * lay.rows_per_seq, allow_none=True)
    need = kka_score_topk_workspace(lay, affinity_out is not None, k_page, k_grid, k_chunk)
    wp, wbytes, keep = _ws(workspace, need, level_buf.device, stream)
    sel = c_select(int(k_grid), int(k_chunk), int(k_page))
    if history is not None:
        if lazy:
            raise ValueError("the stability filter needs every page scored: it runs with the single pass only")
        n_words = S * lay.max_pages
        hp = _dev(history, "history", (torch.int32, torch.uint32), min_numel=n_words)
        so = _dev(stability_out, "stability_out", torch.float32, min_numel=n_words, allow_none=True)
        stab = c_stability(hp.value, None if so is None else so.value, int(window), float(theta))
        _check(lib().kka_score_topk_stable(ctypes.byref(lay.c), lp, npp, anc, ctypes.byref(sel), ctypes.byref(stab),
                                           aff, idx, sc, cnt, wp, wbytes, _stream(stream)), "kka_score_topk_stable")
        return keep
    fn = lib().kka_score_topk_lazy if lazy else lib().kka_score_topk
    _check(fn(ctypes.byref(lay.c), lp, npp, anc, ctypes.byref(sel), aff, idx, sc, cnt, wp, wbytes, _stream(stream)),
           "kka_score_topk_lazy" if lazy else "kka_score_topk")
    return keep


def kka_score_topk_lazy(lay: LevelLayout, level_buf: torch.Tensor, n_pages: torch.Tensor, anchors: torch.Tensor,
                        **kw):
    """kka_score_topk_lazy: same arguments and results as kka_score_topk."""
    return kka_score_topk(lay, level_buf, n_pages, anchors, lazy=True, **kw)


def kka_device_error(stream=None) -> int:
    """Waits for the stream and returns (and clears) the device error bits."""
    v = int(lib().kka_device_error(_stream(stream)))
    if v < 0:
        raise KkaError(5, "kka_device_error")
    return v


def version() -> int:
    return int(lib().kka_version())


def kka_score_topk_stable(lay: LevelLayout, level_buf: torch.Tensor, n_pages: torch.Tensor, anchors: torch.Tensor,
                          *, history: torch.Tensor, **kw):
    """kka_score_topk_stable: kka_score_topk plus the fused stability update."""
    return kka_score_topk(lay, level_buf, n_pages, anchors, history=history, **kw)
