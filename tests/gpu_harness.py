"""Shared plumbing of the GPU parity tests: upload a synthetic workload, run
the library, pull results back, and compare stage by stage with the oracle.

Tolerances (fp32 accumulation on the GPU against fp64 sums rounded once in
the oracle): block vectors, anchors, level vectors and affinities within
1e-5 absolute; head weights within 1e-6 relative; selected indices and
their scores bit-exact when the oracle selects on the GPU's own
affinities.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import kv_cache_block_amd as kka
import oracle
from kv_cache_block_amd.pipeline import Selector

ATOL = 1e-5
WEIGHT_RTOL = 1e-6


def say(msg: str):
    """Progress line that pytest does not hold back (names the case before GPU work)."""
    from conftest import progress
    progress(f"[gpu] {msg}")


def upload(w, device="cuda"):
    """(KPool, Seqs, tensors) of a synth KWorkload."""
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(device)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    sl = torch.from_numpy(np.ascontiguousarray(w.seq_len, dtype=np.int32)).to(device)
    off = torch.from_numpy(np.ascontiguousarray(w.block_offsets, dtype=np.int32)).to(device)
    tab = torch.from_numpy(np.ascontiguousarray(w.block_table, dtype=np.int32)).to(device)
    seqs = kka.Seqs(sl, off, tab, w.total_blocks)
    return kp, seqs


def n_pages_of(w, device="cuda"):
    return torch.from_numpy(np.diff(w.block_offsets).astype(np.int32)).to(device)


def mode_of(w):
    return kka.WEIGHT_VARIANCE if w.mode == "variance" else kka.WEIGHT_UNIFORM


def run_selector(w, device="cuda", mode=None, keep_affinity=True):
    kp, seqs = upload(w, device)
    sel = Selector(kp, seqs, w.select, max_pages=max(1, w.max_pages()), window=w.window,
                   mode=mode_of(w) if mode is None else mode, keep_affinity=keep_affinity, device=device)
    npg = n_pages_of(w, device)
    sel.step(npg)
    torch.cuda.synchronize()
    return sel, npg


def check_selection(sel: Selector, s: int, n_p: int, tag: str = ""):
    """Levels and affinities of sequence s against the oracle run on the
    GPU's own page vectors and anchor; top-K against the oracle's selection
    on the GPU's own affinities (bit-exact)."""
    lay = sel.lay
    cfg = sel.sel
    pages = sel.pages(s, n_p).cpu().numpy()
    anchor = sel.anchors[s].cpu().numpy()
    aff_row = sel.affinity[s].cpu().numpy()
    gpu_aff_pages = aff_row[:n_p]
    if cfg["hierarchical"]:
        ppc, cpg = cfg["pages_per_chunk"], cfg["chunks_per_grid"]
        n_c = -(-n_p // ppc)
        n_g = -(-n_c // cpg)
        oc, og = oracle.build_levels(pages, ppc, cpg) if n_p else (np.zeros((0, lay.head_dim), np.float32),) * 2
        gc = sel.chunks(s, n_c).cpu().numpy()
        gg = sel.grids(s, n_g).cpu().numpy()
        np.testing.assert_allclose(gc, oc, atol=ATOL, rtol=0, err_msg=f"{tag} chunks s={s}")
        np.testing.assert_allclose(gg, og, atol=ATOL, rtol=0, err_msg=f"{tag} grids s={s}")
        gpu_aff_chunks = aff_row[lay.chunk_row0:lay.chunk_row0 + n_c]
        gpu_aff_grids = aff_row[lay.grid_row0:lay.grid_row0 + n_g]
        np.testing.assert_allclose(gpu_aff_chunks, oracle.affinity(gc, anchor), atol=ATOL, rtol=0)
        np.testing.assert_allclose(gpu_aff_grids, oracle.affinity(gg, anchor), atol=ATOL, rtol=0)
    else:
        gpu_aff_chunks = gpu_aff_grids = None
    if n_p:
        np.testing.assert_allclose(gpu_aff_pages, oracle.affinity(pages, anchor), atol=ATOL, rtol=0,
                                   err_msg=f"{tag} page affinities s={s}")
    assert not np.signbit(aff_row[:n_p]).any()
    idx_ref, sc_ref = oracle.select(gpu_aff_pages, gpu_aff_chunks, gpu_aff_grids,
                                    hierarchical=cfg["hierarchical"], k_grid=cfg.get("k_grid", 0),
                                    k_chunk=cfg.get("k_chunk", 0), k_page=cfg["k_page"],
                                    pages_per_chunk=cfg.get("pages_per_chunk", 16),
                                    chunks_per_grid=cfg.get("chunks_per_grid", 16))
    k_eff = len(idx_ref)
    got_idx = sel.page_idx[s].cpu().numpy()
    got_sc = sel.page_score[s].cpu().numpy()
    assert int(sel.n_selected[s].item()) == k_eff, f"{tag} count s={s}"
    np.testing.assert_array_equal(got_idx[:k_eff], idx_ref, err_msg=f"{tag} top-K s={s}")
    np.testing.assert_array_equal(got_sc[:k_eff].view(np.uint32), sc_ref.view(np.uint32))
    if cfg["k_page"] > k_eff:
        assert (got_idx[k_eff:cfg["k_page"]] == -1).all()
        assert (got_sc[k_eff:cfg["k_page"]] == 0).all()
    return idx_ref


def check_end_to_end(sel: Selector, s: int, pages_ref: np.ndarray, anchor_ref: np.ndarray, tag: str = "") -> int:
    """The oracle's own selection of sequence s, from its own block vectors
    and anchor (levels, affinities and top-K all in the oracle), against the
    GPU's: the same count, and the selected scores equal position by
    position within ATOL, so selected indices can differ only between
    blocks whose scores do.  Returns the number of positions whose indices
    differ."""
    cfg = sel.sel
    n_p = len(pages_ref)
    D = sel.lay.head_dim
    ac = ag = None
    if cfg["hierarchical"]:
        ppc, cpg = cfg["pages_per_chunk"], cfg["chunks_per_grid"]
        oc, og = oracle.build_levels(pages_ref, ppc, cpg) if n_p else (np.zeros((0, D), np.float32),) * 2
        ac, ag = oracle.affinity(oc, anchor_ref), oracle.affinity(og, anchor_ref)
    ap = oracle.affinity(pages_ref, anchor_ref)
    idx, sc = oracle.select(ap, ac, ag, hierarchical=cfg["hierarchical"], k_grid=cfg.get("k_grid", 0),
                            k_chunk=cfg.get("k_chunk", 0), k_page=cfg["k_page"],
                            pages_per_chunk=cfg.get("pages_per_chunk", 16), chunks_per_grid=cfg.get("chunks_per_grid", 16))
    k_eff = len(idx)
    assert int(sel.n_selected[s].item()) == k_eff, f"{tag} end-to-end count s={s}"
    got_idx = sel.page_idx[s].cpu().numpy()[:k_eff]
    got_sc = sel.page_score[s].cpu().numpy()[:k_eff]
    np.testing.assert_allclose(got_sc, sc, atol=ATOL, rtol=0, err_msg=f"{tag} end-to-end scores s={s}")
    return int((got_idx != idx).sum())


def oracle_vb(w, blocks, weights=None):
    kp = oracle.KPool.of(w)
    return oracle.pool_blocks(kp, w.seq_len, w.block_offsets, w.block_table, weights, blocks=set(blocks))


def host_threads() -> int:
    """Worker threads for the oracle at full size: the cores this process may
    run on, at most 16 (the GPU host's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pmap(fn, items):
    """[fn(x) for x in items] on host_threads() threads.  The oracle's C
    calls run without Python's lock, so independent blocks and sequences
    pool in parallel; each call is the unchanged single-threaded oracle."""
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        return list(ex.map(fn, items, chunksize=max(1, len(items) // (8 * host_threads()))))


def oracle_vb_all(w, weights=None, seq_len=None, block_offsets=None, block_table=None) -> np.ndarray:
    """Oracle v_b of every logical block [total_blocks][D], in parallel.
    weights: None (uniform) or [S][L*H]; the CSR arrays default to w's."""
    kp = oracle.KPool.of(w)
    T = w.seq_len if seq_len is None else seq_len
    off = w.block_offsets if block_offsets is None else block_offsets
    tab = w.block_table if block_table is None else block_table
    S = len(T)
    seq_of = np.repeat(np.arange(S), np.diff(off))

    def one(b):
        s = int(seq_of[b])
        i = b - int(off[s])
        return oracle.pool_block(kp, int(tab[b]), oracle.n_valid(T, kp.B, i, s),
                                 None if weights is None else weights[s])
    n = int(off[-1])
    return np.stack(pmap(one, range(n))) if n else np.zeros((0, w.D), np.float32)


def oracle_weights_all(w, seq_len=None, block_offsets=None, block_table=None) -> np.ndarray:
    """Oracle head weights [S][L*H] of every sequence, in parallel."""
    kp = oracle.KPool.of(w)
    T = w.seq_len if seq_len is None else seq_len
    off = w.block_offsets if block_offsets is None else block_offsets
    tab = w.block_table if block_table is None else block_table
    rows = pmap(lambda s: oracle.head_weights(kp, oracle.seq_table(off, tab, s), int(T[s])), range(len(T)))
    return np.stack(rows)


def oracle_anchors_all(w, weights=None, seq_len=None, block_offsets=None, block_table=None) -> np.ndarray:
    """Oracle anchors [S][D] of every sequence, in parallel."""
    kp = oracle.KPool.of(w)
    T = w.seq_len if seq_len is None else seq_len
    off = w.block_offsets if block_offsets is None else block_offsets
    tab = w.block_table if block_table is None else block_table
    rows = pmap(lambda s: oracle.pool_anchor(kp, oracle.seq_table(off, tab, s), int(T[s]), w.window,
                                             None if weights is None else weights[s]), range(len(T)))
    return np.stack(rows)


def assert_rows_close(got: np.ndarray, ref: np.ndarray, what: str, atol: float = ATOL):
    """Element-wise |got - ref| <= atol over every row; names the worst row."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    if got.size == 0:
        return
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    if not (err <= atol).all() or not np.isfinite(got).all():
        r = int(np.unravel_index(np.nanargmax(np.where(np.isfinite(err), err, np.inf)), err.shape)[0])
        raise AssertionError(f"{what}: row {r} max abs error {float(np.max(err[r])):.3e} > {atol:g} "
                             f"({int((err > atol).any(axis=-1).sum())} rows over)")
