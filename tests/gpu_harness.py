"""Shared plumbing of the GPU parity tests: upload a synthetic workload, run
the library, pull results back, and compare stage by stage with the oracle.

Tolerances (fp32 accumulation on the GPU against fp64 sums rounded once in
the oracle): block vectors, anchors, level vectors and affinities within
1e-5 absolute; head weights within 1e-6 relative; selected indices and
their scores bit-exact when the oracle selects on the GPU's own
affinities.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import kv_cache_block_amd as kka
import oracle
from kv_cache_block_amd.pipeline import Selector

ATOL = 1e-5
WEIGHT_RTOL = 1e-6


def say(msg: str):
    """Progress line that pytest does not capture (names the case before GPU work)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


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


def oracle_vb(w, blocks, weights=None):
    kp = oracle.KPool.of(w)
    return oracle.pool_blocks(kp, w.seq_len, w.block_offsets, w.block_table, weights, blocks=set(blocks))
