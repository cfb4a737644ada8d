"""GPU parity of kka_score_topk_lazy (coarse-to-fine scoring, page section
5.1) against kka_score_topk on the same level buffer and anchors.

The selection (indices, score bits, counts) must be bit-identical.  The
affinities the lazy pass writes must be bit-identical to the full pass's for
exactly the rows it scores -- every grid, the chunks of kept grids, the pages
of kept chunks (kept sets derived here from the full pass's affinities with
the documented order: score descending, index ascending, unscored rows +0)
-- and every other row must be left as it was.  The full pass itself is
checked against the oracle in the other parity tests; here the oracle also
checks the lazy selection of a few sequences directly.
"""
import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth
from kv_cache_block_amd.pipeline import Selector

from gpu_harness import ATOL, check_selection, run_selector, say

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-3.25)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


def top_kept(score, k):
    """Indices of the top min(k, n) entries by (score desc, index asc)."""
    n = len(score)
    k = min(k, n)
    order = np.lexsort((np.arange(n), -score.astype(np.float64)))
    return order[:k]


def scored_rows(aff, lay, cfg, n_p):
    """Row indices (within a sequence) the lazy pass must score."""
    ppc, cpg = cfg["pages_per_chunk"], cfg["chunks_per_grid"]
    n_c = -(-n_p // ppc)
    n_g = -(-n_c // cpg)
    grid = aff[lay.grid_row0:lay.grid_row0 + n_g]
    kept_g = top_kept(grid, cfg["k_grid"])
    cand_c = np.array(sorted(c for g in kept_g for c in range(g * cpg, min(n_c, g * cpg + cpg))), np.int64)
    chunk_score = np.zeros(n_c, np.float32)
    chunk_score[cand_c] = aff[lay.chunk_row0 + cand_c]
    kept_c = top_kept(chunk_score, cfg["k_chunk"])
    cand_p = np.array(sorted(p for c in kept_c for p in range(c * ppc, min(n_p, c * ppc + ppc))), np.int64)
    return np.concatenate([lay.grid_row0 + np.arange(n_g), lay.chunk_row0 + cand_c, cand_p]).astype(np.int64)


def score_both(lay, level, npg, anchors, cfg, with_affinity=True):
    """(full outputs, lazy outputs) as numpy arrays; lazy outputs start as garbage."""
    S = lay.num_seqs
    kq = max(1, cfg["k_page"])
    kw = dict(k_page=cfg["k_page"], k_grid=cfg["k_grid"], k_chunk=cfg["k_chunk"])
    ws = kka.new_workspace(kka.kka_score_topk_workspace(lay, with_affinity))
    full = dict(idx=torch.full((S, kq), -5, dtype=torch.int32, device="cuda"),
                sc=torch.full((S, kq), 9.0, dtype=torch.float32, device="cuda"),
                cnt=torch.full((S,), -5, dtype=torch.int32, device="cuda"),
                aff=torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda"))
    lazy = dict(idx=torch.full((S, kq), 77, dtype=torch.int32, device="cuda"),
                sc=torch.full((S, kq), -4.0, dtype=torch.float32, device="cuda"),
                cnt=torch.full((S,), 77, dtype=torch.int32, device="cuda"),
                aff=torch.full((S, lay.rows_per_seq), float(SENTINEL), dtype=torch.float32, device="cuda"))
    kka.kka_score_topk(lay, level, npg, anchors, page_idx_out=full["idx"], page_score_out=full["sc"],
                       n_selected_out=full["cnt"], affinity_out=full["aff"], workspace=ws, **kw)
    kka.kka_score_topk_lazy(lay, level, npg, anchors, page_idx_out=lazy["idx"], page_score_out=lazy["sc"],
                            n_selected_out=lazy["cnt"], affinity_out=lazy["aff"] if with_affinity else None,
                            workspace=ws, **kw)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in full.items()}, {k: v.cpu().numpy() for k, v in lazy.items()})


def compare(lay, cfg, npg, full, lazy, with_affinity=True, tag=""):
    k = cfg["k_page"]
    np.testing.assert_array_equal(lazy["cnt"], full["cnt"], err_msg=f"{tag} counts")
    if k:
        np.testing.assert_array_equal(lazy["idx"][:, :k], full["idx"][:, :k], err_msg=f"{tag} indices")
        np.testing.assert_array_equal(lazy["sc"][:, :k].view(np.uint32), full["sc"][:, :k].view(np.uint32),
                                      err_msg=f"{tag} scores")
    if not with_affinity:
        assert (lazy["aff"] == SENTINEL).all()
        return
    for s in range(lay.num_seqs):
        n_p = int(npg[s])
        rows = scored_rows(full["aff"][s], lay, cfg, n_p)
        got = lazy["aff"][s]
        np.testing.assert_array_equal(got[rows].view(np.uint32), full["aff"][s][rows].view(np.uint32),
                                      err_msg=f"{tag} scored affinities s={s}")
        untouched = np.ones(lay.rows_per_seq, bool)
        untouched[rows] = False
        assert (got[untouched] == SENTINEL).all(), f"{tag} s={s}: lazy pass wrote rows it must not score"


def random_levels(seed, S, max_pages, D, cfg, lengths, zero_rows=()):
    lay = kka.LevelLayout(S, max_pages, D, True, cfg["pages_per_chunk"], cfg["chunks_per_grid"])
    rng = np.random.default_rng(seed)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    lvl[:, list(zero_rows)] = 0.0
    anchors = rng.standard_normal((S, D), dtype=np.float32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    kka.kka_build_levels(lay, level, npg)
    return lay, level, npg, torch.from_numpy(anchors).cuda()


CASES = [
    dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3),
    dict(hierarchical=1, k_grid=1, k_chunk=1, k_page=40, pages_per_chunk=4, chunks_per_grid=3),   # zero fill
    dict(hierarchical=1, k_grid=0, k_chunk=2, k_page=6, pages_per_chunk=2, chunks_per_grid=2),    # all masked
    dict(hierarchical=1, k_grid=1000, k_chunk=1000, k_page=7, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=1, k_grid=3, k_chunk=20, k_page=300, pages_per_chunk=64, chunks_per_grid=4),
    dict(hierarchical=1, k_grid=8, k_chunk=40, k_page=900, pages_per_chunk=32, chunks_per_grid=8),
    dict(hierarchical=1, k_grid=7, k_chunk=28, k_page=500, pages_per_chunk=16, chunks_per_grid=8),
    dict(hierarchical=1, k_grid=4, k_chunk=16, k_page=64, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=1, k_grid=4, k_chunk=16, k_page=0, pages_per_chunk=16, chunks_per_grid=16),
]


@pytest.mark.parametrize("cfg", CASES)
def test_lazy_equals_full_ragged(cfg):
    """Ragged lengths (0, a tail page, exact multiples, the maximum)."""
    say(f"lazy ragged {cfg}")
    max_pages = 2300
    lengths = [0, 1, 17, cfg["pages_per_chunk"] * cfg["chunks_per_grid"], 999, max_pages]
    lay, level, npg, anchors = random_levels(21, len(lengths), max_pages, 64, cfg, lengths, zero_rows=(3, 40))
    full, lazy = score_both(lay, level, npg, anchors, cfg)
    compare(lay, cfg, npg.cpu().numpy(), full, lazy, tag=str(cfg))
    full2, lazy2 = score_both(lay, level, npg, anchors, cfg, with_affinity=False)
    compare(lay, cfg, npg.cpu().numpy(), full2, lazy2, with_affinity=False, tag=str(cfg))


@pytest.mark.parametrize("cfg", [CASES[3], CASES[5], CASES[7]])
def test_lazy_equals_full_rows_beyond_lds(cfg):
    """Sequences with more level rows than the selecting group keeps in LDS
    (scored affinities then go through the affinity buffer)."""
    say(f"lazy long {cfg}")
    max_pages = 12000
    lengths = [12000, 9300, 5]
    lay, level, npg, anchors = random_levels(22, 3, max_pages, 128, cfg, lengths)
    assert lay.rows_per_seq > 9216
    full, lazy = score_both(lay, level, npg, anchors, cfg)
    compare(lay, cfg, npg.cpu().numpy(), full, lazy, tag="long")
    full2, lazy2 = score_both(lay, level, npg, anchors, cfg, with_affinity=False)
    compare(lay, cfg, npg.cpu().numpy(), full2, lazy2, with_affinity=False, tag="long")


@pytest.mark.parametrize("D", [8, 24, 256, 520, 1024])
def test_lazy_equals_full_head_dims(D):
    """Both passes at head dims that take every lane layout (8 lanes per row
    up to 512, 16 above); the full pass also against the oracle."""
    cfg = dict(hierarchical=1, k_grid=3, k_chunk=9, k_page=33, pages_per_chunk=8, chunks_per_grid=4)
    say(f"lazy head_dim {D}")
    lengths = [400, 129, 64]
    lay, level, npg, anchors = random_levels(23, 3, 400, D, cfg, lengths)
    full, lazy = score_both(lay, level, npg, anchors, cfg)
    compare(lay, cfg, npg.cpu().numpy(), full, lazy, tag=f"D={D}")
    lv, an = level.cpu().numpy(), anchors.cpu().numpy()
    for s, n_p in enumerate(lengths):
        n_c = -(-n_p // 8)
        n_g = -(-n_c // 4)
        rows = np.concatenate([np.arange(n_p), lay.chunk_row0 + np.arange(n_c), lay.grid_row0 + np.arange(n_g)])
        np.testing.assert_allclose(full["aff"][s][rows], oracle.affinity(lv[s][rows], an[s]), atol=ATOL, rtol=0,
                                   err_msg=f"D={D} s={s}")
        a = full["aff"][s]
        ridx, rsc = oracle.select(a[:n_p], a[lay.chunk_row0:lay.chunk_row0 + n_c],
                                  a[lay.grid_row0:lay.grid_row0 + n_g], hierarchical=1, k_grid=3, k_chunk=9,
                                  k_page=33, pages_per_chunk=8, chunks_per_grid=4)
        assert full["cnt"][s] == len(ridx)
        np.testing.assert_array_equal(full["idx"][s][:len(ridx)], ridx)
        np.testing.assert_array_equal(full["sc"][s][:len(ridx)].view(np.uint32), rsc.view(np.uint32))


def test_lazy_exact_ties():
    """Integer-valued page vectors: exact ties and exact 0 / 0.5 / 1 scores."""
    say("lazy ties")
    S, n_p, D = 3, 300, 8
    cfg = dict(hierarchical=1, k_grid=3, k_chunk=30, k_page=64, pages_per_chunk=4, chunks_per_grid=5)
    lay = kka.LevelLayout(S, 320, D, True, 4, 5)
    rng = np.random.default_rng(9)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :n_p] = rng.integers(-1, 2, (S, n_p, D)).astype(np.float32)
    anchors = np.zeros((S, D), np.float32)
    anchors[:, 0] = 1.0
    level = torch.from_numpy(lvl).cuda()
    npg = torch.full((S,), n_p, dtype=torch.int32, device="cuda")
    kka.kka_build_levels(lay, level, npg)
    full, lazy = score_both(lay, level, npg, torch.from_numpy(anchors).cuda(), cfg)
    compare(lay, cfg, npg.cpu().numpy(), full, lazy, tag="ties")


def test_lazy_flat_layout_is_the_full_pass():
    cfg = dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=50, pages_per_chunk=16, chunks_per_grid=16)
    say("lazy flat")
    lay = kka.LevelLayout(2, 700, 64, False, 16, 16)
    rng = np.random.default_rng(5)
    level = torch.from_numpy(rng.standard_normal((2, 700, 64), dtype=np.float32)).cuda()
    npg = torch.tensor([700, 321], dtype=torch.int32, device="cuda")
    anchors = torch.from_numpy(rng.standard_normal((2, 64), dtype=np.float32)).cuda()
    full, lazy = score_both(lay, level, npg, anchors, cfg)
    np.testing.assert_array_equal(lazy["idx"], full["idx"])
    np.testing.assert_array_equal(lazy["sc"].view(np.uint32), full["sc"].view(np.uint32))
    np.testing.assert_array_equal(lazy["cnt"], full["cnt"])
    for s, n in enumerate((700, 321)):
        np.testing.assert_array_equal(lazy["aff"][s, :n].view(np.uint32), full["aff"][s, :n].view(np.uint32))


def test_lazy_selector_end_to_end_against_oracle():
    """Whole path from a key pool with the lazy scoring step; the lazy
    selection is checked against the oracle directly (selection on the
    full pass's affinities, which the lazy pass reproduces bit for bit)."""
    say("lazy selector end to end")
    w = synth.config1(0)
    w.select = dict(hierarchical=1, k_grid=2, k_chunk=6, k_page=24, pages_per_chunk=4, chunks_per_grid=4)
    sel, npg = run_selector(w)
    full_idx = sel.page_idx.clone()
    lazy_sel = Selector(sel.kp, sel.seqs, w.select, max_pages=sel.lay.max_pages, window=w.window,
                        keep_affinity=True)
    lazy_sel.level.copy_(sel.level)
    lazy_sel.anchors.copy_(sel.anchors)
    lazy_sel.score(npg, lazy=True)
    torch.cuda.synchronize()
    assert torch.equal(lazy_sel.page_idx, full_idx)
    # oracle check on the full affinities, then the lazy outputs are the same
    lazy_sel.affinity.copy_(sel.affinity)
    for s in range(w.S):
        check_selection(lazy_sel, s, int(npg[s]), tag="lazy")


def test_lazy_full_size_serving_batch():
    """64 sequences x 8192 pages x 128, the serving-scale decode batch."""
    say("lazy serving batch 64 x 8192")
    v = synth.config4(0)
    S, n_p, D = v.vb.shape
    lay = kka.LevelLayout(S, n_p, D, True, 16, 16)
    level = lay.new_buffer()
    level[:, :n_p] = torch.from_numpy(v.vb).cuda()
    npg = torch.full((S,), n_p, dtype=torch.int32, device="cuda")
    kka.kka_build_levels(lay, level, npg)
    full, lazy = score_both(lay, level, npg, torch.from_numpy(v.anchors).cuda(), v.select)
    compare(lay, v.select, npg.cpu().numpy(), full, lazy, tag="c4")
    for s in range(S):
        assert (v.page_topic[s][lazy["idx"][s]] == v.anchor_topic[s]).all()
