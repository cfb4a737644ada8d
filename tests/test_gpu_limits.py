"""GPU parity at the documented size limits.

Pooling at head_dim 1024 with 1024 threads per group (8 KV heads), and at
4096 (layer, KV head) pairs, uniform and variance-weighted; selection with
k = 1024 at every level of a hierarchy of 16384 chunks (the largest parent
count a selecting group tracks), full, lazy and stability-filtered passes.
Tolerances and selection checks as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle

from gpu_harness import ATOL, WEIGHT_RTOL, run_selector, say
from test_gpu_parity import ragged_workload, vb_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


@pytest.mark.parametrize("shape,mode", [
    ((2, 2, 8, 1024, 4, 9, 30), "uniform"),     # 8 heads x 128 pieces = 1024 threads per token row
    ((2, 2, 8, 1024, 4, 9, 30), "variance"),
    ((2, 1024, 4, 8, 2, 3, 9), "uniform"),      # 4096 (layer, head) pairs, the largest
    ((2, 1024, 4, 8, 2, 3, 9), "variance"),
])
def test_pool_at_limits(shape, mode):
    S, L, H, D, B, lo, hi = shape
    say(f"pool limits {shape} {mode}")
    w = ragged_workload(80, S, L, H, D, B, lo, hi, mode=mode, offset=0.5 if mode == "variance" else 0.0)
    sel, _ = run_selector(w)
    okp = oracle.KPool.of(w)
    weights = None
    if mode == "variance":
        weights = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
        got_w = sel.head_weight.cpu().numpy()
        np.testing.assert_allclose(got_w, weights, rtol=WEIGHT_RTOL, atol=1e-9)
        weights = got_w  # the frozen fp32 weights the GPU pooled with
    got = vb_rows(sel, w)
    ref = oracle.pool_blocks(okp, w.seq_len, w.block_offsets, w.block_table, weights)
    for b, v in ref.items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")


def _max_levels(seed, S, D, ppc, cpg, n_pages):
    lay = kka.LevelLayout(S, max(n_pages), D, True, ppc, cpg)
    rng = np.random.default_rng(seed)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :lay.max_pages] = rng.standard_normal((S, lay.max_pages, D)).astype(np.float32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.tensor(n_pages, dtype=torch.int32, device="cuda")
    kka.kka_build_levels(lay, level, npg)
    anchors = torch.from_numpy(rng.standard_normal((S, D)).astype(np.float32)).cuda()
    return lay, level, npg, anchors


def test_selection_k1024_at_every_level_of_the_largest_hierarchy():
    """16384 chunks of 4 pages (65536 pages), grids of 4 chunks; k = 1024 at
    each level, so the chunk and page levels select from 4096 candidates."""
    say("selection limits: 65536 pages, k 1024/1024/1024")
    ppc, cpg, D = 4, 4, 8
    n_pages = [65536, 40001]
    lay, level, npg, anchors = _max_levels(81, 2, D, ppc, cpg, n_pages)
    S, K = 2, 1024
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, K), dtype=torch.float32, device="cuda")
    cnt = torch.zeros(S, dtype=torch.int32, device="cuda")
    aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
    kw = dict(k_page=K, k_grid=K, k_chunk=K)
    kka.kka_score_topk(lay, level, npg, anchors, page_idx_out=idx, page_score_out=sc, n_selected_out=cnt,
                       affinity_out=aff, **kw)
    torch.cuda.synchronize()
    lv, an, af = level.cpu().numpy(), anchors.cpu().numpy(), aff.cpu().numpy()
    for s, n_p in enumerate(n_pages):
        n_c = -(-n_p // ppc)
        n_g = -(-n_c // cpg)
        a_pages = af[s, :n_p]
        a_chunks = af[s, lay.chunk_row0:lay.chunk_row0 + n_c]
        a_grids = af[s, lay.grid_row0:lay.grid_row0 + n_g]
        np.testing.assert_allclose(a_pages, oracle.affinity(lv[s, :n_p], an[s]), atol=ATOL, rtol=0)
        np.testing.assert_allclose(a_grids, oracle.affinity(lv[s, lay.grid_row0:lay.grid_row0 + n_g], an[s]),
                                   atol=ATOL, rtol=0)
        ridx, rsc = oracle.select(a_pages, a_chunks, a_grids, hierarchical=1, k_grid=K, k_chunk=K, k_page=K,
                                  pages_per_chunk=ppc, chunks_per_grid=cpg)
        assert int(cnt[s]) == len(ridx) == K
        np.testing.assert_array_equal(idx[s].cpu().numpy(), ridx)
        np.testing.assert_array_equal(sc[s].cpu().numpy().view(np.uint32), rsc.view(np.uint32))
    # the lazy pass and the stability-filtered pass select the same pages
    for variant in ("lazy", "stable"):
        idx2 = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
        sc2 = torch.zeros((S, K), dtype=torch.float32, device="cuda")
        extra = dict(lazy=True) if variant == "lazy" else dict(
            history=torch.zeros((S, lay.max_pages), dtype=torch.int32, device="cuda"), window=32, theta=0.5)
        kka.kka_score_topk(lay, level, npg, anchors, page_idx_out=idx2, page_score_out=sc2, **kw, **extra)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx), variant
        assert torch.equal(sc2.view(torch.int32), sc.view(torch.int32)), variant
