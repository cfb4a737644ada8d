"""GPU parity: the HIP library (called through the C ABI) against the CPU
oracle on the same seeded inputs, stage by stage.  Small cases span several
work-groups, layer splits and ragged tails; edge cases cover empty
sequences, k larger than the level, k = 0, exact ties and masked fills."""
import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth
from kv_cache_block_amd.pipeline import Selector

from gpu_harness import (ATOL, WEIGHT_RTOL, assert_rows_close, check_end_to_end, check_selection, host_threads, mode_of,
                         n_pages_of, oracle_anchors_all, oracle_vb, oracle_vb_all, oracle_weights_all, run_selector, say,
                         upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()  # raises loudly when the library is missing
    yield
    assert kka.kka_device_error() == 0


def ragged_workload(seed, S, L, H, D, B, len_lo, len_hi, mode="uniform", select=None, window=16, noise=1.0,
                    offset=0.0, lengths=None):
    """Random ragged batch over a permuted shared pool (keys N(offset, noise))."""
    if lengths is None:
        T = synth.uniform_int(seed, 101, S, len_lo, len_hi).astype(np.int32)
    else:
        T = np.asarray(lengths, dtype=np.int32)
        S = len(T)
    nb = (T + B - 1) // B
    off = np.zeros(S + 1, np.int32)
    off[1:] = np.cumsum(nb)
    P = int(off[-1]) + 3  # a few physical blocks nobody uses
    table = synth.permutation(seed, 102, P)[:off[-1]].astype(np.int32)
    std = np.full(L * H, noise, np.float32)
    bias = np.full((L, H, D), offset, np.float32) if offset else None
    k = synth._gen_kpool(L, H, D, B, P, T, off, table, None, None, 0.0, 0.0, std, bias, seed)
    sel = select or {"hierarchical": 0, "k_grid": 0, "k_chunk": 0, "k_page": 8, "pages_per_chunk": 4,
                     "chunks_per_grid": 3}
    return synth.KWorkload(name="ragged", L=L, H=H, D=D, B=B, P=P, k=k, seq_len=T, block_offsets=off,
                           block_table=table, window=window, mode=mode, select=sel, seed=seed)


def vb_rows(sel, w):
    out = {}
    lvl = sel.level.cpu().numpy()
    for s in range(w.S):
        for i in range(int(w.block_offsets[s + 1] - w.block_offsets[s])):
            out[int(w.block_offsets[s]) + i] = lvl[s, i]
    return out


# ------------------------------------------------------------------ pooling

POOL_SHAPES = [
    # (S, L, H, D, B, len_lo, len_hi)
    (3, 4, 4, 128, 16, 1, 200),      # ragged tails, splits over layers
    (2, 3, 2, 64, 16, 100, 700),
    (4, 5, 3, 24, 7, 1, 90),         # odd head count / width: 9 threads per token row
    (1, 2, 1, 256, 33, 500, 500),
    (2, 2, 16, 512, 4, 30, 60),      # 1024 threads per group
]


@pytest.mark.parametrize("shape", POOL_SHAPES)
def test_pool_uniform_matches_oracle(shape):
    S, L, H, D, B, lo, hi = shape
    say(f"pool uniform {shape}")
    w = ragged_workload(1, S, L, H, D, B, lo, hi)
    sel, _ = run_selector(w)
    got = vb_rows(sel, w)
    ref = oracle_vb(w, range(w.total_blocks))
    for b, v in ref.items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")


@pytest.mark.parametrize("mode", ["uniform", "given"])
def test_xcd_shares_pool_every_block_once(mode, monkeypatch):
    """A launch of at least 2048 blocks gives XCD x (work-group i mod 8) a
    contiguous range of blocks sized by a weight per XCD (KKA_XCD_WEIGHTS;
    on MI355X 1.1 for even and 1.0 for odd XCDs by default), and groups past
    their XCD's range pool nothing.  Default, equal, uneven and extreme
    weights, the shares off, and malformed values (the default then) all give
    every block vector the same bits, no row is left unwritten, and a sample
    of blocks matches the oracle."""
    say(f"xcd shares {mode}")
    w = ragged_workload(11, 7, 2, 2, 64, 16, 5000, 8000)
    assert w.total_blocks >= 2048
    kp, seqs = upload(w)
    S, LH = w.S, w.L * w.H
    hw = None
    if mode == "given":
        raw = synth.uniform(11, 104, S * LH).reshape(S, LH).astype(np.float64) + 0.1
        hw = (raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
    hw_t = torch.from_numpy(hw).cuda() if hw is not None else None
    kmode = kka.WEIGHT_GIVEN if mode == "given" else kka.WEIGHT_UNIFORM
    outs = {}
    for setting in ("off", None, "1,1,1,1,1,1,1,1", "1,2,3,4,5,6,7,8", "8,0.5,1,1,1,1,1,20", "1,2", "x", "0,1,1,1,1,1,1,1"):
        if setting is None:
            monkeypatch.delenv("KKA_XCD_WEIGHTS", raising=False)
        else:
            monkeypatch.setenv("KKA_XCD_WEIGHTS", setting)
        out = torch.full((w.total_blocks, w.D), 7.0, dtype=torch.float32, device="cuda")
        kka.kka_pool_blocks(kp, seqs, out, mode=kmode, head_weight=hw_t)
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        outs[setting] = out.cpu().numpy()
    ref = outs["off"]
    assert not (ref == 7.0).all(axis=1).any()
    for setting, o in outs.items():
        np.testing.assert_array_equal(o.view(np.uint32), ref.view(np.uint32), err_msg=f"KKA_XCD_WEIGHTS={setting}")
    sample = sorted(set(synth.uniform_int(11, 105, 48, 0, w.total_blocks - 1).tolist()) | {0, w.total_blocks - 1})
    want = oracle_vb(w, sample, hw)
    for b in sample:
        np.testing.assert_allclose(outs[None][b], want[b], atol=ATOL, rtol=0, err_msg=f"block {b}")


@pytest.mark.parametrize("shape", POOL_SHAPES)
def test_pool_variance_weights_match_oracle(shape):
    S, L, H, D, B, lo, hi = shape
    say(f"pool variance {shape}")
    w = ragged_workload(2, S, L, H, D, B, lo, hi, mode="variance", offset=0.75)
    # distinct head scales so the weights are far from uniform
    sc = synth.uniform(2, 103, L * H).astype(np.float32) * 3 + 0.2
    f = synth.bf16_bits_to_f32(w.k).reshape(L, w.P, B, H, D) * sc.reshape(L, 1, 1, H, 1)
    w.k = synth.to_bf16_bits(f)
    sel, _ = run_selector(w)
    okp = oracle.KPool.of(w)
    wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
    wgpu = sel.head_weight.cpu().numpy()
    np.testing.assert_allclose(wgpu, wref, rtol=WEIGHT_RTOL, atol=0)
    got = vb_rows(sel, w)
    ref = oracle_vb(w, range(w.total_blocks), wref)
    for b, v in ref.items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")
    anc = sel.anchors.cpu().numpy()
    for s in range(w.S):
        a = oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]),
                               w.window, wref[s])
        np.testing.assert_allclose(anc[s], a, atol=ATOL, rtol=0)


def test_pool_physical_permutation_is_bitwise_invariant():
    say("pool permutation invariance")
    w = ragged_workload(3, 2, 4, 4, 128, 16, 300, 600)
    sel0, _ = run_selector(w)
    v0 = vb_rows(sel0, w)
    a0 = sel0.anchors.cpu().numpy()
    # move every block to another physical slot, content unchanged
    perm = synth.permutation(3, 104, w.P)
    k = w.k.reshape(w.L, w.P, -1)
    moved = np.empty_like(k)
    moved[:, perm] = k
    w2 = synth.KWorkload(**{**w.__dict__, "k": moved.reshape(w.k.shape),
                            "block_table": perm[w.block_table].astype(np.int32)})
    sel1, _ = run_selector(w2)
    v1 = vb_rows(sel1, w2)
    for b in v0:
        np.testing.assert_array_equal(v0[b].view(np.uint32), v1[b].view(np.uint32))
    np.testing.assert_array_equal(a0.view(np.uint32), sel1.anchors.cpu().numpy().view(np.uint32))


def test_pool_token_order_within_block():
    say("pool token order")
    w = ragged_workload(4, 1, 3, 4, 128, 16, 160, 160)
    sel0, _ = run_selector(w)
    v0 = vb_rows(sel0, w)
    k = w.k.reshape(w.L, w.P, w.B, -1).copy()
    rng = np.random.default_rng(0)
    for p in range(w.P):
        k[:, p] = k[:, p][:, rng.permutation(w.B)]
    w2 = synth.KWorkload(**{**w.__dict__, "k": k.reshape(w.k.shape)})
    sel1, _ = run_selector(w2)
    v1 = vb_rows(sel1, w2)
    for b in v0:
        np.testing.assert_allclose(v0[b], v1[b], atol=1e-6, rtol=0)


def test_pool_is_deterministic():
    say("pool determinism")
    w = ragged_workload(5, 3, 4, 4, 128, 16, 10, 900, mode="variance")
    s0, _ = run_selector(w)
    s1, _ = run_selector(w)
    assert torch.equal(s0.level, s1.level)
    assert torch.equal(s0.head_weight, s1.head_weight)
    assert torch.equal(s0.affinity, s1.affinity)


def test_incremental_repool_equals_scratch():
    """Append one token per sequence, re-pool only each sequence's newest
    block with the frozen weights: equals pooling that block from scratch
    (oracle) and the GPU's full pool with the same weights."""
    say("incremental repool")
    w = synth.config5(6, n_seqs=5, len_lo=60, len_hi=400, L=3, H=4, D=128, B=16)
    after = w.extra["after"]
    kp, seqs_before = upload(w)
    sel = Selector(kp, seqs_before, w.select, max_pages=int(np.max(np.diff(after["block_offsets"]))),
                   window=w.window, mode=kka.WEIGHT_VARIANCE)
    sel.pool()
    frozen = sel.head_weight.clone()
    # state after the append
    dev = "cuda"
    seqs_after = kka.Seqs(torch.from_numpy(after["seq_len"]).to(dev),
                          torch.from_numpy(after["block_offsets"]).to(dev),
                          torch.from_numpy(after["block_table"]).to(dev), int(after["block_offsets"][-1]))
    sel.seqs = seqs_after
    newest = (after["block_offsets"][1:] - 1).astype(np.int32)
    sel.repool(torch.from_numpy(newest).to(dev))
    torch.cuda.synchronize()
    assert torch.equal(sel.head_weight, frozen)
    lvl = sel.level.cpu().numpy()
    okp = oracle.KPool.of(w)
    wf = frozen.cpu().numpy()
    full = torch.zeros_like(sel.level)
    kka.kka_pool_blocks(kp, seqs_after, full, mode=kka.WEIGHT_GIVEN, head_weight=frozen,
                        vb_seq_stride=sel.lay.rows_per_seq)
    full = full.cpu().numpy()
    for s in range(w.S):
        i = int(newest[s] - after["block_offsets"][s])
        n_b = int(after["seq_len"][s]) - i * w.B
        ref = oracle.pool_block(okp, int(after["block_table"][newest[s]]), n_b, wf[s])
        np.testing.assert_allclose(lvl[s, i], ref, atol=ATOL, rtol=0)
        np.testing.assert_allclose(lvl[s, i], full[s, i], atol=1e-6, rtol=0)


def test_repool_on_a_side_stream_matches_the_current_stream():
    """Pool, re-pool (workspace allocated by the binding) and anchor on a
    stream that is not torch's current one: the zero-filled workspaces are
    ordered before the launches and the results equal the same calls on the
    current stream, bit for bit."""
    say("repool on a side stream")
    w = synth.config5(7, n_seqs=5, len_lo=60, len_hi=400, L=3, H=4, D=128, B=16)
    after = w.extra["after"]
    dev = "cuda"
    newest = torch.from_numpy((after["block_offsets"][1:] - 1).astype(np.int32)).to(dev)
    results = []
    for use_side in (False, True):
        kp, seqs_before = upload(w)
        seqs_after = kka.Seqs(torch.from_numpy(after["seq_len"]).to(dev),
                              torch.from_numpy(after["block_offsets"]).to(dev),
                              torch.from_numpy(after["block_table"]).to(dev), int(after["block_offsets"][-1]))
        sel = Selector(kp, seqs_before, w.select, max_pages=int(np.max(np.diff(after["block_offsets"]))),
                       window=w.window, mode=kka.WEIGHT_VARIANCE)
        side = torch.cuda.Stream() if use_side else None
        sel.pool(stream=side)
        sel.seqs = seqs_after
        sel.repool(newest, stream=side)
        sel.anchor(stream=side)
        if side is not None:
            side.synchronize()
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        results.append((sel.level.cpu().numpy(), sel.anchors.cpu().numpy(), sel.head_weight.cpu().numpy()))
    for a, b in zip(*results):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("hier", [False, True])
def test_decode_step_equals_its_calls(hier):
    """Selector.decode_step (re-pool of the newest blocks, anchor, levels
    above each sequence's newest page for hierarchical layouts, score)
    gives the same bits as the calls made one by one with a full level
    rebuild (block vectors, levels, anchors, affinities, selections), and
    its selections follow the oracle's rules on its own affinities; flat
    and hierarchical layouts."""
    say(f"decode step hier={hier}")
    w = synth.config5(8, n_seqs=6, len_lo=100, len_hi=900, L=3, H=4, D=128, B=16)
    after = w.extra["after"]
    dev = "cuda"
    select = (dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3) if hier
              else dict(w.select))
    newest_np = (after["block_offsets"][1:] - 1).astype(np.int32)
    newest = torch.from_numpy(newest_np).to(dev)
    first_dirty = torch.from_numpy((newest_np - after["block_offsets"][:-1]).astype(np.int32)).to(dev)
    npg_before = torch.from_numpy(np.diff(w.block_offsets).astype(np.int32)).to(dev)
    npg_after = torch.from_numpy(np.diff(after["block_offsets"]).astype(np.int32)).to(dev)
    results = []
    for one_call in (False, True):
        kp, seqs_before = upload(w)
        seqs_after = kka.Seqs(torch.from_numpy(after["seq_len"]).to(dev),
                              torch.from_numpy(after["block_offsets"]).to(dev),
                              torch.from_numpy(after["block_table"]).to(dev), int(after["block_offsets"][-1]))
        sel = Selector(kp, seqs_before, select, max_pages=int(np.max(np.diff(after["block_offsets"]))),
                       window=w.window, mode=kka.WEIGHT_VARIANCE)
        sel.pool()
        sel.levels(npg_before)
        sel.seqs = seqs_after
        if one_call:
            sel.decode_step(newest, npg_after, first_dirty_page=first_dirty if hier else None)
        else:
            sel.repool(newest)
            sel.anchor()
            sel.levels(npg_after)
            sel.score(npg_after)
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        results.append(tuple(t.cpu().numpy() for t in (sel.level, sel.anchors, sel.affinity, sel.page_idx,
                                                       sel.page_score, sel.n_selected)))
        if one_call:
            for s in range(w.S):
                check_selection(sel, s, int(npg_after[s]), "decode step")
    for a, b in zip(*results):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ anchor

@pytest.mark.parametrize("W", [0, 1, 5, 16, 17, 40, 1000])
def test_anchor_windows(W):
    """Windows inside one block, straddling blocks, longer than the
    sequence, and an empty sequence (zero anchor)."""
    say(f"anchor W={W}")
    w = ragged_workload(7, 4, 3, 2, 64, 16, 0, 0, window=W, lengths=[37, 0, 16, 70])
    kp, seqs = upload(w)
    out = torch.full((w.S, w.D), 5.0, dtype=torch.float32, device="cuda")
    kka.kka_pool_anchor(kp, seqs, W, out)
    torch.cuda.synchronize()
    okp = oracle.KPool.of(w)
    for s in range(w.S):
        ref = oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]), W)
        np.testing.assert_allclose(out[s].cpu().numpy(), ref, atol=ATOL, rtol=0)
    assert (out[1] == 0).all()


# ------------------------------------------------------------------ levels + selection

@pytest.mark.parametrize("case", [
    dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3),
    dict(hierarchical=1, k_grid=1, k_chunk=1, k_page=40, pages_per_chunk=4, chunks_per_grid=3),  # zero fill
    dict(hierarchical=1, k_grid=0, k_chunk=2, k_page=6, pages_per_chunk=2, chunks_per_grid=2),   # all masked
    dict(hierarchical=1, k_grid=1000, k_chunk=1000, k_page=7, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=0, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=1024, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=13, pages_per_chunk=16, chunks_per_grid=16),
])
def test_levels_and_selection_match_oracle(case):
    say(f"select {case}")
    w = ragged_workload(8, 5, 2, 2, 64, 4, 0, 900, select=case)
    sel, npg = run_selector(w)
    for s in range(w.S):
        check_selection(sel, s, int(npg[s]), tag=str(case))


@pytest.mark.parametrize("case", [
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=100, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=1000, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=1, k_grid=3, k_chunk=20, k_page=300, pages_per_chunk=64, chunks_per_grid=4),
    dict(hierarchical=1, k_grid=8, k_chunk=40, k_page=900, pages_per_chunk=32, chunks_per_grid=8),
    dict(hierarchical=1, k_grid=4, k_chunk=10, k_page=50, pages_per_chunk=16, chunks_per_grid=8),   # 160 live
    dict(hierarchical=1, k_grid=6, k_chunk=20, k_page=200, pages_per_chunk=16, chunks_per_grid=8),  # 320 live
    dict(hierarchical=1, k_grid=7, k_chunk=28, k_page=500, pages_per_chunk=16, chunks_per_grid=8),  # 448 live
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=77, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=48, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=64, pages_per_chunk=16, chunks_per_grid=16),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=1, pages_per_chunk=16, chunks_per_grid=16),
])
def test_selection_large_candidate_sets(case):
    """Levels with more candidates than the selecting group has threads
    (radix-select path), including k larger than the positive candidates."""
    say(f"select large {case}")
    w = ragged_workload(13, 3, 1, 2, 64, 4, 2000, 9000, select=case)
    if not case["hierarchical"] and case["k_page"] == 77:
        # flat levels of 129-512 pages: 3 to 8 groups of candidates
        w = ragged_workload(14, 6, 1, 2, 64, 4, 516, 2048, select=case)
    sel, npg = run_selector(w)
    for s in range(w.S):
        check_selection(sel, s, int(npg[s]), tag=str(case))


def test_selection_exact_ties_and_zero_scores():
    """Integer-valued page vectors force exact ties and exact 0/0.5/1
    affinities; the anchor is orthogonal to some pages and opposite to
    others."""
    say("select ties")
    S, n_p, D = 3, 300, 8
    lay = kka.LevelLayout(S, 320, D, True, 4, 5)
    rng = np.random.default_rng(9)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :n_p] = rng.integers(-1, 2, (S, n_p, D)).astype(np.float32)
    lvl[:, 7] = 0.0
    anchors = np.zeros((S, D), np.float32)
    anchors[:, 0] = 1.0
    lvl[:, 11] = -anchors[:, None, :][:, 0]
    dev = "cuda"
    sels = [dict(hierarchical=1, k_grid=2, k_chunk=4, k_page=9, pages_per_chunk=4, chunks_per_grid=5),
            dict(hierarchical=1, k_grid=3, k_chunk=30, k_page=64, pages_per_chunk=4, chunks_per_grid=5)]
    for cfg in sels:
        level = torch.from_numpy(lvl).to(dev)
        npg = torch.full((S,), n_p, dtype=torch.int32, device=dev)
        kka.kka_build_levels(lay, level, npg)
        sel = Selector.__new__(Selector)
        sel.lay, sel.sel, sel.level = lay, cfg, level
        sel.anchors = torch.from_numpy(anchors).to(dev)
        sel.page_idx = torch.zeros((S, cfg["k_page"]), dtype=torch.int32, device=dev)
        sel.page_score = torch.zeros((S, cfg["k_page"]), dtype=torch.float32, device=dev)
        sel.n_selected = torch.zeros(S, dtype=torch.int32, device=dev)
        sel.affinity = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device=dev)
        sel.ws_score = kka.new_workspace(kka.kka_score_topk_workspace(lay, True))
        sel.score(npg)
        torch.cuda.synchronize()
        for s in range(S):
            check_selection(sel, s, n_p, tag="ties")


def test_dirty_rebuild_equals_full_rebuild():
    say("levels dirty rebuild")
    w = ragged_workload(10, 4, 2, 2, 64, 4, 50, 700,
                        select=dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4,
                                    chunks_per_grid=3))
    sel, npg = run_selector(w)
    ref = sel.level.clone()
    # scribble over chunk and grid rows, then rebuild only from a dirty page on
    fd = torch.tensor([0, 5, 37, 10_000], dtype=torch.int32, device="cuda")
    lay = sel.lay
    sel.level[:, lay.chunk_row0:] = -7.0
    kka.kka_build_levels(lay, sel.level, npg, fd)
    torch.cuda.synchronize()
    ppc, cpg = lay.pages_per_chunk, lay.chunks_per_grid
    for s in range(w.S):
        n_p = int(npg[s])
        n_c = -(-n_p // ppc)
        n_g = -(-n_c // cpg)
        g0 = (int(fd[s]) // ppc) // cpg
        for g in range(n_g):
            rows_c = range(lay.chunk_row0 + g * cpg, lay.chunk_row0 + min(n_c, (g + 1) * cpg))
            row_g = lay.grid_row0 + g
            if g >= g0:
                assert torch.equal(sel.level[s, row_g], ref[s, row_g])
                for r in rows_c:
                    assert torch.equal(sel.level[s, r], ref[s, r])
            else:
                assert (sel.level[s, row_g] == -7.0).all()


def test_score_workspace_reuse_and_smaller_batch():
    """Repeated calls on the same buffers, then a call with fewer sequences
    and pages on the same workspace, still match the oracle."""
    say("score workspace reuse")
    w = ragged_workload(11, 6, 2, 2, 64, 4, 100, 800,
                        select=dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=6, pages_per_chunk=4,
                                    chunks_per_grid=3))
    sel, npg = run_selector(w)
    for _ in range(2):
        sel.score(npg)
        torch.cuda.synchronize()
        for s in range(w.S):
            check_selection(sel, s, int(npg[s]))
    ws = sel.ws_score
    lay2 = kka.LevelLayout(3, sel.lay.max_pages, w.D, True, 4, 3)
    npg2 = torch.clamp(npg[:3] // 2, min=1)
    level2 = sel.level[:3].contiguous()
    kka.kka_build_levels(lay2, level2, npg2)
    sel2 = Selector.__new__(Selector)
    sel2.lay, sel2.sel, sel2.level, sel2.anchors = lay2, sel.sel, level2, sel.anchors[:3].contiguous()
    sel2.page_idx, sel2.page_score = sel.page_idx[:3].contiguous(), sel.page_score[:3].contiguous()
    sel2.n_selected, sel2.affinity = sel.n_selected[:3].contiguous(), sel.affinity[:3].contiguous()
    sel2.ws_score = ws
    sel2.score(npg2)
    torch.cuda.synchronize()
    for s in range(3):
        check_selection(sel2, s, int(npg2[s]))


def test_device_error_flags_bad_table_entries():
    """Block-table entries outside the pool are skipped (zero vectors) and
    reported through the device flag; nothing outside the pool is read."""
    say("device error flags")
    w = ragged_workload(12, 2, 2, 2, 64, 16, 40, 90)
    w.block_table = w.block_table.copy()
    w.block_table[1] = w.P + 5
    kp, seqs = upload(w)
    out = torch.full((w.total_blocks, w.D), 3.0, dtype=torch.float32, device="cuda")
    kka.kka_pool_blocks(kp, seqs, out)
    assert kka.kka_device_error() & kka.DEVERR_BLOCK_TABLE
    assert (out[1] == 0).all()
    assert kka.kka_device_error() == 0
    lay = kka.LevelLayout(2, 8, w.D, True, 2, 2)
    level = lay.new_buffer()
    kka.kka_build_levels(lay, level, torch.tensor([3, 9], dtype=torch.int32, device="cuda"))
    assert kka.kka_device_error() & kka.DEVERR_PAGES


# ------------------------------------------------------------------ configs (reduced + full)

def test_config1_parity_and_recovery():
    say("config1")
    w = synth.config1(0)
    sel, npg = run_selector(w)
    ref = oracle_vb(w, range(w.total_blocks))
    got = vb_rows(sel, w)
    for b in ref:
        np.testing.assert_allclose(got[b], ref[b], atol=ATOL, rtol=0)
    okp = oracle.KPool.of(w)
    a = oracle.pool_anchor(okp, w.block_table, int(w.seq_len[0]), w.window)
    np.testing.assert_allclose(sel.anchors[0].cpu().numpy(), a, atol=ATOL, rtol=0)
    idx = check_selection(sel, 0, int(npg[0]), "c1")
    prec = np.mean(w.block_topic[0][idx] == w.anchor_topic[0])
    assert prec >= 0.75
    pages = np.stack([ref[b] for b in range(w.total_blocks)])
    say(f"config1 end to end: {check_end_to_end(sel, 0, pages, a, 'c1')} positions differ")


def test_config1_variance_mode_parity():
    say("config1 variance")
    w = synth.config1(0)
    w.mode = "variance"
    sel, npg = run_selector(w)
    okp = oracle.KPool.of(w)
    wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
    np.testing.assert_allclose(sel.head_weight.cpu().numpy(), wref, rtol=WEIGHT_RTOL, atol=0)
    ref = oracle_vb(w, range(w.total_blocks), wref)
    got = vb_rows(sel, w)
    for b in ref:
        np.testing.assert_allclose(got[b], ref[b], atol=ATOL, rtol=0)
    check_selection(sel, 0, int(npg[0]), "c1v")


def test_config2_parity_and_recovery():
    say("config2 (939 MB keys)")
    w = synth.config2(0)
    sel, npg = run_selector(w)
    ref = oracle_vb(w, range(w.total_blocks))
    got = vb_rows(sel, w)
    for b in ref:
        np.testing.assert_allclose(got[b], ref[b], atol=ATOL, rtol=0)
    idx = check_selection(sel, 0, int(npg[0]), "c2")
    assert (w.block_topic[0][idx[:8]] == w.anchor_topic[0]).all()
    okp = oracle.KPool.of(w)
    a = oracle.pool_anchor(okp, w.block_table, int(w.seq_len[0]), w.window)
    np.testing.assert_allclose(sel.anchors[0].cpu().numpy(), a, atol=ATOL, rtol=0)
    pages = np.stack([ref[b] for b in range(w.total_blocks)])
    say(f"config2 end to end: {check_end_to_end(sel, 0, pages, a, 'c2')} positions differ")


def test_config3_full_size_parity_and_recovery():
    """7B shape at 131072 tokens (3.76 GB of keys), launched exactly as the
    benchmark launches it: every one of the 8192 block vectors against the
    oracle (run on the host's cores, one unchanged single-threaded oracle
    call per block), the anchor, every level row and affinity, and the
    selection."""
    say("config3 generate (3.76 GB keys)")
    w = synth.config3(0)
    say("config3 run")
    sel, npg = run_selector(w)
    say(f"config3 oracle: {w.total_blocks} blocks on {host_threads()} threads")
    ref = oracle_vb_all(w)
    got = sel.level[0, :w.total_blocks].cpu().numpy()
    assert_rows_close(got, ref, "config3 v_b")
    okp = oracle.KPool.of(w)
    a = oracle.pool_anchor(okp, w.block_table, int(w.seq_len[0]), w.window)
    np.testing.assert_allclose(sel.anchors[0].cpu().numpy(), a, atol=ATOL, rtol=0)
    idx = check_selection(sel, 0, int(npg[0]), "c3")
    run = w.extra["anchor_run"]
    assert set(range(run * 32, run * 32 + 32)) <= set(idx.tolist())
    say(f"config3 end to end: {check_end_to_end(sel, 0, ref, a, 'c3')} positions differ")


def test_config4_full_size_parity_and_recovery():
    """64 sequences x 8192 fp32 block vectors written directly."""
    say("config4")
    v = synth.config4(0)
    S, n_p, D = v.vb.shape
    lay = kka.LevelLayout(S, n_p, D, True, 16, 16)
    level = lay.new_buffer()
    level[:, :n_p] = torch.from_numpy(v.vb).cuda()
    npg = torch.full((S,), n_p, dtype=torch.int32, device="cuda")
    kka.kka_build_levels(lay, level, npg)
    sel = Selector.__new__(Selector)
    sel.lay, sel.sel, sel.level = lay, v.select, level
    sel.anchors = torch.from_numpy(v.anchors).cuda()
    sel.page_idx = torch.zeros((S, 64), dtype=torch.int32, device="cuda")
    sel.page_score = torch.zeros((S, 64), dtype=torch.float32, device="cuda")
    sel.n_selected = torch.zeros(S, dtype=torch.int32, device="cuda")
    sel.affinity = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
    sel.ws_score = kka.new_workspace(kka.kka_score_topk_workspace(lay, True))
    sel.score(npg)
    torch.cuda.synchronize()
    for s in range(S):
        idx = check_selection(sel, s, n_p, "c4")
        assert (v.page_topic[s][idx] == v.anchor_topic[s]).all()


def _level_pages(lvl: np.ndarray, block_offsets) -> np.ndarray:
    """Page rows of every sequence of a level buffer, in global block order."""
    nb = np.diff(block_offsets)
    return np.concatenate([lvl[s, :int(nb[s])] for s in range(len(nb))])


@pytest.mark.timeout(900)
def test_ragged_variance_batch_full_size_and_decode_step():
    """32 sequences of 4096-65536 tokens (about 32 GB of bf16 keys), blocks of
    64, one shared permuted pool, head-variance weighting, flat top-48; then
    one decode step: one token appended per sequence, the newest block of
    each re-pooled with the frozen weights, anchor, score and select again.
    Everything against the oracle (run on the host's cores): the weights of
    all 32 sequences, the longest (64,866 tokens) included, every block
    vector before the append, every anchor before and after it, every
    re-pooled block, every selection; blocks the append did not touch keep
    their bits."""
    say("ragged variance batch: generate (~32 GB of keys)")
    w = synth.config5(0)
    after = w.extra["after"]
    say(f"ragged variance batch: upload {w.k.nbytes / 1e9:.1f} GB, {w.S} sequences, {w.P} blocks, "
        f"lengths {int(w.seq_len.min())}..{int(w.seq_len.max())}")
    kp, seqs = upload(w)
    max_pages = int(np.max(np.diff(after["block_offsets"])))
    sel = Selector(kp, seqs, w.select, max_pages=max_pages, window=w.window, mode=kka.WEIGHT_VARIANCE)
    npg = n_pages_of(w)
    say("ragged variance batch: pool + anchor + score")
    sel.pool()
    sel.anchor()
    sel.score(npg)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    wg = sel.head_weight.cpu().numpy()
    lvl_before = sel.level.cpu().numpy()
    anc = sel.anchors.cpu().numpy()
    say(f"ragged variance batch: oracle weights of {w.S} sequences on {host_threads()} threads")
    wref = oracle_weights_all(w)
    np.testing.assert_allclose(wg, wref, rtol=WEIGHT_RTOL, atol=0)
    say(f"ragged variance batch: oracle v_b of {w.total_blocks} blocks")
    # end to end: the oracle pools with its own weights
    ref_vb = oracle_vb_all(w, weights=wref)
    assert_rows_close(_level_pages(lvl_before, w.block_offsets), ref_vb, "ragged v_b before the append")
    assert_rows_close(anc, oracle_anchors_all(w, weights=wref), "ragged anchors before the append")
    for s in range(w.S):
        check_selection(sel, s, int(npg[s]), "ragged")

    say("ragged variance batch: decode step")
    dev = "cuda"
    seqs_after = kka.Seqs(torch.from_numpy(after["seq_len"]).to(dev), torch.from_numpy(after["block_offsets"]).to(dev),
                          torch.from_numpy(after["block_table"]).to(dev), int(after["block_offsets"][-1]))
    frozen = sel.head_weight.clone()
    sel.seqs = seqs_after
    newest = (after["block_offsets"][1:] - 1).astype(np.int32)
    npg_after = torch.from_numpy(np.diff(after["block_offsets"]).astype(np.int32)).to(dev)
    sel.repool(torch.from_numpy(newest).to(dev))
    sel.anchor()
    sel.score(npg_after)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    assert torch.equal(sel.head_weight, frozen)
    lvl = sel.level.cpu().numpy()
    okp = oracle.KPool.of(w)
    nb_before = np.diff(w.block_offsets)
    for s in range(w.S):
        i = int(newest[s] - after["block_offsets"][s])
        n_b = int(after["seq_len"][s]) - i * w.B
        ref = oracle.pool_block(okp, int(after["block_table"][newest[s]]), n_b, wref[s])
        np.testing.assert_allclose(lvl[s, i], ref, atol=ATOL, rtol=0, err_msg=f"seq {s} newest block")
        # every older block keeps the bits it had before the append
        np.testing.assert_array_equal(lvl[s, :i].view(np.uint32), lvl_before[s, :i].view(np.uint32),
                                      err_msg=f"seq {s} blocks untouched by the append")
        assert i in (nb_before[s] - 1, nb_before[s])
        check_selection(sel, s, int(npg_after[s]), "ragged decode")
    anc_ref = oracle_anchors_all(w, weights=wref, seq_len=after["seq_len"], block_offsets=after["block_offsets"],
                                 block_table=after["block_table"])
    assert_rows_close(sel.anchors.cpu().numpy(), anc_ref, "ragged anchors after the append")


@pytest.mark.parametrize("case", [
    dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3),
    dict(hierarchical=1, k_grid=1, k_chunk=1, k_page=40, pages_per_chunk=4, chunks_per_grid=3),  # zero fill
    dict(hierarchical=1, k_grid=0, k_chunk=2, k_page=6, pages_per_chunk=2, chunks_per_grid=2),   # all masked
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=9, pages_per_chunk=16, chunks_per_grid=16),
])
@pytest.mark.parametrize("S", [5, 600])
@pytest.mark.parametrize("path", ["one_launch", "two_launch"])
def test_selection_both_launch_shapes(case, S, path, monkeypatch):
    """Three paths on the same inputs, all against the oracle on the same
    rules: 5 sequences score and select in one launch with the selection
    handed to the group that finishes a sequence's last tile; 600 short
    sequences (more tiles than fit on the chip at once) score and select in
    one launch with a selecting group per sequence beside the scoring tiles;
    KKA_SCORE_TWO_LAUNCH=1 forces the scoring launch then the selection
    launch."""
    if path == "two_launch":
        monkeypatch.setenv("KKA_SCORE_TWO_LAUNCH", "1")
    say(f"launch shapes S={S} {path} {case}")
    max_pages, D = 60, 8
    lay = kka.LevelLayout(S, max_pages, D, bool(case["hierarchical"]), case["pages_per_chunk"],
                          case["chunks_per_grid"])
    rng = np.random.default_rng(31 + S)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    n_pages = rng.integers(0, max_pages + 1, S).astype(np.int32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    kka.kka_build_levels(lay, level, npg)
    anchors = torch.from_numpy(rng.standard_normal((S, D), dtype=np.float32)).cuda()
    K = max(1, case["k_page"])
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.full((S, K), 7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
    ws = kka.new_workspace(kka.kka_score_topk_workspace(lay, True))
    for _ in range(2):  # the tile counters are left ready for the next call
        kka.kka_score_topk(lay, level, npg, anchors, k_page=case["k_page"], k_grid=case["k_grid"],
                           k_chunk=case["k_chunk"], page_idx_out=idx, page_score_out=sc, n_selected_out=cnt,
                           affinity_out=aff, workspace=ws)
        torch.cuda.synchronize()
        lv, an, af = level.cpu().numpy(), anchors.cpu().numpy(), aff.cpu().numpy()
        gi, gs, gc = idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy()
        for s in range(S):
            n_p = int(n_pages[s])
            if case["hierarchical"]:
                n_c = -(-n_p // case["pages_per_chunk"])
                n_g = -(-n_c // case["chunks_per_grid"])
                rows = np.concatenate([np.arange(n_p), lay.chunk_row0 + np.arange(n_c),
                                       lay.grid_row0 + np.arange(n_g)]).astype(np.int64)
                a_c = af[s, lay.chunk_row0:lay.chunk_row0 + n_c]
                a_g = af[s, lay.grid_row0:lay.grid_row0 + n_g]
            else:
                rows, a_c, a_g = np.arange(n_p), None, None
            if len(rows):
                np.testing.assert_allclose(af[s, rows], oracle.affinity(lv[s, rows], an[s]), atol=ATOL, rtol=0,
                                           err_msg=f"S={S} s={s}")
            ridx, rsc = oracle.select(af[s, :n_p], a_c, a_g, **case)
            assert gc[s] == len(ridx), f"S={S} s={s}"
            np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"S={S} s={s}")
            np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32))
            if case["k_page"] > len(ridx):
                assert (gi[s, len(ridx):case["k_page"]] == -1).all()


@pytest.mark.parametrize("case,S,max_pages", [
    (dict(hierarchical=1, k_grid=3, k_chunk=12, k_page=70, pages_per_chunk=16, chunks_per_grid=16), 1, 12000),
    (dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=100, pages_per_chunk=16, chunks_per_grid=16), 2, 10000),
])
def test_one_launch_selection_beyond_lds_rows(case, S, max_pages):
    """Few sequences whose rows exceed what the selecting work-group stages in
    LDS: scoring and selection still share one launch, and the selection
    reads the affinities from memory.  Against the oracle."""
    say(f"one launch beyond LDS rows S={S} max_pages={max_pages}")
    D = 16
    lay = kka.LevelLayout(S, max_pages, D, bool(case["hierarchical"]), case["pages_per_chunk"],
                          case["chunks_per_grid"])
    assert lay.rows_per_seq > 9216
    rng = np.random.default_rng(41)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    n_pages = np.array([max_pages - 7 * s for s in range(S)], np.int32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    kka.kka_build_levels(lay, level, npg)
    anchors = torch.from_numpy(rng.standard_normal((S, D), dtype=np.float32)).cuda()
    K = case["k_page"]
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, K), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((S,), dtype=torch.int32, device="cuda")
    for with_aff in (True, False):
        aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda") if with_aff else None
        kka.kka_score_topk(lay, level, npg, anchors, k_page=K, k_grid=case["k_grid"], k_chunk=case["k_chunk"],
                           page_idx_out=idx, page_score_out=sc, n_selected_out=cnt, affinity_out=aff)
        torch.cuda.synchronize()
        if with_aff:
            af = aff.cpu().numpy()
            ref_idx = idx.cpu().numpy().copy()
        lv, an = level.cpu().numpy(), anchors.cpu().numpy()
        gi, gs, gc = idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy()
        for s in range(S):
            n_p = int(n_pages[s])
            if case["hierarchical"]:
                n_c = -(-n_p // case["pages_per_chunk"])
                n_g = -(-n_c // case["chunks_per_grid"])
                rows = np.concatenate([np.arange(n_p), lay.chunk_row0 + np.arange(n_c), lay.grid_row0 + np.arange(n_g)])
                a_c, a_g = af[s, lay.chunk_row0:lay.chunk_row0 + n_c], af[s, lay.grid_row0:lay.grid_row0 + n_g]
            else:
                rows, a_c, a_g = np.arange(n_p), None, None
            np.testing.assert_allclose(af[s, rows], oracle.affinity(lv[s, rows], an[s]), atol=ATOL, rtol=0)
            ridx, rsc = oracle.select(af[s, :n_p], a_c, a_g, **case)
            assert gc[s] == len(ridx)
            np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"s={s} with_aff={with_aff}")
            np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32))
        if not with_aff:
            np.testing.assert_array_equal(gi, ref_idx)  # scratch affinities in the workspace: same selection


def test_unzeroed_score_workspace_raises_flag():
    """A scoring workspace whose tile counters hold garbage: the one-launch
    call raises the workspace flag (the kernel still completes); after the
    counters are re-zeroed the same call selects as the oracle does."""
    say("score workspace garbage counters")
    case = dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3)
    w = ragged_workload(12, 3, 2, 2, 64, 4, 100, 800, select=case)
    sel, npg = run_selector(w)
    sel.ws_score.fill_(0xFF)
    sel.score(npg)
    assert kka.kka_device_error() & kka.DEVERR_WORKSPACE
    sel.ws_score.zero_()
    sel.score(npg)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    for s in range(w.S):
        check_selection(sel, s, int(npg[s]))


def test_concurrent_calls_on_two_streams_with_own_workspaces():
    """Two one-launch score+top-K calls in flight at once on two streams
    (default priority), each with its own workspace: both select as the
    oracle does, repeatedly."""
    say("concurrent score calls on two streams")
    case = dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=6, pages_per_chunk=4, chunks_per_grid=3)
    w1 = ragged_workload(21, 3, 2, 2, 64, 4, 100, 900, select=case)
    w2 = ragged_workload(22, 4, 2, 2, 64, 4, 100, 900, select=case)
    sel1, npg1 = run_selector(w1)
    sel2, npg2 = run_selector(w2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(20):
        sel1.score(npg1, stream=s1)
        sel2.score(npg2, stream=s2)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    for sel, w, npg in ((sel1, w1, npg1), (sel2, w2, npg2)):
        for s in range(w.S):
            check_selection(sel, s, int(npg[s]))


@pytest.mark.parametrize("K", [100, 400])
def test_flat_selection_many_rows_few_positive(K):
    """A flat level of 1000 pages of which 700 point exactly away from the
    anchor (affinity exactly 0): more rows than the ranking path takes but
    only 300 positive scores, so those are compacted and ranked; with k
    above 300 the lowest-index zero rows fill the remaining slots."""
    say(f"flat few positive K={K}")
    S, NP, D = 2, 1000, 8
    lay = kka.LevelLayout(S, NP, D, False, 16, 16)
    rng = np.random.default_rng(61)
    anc = np.zeros((S, D), np.float32)
    anc[:, 0] = 1.0
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :NP] = rng.standard_normal((S, NP, D), dtype=np.float32)
    for s in range(S):
        neg = rng.permutation(NP)[:700]
        lvl[s, neg] = 0.0
        lvl[s, neg, 0] = -rng.uniform(0.5, 2.0, 700).astype(np.float32)  # cos = -1 exactly
    level = torch.from_numpy(lvl).cuda()
    npg = torch.full((S,), NP, dtype=torch.int32, device="cuda")
    anchors = torch.from_numpy(anc).cuda()
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, K), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((S,), dtype=torch.int32, device="cuda")
    aff = torch.zeros((S, NP), dtype=torch.float32, device="cuda")
    kka.kka_score_topk(lay, level, npg, anchors, k_page=K, page_idx_out=idx, page_score_out=sc,
                       n_selected_out=cnt, affinity_out=aff)
    torch.cuda.synchronize()
    af = aff.cpu().numpy()
    for s in range(S):
        assert int((af[s] > 0).sum()) <= 300
        np.testing.assert_allclose(af[s], oracle.affinity(lvl[s, :NP], anc[s]), atol=ATOL, rtol=0)
        ridx, rsc = oracle.select(af[s], hierarchical=0, k_page=K)
        assert int(cnt[s]) == len(ridx)
        np.testing.assert_array_equal(idx[s].cpu().numpy()[:len(ridx)], ridx)
        np.testing.assert_array_equal(sc[s].cpu().numpy()[:len(ridx)].view(np.uint32), rsc.view(np.uint32))


# page counts at the edges of the ranking paths: one group of up to 64, and
# 2 to 8 groups of 64, each group count with a ragged, a full and a
# just-started last group
GROUP_EDGES = [1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 191, 192, 193, 255, 256, 257, 319, 320,
               321, 383, 384, 385, 447, 448, 449, 511, 512]


@pytest.mark.parametrize("K", [1, 17, 64, 200])
@pytest.mark.parametrize("reps", [1, 8])
def test_flat_selection_group_edges(K, reps):
    """Flat levels of 1-512 pages (one group, every group count of the
    ranking path and the edges between them) with exact ties, exact 0 and exact 0.5
    affinities: integer-valued vectors, some exactly opposite the anchor,
    some zero.  reps = 8 repeats the batch so that it takes the two-launch
    path; bit-exact against the oracle's selection of the GPU's own
    affinities."""
    say(f"flat group edges K={K} reps={reps}")
    base = len(GROUP_EDGES)
    S, NP, D = base * reps, 512, 8
    lay = kka.LevelLayout(S, NP, D, False, 16, 16)
    rng = np.random.default_rng(71 + K)
    anc = np.zeros((S, D), np.float32)
    anc[:, 0] = 1.0
    anc[:, 1] = 1.0
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :NP] = rng.integers(-1, 2, (S, NP, D)).astype(np.float32)
    for s in range(S):
        opp = rng.permutation(NP)[:NP // 3]
        lvl[s, opp] = 0.0
        lvl[s, opp, 0] = -1.0
        lvl[s, opp, 1] = -1.0  # cos = -1 exactly: affinity 0
        lvl[s, rng.permutation(NP)[:5]] = 0.0  # zero norm: affinity 0.5
    n_pages = np.array([GROUP_EDGES[s % base] for s in range(S)], np.int32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    anchors = torch.from_numpy(anc).cuda()
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, K), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((S,), dtype=torch.int32, device="cuda")
    aff = torch.zeros((S, NP), dtype=torch.float32, device="cuda")
    kka.kka_score_topk(lay, level, npg, anchors, k_page=K, page_idx_out=idx, page_score_out=sc,
                       n_selected_out=cnt, affinity_out=aff)
    torch.cuda.synchronize()
    af = aff.cpu().numpy()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    for s in range(S):
        n = int(n_pages[s])
        np.testing.assert_allclose(af[s, :n], oracle.affinity(lvl[s, :n], anc[s]), atol=ATOL, rtol=0)
        ridx, rsc = oracle.select(af[s, :n], hierarchical=0, k_page=K)
        assert int(cnt[s]) == len(ridx) == min(K, n)
        np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"s={s} n={n}")
        np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32))
        if K > n:
            assert (gi[s, n:] == -1).all()


@pytest.mark.parametrize("case", [
    dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3),
    dict(hierarchical=1, k_grid=5, k_chunk=8, k_page=20, pages_per_chunk=4, chunks_per_grid=3),
])
def test_parented_small_levels_many_sequences(case):
    """A level of at most 64 candidates that both reads the parent list (its
    candidates are children of kept parents) and rewrites it (its kept
    elements parent the next level) must let every wave finish reading
    before the list is rewritten.  4000 sequences of ragged lengths take the
    selection launch (work-groups sharing a compute unit at different
    phases), six calls, every sequence bit-exact against the oracle's
    selection of the GPU's own affinities."""
    say(f"parented small levels {case}")
    S, max_pages, D = 4000, 60, 8
    lay = kka.LevelLayout(S, max_pages, D, True, case["pages_per_chunk"], case["chunks_per_grid"])
    rng = np.random.default_rng(83)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    n_pages = rng.integers(1, max_pages + 1, S).astype(np.int32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    kka.kka_build_levels(lay, level, npg)
    anchors = torch.from_numpy(rng.standard_normal((S, D), dtype=np.float32)).cuda()
    K = case["k_page"]
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.zeros((S, K), dtype=torch.float32, device="cuda")
    aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
    for call in range(6):
        kka.kka_score_topk(lay, level, npg, anchors, k_page=K, k_grid=case["k_grid"], k_chunk=case["k_chunk"],
                           page_idx_out=idx, page_score_out=sc, affinity_out=aff)
        torch.cuda.synchronize()
        af, gi, gs = aff.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
        for s in range(S):
            n_p = int(n_pages[s])
            n_c = -(-n_p // case["pages_per_chunk"])
            n_g = -(-n_c // case["chunks_per_grid"])
            ridx, rsc = oracle.select(af[s, :n_p], af[s, lay.chunk_row0:lay.chunk_row0 + n_c],
                                      af[s, lay.grid_row0:lay.grid_row0 + n_g], **case)
            np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"call={call} s={s}")
            np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32))


@pytest.mark.parametrize("one_launch", [True, False])
def test_layer_split_shares_and_counters(one_launch):
    """A small batch splits every block's and every sequence's layers over
    several work-groups (blocks of 16 KiB per layer: shares of 8 layers).
    With at most one work-group per compute unit (13 blocks, 2 sequences)
    the one that finishes an item's last share adds the shares in split
    order in the same launch, else (151 blocks, 302 work-groups) a second
    kernel does.  v_b and anchors match
    the oracle over three steps on one set of workspaces (the arrival
    counters are left zero) and are bit-identical from step to step; in the
    one-launch case garbage counters raise the workspace flag until they
    are re-zeroed."""
    say(f"layer split one_launch={one_launch}")
    w = ragged_workload(16, 2, 12, 4, 128, 16, 80, 120, window=24) if one_launch else \
        ragged_workload(16, 10, 12, 4, 128, 16, 200, 280, window=24)
    sel, npg = run_selector(w)
    assert sel.ws_pool is not None and sel.ws_anchor is not None  # both launches are split
    okp = oracle.KPool.of(w)
    ref = oracle_vb(w, range(w.total_blocks))
    ref_anc = [oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]),
                                  w.window) for s in range(w.S)]
    first = None
    for step in range(3):
        if step:
            sel.step(npg)
            torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        got = vb_rows(sel, w)
        for b, v in ref.items():
            np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"step {step} block {b}")
        anc = sel.anchors.cpu().numpy()
        for s in range(w.S):
            np.testing.assert_allclose(anc[s], ref_anc[s], atol=ATOL, rtol=0, err_msg=f"step {step} seq {s}")
        now = (sel.level.cpu().numpy().copy(), anc.copy())
        if first is None:
            first = now
        else:
            np.testing.assert_array_equal(now[0].view(np.uint32), first[0].view(np.uint32))
            np.testing.assert_array_equal(now[1].view(np.uint32), first[1].view(np.uint32))
    if not one_launch:
        return
    for ws in (sel.ws_pool, sel.ws_anchor):
        ws.fill_(0xFF)
        sel.step(npg)
        assert kka.kka_device_error() & kka.DEVERR_WORKSPACE
        ws.zero_()
        sel.step(npg)
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
    got = vb_rows(sel, w)
    for b, v in ref.items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"after re-zero block {b}")


def test_no_handoff_switch_gives_the_same_bits(monkeypatch):
    """Launches that hand values between work-groups (a small layer-split
    pool and anchor, a scoring batch that fits on the chip) against the same
    calls with KKA_NO_HANDOFF=1, which adds the shares and selects in a
    second launch: the same bits for every block vector, anchor, affinity
    and selection."""
    say("no-handoff switch")
    case = dict(hierarchical=1, k_grid=2, k_chunk=3, k_page=5, pages_per_chunk=4, chunks_per_grid=3)
    w = ragged_workload(17, 2, 12, 4, 128, 16, 80, 120, window=24, select=case)
    outs = []
    for flag in ("0", "1"):
        monkeypatch.setenv("KKA_NO_HANDOFF", flag)
        sel, npg = run_selector(w)
        assert kka.kka_device_error() == 0
        outs.append([t.cpu().numpy() for t in (sel.level, sel.anchors, sel.affinity, sel.page_idx, sel.page_score,
                                                sel.n_selected)])
        if flag == "1":
            for s in range(w.S):
                check_selection(sel, s, int(npg[s]), "no handoff")
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("seed", range(40))
def test_selection_random_configurations(seed):
    """Seeded sweep over selection configurations: flat or hierarchical,
    fan-outs 1-20, k per level from 0 to beyond the level's size, 1-300
    sequences of 0-700 pages (so one-launch and two-launch batches, levels
    of every ranking path, parented and not), head_dim 8-256, and a share
    of exactly-zero and tied scores.  Chunk and grid vectors and every
    present row's affinity against the oracle (from the GPU's own page
    vectors and anchor); every selection bit-exact against the oracle's
    selection of the GPU's own affinities, and the lazy pass bit-identical
    to the full pass."""
    rng = np.random.default_rng(1000 + seed)
    hier = int(rng.integers(0, 2))
    ppc, cpg = int(rng.integers(1, 21)), int(rng.integers(1, 21))
    S = int(rng.choice([1, 3, 17, 64, 300]))
    max_pages = int(rng.integers(1, 701))
    D = int(rng.choice([8, 16, 64, 128, 256]))
    kp_ = int(rng.integers(1, 1025)) if rng.random() < 0.3 else int(rng.integers(1, 129))
    case = dict(hierarchical=hier, k_grid=int(rng.integers(0, 40)) if hier else 0,
                k_chunk=int(rng.integers(0, 200)) if hier else 0, k_page=kp_, pages_per_chunk=ppc,
                chunks_per_grid=cpg)
    say(f"random selection seed={seed} S={S} max_pages={max_pages} D={D} {case}")
    lay = kka.LevelLayout(S, max_pages, D, bool(hier), ppc, cpg)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    if rng.random() < 0.3:  # integer-valued vectors: exact ties, exact 0 / 0.5 / 1 affinities
        lvl[:, :max_pages] = rng.integers(-1, 2, (S, max_pages, D)).astype(np.float32)
    else:
        lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    anc = rng.standard_normal((S, D), dtype=np.float32)
    n_pages = rng.integers(0, max_pages + 1, S).astype(np.int32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    kka.kka_build_levels(lay, level, npg)
    K = case["k_page"]
    idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc = torch.full((S, K), 7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
    kka.kka_score_topk(lay, level, npg, torch.from_numpy(anc).cuda(), k_page=K, k_grid=case["k_grid"],
                       k_chunk=case["k_chunk"], page_idx_out=idx, page_score_out=sc, n_selected_out=cnt,
                       affinity_out=aff)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    af, gi, gs, gc = aff.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy()
    lv = level.cpu().numpy()
    for s in range(S):
        n_p = int(n_pages[s])
        rows = np.arange(n_p)
        if hier:
            n_c = -(-n_p // ppc)
            n_g = -(-n_c // cpg)
            a_c = af[s, lay.chunk_row0:lay.chunk_row0 + n_c]
            a_g = af[s, lay.grid_row0:lay.grid_row0 + n_g]
            if n_p:
                oc, og = oracle.build_levels(lv[s, :n_p], ppc, cpg)
                np.testing.assert_allclose(lv[s, lay.chunk_row0:lay.chunk_row0 + n_c], oc, atol=ATOL, rtol=0)
                np.testing.assert_allclose(lv[s, lay.grid_row0:lay.grid_row0 + n_g], og, atol=ATOL, rtol=0)
            rows = np.concatenate([rows, lay.chunk_row0 + np.arange(n_c), lay.grid_row0 + np.arange(n_g)])
        else:
            a_c = a_g = None
        if len(rows):
            np.testing.assert_allclose(af[s, rows], oracle.affinity(lv[s, rows], anc[s]), atol=ATOL, rtol=0,
                                       err_msg=f"s={s}")
        ridx, rsc = oracle.select(af[s, :n_p], a_c, a_g, **case)
        assert gc[s] == len(ridx), f"s={s}"
        np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"s={s} n_p={n_p}")
        np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32), err_msg=f"s={s}")
        assert (gi[s, len(ridx):] == -1).all() and (gs[s, len(ridx):] == 0).all()
    # the lazy pass (one work-group per sequence, children of kept parents
    # only) selects exactly what the full pass selects
    idx2 = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
    sc2 = torch.full((S, K), 7.0, dtype=torch.float32, device="cuda")
    cnt2 = torch.full((S,), -9, dtype=torch.int32, device="cuda")
    kka.kka_score_topk(lay, level, npg, torch.from_numpy(anc).cuda(), k_page=K, k_grid=case["k_grid"],
                       k_chunk=case["k_chunk"], page_idx_out=idx2, page_score_out=sc2, n_selected_out=cnt2,
                       lazy=True)
    torch.cuda.synchronize()
    assert kka.kka_device_error() == 0
    np.testing.assert_array_equal(idx2.cpu().numpy(), gi)
    np.testing.assert_array_equal(sc2.cpu().numpy().view(np.uint32), gs.view(np.uint32))
    np.testing.assert_array_equal(cnt2.cpu().numpy(), gc)


@pytest.mark.parametrize("seed", range(16))
def test_pool_and_anchor_random_shapes(seed):
    """Seeded sweep over key-pool shapes (layers 1-32, KV heads 1-8,
    head_dim 8-256, blocks of 1-64 tokens, 1-24 ragged sequences, windows
    1-40; at most 16M key elements), so that pooling and anchors run unsplit,
    split and combined in one launch, and split with a second launch;
    uniform or head-variance weights.  v_b, weights and anchors against the
    oracle."""
    rng = np.random.default_rng(2000 + seed)
    L = int(rng.integers(1, 33))
    H = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([8, 16, 32, 64, 128, 256]))
    B = int(rng.choice([1, 4, 8, 16, 32, 64]))
    S = int(rng.integers(1, 25))
    per_token = L * H * D
    max_len = max(1, min(600, (16 << 20) // (per_token * S)))
    lengths = rng.integers(0, max_len + 1, S)
    lengths[0] = max(1, lengths[0])
    mode = "variance" if rng.random() < 0.4 else "uniform"
    window = int(rng.integers(1, 41))
    say(f"pool random seed={seed} L={L} H={H} D={D} B={B} S={S} max_len={max_len} {mode} W={window}")
    w = ragged_workload(3000 + seed, S, L, H, D, B, 0, 0, mode=mode, window=window, lengths=lengths,
                        offset=0.5 if mode == "variance" else 0.0)
    sel, _ = run_selector(w)
    assert kka.kka_device_error() == 0
    okp = oracle.KPool.of(w)
    wref = None
    if mode == "variance":
        wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
        np.testing.assert_allclose(sel.head_weight.cpu().numpy(), wref, rtol=WEIGHT_RTOL, atol=0)
    got = vb_rows(sel, w)
    ref = oracle_vb(w, range(w.total_blocks), wref)
    for b, v in ref.items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")
    anc = sel.anchors.cpu().numpy()
    for s in range(w.S):
        a = oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]),
                               w.window, None if wref is None else wref[s])
        np.testing.assert_allclose(anc[s], a, atol=ATOL, rtol=0, err_msg=f"anchor {s}")


@pytest.mark.parametrize("seed", range(12))
def test_pool_odd_heads_and_many_sequences(seed):
    """Pooling and anchors where a work-group's last wavefront is partial
    (3, 5, 6 or 7 KV heads, so a token row is not a power-of-two number of
    16-byte pieces) and batches of 64-100 sequences: the block lookup then
    takes its binary-search path for some or all wavefronts, and must agree
    with the one-round path.  v_b, weights and anchors against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    L = int(rng.integers(1, 17))
    H = int(rng.choice([3, 5, 6, 7]))
    D = int(rng.choice([8, 16, 24, 64, 128]))
    B = int(rng.choice([1, 4, 16, 64]))
    S = int(rng.choice([5, 64, 65, 100]))
    max_len = max(1, min(400, (8 << 20) // (L * H * D * S)))
    lengths = rng.integers(0, max_len + 1, S)
    lengths[0] = max(1, lengths[0])
    mode = "variance" if rng.random() < 0.4 else "uniform"
    window = int(rng.integers(1, 41))
    say(f"pool odd heads seed={seed} L={L} H={H} D={D} B={B} S={S} max_len={max_len} {mode} W={window}")
    w = ragged_workload(9000 + seed, S, L, H, D, B, 0, 0, mode=mode, window=window, lengths=lengths,
                        offset=0.5 if mode == "variance" else 0.0)
    sel, _ = run_selector(w)
    assert kka.kka_device_error() == 0
    okp = oracle.KPool.of(w)
    wref = None
    if mode == "variance":
        wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
        np.testing.assert_allclose(sel.head_weight.cpu().numpy(), wref, rtol=WEIGHT_RTOL, atol=0)
    got = vb_rows(sel, w)
    for b, v in oracle_vb(w, range(w.total_blocks), wref).items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")
    anc = sel.anchors.cpu().numpy()
    for s in range(w.S):
        a = oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]),
                               w.window, None if wref is None else wref[s])
        np.testing.assert_allclose(anc[s], a, atol=ATOL, rtol=0, err_msg=f"anchor {s}")


def test_variance_weights_of_constant_sequences_are_uniform():
    """Head-variance weights where the temporal variance is exactly 0: a
    sequence of one token, and a sequence whose keys repeat the same token
    at every position (over several blocks).  The definition then gives
    uniform weights; the GPU must find exactly 0 (not fp32 rounding noise,
    which the normalisation would turn into arbitrary weights).  The other
    sequences' weights and every v_b against the oracle."""
    say("variance weights of constant sequences")
    L, H, D, B = 22, 8, 128, 32
    w = ragged_workload(41, 4, L, H, D, B, 0, 0, mode="variance", lengths=[63, 1, 150, 40])
    f = synth.bf16_bits_to_f32(w.k).reshape(L, w.P, B, H, D)
    # sequence 2: every token repeats its first token
    for i in range(int(w.block_offsets[2]), int(w.block_offsets[3])):
        p = int(w.block_table[i])
        p0 = int(w.block_table[w.block_offsets[2]])
        f[:, p, :, :, :] = f[:, p0, 0:1, :, :]
    w.k = synth.to_bf16_bits(f)
    sel, _ = run_selector(w)
    assert kka.kka_device_error() == 0
    okp = oracle.KPool.of(w)
    wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
    wgpu = sel.head_weight.cpu().numpy()
    uniform = np.float32(1.0 / (L * H))
    for s in (1, 2):
        np.testing.assert_array_equal(wref[s], np.full(L * H, uniform, np.float32))
        np.testing.assert_array_equal(wgpu[s], np.full(L * H, uniform, np.float32), err_msg=f"seq {s}")
    np.testing.assert_allclose(wgpu, wref, rtol=WEIGHT_RTOL, atol=0)
    got = vb_rows(sel, w)
    for b, v in oracle_vb(w, range(w.total_blocks), wref).items():
        np.testing.assert_allclose(got[b], v, atol=ATOL, rtol=0, err_msg=f"block {b}")


def test_variance_weights_of_large_offset_low_variance_heads():
    """Heads whose keys sit at a large offset and change by one bf16 ulp in a
    few tokens only, on a 65,536-token sequence (every head like that) and a
    shorter one (mixed with ordinary heads): the spread is far below the
    mean square (down to ~1e-12 of it), where E[x^2] - E[x]^2 would cancel.
    Weights against the oracle's two-pass fp64 variance at rtol 1e-6; block
    vectors (magnitudes up to 4e4) within 3e-7 relative plus 1e-5."""
    say("variance weights of large-offset, low-variance heads (65,536 tokens)")
    L, H, D, B = 2, 4, 64, 64
    w = ragged_workload(43, 2, L, H, D, B, 0, 0, mode="variance", lengths=[65536, 3000])
    LH = L * H
    offsets = np.array([1000.0, -300.0, 77.5, 4096.0, 0.75, -12.0, 250.0, 30000.0], np.float32)
    p_dev = np.array([1e-4, 1e-3, 3e-3, 1e-2, 3e-4, 3e-2, 2e-3, 5e-4], np.float32)
    ulp = np.float32(2.0) ** (np.floor(np.log2(np.abs(offsets))) - 7)  # bf16 spacing at the offset
    n = L * w.P * B * H * D
    u = synth.uniform(43, 120, n).reshape(L, w.P, B, H, D)
    sign = np.where(synth.uniform(43, 121, n).reshape(L, w.P, B, H, D) < 0.5, -1.0, 1.0).astype(np.float32)
    f = np.empty((L, w.P, B, H, D), np.float32)
    for l in range(L):
        for h in range(H):
            lh = l * H + h
            f[l, :, :, h, :] = offsets[lh] + np.where(u[l, :, :, h, :] < p_dev[lh], sign[l, :, :, h, :] * ulp[lh], 0.0)
    # the shorter sequence: two of its heads are ordinary (noise of unit size around the offset)
    noise = synth.normal(43, 122, n).reshape(L, w.P, B, H, D).astype(np.float32)
    for i in range(int(w.block_offsets[1]), int(w.block_offsets[2])):
        p = int(w.block_table[i])
        f[0, p, :, 1, :] += noise[0, p, :, 1, :]
        f[1, p, :, 2, :] += noise[1, p, :, 2, :]
    w.k = synth.to_bf16_bits(f)
    sel, _ = run_selector(w)
    assert kka.kka_device_error() == 0
    okp = oracle.KPool.of(w)
    wref = oracle.weights_all(okp, w.seq_len, w.block_offsets, w.block_table)
    wgpu = sel.head_weight.cpu().numpy()
    # the long sequence's weights are far from uniform: every head varies, by different amounts
    assert np.ptp(wref[0]) > 0.1 and (wref[0] > 0).all()
    np.testing.assert_allclose(wgpu, wref, rtol=WEIGHT_RTOL, atol=0)
    got = vb_rows(sel, w)
    for b, v in oracle_vb(w, range(w.total_blocks), wref).items():
        np.testing.assert_allclose(got[b], v, rtol=3e-7, atol=1e-5, err_msg=f"block {b}")


# Layouts at the limits of the lean selection (at most 64 grids, 64 chunk
# candidates, 256 page candidates and k = 64 a level) and one step past
# each (the general path): head_dim 32 and 128, ragged and empty
# sequences, integer-valued vectors for exact affinity ties.  The single
# pass is checked against the oracle, the lazy pass bit for bit against
# the single pass.
@pytest.mark.parametrize("seed", range(48))
def test_lean_random_configurations(seed):
    """Seeded sweep over hierarchical layouts within the lean limits (fan-outs
    1-16, up to 64 grids, k_grid * chunks_per_grid <= 64, k_chunk <= 64 with
    at most 256 page candidates, k_page <= 64), 1-17 ragged or full
    sequences, head_dim 8-128 (some not a multiple of 32, so lanes whose
    row pieces lie past head_dim), a share of tied scores: the one-launch
    single pass (tiles whose first rows go out with the page count, lean
    selection) and the lazy pass (one round of rows per level) against the
    oracle's affinities and selection, and the lazy pass's scored rows and
    selections bit-identical to the single pass's."""
    rng = np.random.default_rng(50000 + seed)
    ppc = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    cpg = int(rng.choice([1, 2, 3, 4, 7, 8, 16]))
    max_pages = int(rng.integers(1, min(8192, ppc * cpg * 64) + 1))
    S = int(rng.choice([1, 2, 3, 6, 17]))
    D = int(rng.choice([8, 16, 24, 32, 40, 64, 96, 128]))  # 24, 40, 96: lanes whose pieces lie past the row
    case = dict(hierarchical=1, k_grid=int(rng.integers(0, 64 // cpg + 1)),
                k_chunk=int(rng.integers(0, min(64, 256 // ppc) + 1)), k_page=int(rng.integers(1, 65)),
                pages_per_chunk=ppc, chunks_per_grid=cpg)
    ties = rng.random() < 0.3
    say(f"lean random seed={seed} S={S} max_pages={max_pages} D={D} {case} ties={ties}")
    lay = kka.LevelLayout(S, max_pages, D, True, ppc, cpg)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    if ties:
        lvl[:, :max_pages] = rng.integers(-1, 2, (S, max_pages, D)).astype(np.float32)
    else:
        lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D), dtype=np.float32)
    anc = rng.standard_normal((S, D), dtype=np.float32)
    n_pages = rng.integers(0, max_pages + 1, S).astype(np.int32)
    if rng.random() < 0.3:
        n_pages[:] = max_pages  # every level full: the tiles' first-row guess holds
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(n_pages).cuda()
    kka.kka_build_levels(lay, level, npg)
    K = case["k_page"]
    outs = []
    for lazy in (False, True):
        idx = torch.full((S, K), -9, dtype=torch.int32, device="cuda")
        sc = torch.full((S, K), 7.0, dtype=torch.float32, device="cuda")
        cnt = torch.full((S,), -9, dtype=torch.int32, device="cuda")
        aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
        kka.kka_score_topk(lay, level, npg, torch.from_numpy(anc).cuda(), k_page=K, k_grid=case["k_grid"],
                           k_chunk=case["k_chunk"], page_idx_out=idx, page_score_out=sc, n_selected_out=cnt,
                           affinity_out=aff, lazy=lazy)
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        outs.append(tuple(t.cpu().numpy() for t in (aff, idx, sc, cnt)))
    (af, gi, gs, gc), (af2, gi2, gs2, gc2) = outs
    lv = level.cpu().numpy()
    for s in range(S):
        n_p = int(n_pages[s])
        n_c = -(-n_p // ppc)
        n_g = -(-n_c // cpg)
        rows = np.concatenate([np.arange(n_p), lay.chunk_row0 + np.arange(n_c), lay.grid_row0 + np.arange(n_g)])
        if len(rows):
            np.testing.assert_allclose(af[s, rows], oracle.affinity(lv[s, rows], anc[s]), atol=ATOL, rtol=0,
                                       err_msg=f"s={s}")
        a_c = af[s, lay.chunk_row0:lay.chunk_row0 + n_c]
        a_g = af[s, lay.grid_row0:lay.grid_row0 + n_g]
        ridx, rsc = oracle.select(af[s, :n_p], a_c, a_g, **case)
        assert gc[s] == len(ridx), f"s={s}"
        np.testing.assert_array_equal(gi[s, :len(ridx)], ridx, err_msg=f"s={s} n_p={n_p}")
        np.testing.assert_array_equal(gs[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32), err_msg=f"s={s}")
        assert (gi[s, len(ridx):] == -1).all() and (gs[s, len(ridx):] == 0).all()
        scored = af2[s] != 0  # rows the lazy pass scored (others left at 0)
        np.testing.assert_array_equal(af2[s][scored].view(np.uint32), af[s][scored].view(np.uint32))
    np.testing.assert_array_equal(gi2, gi)
    np.testing.assert_array_equal(gs2.view(np.uint32), gs.view(np.uint32))
    np.testing.assert_array_equal(gc2, gc)


LEAN_LIMITS = [
    # (pages_per_chunk, chunks_per_grid, max_pages, k_grid, k_chunk, k_page)
    (4, 4, 1024, 16, 64, 64),    # 64 grids, 64 chunk and 256 page candidates, k = 64: lean
    (4, 4, 1024, 16, 64, 65),    # k_page past the limit: general
    (4, 4, 1024, 17, 64, 64),    # 68 chunk candidates: general
    (16, 16, 8192, 4, 16, 64),   # the serving shape: lean
    (5, 3, 900, 7, 21, 40),      # fan-outs that are not powers of two: lean
    (16, 4, 4096, 16, 65, 64),   # k_chunk past the limit: general
]


def _lean_case_levels(S, max_pages, D, ppc, cpg, n_pages, ties, seed):
    lay = kka.LevelLayout(S, max_pages, D, True, ppc, cpg)
    rng = np.random.default_rng(seed)
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    if ties:
        lvl[:, :max_pages] = rng.integers(-1, 2, (S, max_pages, D)).astype(np.float32)
        anchors = rng.integers(-1, 2, (S, D)).astype(np.float32)
    else:
        lvl[:, :max_pages] = rng.standard_normal((S, max_pages, D)).astype(np.float32)
        anchors = rng.standard_normal((S, D)).astype(np.float32)
    for s, n in enumerate(n_pages):
        lvl[s, n:max_pages] = 0.0
    return lay, lvl, anchors


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("geom", LEAN_LIMITS)
def test_lean_level_limits(geom, D, ties):
    ppc, cpg, max_pages, kg, kc, kp = geom
    say(f"lean limits {geom} D={D} ties={ties}")
    n_pages = [max_pages, max_pages - 1, 1, 0, 17, max_pages // 2 + 3]
    S = len(n_pages)
    lay, lvl, anchors = _lean_case_levels(S, max_pages, D, ppc, cpg, n_pages, ties, seed=max_pages + D + kp)
    cfg = dict(hierarchical=1, k_grid=kg, k_chunk=kc, k_page=kp, pages_per_chunk=ppc, chunks_per_grid=cpg)
    dev = "cuda"
    level = torch.from_numpy(lvl).to(dev)
    npg = torch.tensor(n_pages, dtype=torch.int32, device=dev)
    kka.kka_build_levels(lay, level, npg)
    sel = Selector.__new__(Selector)
    sel.lay, sel.sel, sel.level = lay, cfg, level
    sel.anchors = torch.from_numpy(anchors).to(dev)
    sel.page_idx = torch.zeros((S, kp), dtype=torch.int32, device=dev)
    sel.page_score = torch.zeros((S, kp), dtype=torch.float32, device=dev)
    sel.n_selected = torch.zeros(S, dtype=torch.int32, device=dev)
    sel.affinity = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device=dev)
    sel.ws_score = kka.new_workspace(kka.kka_score_topk_workspace(lay, True))
    sel.score(npg)
    torch.cuda.synchronize()
    for s in range(S):
        check_selection(sel, s, n_pages[s], tag=f"lean {geom} D={D}")
    full = (sel.page_idx.clone(), sel.page_score.clone(), sel.n_selected.clone())
    sel.page_idx.fill_(-7)
    sel.page_score.fill_(-7.0)
    sel.n_selected.fill_(-7)
    sel.score(npg, lazy=True)
    torch.cuda.synchronize()
    assert torch.equal(sel.page_idx, full[0]), "lazy indices differ from the single pass"
    assert torch.equal(sel.page_score.view(torch.int32), full[1].view(torch.int32)), "lazy scores differ"
    assert torch.equal(sel.n_selected, full[2])
