"""GPU parity of the attention reference (kka_attention_topk): the attention
mass of every block for one decode query per sequence, QK^T softmax
averaged over every layer and query head (page section 3.3), and its top-k.

Block scores against the oracle (fp64 softmax, rounded once) within
rtol 2e-5 + atol 1e-7: fp32 logits carry a relative error of a few ulp of
|logit|, which exp turns into the same relative error of the mass.  The
top-k against the oracle's selection on the GPU's own scores, bit-exact.
Both logit kernels are covered: the matrix-core one (head_dim 32-256, up to
16 query heads per KV head, blocks dividing or divisible by 16) and the
vector one (everything else).  At 128K tokens with all 28 layers the
oracle is too slow, so that case is
checked through properties that hold at any size (unit total mass,
non-negative scores, selection on the GPU's scores, planted-topic blocks on
top) plus full parity of the same 131072-token sequence at 4 layers.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth

from gpu_harness import say, upload
from test_gpu_parity import ragged_workload

pytestmark = pytest.mark.gpu

RTOL, ATOL_MASS = 2e-5, 1e-7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


def run_attention(w, q, Hq, k, scale=None, stride=None):
    kp, seqs = upload(w)
    nb = np.diff(w.block_offsets)
    stride = stride or max(1, int(nb.max()))
    out = torch.full((w.S, stride), -1.0, dtype=torch.float32, device="cuda")
    idx = torch.full((w.S, max(1, k)), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((w.S, max(1, k)), dtype=torch.float32, device="cuda")
    cnt = torch.full((w.S,), -7, dtype=torch.int32, device="cuda")
    qd = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    kka.kka_attention_topk(kp, seqs, qd, Hq, out, stride, scale=scale, k=k, idx_out=idx, score_out=sc,
                           n_selected_out=cnt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy(), cnt.cpu().numpy()


def check(w, q, Hq, k, scale, out, idx, sc, cnt, tag, seqs_to_check=None):
    okp = oracle.KPool.of(w)
    for s in (range(w.S) if seqs_to_check is None else seqs_to_check):
        T = int(w.seq_len[s])
        tab = oracle.seq_table(w.block_offsets, w.block_table, s)
        ref = oracle.attention_blocks(okp, tab, T, q[s], scale)
        n = len(ref)
        np.testing.assert_allclose(out[s, :n], ref, rtol=RTOL, atol=ATOL_MASS, err_msg=f"{tag} s={s}")
        if T:
            assert abs(float(out[s, :n].astype(np.float64).sum()) - 1.0) < 1e-5
        # selection on the GPU's own scores, bit-exact
        ridx, rsc = oracle.select(out[s, :n], hierarchical=0, k_page=k)
        assert int(cnt[s]) == len(ridx), f"{tag} s={s} count"
        np.testing.assert_array_equal(idx[s, :len(ridx)], ridx, err_msg=f"{tag} s={s} top-k")
        np.testing.assert_array_equal(sc[s, :len(ridx)].view(np.uint32), rsc.view(np.uint32))
        if k > len(ridx):
            assert (idx[s, len(ridx):k] == -1).all()


@pytest.mark.parametrize("D,B,H,Hq", [(64, 16, 2, 14), (128, 5, 4, 28), (8, 1, 1, 8), (32, 128, 2, 2),
                                      (512, 16, 1, 4), (128, 64, 4, 4), (128, 16, 2, 32), (64, 8, 1, 12),
                                      (256, 4, 3, 9), (16, 32, 4, 8), (128, 48, 8, 8)])
def test_attention_matches_oracle_ragged(D, B, H, Hq):
    say(f"attention ragged D={D} B={B} H={H} Hq={Hq}")
    lengths = [0, 1, 37, 300, B * 3]
    w = ragged_workload(70, 5, 3, H, D, B, 0, 0, lengths=lengths)
    rng = np.random.default_rng(71)
    q = rng.standard_normal((w.S, w.L, Hq, D)).astype(np.float32)
    k = 7
    scale = 1.0 / math.sqrt(D)
    out, idx, sc, cnt = run_attention(w, q, Hq, k, scale)
    check(w, q, Hq, k, scale, out, idx, sc, cnt, "ragged")
    assert cnt[0] == 0 and (idx[0] == -1).all()


def test_attention_peaked_and_flat_extremes():
    """A sharp softmax (logits with standard deviation 8) and scale 0
    (uniform: n_b / T)."""
    say("attention extremes")
    w = ragged_workload(72, 3, 2, 2, 64, 16, 0, 0, lengths=[50, 161, 16])
    rng = np.random.default_rng(73)
    q = rng.standard_normal((w.S, w.L, 4, 64)).astype(np.float32)
    for scale in (1.0, 0.0):
        out, idx, sc, cnt = run_attention(w, q, 4, 5, scale)
        check(w, q, 4, 5, scale, out, idx, sc, cnt, f"scale={scale}")
    for s, T in enumerate(w.seq_len):
        nb = -(-int(T) // 16)
        expect = np.array([min(16, int(T) - 16 * b) for b in range(nb)], np.float64) / int(T)
        np.testing.assert_allclose(out[s, :nb], expect, rtol=1e-6)


def test_attention_planted_topic_and_overlap_with_kka():
    """0.5B shape with planted topics and queries aimed at the anchor topic:
    the attention top-16 is on the anchor topic, and the overlap between the
    attention top-16 and the key-key top-16 (the page's quality metric)
    equals the oracle's wherever neither ranking has a near-tie at the
    16th place (then several overlaps are correct)."""
    say("attention planted 0.5B shape")
    from gpu_harness import run_selector
    w = synth.config1(0)
    q = synth.planted_queries(w, 14, 8.0, 0.5)[None]
    out, idx, sc, cnt = run_attention(w, q, 14, 16, 1 / 8)
    check(w, q, 14, 16, 1 / 8, out, idx, sc, cnt, "c1")
    assert (w.block_topic[0][idx[0]] == w.anchor_topic[0]).all()
    sel, npg = run_selector(w)
    o_gpu = oracle.overlap(sel.page_idx[0, :16].cpu().numpy(), idx[0], 16)
    okp = oracle.KPool.of(w)
    vb = oracle.pool_blocks(okp, w.seq_len, w.block_offsets, w.block_table)
    r = oracle.score_select(np.stack([vb[b] for b in range(w.total_blocks)]),
                            oracle.pool_anchor(okp, w.block_table, int(w.seq_len[0]), w.window), w.select)
    att = oracle.attention_blocks(okp, w.block_table, int(w.seq_len[0]), q[0], 1 / 8)
    oatt, _ = oracle.select(att, hierarchical=0, k_page=16)

    def gap16(x):
        v = np.sort(np.asarray(x, np.float64))[::-1]
        return v[15] - v[16]

    if min(gap16(r["aff_pages"]) / r["aff_pages"].max(), gap16(att) / att.max()) > 1e-4:
        assert o_gpu == oracle.overlap(r["idx"], oatt, 16)


def test_attention_bad_block_table_entry_raises_flag():
    say("attention bad table")
    w = ragged_workload(74, 2, 1, 2, 64, 16, 0, 0, lengths=[40, 40])
    kp, seqs = upload(w)
    seqs.tensors[2][1] = w.P + 5  # block 1 of sequence 0
    out = torch.zeros((2, 3), dtype=torch.float32, device="cuda")
    idx = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    q = torch.randn((2, 1, 2, 64), device="cuda")
    kka.kka_attention_topk(kp, seqs, q, 2, out, 3, k=2, idx_out=idx)
    assert kka.kka_device_error() == kka.DEVERR_BLOCK_TABLE
    o = out.cpu().numpy()
    assert o[0, 1] == 0.0  # the bad block holds no mass
    assert abs(float(o[1].sum()) - 1.0) < 1e-5


def test_attention_128k_four_layers_full_parity():
    """The benchmark's 131072-token sequence (8192 blocks of 16, permuted
    physical blocks) at 4 layers: every block against the oracle."""
    say("attention 128K x 4 layers: generate")
    w = synth.config3(0, L=4)
    q = synth.planted_queries(w, 28, 12.0, 1.0)[None]
    scale = 1 / math.sqrt(128)
    say("attention 128K x 4 layers: run")
    out, idx, sc, cnt = run_attention(w, q, 28, 64, scale)
    say("attention 128K x 4 layers: oracle")
    check(w, q, 28, 64, scale, out, idx, sc, cnt, "c3 L=4")


@pytest.mark.timeout(600)
def test_attention_128k_full_size_properties():
    """28 layers x 4 KV heads x 128, 28 query heads, 131072 tokens: unit
    total mass, non-negative scores, selection bit-exact on the GPU's
    scores, and the anchor topic's run of 32 blocks inside the top 64."""
    say("attention 128K x 28 layers: generate")
    w = synth.config3(0)
    q = synth.planted_queries(w, 28, 12.0, 1.0)[None]
    say("attention 128K x 28 layers: run")
    out, idx, sc, cnt = run_attention(w, q, 28, 64, 1 / math.sqrt(128))
    s = out[0, :w.total_blocks]
    assert (s >= 0).all()
    assert abs(float(s.astype(np.float64).sum()) - 1.0) < 1e-4
    ridx, rsc = oracle.select(s, hierarchical=0, k_page=64)
    np.testing.assert_array_equal(idx[0], ridx)
    np.testing.assert_array_equal(sc[0].view(np.uint32), rsc.view(np.uint32))
    run = w.extra["anchor_run"]
    assert set(range(run * 32, run * 32 + 32)) <= set(idx[0].tolist())


def _attention_shape(rng):
    """One random shape that one of the two logit kernels accepts (the rules of
    kka_attention_topk), and the kernel it goes to."""
    while True:
        D = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
        H = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.integers(1, 17))
        B = int(rng.choice([1, 2, 4, 8, 16, 24, 32, 48, 64, 5, 12]))
        mfma = D in (32, 64, 128, 256) and G <= 16 and (16 % B == 0 or B % 16 == 0)
        vector = G <= 8 and (D // 8) * H <= 256 and H * G * (B + 1) <= 15360
        if mfma or vector:
            return D, H, G, B, "matrix" if mfma else "vector"


@pytest.mark.parametrize("seed", range(12))
def test_attention_random_shapes(seed):
    """Seeded sweep over shapes both logit kernels take (head_dim 8-512, KV
    heads 1-8, 1-16 query heads per KV head, blocks of 1-64 tokens, 1-12 ragged
    sequences with empty ones and ragged tails, k 0-40, scale 0.25-2 over
    sqrt(head_dim)): block masses and the top-k against the oracle."""
    rng = np.random.default_rng(5000 + seed)
    D, H, G, B, path = _attention_shape(rng)
    L = int(rng.integers(1, 7))
    S = int(rng.integers(1, 13))
    Hq = H * G
    max_len = max(1, min(900, (2 << 20) // (L * H * D * S)))
    lengths = rng.integers(0, max_len + 1, S)
    if S > 1:
        lengths[int(rng.integers(0, S))] = 0
    k = int(rng.integers(0, 41))
    scale = float(rng.uniform(0.25, 2.0)) / math.sqrt(D)
    say(f"attention random seed={seed} {path} D={D} H={H} G={G} B={B} L={L} S={S} max_len={max_len} k={k}")
    w = ragged_workload(5100 + seed, S, L, H, D, B, 0, 0, lengths=lengths)
    q = rng.standard_normal((w.S, L, Hq, D)).astype(np.float32)
    out, idx, sc, cnt = run_attention(w, q, Hq, k, scale)
    if k == 0:
        okp = oracle.KPool.of(w)
        for s in range(w.S):
            T = int(w.seq_len[s])
            tab = oracle.seq_table(w.block_offsets, w.block_table, s)
            ref = oracle.attention_blocks(okp, tab, T, q[s], scale)
            np.testing.assert_allclose(out[s, :len(ref)], ref, rtol=RTOL, atol=ATOL_MASS, err_msg=f"s={s}")
    else:
        check(w, q, Hq, k, scale, out, idx, sc, cnt, f"random seed={seed}")
