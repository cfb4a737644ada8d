"""Pins for the CPU oracle, checked against things other than the oracle.

Each test names what fixes the expected value: a hand-worked example
(tests/golden/), a closed form, an invariant, an independent library routine
(numpy / scipy written differently from the oracle's C loops), or brute force
over all subsets on tiny inputs.  Page citations refer to "Key-Key Semantic
Affinity: Key vectors replace attention scores for KV-cache importance"
(10100.com).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def kp_from_f32(keys):
    """keys [L][P][B][H][D] fp32 -> oracle KPool over their bf16 rounding."""
    keys = np.asarray(keys, dtype=np.float32)
    L, P, B, H, D = keys.shape
    return oracle.KPool(synth.to_bf16_bits(keys), L, H, D, B, P)


def bf16_round(x):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(np.asarray(x, dtype=np.float32)))


def rand_keys(rng, L, P, B, H, D, scale=1.0):
    return bf16_round(rng.standard_normal((L, P, B, H, D)).astype(np.float32) * scale)


# ------------------------------------------------------------ hand examples

def test_w1_hand_example():
    """Section 2.2 steps 1-3 and section 3.3 under the stated readings."""
    g = json.load(open(os.path.join(GOLDEN, "w1_pool_weights_affinity.json")))
    tol = g["tolerance"]
    keys = np.zeros((1, 1, 2, 2, 2), dtype=np.float32)
    for t, row in enumerate(g["keys_t_h"]):
        for h, v in enumerate(row):
            keys[0, 0, t, h, :] = v
    kp = kp_from_f32(keys)
    ex = g["expected"]
    w = oracle.head_weights(kp, np.array([0]), 2)
    np.testing.assert_allclose(w, ex["weights"], atol=tol)
    vu = oracle.pool_block(kp, 0, 2)
    vw = oracle.pool_block(kp, 0, 2, w)
    np.testing.assert_allclose(vu, ex["vb_uniform"], atol=tol)
    np.testing.assert_allclose(vw, ex["vb_weighted"], atol=tol)
    au = oracle.pool_anchor(kp, np.array([0]), 2, 1)
    aw = oracle.pool_anchor(kp, np.array([0]), 2, 1, w)
    np.testing.assert_allclose(au, ex["anchor_uniform_w1"], atol=tol)
    np.testing.assert_allclose(aw, ex["anchor_weighted_w1"], atol=tol)
    e = np.eye(2, dtype=np.float32)
    np.testing.assert_allclose(oracle.affinity(np.stack([vu]), e[0])[0], ex["aff_uniform_e0"], atol=tol)
    np.testing.assert_allclose(oracle.affinity(np.stack([vu]), e[1])[0], ex["aff_uniform_e1"], atol=tol)
    np.testing.assert_allclose(oracle.affinity(np.stack([vw]), e[0])[0], ex["aff_weighted_e0"], atol=tol)
    np.testing.assert_allclose(oracle.affinity(np.stack([vw]), e[1])[0], ex["aff_weighted_e1"], atol=tol)
    np.testing.assert_allclose(oracle.affinity(np.stack([vu]), au)[0], ex["aff_uniform_anchor"], atol=tol)
    np.testing.assert_allclose(oracle.affinity(np.stack([vw]), aw)[0], ex["aff_weighted_anchor"], atol=tol)


def test_w2_hierarchy_example():
    """Section 5.1 (grid = mean of chunks; masking) and section 5.2 step 4."""
    g = json.load(open(os.path.join(GOLDEN, "w2_hierarchy.json")))
    tol = g["tolerance"]
    pages = np.array(g["pages"], dtype=np.float32)
    anchor = np.array(g["anchor"], dtype=np.float32)
    ppc, cpg = g["pages_per_chunk"], g["chunks_per_grid"]
    chunks, grids = oracle.build_levels(pages, ppc, cpg)
    ex = g["expected"]
    ap = oracle.affinity(pages, anchor)
    ac = oracle.affinity(chunks, anchor)
    ag = oracle.affinity(grids, anchor)
    np.testing.assert_allclose(ap, ex["aff_pages"], atol=tol)
    np.testing.assert_allclose(ac, ex["aff_chunks"], atol=tol)
    np.testing.assert_allclose(ag, ex["aff_grids"], atol=tol)
    for key, kp_ in (("hier_k1_1_2", 2), ("hier_k1_1_4", 4)):
        idx, sc = oracle.select(ap, ac, ag, hierarchical=1, k_grid=1, k_chunk=1, k_page=kp_,
                                pages_per_chunk=ppc, chunks_per_grid=cpg)
        assert idx.tolist() == ex[key]["idx"]
        np.testing.assert_allclose(sc, ex[key]["score"], atol=tol)
    for key, k in (("flat_k2", 2), ("flat_k7", 7)):
        idx, _ = oracle.select(ap, hierarchical=0, k_page=k)
        assert idx.tolist() == ex[key]["idx"]


# ------------------------------------------------------------ pooling pins

@pytest.mark.parametrize("shape", [(3, 2, 4, 2, 16), (2, 3, 16, 4, 8)])
def test_constant_keys_pool_to_constant(shape):
    """Closed form: the mean of identical vectors is that vector; with every
    temporal variance 0 the weights fall back to uniform."""
    L, P, B, H, D = shape
    c = bf16_round(np.linspace(-2, 3, D).astype(np.float32))
    keys = np.broadcast_to(c, (L, P, B, H, D)).copy()
    kp = kp_from_f32(keys)
    table = np.arange(P, dtype=np.int32)
    T = P * B - 3
    w = oracle.head_weights(kp, table, T)
    np.testing.assert_array_equal(w, np.float32(1.0 / (L * H)))
    for p in range(P):
        for n in (1, B):
            np.testing.assert_allclose(oracle.pool_block(kp, p, n), c, rtol=1e-7, atol=0)
            np.testing.assert_allclose(oracle.pool_block(kp, p, n, w), c, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(oracle.pool_anchor(kp, table, T, 5), c, rtol=1e-7)


def test_pool_is_linear_in_keys():
    """Invariant: pool(a*K1 + b*K2) = a*pool(K1) + b*pool(K2) for fixed weights
    (small integer keys so every combination is exact in bf16)."""
    rng = np.random.default_rng(1)
    L, P, B, H, D = 3, 2, 8, 2, 16
    k1 = rng.integers(-8, 9, (L, P, B, H, D)).astype(np.float32)
    k2 = rng.integers(-8, 9, (L, P, B, H, D)).astype(np.float32)
    a, b = 2.0, -3.0
    w = rng.random(L * H).astype(np.float32)
    w /= w.sum()
    for weights in (None, w):
        for n in (B, 5):
            p1 = oracle.pool_block(kp_from_f32(k1), 1, n, weights).astype(np.float64)
            p2 = oracle.pool_block(kp_from_f32(k2), 1, n, weights).astype(np.float64)
            p3 = oracle.pool_block(kp_from_f32(a * k1 + b * k2), 1, n, weights).astype(np.float64)
            np.testing.assert_allclose(p3, a * p1 + b * p2, rtol=1e-6, atol=1e-5)


def test_pool_matches_numpy_mean():
    """Library routine: uniform v_b is numpy's float64 mean over (layer,
    token, head) of the stored bf16 keys; weighted v_b is the weighted sum of
    numpy per-head token means."""
    rng = np.random.default_rng(2)
    L, P, B, H, D = 4, 5, 16, 4, 32
    keys = rand_keys(rng, L, P, B, H, D, 2.0)
    kp = kp_from_f32(keys)
    w = rng.random(L * H).astype(np.float32)
    w /= w.sum()
    for p in range(P):
        for n in (B, 1, 7):
            x = keys[:, p, :n].astype(np.float64)  # [L][n][H][D]
            np.testing.assert_allclose(oracle.pool_block(kp, p, n), x.mean(axis=(0, 1, 2)), rtol=0, atol=1e-6)
            head_means = x.mean(axis=1)  # [L][H][D]
            ref = np.einsum("lh,lhd->d", w.reshape(L, H).astype(np.float64), head_means)
            np.testing.assert_allclose(oracle.pool_block(kp, p, n, w), ref, rtol=0, atol=1e-6)


def test_token_order_invariance():
    """Invariant: permuting the tokens inside a block changes nothing (the
    oracle sums exactly in fp64, so the bits agree; the stated bound is 1 ulp)."""
    rng = np.random.default_rng(3)
    L, P, B, H, D = 3, 2, 16, 2, 32
    keys = rand_keys(rng, L, P, B, H, D)
    n = 11
    perm = np.concatenate([rng.permutation(n), np.arange(n, B)])
    keys2 = keys.copy()
    keys2[:, 0] = keys[:, 0][:, perm]
    w = rng.random(L * H).astype(np.float32)
    w /= w.sum()
    for weights in (None, w):
        a = oracle.pool_block(kp_from_f32(keys), 0, n, weights)
        b = oracle.pool_block(kp_from_f32(keys2), 0, n, weights)
        ulp = np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1


def test_physical_permutation_invariance():
    """Invariant: moving blocks to other physical slots behind the table gives
    bit-identical block vectors and anchors."""
    rng = np.random.default_rng(4)
    L, P, B, H, D = 2, 6, 8, 2, 16
    keys = rand_keys(rng, L, P, B, H, D)
    perm = rng.permutation(P)
    moved = np.empty_like(keys)
    moved[:, perm] = keys  # logical block i now sits in physical slot perm[i]
    kp0, kp1 = kp_from_f32(keys), kp_from_f32(moved)
    T = P * B - 3
    t0 = np.arange(P, dtype=np.int32)
    t1 = perm.astype(np.int32)
    w0 = oracle.head_weights(kp0, t0, T)
    w1 = oracle.head_weights(kp1, t1, T)
    np.testing.assert_array_equal(w0, w1)
    for i in range(P):
        n = min(B, T - i * B)
        np.testing.assert_array_equal(oracle.pool_block(kp0, i, n), oracle.pool_block(kp1, perm[i], n))
        np.testing.assert_array_equal(oracle.pool_block(kp0, i, n, w0), oracle.pool_block(kp1, perm[i], n, w1))
    np.testing.assert_array_equal(oracle.pool_anchor(kp0, t0, T, 13), oracle.pool_anchor(kp1, t1, T, 13))


def test_pure_noise_pool_variance():
    """Closed-form statistic (section 3.1: independent per-token noise
    averages out; section 3.2: the deviation shrinks with the block size):
    for N(0, v_lh) keys, uniform v_b entries are N(0, mean(v)/(n_b*L*H)) and
    weighted ones N(0, sum w^2 v / n_b).  Sample variance within 3% over
    131072 entries (its relative standard error is 0.4%)."""
    L, H, D, B, n_blocks = 2, 2, 64, 16, 2048
    v = np.array([0.5, 1.0, 2.0, 4.0], dtype=np.float64)
    std = np.sqrt(v).astype(np.float32)
    off = np.array([0, n_blocks], dtype=np.int32)
    table = np.arange(n_blocks, dtype=np.int32)
    seq_len = np.array([n_blocks * B], dtype=np.int32)
    k = synth._gen_kpool(L, H, D, B, n_blocks, seq_len, off, table, None, None, 0.0, 0.0, std, None, 7)
    kp = oracle.KPool(k, L, H, D, B, n_blocks)
    w = (v / v.sum()).astype(np.float32)
    uni = np.stack([oracle.pool_block(kp, p, B) for p in range(n_blocks)]).astype(np.float64)
    wtd = np.stack([oracle.pool_block(kp, p, B, w) for p in range(n_blocks)]).astype(np.float64)
    exp_u = v.mean() / (B * L * H)
    exp_w = float(np.sum(w.astype(np.float64) ** 2 * v)) / B
    assert abs(uni.var() / exp_u - 1) < 0.03
    assert abs(wtd.var() / exp_w - 1) < 0.03
    assert abs(uni.mean()) < 4 * math.sqrt(exp_u / uni.size)


# ------------------------------------------------------------ weight pins

def test_weights_match_numpy_variance():
    """Library routine: per-head temporal variance = mean over d of
    numpy.var over the sequence's tokens, normalised to sum 1."""
    rng = np.random.default_rng(5)
    L, P, B, H, D = 3, 5, 8, 4, 16
    scales = rng.uniform(0.2, 3.0, (L, 1, 1, H, 1)).astype(np.float32)
    keys = bf16_round(rng.standard_normal((L, P, B, H, D)).astype(np.float32) * scales + 0.7)
    table = rng.permutation(P).astype(np.int32)
    kp = kp_from_f32(keys)
    T = P * B - 5
    w = oracle.head_weights(kp, table, T).astype(np.float64)
    x = keys[:, table].reshape(L, P * B, H, D)[:, :T].astype(np.float64)  # [L][T][H][D]
    var = np.var(x, axis=1).mean(axis=-1).reshape(L * H)
    np.testing.assert_allclose(w, var / var.sum(), rtol=1e-6)


def test_weights_equal_variances_are_uniform():
    """Special case: when every head carries the same keys, the weights are
    uniform and weighted pooling equals uniform pooling."""
    rng = np.random.default_rng(6)
    L, P, B, H, D = 2, 3, 8, 4, 16
    base = rand_keys(rng, 1, P, B, 1, D)
    keys = np.broadcast_to(base, (L, P, B, H, D)).copy()
    kp = kp_from_f32(keys)
    table = np.arange(P, dtype=np.int32)
    w = oracle.head_weights(kp, table, P * B)
    np.testing.assert_allclose(w, 1.0 / (L * H), rtol=1e-7)
    for p in range(P):
        np.testing.assert_allclose(oracle.pool_block(kp, p, B, w), oracle.pool_block(kp, p, B), rtol=1e-6,
                                   atol=1e-7)


def test_weights_ignore_constant_offset():
    """Invariant behind the temporal reading (section 3.3: low-variance heads
    act like positional bias): adding a vector that is constant over tokens
    to one head leaves every weight unchanged."""
    rng = np.random.default_rng(8)
    L, P, B, H, D = 2, 4, 8, 2, 16
    keys = rng.integers(-16, 17, (L, P, B, H, D)).astype(np.float32) / 8.0
    shifted = keys.copy()
    shifted[1, :, :, 0, :] += rng.integers(-4, 5, D).astype(np.float32)
    table = np.arange(P, dtype=np.int32)
    w0 = oracle.head_weights(kp_from_f32(keys), table, P * B)
    w1 = oracle.head_weights(kp_from_f32(shifted), table, P * B)
    np.testing.assert_allclose(w1, w0, rtol=1e-7)


# ------------------------------------------------------------ anchor pins

def test_anchor_aligned_window_is_block_vector():
    """Special case: a window of exactly the last full block equals that
    block's vector (same tokens, same sums), uniform and weighted."""
    rng = np.random.default_rng(9)
    L, P, B, H, D = 3, 4, 8, 2, 16
    keys = rand_keys(rng, L, P, B, H, D)
    kp = kp_from_f32(keys)
    table = np.array([2, 0, 3, 1], dtype=np.int32)
    T = P * B
    w = oracle.head_weights(kp, table, T)
    np.testing.assert_array_equal(oracle.pool_anchor(kp, table, T, B), oracle.pool_block(kp, table[-1], B))
    np.testing.assert_array_equal(oracle.pool_anchor(kp, table, T, B, w), oracle.pool_block(kp, table[-1], B, w))


def test_anchor_straddling_window_matches_numpy():
    """Library routine: a window spanning blocks is numpy's mean over the
    last W tokens gathered through the table; W > T clips to T."""
    rng = np.random.default_rng(10)
    L, P, B, H, D = 2, 4, 8, 2, 16
    keys = rand_keys(rng, L, P, B, H, D)
    kp = kp_from_f32(keys)
    table = np.array([3, 1, 0, 2], dtype=np.int32)
    T = 3 * B + 3
    flat = keys[:, table].reshape(L, P * B, H, D).astype(np.float64)
    for W in (1, 5, 11, 40):
        n = min(W, T)
        ref = flat[:, T - n:T].mean(axis=(0, 1, 2))
        np.testing.assert_allclose(oracle.pool_anchor(kp, table, T, W), ref, atol=1e-6)
    np.testing.assert_array_equal(oracle.pool_anchor(kp, table, 0, 4), np.zeros(D, np.float32))


# ------------------------------------------------------------ level pins

def test_levels_full_grid_is_mean_of_pages():
    """Closed form (section 5.1): for a full grid, the mean of its chunk
    means equals the mean of its ppc*cpg pages; chunks are numpy means."""
    rng = np.random.default_rng(11)
    ppc, cpg, D = 4, 3, 16
    n_p = ppc * cpg * 5
    pages = rng.standard_normal((n_p, D)).astype(np.float32)
    chunks, grids = oracle.build_levels(pages, ppc, cpg)
    p64 = pages.astype(np.float64)
    np.testing.assert_allclose(chunks, p64.reshape(-1, ppc, D).mean(axis=1), atol=1e-6)
    np.testing.assert_allclose(grids, p64.reshape(-1, ppc * cpg, D).mean(axis=1), atol=1e-6)


def test_levels_ragged_tail_uses_present_children():
    rng = np.random.default_rng(12)
    ppc, cpg, D = 4, 3, 8
    n_p = ppc * cpg * 2 + 1  # 7 chunks, the last with 1 page; 3 grids, the last with 1 chunk
    pages = rng.standard_normal((n_p, D)).astype(np.float32)
    chunks, grids = oracle.build_levels(pages, ppc, cpg)
    assert chunks.shape == (7, D) and grids.shape == (3, D)
    np.testing.assert_allclose(chunks[-1], pages[-1], atol=1e-7)
    np.testing.assert_allclose(chunks[-2], pages[-5:-1].astype(np.float64).mean(0), atol=1e-6)
    np.testing.assert_allclose(grids[-1], chunks[-1], atol=1e-7)
    np.testing.assert_allclose(grids[1], chunks[3:6].astype(np.float64).mean(0), atol=1e-6)


# ------------------------------------------------------------ affinity pins

def test_affinity_closed_forms():
    """Section 3.2: related vectors score 1, unrelated (orthogonal) 0.5 after
    the [0, 1] map, opposite 0; the score ignores positive scaling."""
    rng = np.random.default_rng(13)
    D = 128
    v = rng.standard_normal(D).astype(np.float32)
    u = rng.standard_normal(D)
    u -= u.dot(v) / v.astype(np.float64).dot(v) * v
    u = u.astype(np.float32)
    rows = np.stack([v, -v, u, 3.5 * v, np.zeros(D, np.float32)])
    a = oracle.affinity(rows, v)
    assert abs(a[0] - 1) <= 1e-7 and a[1] == 0.0 and abs(a[2] - 0.5) <= 1e-7
    assert abs(a[3] - 1) <= 1e-7 and a[4] == 0.5
    assert not np.signbit(a[1])
    w = rng.standard_normal(D).astype(np.float32)
    base = oracle.affinity(np.stack([w]), v)[0]
    scaled = oracle.affinity(np.stack([np.float32(0.37) * w]), np.float32(12.0) * v)[0]
    assert abs(base - scaled) <= 1e-7
    assert oracle.affinity(np.stack([v]), np.zeros(D, np.float32))[0] == 0.5


def test_affinity_matches_scipy_cosine():
    """Library routine: (1 + (1 - scipy cosine distance)) / 2."""
    from scipy.spatial.distance import cosine
    rng = np.random.default_rng(14)
    rows = rng.standard_normal((50, 64)).astype(np.float32)
    a = rng.standard_normal(64).astype(np.float32)
    got = oracle.affinity(rows, a)
    ref = np.array([(2.0 - cosine(r.astype(np.float64), a.astype(np.float64))) / 2 for r in rows])
    np.testing.assert_allclose(got, ref, atol=1e-7)


# ------------------------------------------------------------ selection pins

def brute_top(scores, k):
    """The unique size-k subset whose every member beats every non-member
    under (score desc, index asc), found by enumerating all subsets, then
    listed in that order."""
    n = len(scores)
    beats = lambda i, j: scores[i] > scores[j] or (scores[i] == scores[j] and i < j)
    k = min(k, n)
    found = []
    for sub in itertools.combinations(range(n), k):
        rest = set(range(n)) - set(sub)
        if all(beats(i, j) for i in sub for j in rest):
            found.append(sub)
    assert len(found) == 1
    sub = list(found[0])
    # order inside the subset: count how many members each one beats
    return sorted(sub, key=lambda i: -sum(beats(i, j) for j in sub))


def test_select_flat_brute_force():
    rng = np.random.default_rng(15)
    vals = np.array([0.0, 0.25, 0.5, 0.75, 1.0], dtype=np.float32)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        s = vals[rng.integers(0, len(vals), n)]
        k = int(rng.integers(0, n + 2))
        idx, sc = oracle.select(s, hierarchical=0, k_page=k)
        ref = brute_top(s.tolist(), k)
        assert idx.tolist() == ref
        np.testing.assert_array_equal(sc, s[ref])


def test_select_hierarchical_brute_force():
    """Brute force per level with the masks of section 5.1 recomputed from
    the brute-force parent choice."""
    rng = np.random.default_rng(16)
    vals = np.array([0.0, 0.2, 0.5, 0.6, 0.9, 1.0], dtype=np.float32)
    for trial in range(150):
        ppc, cpg = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        n_p = int(rng.integers(1, 13))
        n_c = -(-n_p // ppc)
        n_g = -(-n_c // cpg)
        ap = vals[rng.integers(0, len(vals), n_p)]
        ac = vals[rng.integers(0, len(vals), n_c)]
        ag = vals[rng.integers(0, len(vals), n_g)]
        kg, kc, kp_ = (int(rng.integers(0, n_g + 1)), int(rng.integers(0, n_c + 1)), int(rng.integers(0, n_p + 2)))
        gsel = set(brute_top(ag.tolist(), kg))
        cs = [float(ac[j]) if (j // cpg) in gsel else 0.0 for j in range(n_c)]
        csel = set(brute_top(cs, kc))
        ps = [float(ap[i]) if (i // ppc) in csel else 0.0 for i in range(n_p)]
        ref = brute_top(ps, kp_)
        idx, sc = oracle.select(ap, ac, ag, hierarchical=1, k_grid=kg, k_chunk=kc, k_page=kp_,
                                pages_per_chunk=ppc, chunks_per_grid=cpg)
        assert idx.tolist() == ref
        np.testing.assert_array_equal(sc, np.array([ps[i] for i in ref], dtype=np.float32))


def test_select_full_keep_equals_flat():
    """Special case: keeping every grid and chunk makes the hierarchy flat."""
    rng = np.random.default_rng(17)
    n_p, ppc, cpg = 300, 16, 4
    n_c = -(-n_p // ppc)
    n_g = -(-n_c // cpg)
    ap = rng.random(n_p).astype(np.float32)
    ac = rng.random(n_c).astype(np.float32)
    ag = rng.random(n_g).astype(np.float32)
    h = oracle.select(ap, ac, ag, hierarchical=1, k_grid=n_g, k_chunk=n_c, k_page=40, pages_per_chunk=ppc,
                      chunks_per_grid=cpg)
    f = oracle.select(ap, hierarchical=0, k_page=40)
    np.testing.assert_array_equal(h[0], f[0])
    np.testing.assert_array_equal(h[1], f[1])


def test_select_flat_matches_lexsort():
    """Library routine: numpy lexsort on (index, -score)."""
    rng = np.random.default_rng(18)
    s = np.round(rng.random(5000) * 50).astype(np.float32) / 50
    for k in (0, 1, 64, 4999, 5000, 6000):
        idx, sc = oracle.select(s, hierarchical=0, k_page=k)
        ref = np.lexsort((np.arange(len(s)), -s.astype(np.float64)))[:k]
        np.testing.assert_array_equal(idx, ref)
        np.testing.assert_array_equal(sc, s[ref])


# ------------------------------------------------------------ end to end

def oracle_pipeline(w, weights=None):
    kp = oracle.KPool.of(w)
    vb = oracle.pool_blocks(kp, w.seq_len, w.block_offsets, w.block_table, weights)
    out = []
    for s in range(w.S):
        lo, hi = int(w.block_offsets[s]), int(w.block_offsets[s + 1])
        pages = np.stack([vb[b] for b in range(lo, hi)])
        a = oracle.pool_anchor(kp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]),
                               w.window, None if weights is None else weights[s])
        out.append(oracle.score_select(pages, a, w.select))
    return out


@pytest.mark.slow
def test_recovery_config1_mean_precision():
    """0.5B shape, 8 balanced topics: mean fraction of the 16 selected blocks
    that carry the anchor topic, over seeds 0-63, at least 0.95."""
    precs = []
    for seed in range(64):
        w = synth.config1(seed)
        r = oracle_pipeline(w)[0]
        precs.append(np.mean(w.block_topic[0][r["idx"]] == w.anchor_topic[0]))
    assert np.mean(precs) >= 0.95, np.mean(precs)


@pytest.mark.slow
def test_recovery_config2():
    """7B shape, blocks of 128: the 8 anchor-topic blocks come first among the 32."""
    w = synth.config2(0)
    r = oracle_pipeline(w)[0]
    top = w.block_topic[0][r["idx"][:8]]
    assert (top == w.anchor_topic[0]).all()
    assert len(r["idx"]) == 32


@pytest.mark.slow
def test_recovery_config3_reduced():
    """7B head shape with runs of 32 blocks (2048 blocks, 8 layers): every
    page of the planted anchor run is among the 64 selected."""
    w = synth.config3(0, n_blocks=2048, L=8)
    r = oracle_pipeline(w)[0]
    run = w.extra["anchor_run"]
    planted = set(range(run * 32, run * 32 + 32))
    assert planted <= set(r["idx"].tolist())


@pytest.mark.slow
def test_recovery_config4():
    """Serving scale: all 64 selected pages of every sequence carry its anchor topic."""
    v = synth.config4(0)
    for s in range(v.vb.shape[0]):
        r = oracle.score_select(v.vb[s], v.anchors[s], v.select)
        assert len(r["idx"]) == 64
        assert (v.page_topic[s][r["idx"]] == v.anchor_topic[s]).all()


# ------------------------------------------------------------ stability filter (section 5.3)

def test_w3_stability_example():
    """The page's two worked values (1/20 = 0.05 for a single spike, 1.0 for
    twenty steps above 0.6) and three blocks worked by hand."""
    g = json.load(open(os.path.join(GOLDEN, "w3_stability.json")))
    for blk in g["blocks"]:
        hist = np.asarray(blk["steps"], np.float32)[:, None]
        score, bits = oracle.stability(hist, g["window"], g["theta"])
        assert score[0] == np.float32(blk["expected_score"]), blk["name"]
        assert int(bits[0]) == blk["expected_bits"], blk["name"]


def test_stability_closed_forms():
    W = 20
    # fewer steps than the window: the missing steps count as not high
    hist = np.full((7, 1), 0.9, np.float32)
    assert oracle.stability(hist, W, 0.5)[0][0] == np.float32(7 / 20)
    # W = 1 sees only the newest step
    hist = np.array([[0.9], [0.9], [0.1]], np.float32)
    assert oracle.stability(hist, 1, 0.5)[0][0] == 0.0
    assert oracle.stability(hist[:2], 1, 0.5)[0][0] == 1.0
    # a full 32-step window of high steps fills the word
    score, bits = oracle.stability(np.full((40, 3), 0.75, np.float32), 32, 0.5)
    assert (score == 1.0).all() and (bits == 0xFFFFFFFF).all()
    # no steps yet
    score, bits = oracle.stability(np.zeros((0, 4), np.float32), 20, 0.5)
    assert (score == 0).all() and (bits == 0).all()


def test_stability_matches_box_filter():
    """Every prefix of a random history against a numpy box filter (a
    length-W convolution of the high-step indicator) divided by W."""
    rng = np.random.default_rng(31)
    n_steps, n = 45, 9
    for W, theta in ((20, 0.5), (1, 0.5), (32, 0.3), (7, 0.65)):
        hist = rng.uniform(0, 1, (n_steps, n)).astype(np.float32)
        high = (hist > np.float32(theta)).astype(np.int64)
        for t in range(n_steps + 1):
            score, bits = oracle.stability(hist[:t], W, theta)
            if t == 0:
                assert (score == 0).all()
                continue
            windowed = np.stack([np.convolve(high[:t, b], np.ones(W, np.int64))[t - 1] for b in range(n)])
            np.testing.assert_array_equal(score, (windowed / W).astype(np.float32))
            # bit i of the word is the step i before the newest
            for i in range(min(W, t)):
                np.testing.assert_array_equal((bits >> np.uint32(i)) & np.uint32(1), high[t - 1 - i])


def test_stability_shift_invariant_and_threshold_monotone():
    """One more step shifts the window word left by one and brings in the new
    step's bit; raising theta never raises a score."""
    rng = np.random.default_rng(32)
    hist = rng.uniform(0, 1, (30, 50)).astype(np.float32)
    W = 20
    mask = np.uint32((1 << W) - 1)
    for t in range(1, 30):
        _, before = oracle.stability(hist[:t], W, 0.5)
        _, after = oracle.stability(hist[:t + 1], W, 0.5)
        new = (hist[t] > np.float32(0.5)).astype(np.uint32)
        np.testing.assert_array_equal(after, ((before << np.uint32(1)) | new) & mask)
    prev = None
    for theta in (0.0, 0.25, 0.5, 0.75, 1.0):
        score, _ = oracle.stability(hist, W, theta)
        if prev is not None:
            assert (score <= prev).all()
        prev = score
    assert (oracle.stability(hist, W, 1.0)[0] == 0).all()  # affinities never exceed 1


# ------------------------------------------------------------ attention mass per block (section 3.3)

def _kp_const(L, H, D, B, P, fill):
    keys = np.zeros((L, P, B, H, D), np.float32)
    keys[...] = fill
    return kp_from_f32(keys)


def test_attention_uniform_cases():
    """Equal logits give every token 1/T, so a block holds n_b / T: constant
    keys, a zero query, and scale 0 all reduce to that."""
    L, H, D, B, P, T = 2, 2, 16, 4, 5, 18
    rng = np.random.default_rng(60)
    table = np.array([3, 0, 4, 1, 2], np.int32)
    expect = np.array([4, 4, 4, 4, 2], np.float64) / T
    kp = _kp_const(L, H, D, B, P, 0.75)
    q = rng.standard_normal((L, 4, D)).astype(np.float32)
    np.testing.assert_allclose(oracle.attention_blocks(kp, table, T, q, 0.25), expect, rtol=0, atol=1e-7)
    kp2 = kp_from_f32(rand_keys(rng, L, P, B, H, D))
    np.testing.assert_allclose(oracle.attention_blocks(kp2, table, T, np.zeros_like(q), 0.25), expect, atol=1e-7)
    np.testing.assert_allclose(oracle.attention_blocks(kp2, table, T, q, 0.0), expect, atol=1e-7)


def test_attention_two_token_closed_form():
    """Two tokens, one head: p0 = 1 / (1 + exp(scale * (b - a)))."""
    D = 8
    keys = np.zeros((1, 2, 1, 1, D), np.float32)
    a, b = 1.5, -0.75
    keys[0, 0, 0, 0, 0] = a
    keys[0, 1, 0, 0, 0] = b
    kp = kp_from_f32(keys)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    for scale in (0.1, 1.0, 3.0):
        got = oracle.attention_blocks(kp, np.array([0, 1], np.int32), 2, q, scale)
        p0 = 1.0 / (1.0 + math.exp(scale * (b - a)))
        np.testing.assert_allclose(got, [p0, 1.0 - p0], rtol=1e-7, atol=0)


def test_attention_shift_invariance_and_unit_mass():
    """Adding one vector to every key of a (layer, KV head) shifts all its
    logits equally and leaves the softmax unchanged; the block masses sum
    to 1."""
    rng = np.random.default_rng(61)
    L, H, D, B, P, T = 2, 2, 16, 4, 6, 22
    base = np.round(rng.standard_normal((L, P, B, H, D)) * 4).astype(np.float32)  # small integers: exact in bf16
    shift = np.round(rng.standard_normal((L, 1, 1, H, D)) * 3).astype(np.float32)
    table = np.array([5, 2, 0, 4, 1, 3], np.int32)
    q = (rng.standard_normal((L, 4, D)) * 0.3).astype(np.float32)
    a = oracle.attention_blocks(kp_from_f32(base), table, T, q, 0.5)
    b = oracle.attention_blocks(kp_from_f32(base + shift), table, T, q, 0.5)
    np.testing.assert_allclose(b, a, rtol=1e-6, atol=1e-9)
    assert abs(float(np.sum(a, dtype=np.float64)) - 1.0) < 1e-6


def test_attention_gqa_head_mapping():
    """Query heads 0-1 read KV head 0 and heads 2-3 read KV head 1 (four
    query heads over two KV heads).  KV head 0 matches the query only at
    token 0, KV head 1 only at token 1; with only query head 1 non-zero and
    a large scale, query head 1 puts all its mass on token 0 and the other
    three spread evenly: block 0 holds (1 + 3/T) / 4."""
    D, T = 8, 4
    keys = np.zeros((1, T, 1, 2, D), np.float32)
    keys[0, 0, 0, 0, 0] = 1.0
    keys[0, 1, 0, 1, 0] = 1.0
    kp = kp_from_f32(keys)
    q = np.zeros((1, 4, D), np.float32)
    q[0, 1, 0] = 1.0
    got = oracle.attention_blocks(kp, np.arange(T, dtype=np.int32), T, q, 200.0)
    expect = np.array([1 + 3 / T, 3 / T, 3 / T, 3 / T]) / 4
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-7)


def test_attention_matches_scipy_softmax():
    """Random pool through a table against scipy's softmax of numpy dot
    products, averaged over heads and summed per block."""
    from scipy.special import softmax
    rng = np.random.default_rng(62)
    L, H, Hq, D, B, P, T = 3, 2, 6, 32, 5, 9, 41
    keys = rand_keys(rng, L, P, B, H, D)
    table = synth.permutation(63, 1, P)[: -(-T // B)].astype(np.int32)
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    got = oracle.attention_blocks(kp_from_f32(keys), table, T, q, 1 / math.sqrt(D))
    tok = np.stack([keys[:, table[t // B], t % B] for t in range(T)], axis=1).astype(np.float64)  # [L][T][H][D]
    mass = np.zeros(T)
    for l in range(L):
        for hq in range(Hq):
            mass += softmax(tok[l, :, hq // (Hq // H)] @ q[l, hq].astype(np.float64) / math.sqrt(D))
    mass /= L * Hq
    expect = np.array([mass[b * B:(b + 1) * B].sum() for b in range(-(-T // B))])
    np.testing.assert_allclose(got, expect, rtol=1e-6, atol=1e-9)


def test_overlap_rate():
    assert oracle.overlap([3, 1, 2, 9], [2, 3, 4, 5], 4) == 0.5
    assert oracle.overlap([1, 2], [2, 1], 2) == 1.0
    assert oracle.overlap([], [], 0) == 0.0


def test_variance_weighting_raises_attention_overlap_on_positional_heads():
    """The page's quality experiment (sections 3.3 and 6.1) on a planted
    0.5B-shape workload: two thirds of the heads are positional (a component
    that drifts with position and is shared by every such head, small spread
    over the context), one third carry graded topic relevance (large
    spread), and the decode query attends through the topic heads only.  A
    plain mean is pulled toward recent blocks by the coherent positional
    heads; weighting heads by their temporal variance recovers the blocks
    attention ranks highest.  The attention top-16 is unique (graded
    relevance, no ties), and the variance-weighted top-16 overlaps it far
    more than the uniform one."""
    w, q, rel, role = synth.positional_heads_workload(0)
    kp = oracle.KPool.of(w)
    T, nb, k = int(w.seq_len[0]), w.total_blocks, 16
    att = oracle.attention_blocks(kp, w.block_table, T, q, 1.0 / np.sqrt(w.D))
    order = np.lexsort((np.arange(nb), -att.astype(np.float64)))
    assert att[order[k - 1]] > att[order[k]]  # the attention top-k is unique
    a_idx = order[:k]
    assert rel[a_idx].min() > 0.9  # attention follows the planted relevance
    ov = {}
    for mode in ("uniform", "variance"):
        wts = oracle.weights_all(kp, w.seq_len, w.block_offsets, w.block_table) if mode == "variance" else None
        vb = oracle.pool_blocks(kp, w.seq_len, w.block_offsets, w.block_table, wts)
        pages = np.stack([vb[b] for b in range(nb)])
        anc = oracle.pool_anchor(kp, w.block_table, T, w.window, None if wts is None else wts[0])
        idx, _ = oracle.select(oracle.affinity(pages, anc), hierarchical=0, k_page=k)
        ov[mode] = oracle.overlap(idx, a_idx, k)
        if wts is not None:  # topic heads weigh more than positional ones
            assert wts[0][role.ravel()].min() > 3 * wts[0][~role.ravel()].max()
    assert ov["variance"] >= 0.6 and ov["variance"] >= ov["uniform"] + 0.3, ov
