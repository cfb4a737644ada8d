"""GPU parity of the stability filter (page section 5.3) fused into the
scoring pass (kka_score_topk_stable).

Over many decode steps with a changing anchor, every present page's window
word and stability score must equal the oracle's on the GPU's own page
affinities of all steps so far (bit-exact: the decision is the fp32
affinity against theta on both sides, the score count / W rounded once).
The selection and the affinities must equal kka_score_topk's, and words of
absent pages must stay untouched.
"""
import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth

from gpu_harness import say

pytestmark = pytest.mark.gpu

SENTINEL_WORD = np.int32(0x5A5A5A5A)
SENTINEL_SCORE = -2.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


def levels(seed, S, max_pages, D, cfg, lengths, topics=8):
    """Level buffer with planted topics so affinities straddle any threshold."""
    lay = kka.LevelLayout(S, max_pages, D, bool(cfg["hierarchical"]), cfg["pages_per_chunk"],
                          cfg["chunks_per_grid"])
    rng = np.random.default_rng(seed)
    dirs = rng.standard_normal((topics, D)).astype(np.float32)
    topic = rng.integers(0, topics, (S, max_pages))
    lvl = np.zeros((S, lay.rows_per_seq, D), np.float32)
    lvl[:, :max_pages] = dirs[topic] + rng.standard_normal((S, max_pages, D)).astype(np.float32)
    level = torch.from_numpy(lvl).cuda()
    npg = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    if cfg["hierarchical"]:
        kka.kka_build_levels(lay, level, npg)
    return lay, level, npg, dirs


def run_steps(lay, level, npg_steps, anchors_steps, cfg, W, theta, history, stab):
    """Runs one stable and one plain scoring call per step; yields (step,
    page affinities [S][max_pages] of the stable call) after checking that
    both calls agree."""
    S, kq = lay.num_seqs, max(1, cfg["k_page"])
    kw = dict(k_page=cfg["k_page"], k_grid=cfg["k_grid"], k_chunk=cfg["k_chunk"])
    ws = kka.new_workspace(kka.kka_score_topk_workspace(lay, True))
    for t, (npg, anc) in enumerate(zip(npg_steps, anchors_steps)):
        outs = []
        for stable in (True, False):
            o = dict(idx=torch.full((S, kq), -9, dtype=torch.int32, device="cuda"),
                     sc=torch.zeros((S, kq), dtype=torch.float32, device="cuda"),
                     cnt=torch.zeros(S, dtype=torch.int32, device="cuda"),
                     aff=torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda"))
            extra = dict(history=history, stability_out=stab, window=W, theta=theta) if stable else {}
            kka.kka_score_topk(lay, level, npg, anc, page_idx_out=o["idx"], page_score_out=o["sc"],
                               n_selected_out=o["cnt"], affinity_out=o["aff"], workspace=ws, **kw, **extra)
            outs.append(o)
        torch.cuda.synchronize()
        a, b = outs
        assert torch.equal(a["cnt"], b["cnt"]) and torch.equal(a["idx"], b["idx"])
        assert torch.equal(a["sc"].view(torch.int32), b["sc"].view(torch.int32))
        assert torch.equal(a["aff"].view(torch.int32), b["aff"].view(torch.int32))
        yield t, a["aff"][:, :lay.max_pages].cpu().numpy()


def check_against_oracle(aff_hist, npg_hist, W, theta, history, stab, tag, absent_sentinel=True):
    """aff_hist: list of [S][max_pages] page affinities per step; npg_hist:
    page counts per step.  A page absent at a step gets affinity 0 there."""
    words = history.cpu().numpy().view(np.uint32)
    scores = stab.cpu().numpy() if stab is not None else None
    S, max_pages = words.shape
    for s in range(S):
        n_now = int(npg_hist[-1][s])
        steps = np.stack([np.where(np.arange(max_pages) < int(n[s]), a[s], 0.0).astype(np.float32)
                          for a, n in zip(aff_hist, npg_hist)])[:, :n_now]
        ref_score, ref_bits = oracle.stability(steps, W, theta)
        np.testing.assert_array_equal(words[s, :n_now], ref_bits, err_msg=f"{tag} window words s={s}")
        if scores is not None:
            np.testing.assert_array_equal(scores[s, :n_now].view(np.uint32), ref_score.view(np.uint32),
                                          err_msg=f"{tag} stability s={s}")
        if absent_sentinel:
            assert (words[s, n_now:] == np.uint32(SENTINEL_WORD)).all(), f"{tag} s={s}: absent words touched"
            if scores is not None:
                assert (scores[s, n_now:] == SENTINEL_SCORE).all(), f"{tag} s={s}: absent scores touched"


def fresh_state(lay, lengths):
    hist = np.full((lay.num_seqs, lay.max_pages), SENTINEL_WORD, np.int32)
    for s, n in enumerate(lengths):
        hist[s, :n] = 0
    history = torch.from_numpy(hist).cuda()
    stab = torch.full((lay.num_seqs, lay.max_pages), SENTINEL_SCORE, dtype=torch.float32, device="cuda")
    return history, stab


def drifting_anchors(seed, dirs, S, steps, noise=0.6):
    """Per step, each sequence's anchor is one topic direction plus noise;
    the topic changes now and then (a spike lasts one step)."""
    rng = np.random.default_rng(seed)
    T, D = dirs.shape
    base = rng.integers(0, T, S)
    out = []
    for t in range(steps):
        topic = base.copy()
        spike = rng.random(S) < 0.15
        topic[spike] = rng.integers(0, T, int(spike.sum()))
        a = dirs[topic] + noise * rng.standard_normal((S, D)).astype(np.float32)
        out.append(torch.from_numpy(a.astype(np.float32)).cuda())
    return out


CFGS = [
    dict(hierarchical=1, k_grid=2, k_chunk=6, k_page=20, pages_per_chunk=8, chunks_per_grid=4),
    dict(hierarchical=0, k_grid=0, k_chunk=0, k_page=33, pages_per_chunk=16, chunks_per_grid=16),
]


@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("W,theta", [(20, 0.5), (1, 0.5), (32, 0.55), (7, 0.0)])
def test_stability_matches_oracle_over_steps(cfg, W, theta):
    say(f"stability W={W} theta={theta} {cfg}")
    lengths = [0, 5, 300, 1000, 1]
    lay, level, npg, dirs = levels(40, len(lengths), 1000, 64, cfg, lengths)
    history, stab = fresh_state(lay, lengths)
    steps = 27
    anchors = drifting_anchors(41, dirs, len(lengths), steps)
    aff_hist, npg_hist = [], []
    for t, aff in run_steps(lay, level, [npg] * steps, anchors, cfg, W, theta, history, stab):
        aff_hist.append(aff)
        npg_hist.append(lengths)
        if t in (0, 4, W - 1, 19, steps - 1):
            check_against_oracle(aff_hist, npg_hist, W, theta, history, stab, f"t={t}")


def test_stability_without_score_output_and_growing_sequence():
    """Pages appear one per step (their words zero-filled beforehand, as the
    caller must); no score buffer: only the words advance."""
    cfg = CFGS[0]
    say("stability growing sequence")
    max_pages, start, steps = 64, 10, 30
    lay, level, _, dirs = levels(42, 2, max_pages, 64, cfg, [max_pages, max_pages])
    history = torch.zeros((2, max_pages), dtype=torch.int32, device="cuda")
    npg_list = [[min(max_pages, start + t), start] for t in range(steps)]
    npg_steps = [torch.tensor(n, dtype=torch.int32, device="cuda") for n in npg_list]
    anchors = drifting_anchors(43, dirs, 2, steps)
    aff_hist = []
    S = 2
    kw = dict(k_page=cfg["k_page"], k_grid=cfg["k_grid"], k_chunk=cfg["k_chunk"])
    for t in range(steps):
        kka.kka_build_levels(lay, level, npg_steps[t])
        aff = torch.zeros((S, lay.rows_per_seq), dtype=torch.float32, device="cuda")
        idx = torch.zeros((S, cfg["k_page"]), dtype=torch.int32, device="cuda")
        kka.kka_score_topk_stable(lay, level, npg_steps[t], anchors[t], history=history, window=20, theta=0.5,
                                  page_idx_out=idx, affinity_out=aff, **kw)
        torch.cuda.synchronize()
        aff_hist.append(aff[:, :max_pages].cpu().numpy())
    check_against_oracle(aff_hist, npg_list, 20, 0.5, history, None, "growing", absent_sentinel=False)
    words = history.cpu().numpy()
    assert (words[1, start:] == 0).all() and (words[0, npg_list[-1][0]:] == 0).all()


def test_stability_serving_batch_spike_and_parity():
    """64 sequences x 8192 pages: 20 steps with the planted anchor plus
    noise; at one step (the 10th) the anchor also takes in a second topic (a
    transient shift of focus).  At theta = 0.7 the anchor topic's pages
    stay high every step (20/20 = 1.0), the second topic's pages are high in
    that one step only (1/20 = 0.05) and every other page never is -- the
    page's two worked values -- and every word and score equals the
    oracle's on the GPU's affinities."""
    say("stability serving batch")
    v = synth.config4(0)
    S, n_p, D = v.vb.shape
    cfg = v.select
    lay = kka.LevelLayout(S, n_p, D, True, cfg["pages_per_chunk"], cfg["chunks_per_grid"])
    level = lay.new_buffer()
    level[:, :n_p] = torch.from_numpy(v.vb).cuda()
    npg = torch.full((S,), n_p, dtype=torch.int32, device="cuda")
    kka.kka_build_levels(lay, level, npg)
    rng = np.random.default_rng(44)
    other = np.array([int(v.page_topic[s][(np.asarray(v.page_topic[s]) != v.anchor_topic[s]).argmax()])
                      for s in range(S)])
    spike = np.stack([v.vb[s][np.asarray(v.page_topic[s]) == other[s]].mean(0) for s in range(S)]).astype(np.float32)
    # seeded data: anchor-topic pages stay >= 0.748, the second topic's reach
    # >= 0.763 at its step and <= 0.612 otherwise, all other pages <= 0.682
    steps, W, theta = 20, 20, 0.7
    anchors = []
    for t in range(steps):
        base = v.anchors + spike if t == 9 else v.anchors
        anchors.append(torch.from_numpy((base + 0.3 * rng.standard_normal((S, D))).astype(np.float32)).cuda())
    history, stab = fresh_state(lay, [n_p] * S)
    aff_hist = []
    for t, aff in run_steps(lay, level, [npg] * steps, anchors, cfg, W, theta, history, stab):
        aff_hist.append(aff)
    check_against_oracle(aff_hist, [[n_p] * S] * steps, W, theta, history, stab, "serving")
    scores = stab.cpu().numpy()
    for s in range(S):
        topic = np.asarray(v.page_topic[s])
        assert (scores[s][topic == v.anchor_topic[s]] == 1.0).all()
        assert (scores[s][topic == other[s]] == np.float32(0.05)).all()
        assert (scores[s][(topic != v.anchor_topic[s]) & (topic != other[s])] == 0.0).all()


@pytest.mark.parametrize("seed", range(10))
def test_stability_random_configurations(seed):
    """Seeded sweep: 1-40 sequences of up to 3000 pages (so that both the
    one-launch and the two-launch scoring paths run), head_dim 8-520, flat
    or hierarchical layouts with random fan-outs and k, window 1-32, theta
    0.3-0.7, 6-24 steps; on odd seeds sequences gain pages between steps
    (their words zero-filled beforehand).  Words and scores against the
    oracle on the GPU's own affinities, the selection against the plain
    pass."""
    rng = np.random.default_rng(6000 + seed)
    S = int(rng.integers(1, 41))
    max_pages = int(rng.integers(1, 3001))
    D = int(rng.choice([8, 24, 64, 128, 256, 520]))
    hier = bool(rng.random() < 0.6)
    ppc, cpg = int(rng.integers(1, 33)), int(rng.integers(1, 17))
    cfg = dict(hierarchical=int(hier), pages_per_chunk=ppc, chunks_per_grid=cpg,
               k_grid=int(rng.integers(1, 9)) if hier else 0, k_chunk=int(rng.integers(1, 33)) if hier else 0,
               k_page=int(rng.integers(0, 97)))
    W = int(rng.integers(1, 33))
    theta = float(rng.uniform(0.3, 0.7))
    steps = int(rng.integers(6, 25))
    grow = seed % 2 == 1
    final = rng.integers(0, max_pages + 1, S)
    if grow:
        start = np.minimum(final, rng.integers(0, max_pages + 1, S))
        npg_list = [np.minimum(final, start + (final - start) * t // max(1, steps - 1)).astype(np.int32)
                    for t in range(steps)]
    else:
        npg_list = [final.astype(np.int32)] * steps
    say(f"stability random seed={seed} S={S} max_pages={max_pages} D={D} {cfg} W={W} theta={theta:.3f} "
        f"steps={steps} grow={grow}")
    lay, level, _, dirs = levels(6100 + seed, S, max_pages, D, cfg, final)
    if grow:
        history = torch.zeros((S, max_pages), dtype=torch.int32, device="cuda")
        stab = torch.full((S, max_pages), SENTINEL_SCORE, dtype=torch.float32, device="cuda")
    else:
        history, stab = fresh_state(lay, final)
    npg_steps = [torch.from_numpy(n).cuda() for n in npg_list]
    if grow and cfg["hierarchical"]:
        kka.kka_build_levels(lay, level, npg_steps[0])
    anchors = drifting_anchors(6200 + seed, dirs, S, steps)
    aff_hist = []
    for t, aff in run_steps(lay, level, npg_steps, anchors, cfg, W, theta, history, stab):
        if grow and cfg["hierarchical"] and t + 1 < steps:
            kka.kka_build_levels(lay, level, npg_steps[t + 1])
        aff_hist.append(aff)
    check_against_oracle(aff_hist, npg_list, W, theta, history, stab, f"seed={seed}", absent_sentinel=not grow)
    if grow:
        words = history.cpu().numpy()
        for s in range(S):
            assert (words[s, int(final[s]):] == 0).all(), f"s={s}: absent words touched"
