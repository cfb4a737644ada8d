"""The seeded input generator: determinism, counter addressability and the
distributions the workload recipes ask for."""
import math

import numpy as np

import synth


def test_normal_stream_is_standard_and_deterministic():
    a = synth.normal(3, 5, 200000)
    b = synth.normal(3, 5, 200000)
    np.testing.assert_array_equal(a, b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert not np.array_equal(a[:1000], synth.normal(4, 5, 1000))
    # element i depends only on (seed, tag, i)
    assert synth.lib().synth_normal(3, 5, 12345) == a[12345]


def test_permutation_and_uniform_int():
    p = synth.permutation(1, 2, 1000)
    assert sorted(p.tolist()) == list(range(1000))
    u = synth.uniform_int(1, 3, 100000, 4, 9)
    assert u.min() == 4 and u.max() == 9
    assert np.all(np.abs(np.bincount(u - 4) / 1e5 - 1 / 6) < 0.01)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 1e-3], dtype=np.float32)
    back = synth.bf16_bits_to_f32(synth.to_bf16_bits(x))
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == -2.5
    assert abs(back[5] - 1e-3) / 1e-3 < 2 ** -8


def test_kpool_blocks_regenerate_independently():
    """A block's keys depend only on its logical position, not on where it
    sits physically or on the other blocks."""
    L, H, D, B, n = 2, 2, 16, 4, 6
    off = np.array([0, n], dtype=np.int32)
    gl = np.array([n * B], dtype=np.int32)
    std = np.ones(L * H, np.float32)
    ident = np.arange(n, dtype=np.int32)
    perm = synth.permutation(0, 9, n)
    k0 = synth._gen_kpool(L, H, D, B, n, gl, off, ident, None, None, 0.0, 0.0, std, None, 5)
    k1 = synth._gen_kpool(L, H, D, B, n, gl, off, perm, None, None, 0.0, 0.0, std, None, 5)
    for i in range(n):
        np.testing.assert_array_equal(k0[:, i], k1[:, perm[i]])


def test_config_shapes_and_topics():
    w = synth.config1(0)
    assert w.k.shape == (24, 256, 16, 2, 64) and w.window == 8 and w.select["k_page"] == 16
    assert np.bincount(w.block_topic[0]).tolist() == [32] * 8
    assert w.anchor_topic[0] == w.block_topic[0][-1]
    w3 = synth.config3(0, n_blocks=256, L=2)
    run = w3.extra["anchor_run"]
    assert run < 4 and w3.block_topic[0][-1] == w3.block_topic[0][run * 32]
    assert sorted(w3.block_table.tolist()) == list(range(256))
    v = synth.config4(0, n_seqs=2, n_pages=256)
    assert v.vb.shape == (2, 256, 128)
    assert abs(np.linalg.norm(v.vb[0, 0]) - math.sqrt(128 + 128 * 0.09)) < 2.0


def test_config5_ragged_state():
    w = synth.config5(0, n_seqs=4, len_lo=100, len_hi=300, L=2, H=2, D=8, B=16)
    after = w.extra["after"]
    assert (after["seq_len"] == w.seq_len + 1).all()
    assert (np.diff(w.block_offsets) == (w.seq_len + 15) // 16).all()
    assert (np.diff(after["block_offsets"]) == (w.seq_len + 16) // 16).all()
    assert sorted(after["block_table"].tolist()) == list(range(w.P))
    v = w.extra["head_var"]
    assert v.min() >= 0.1 and v.max() <= 4.0


def test_planted_queries_share_their_kv_head_direction():
    w = synth.config1(0)
    q = synth.planted_queries(w, 14, 8.0, 0.0)
    assert q.shape == (24, 14, 64)
    np.testing.assert_allclose(np.linalg.norm(q, axis=2), 8.0, rtol=1e-5)
    for g in range(7):  # query heads 0-6 read KV head 0, 7-13 read KV head 1
        np.testing.assert_array_equal(q[:, g], q[:, 0])
        np.testing.assert_array_equal(q[:, 7 + g], q[:, 7])
    assert np.abs(q[:, 0] - q[:, 7]).max() > 0.1
    noisy = synth.planted_queries(w, 14, 8.0, 0.5, seed=3)
    assert 0.4 < float((noisy - q).std()) < 0.6
