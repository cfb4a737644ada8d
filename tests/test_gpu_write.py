"""GPU parity of pool-on-write (kka_pool_on_write).

Every decode step appends one token per sequence.  After each step the
paged pool must hold the new keys bit for bit at (layer, block_table[j],
slot, head), and the open block's vector must equal the oracle's block
mean over the block's tokens so far (within 1e-5; fp32 running sums
against fp64 sums rounded once).  Closed blocks keep their vectors.
Covers starting from empty sequences, seeding after a prefill that
kka_pool_blocks pooled, frozen variance weights, keys already in the pool
(new_k = NULL), bad device metadata, and the 7B key shape with 64
sequences.
"""
import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth

from gpu_harness import ATOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


class Batch:
    """Sequences with room to grow: `cap` logical blocks each, behind a
    permuted physical pool; a host mirror of the pool for the oracle."""

    def __init__(self, seed, L, H, D, B, cap, prefill):
        self.L, self.H, self.D, self.B = L, H, D, B
        self.S = len(cap)
        self.cap = np.asarray(cap, np.int32)
        self.off = np.zeros(self.S + 1, np.int32)
        self.off[1:] = np.cumsum(self.cap)
        self.P = int(self.off[-1]) + 2
        self.table = synth.permutation(seed, 7, self.P)[:self.off[-1]].astype(np.int32)
        self.host = np.zeros((L, self.P, B, H, D), np.uint16)
        self.len = np.asarray(prefill, np.int32).copy()
        self.rng = np.random.default_rng(seed)
        for s in range(self.S):
            for t in range(int(self.len[s])):
                self.host_write(s, t, self.random_token())
        self.k = torch.from_numpy(self.host.reshape(-1).view(np.int16).copy()).cuda()
        self.kp = kka.KPool(self.k, L, H, D, B, self.P)
        self.offs_dev = torch.from_numpy(self.off).cuda()
        self.table_dev = torch.from_numpy(self.table).cuda()
        self.len_dev = torch.from_numpy(self.len).cuda()
        self.seqs = kka.Seqs(self.len_dev, self.offs_dev, self.table_dev, int(self.off[-1]))
        self.okp = oracle.KPool(self.host, L, H, D, B, self.P)

    def random_token(self):
        x = self.rng.standard_normal((self.L, self.H, self.D)).astype(np.float32)
        return synth.to_bf16_bits(x)

    def host_write(self, s, t, tok):
        p = self.table[self.off[s] + t // self.B]
        self.host[:, p, t % self.B] = tok

    def prefill_seqs(self):
        """Seqs listing only the blocks that hold tokens (for kka_pool_blocks)."""
        nb = (self.len + self.B - 1) // self.B
        off = np.zeros(self.S + 1, np.int32)
        off[1:] = np.cumsum(nb)
        tab = np.concatenate([self.table[self.off[s]:self.off[s] + nb[s]] for s in range(self.S)]).astype(np.int32)
        return kka.Seqs(torch.from_numpy(self.len.copy()).cuda(), torch.from_numpy(off).cuda(),
                        torch.from_numpy(tab).cuda(), int(off[-1]))

    def step_tokens(self):
        """One new token per sequence: host mirror updated, lengths advanced."""
        toks = np.stack([self.random_token() for _ in range(self.S)])
        for s in range(self.S):
            self.host_write(s, int(self.len[s]), toks[s])
        self.len += 1
        self.len_dev.copy_(torch.from_numpy(self.len))
        return torch.from_numpy(toks.reshape(-1).view(np.int16).copy()).cuda()

    def check(self, vb, weights=None, tag=""):
        """Pool bit for bit; every block holding tokens against the oracle."""
        got = self.k.cpu().numpy().view(np.uint16).reshape(self.host.shape)
        np.testing.assert_array_equal(got, self.host, err_msg=f"{tag} pool contents")
        rows = vb.cpu().numpy()
        for s in range(self.S):
            w = None if weights is None else weights[s]
            for j in range(-(-int(self.len[s]) // self.B)):
                n_valid = min(self.B, int(self.len[s]) - j * self.B)
                ref = oracle.pool_block(self.okp, int(self.table[self.off[s] + j]), n_valid, w)
                np.testing.assert_allclose(rows[s, j], ref, atol=ATOL, rtol=0, err_msg=f"{tag} s={s} block {j}")


def test_from_empty_sequences_token_by_token():
    """Four sequences grow from 0 to 20 tokens in blocks of 8 (two block
    boundaries crossed); the first step opens every block at slot 0."""
    say("pool-on-write from empty")
    b = Batch(50, L=3, H=2, D=64, B=8, cap=[3, 3, 3, 3], prefill=[0, 0, 0, 0])
    vb = torch.full((b.S, 3, b.D), 7.0, dtype=torch.float32, device="cuda")
    running = torch.full((b.S, b.D), 123.0, dtype=torch.float32, device="cuda")  # ignored at slot 0
    for t in range(20):
        nk = b.step_tokens()
        kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, vb_seq_stride=3)
        torch.cuda.synchronize()
        b.check(vb, tag=f"t={t}")
    # tokens 16..19 opened block 2 of every sequence
    assert (vb[:, 2].cpu().numpy() != 7.0).all()


@pytest.mark.parametrize("D,B", [(64, 8), (128, 16), (8, 4), (24, 5), (1024, 2)])
def test_after_prefill_seeded_then_running(D, B):
    """Ragged prefills pooled by kka_pool_blocks, one seeded step, then
    running steps; lengths include 0, a full block and a partial block."""
    say(f"pool-on-write after prefill D={D} B={B}")
    L, H = (2, 2) if D < 1024 else (2, 1)
    prefill = [0, B, 3 * B - 1, 1, 2 * B + 2]
    steps = 2 * B + 3
    cap = [-(-(n + steps) // B) for n in prefill]
    b = Batch(51, L, H, D, B, cap=cap, prefill=prefill)
    stride = max(cap)
    vb = torch.zeros((b.S, stride, D), dtype=torch.float32, device="cuda")
    kka.kka_pool_blocks(b.kp, b.prefill_seqs(), vb, vb_seq_stride=stride)
    running = torch.zeros((b.S, D), dtype=torch.float32, device="cuda")
    for t in range(steps):
        nk = b.step_tokens()
        kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, seed=(t == 0), vb_seq_stride=stride)
        torch.cuda.synchronize()
        if t in (0, 1, B - 1, B, steps - 1):
            b.check(vb, tag=f"t={t}")


def test_frozen_variance_weights():
    """Weights computed by kka_pool_blocks in variance mode, then used
    frozen for every appended token (given-weight mode)."""
    say("pool-on-write frozen variance weights")
    L, H, D, B = 3, 4, 64, 8
    prefill = [40, 17, 9]
    steps = 12
    cap = [-(-(n + steps) // B) for n in prefill]
    b = Batch(52, L, H, D, B, cap=cap, prefill=prefill)
    # give the heads different variances
    scale = np.exp(np.linspace(-1.5, 1.5, L * H)).reshape(L, 1, 1, H, 1).astype(np.float32)
    f = synth.bf16_bits_to_f32(b.host) * scale
    b.host[...] = synth.to_bf16_bits(f)
    b.k.copy_(torch.from_numpy(b.host.reshape(-1).view(np.int16).copy()))
    stride = max(cap)
    vb = torch.zeros((b.S, stride, D), dtype=torch.float32, device="cuda")
    hw = torch.zeros((b.S, L * H), dtype=torch.float32, device="cuda")
    kka.kka_pool_blocks(b.kp, b.prefill_seqs(), vb, mode=kka.WEIGHT_VARIANCE, head_weight=hw, vb_seq_stride=stride)
    weights = hw.cpu().numpy()
    assert weights.std(axis=1).min() > 0.01  # not uniform
    running = torch.zeros((b.S, D), dtype=torch.float32, device="cuda")
    b.rng = np.random.default_rng(53)
    for t in range(steps):
        nk = b.step_tokens()
        kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, mode=kka.WEIGHT_GIVEN, head_weight=hw,
                              seed=(t == 0), vb_seq_stride=stride)
        torch.cuda.synchronize()
        b.check(vb, weights=weights, tag=f"t={t}")


def test_keys_already_in_pool_match_new_k_bitwise():
    """new_k = NULL reads the token the caller already stored: the same
    arithmetic in the same order, so the vectors are bit-identical."""
    say("pool-on-write without new_k")
    prefill = [3, 0, 9]
    a = Batch(54, 2, 2, 64, 4, cap=[6, 6, 6], prefill=prefill)
    c = Batch(54, 2, 2, 64, 4, cap=[6, 6, 6], prefill=prefill)
    va = torch.zeros((3, 6, 64), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(va)
    ra = torch.zeros((3, 64), dtype=torch.float32, device="cuda")
    rc = torch.zeros_like(ra)
    kka.kka_pool_blocks(a.kp, a.prefill_seqs(), va, vb_seq_stride=6)
    kka.kka_pool_blocks(c.kp, c.prefill_seqs(), vc, vb_seq_stride=6)
    for t in range(10):
        nk = a.step_tokens()
        c.step_tokens()  # same seed: same tokens in c's host mirror
        c.k.copy_(torch.from_numpy(c.host.reshape(-1).view(np.int16).copy()))
        kka.kka_pool_on_write(a.kp, a.seqs, va, ra, new_k=nk, seed=(t == 0), vb_seq_stride=6)
        kka.kka_pool_on_write(c.kp, c.seqs, vc, rc, new_k=None, seed=(t == 0), vb_seq_stride=6)
        torch.cuda.synchronize()
        assert torch.equal(va.view(torch.int32), vc.view(torch.int32))
        assert torch.equal(a.k, c.k)
    a.check(va, tag="no new_k")


def test_bad_metadata_raises_flag_and_skips_only_that_sequence():
    say("pool-on-write bad metadata")
    b = Batch(55, 2, 2, 64, 4, cap=[1, 2], prefill=[4, 3])  # sequence 0 is full
    vb = torch.zeros((2, 2, 64), dtype=torch.float32, device="cuda")
    running = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    before = b.k.clone()
    b.len_dev.copy_(torch.tensor([5, 4], dtype=torch.int32))  # sequence 0 has no block for token 4
    nk = torch.from_numpy(np.stack([b.random_token() for _ in range(2)]).reshape(-1).view(np.int16).copy()).cuda()
    kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, seed=True, vb_seq_stride=2)
    assert kka.kka_device_error() == kka.DEVERR_SEQ_LEN
    assert (vb[0] == 0).all()
    # sequence 1 went through: its token 3 (slot 3 of block 0) is stored
    p1 = int(b.table[b.off[1]])
    got = b.k.cpu().numpy().view(np.uint16).reshape(b.host.shape)
    np.testing.assert_array_equal(got[:, p1, 3], nk.cpu().numpy().view(np.uint16).reshape(2, 2, 2, 64)[1])
    p0 = int(b.table[b.off[0]])
    np.testing.assert_array_equal(got[:, p0], before.cpu().numpy().view(np.uint16).reshape(b.host.shape)[:, p0])


def test_7b_shape_64_sequences():
    """28 layers x 4 KV heads x 128, blocks of 16, 64 sequences with ragged
    prefills (1-31 tokens); one seeded step then 20 running steps."""
    say("pool-on-write 7B shape, 64 sequences")
    rng = np.random.default_rng(56)
    prefill = rng.integers(1, 32, 64).tolist()
    steps = 21
    cap = [-(-(n + steps) // 16) for n in prefill]
    b = Batch(57, 28, 4, 128, 16, cap=cap, prefill=prefill)
    stride = max(cap)
    vb = torch.zeros((b.S, stride, 128), dtype=torch.float32, device="cuda")
    kka.kka_pool_blocks(b.kp, b.prefill_seqs(), vb, vb_seq_stride=stride)
    running = torch.zeros((b.S, 128), dtype=torch.float32, device="cuda")
    for t in range(steps):
        nk = b.step_tokens()
        kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, seed=(t == 0), vb_seq_stride=stride)
        torch.cuda.synchronize()
        if t in (0, 7, steps - 1):
            b.check(vb, tag=f"t={t}")


@pytest.mark.parametrize("seed", range(10))
def test_pool_on_write_random_shapes(seed):
    """Seeded sweep: layers 1-12, KV heads 1-8, head_dim 8-512 (at most 1024
    16-byte pieces per token), blocks of 1-33 tokens, 1-12 sequences with
    ragged prefills (0 to a few blocks, pooled by kka_pool_blocks), uniform
    or frozen random weights, a seeded first step and 1-40 running steps
    crossing block boundaries; pool contents bit for bit and every block
    vector against the oracle after the first, a middle and the last step."""
    rng = np.random.default_rng(4000 + seed)
    L = int(rng.integers(1, 13))
    H = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([8, 16, 24, 64, 128, 256, 512]))
    while H * D // 8 > 1024:
        H //= 2
    B = int(rng.integers(1, 34))
    S = int(rng.integers(1, 13))
    steps = int(rng.integers(1, 41))
    prefill = rng.integers(0, 3 * B + 1, S).astype(np.int32)
    given = rng.random() < 0.5
    say(f"pool-on-write random seed={seed} L={L} H={H} D={D} B={B} S={S} steps={steps} given={given}")
    cap = [-(-(int(n) + steps) // B) for n in prefill]
    b = Batch(4100 + seed, L, H, D, B, cap=cap, prefill=prefill)
    stride = max(cap)
    weights = None
    hw = None
    if given:
        wr = rng.random((S, L * H)).astype(np.float32) + 0.05
        weights = (wr / wr.sum(axis=1, keepdims=True)).astype(np.float32)
        hw = torch.from_numpy(weights).cuda()
    vb = torch.zeros((S, stride, D), dtype=torch.float32, device="cuda")
    kka.kka_pool_blocks(b.kp, b.prefill_seqs(), vb, mode=kka.WEIGHT_GIVEN if given else kka.WEIGHT_UNIFORM,
                        head_weight=hw, vb_seq_stride=stride)
    running = torch.zeros((S, D), dtype=torch.float32, device="cuda")
    for t in range(steps):
        nk = b.step_tokens()
        kka.kka_pool_on_write(b.kp, b.seqs, vb, running, new_k=nk, seed=(t == 0), vb_seq_stride=stride,
                              mode=kka.WEIGHT_GIVEN if given else kka.WEIGHT_UNIFORM, head_weight=hw)
        torch.cuda.synchronize()
        if t in (0, steps // 2, steps - 1):
            b.check(vb, weights=weights, tag=f"t={t}")
    assert kka.kka_device_error() == 0
