"""The allocation-free anchor (kka_pool_anchor_noalloc, called through the
C ABI) against kka_pool_anchor with its own workspace on the same inputs,
and against the oracle: two calls in a row, the second with a smaller
input, both using the library's fixed scratch array (layer-split partial
sums); then a third, uniform-weight call."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_block_amd as kka
import oracle
import synth

from gpu_harness import ATOL, say, upload
from test_gpu_parity import ragged_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kka.lib()
    yield
    assert kka.kka_device_error() == 0


def _noalloc(kp, seqs, W, weights, out):
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return kka.lib().kka_pool_anchor_noalloc(ctypes.byref(kp.c), ctypes.byref(seqs.c), int(W), p(weights), p(out),
                                             stream)


def test_noalloc_anchor_matches_the_workspace_entry_point():
    L, H, D, B = 28, 4, 128, 16
    for seed, S, lo, hi, W, weighted in ((51, 8, 100, 3000, 16, True), (52, 3, 20, 400, 5, True),
                                         (53, 2, 1, 90, 40, False)):
        say(f"noalloc anchor: seed {seed}, {S} sequences, lengths {lo}..{hi}, window {W}, weighted {weighted}")
        w = ragged_workload(seed, S, L, H, D, B, lo, hi, window=W)
        kp, seqs = upload(w)
        need = kka.kka_pool_anchor_noalloc_scratch(kp, seqs)
        assert 0 < need <= 4 << 20  # the scratch array is in use
        hw = None
        if weighted:
            u = synth.uniform(seed, 130, S * L * H).astype(np.float32).reshape(S, L * H) + 0.1
            hw = torch.from_numpy((u / u.sum(axis=1, keepdims=True)).astype(np.float32)).cuda()
        ref = torch.zeros((S, D), dtype=torch.float32, device="cuda")
        kka.kka_pool_anchor(kp, seqs, W, ref, head_weight=hw)
        got = torch.full((S, D), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(kp, seqs, W, hw, got) == 0
        torch.cuda.synchronize()
        assert kka.kka_device_error() == 0
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        np.testing.assert_allclose(g, r, atol=ATOL, rtol=0)
        # the shares are added in the same order either way: the same bits
        np.testing.assert_array_equal(g.view(np.uint32), r.view(np.uint32))
        okp = oracle.KPool.of(w)
        hwn = None if hw is None else hw.cpu().numpy()
        for s in range(S):
            a = oracle.pool_anchor(okp, oracle.seq_table(w.block_offsets, w.block_table, s), int(w.seq_len[s]), W,
                                   None if hwn is None else hwn[s])
            np.testing.assert_allclose(g[s], a, atol=ATOL, rtol=0, err_msg=f"seed {seed} seq {s}")
