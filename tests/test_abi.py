"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before anything
reaches the device.

Every validation case below breaks at least one rule that is checked before
the library's first HIP call, so the fake (never dereferenced) pointers are
never handed to a kernel.
"""
import ctypes
import os
import re

import pytest

import kv_cache_block_amd as kka

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kka.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced
FAKE_ODD = 0x10004


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kka.LIB_PATH):
        pytest.skip("libkka.so not built")
    return kka.lib()


def declared():
    text = open(HEADER).read()
    return re.findall(r"KKA_API\s+[\w\s\*]+?\b(kka_\w+)\s*\(", text)


def test_binding_constants_match_header():
    """Device error bits, weight modes and status codes: the binding's
    values are the header's."""
    text = open(HEADER).read()
    bits = dict(re.findall(r"#define KKA_DEVERR_(\w+) (\d+)u", text))
    assert bits and {k: int(v) for k, v in bits.items()} == \
        {k[len("DEVERR_"):]: getattr(kka, k) for k in dir(kka) if k.startswith("DEVERR_")}
    modes = dict(re.findall(r"KKA_WEIGHT_(\w+) = (\d+)", text))
    assert modes and all(getattr(kka, "WEIGHT_" + k) == int(v) for k, v in modes.items())


def test_header_declares_all_entry_points():
    names = declared()
    assert sorted(names) == sorted(kka.ENTRY_POINTS)
    for n in ("kka_pool_blocks", "kka_pool_anchor", "kka_build_levels", "kka_score_topk"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared():
        assert hasattr(L, name), name
    assert L.kka_version() == int(re.search(r"#define KKA_VERSION (\d+)", open(HEADER).read()).group(1)) == 400
    assert L.kka_status_string(0) == b"ok"
    assert L.kka_status_string(4).startswith(b"workspace")
    assert b"scratch" in L.kka_status_string(6)


def kpool(**kw):
    d = dict(k=FAKE, num_layers=28, num_kv_heads=4, head_dim=128, block_size=16, num_phys_blocks=64)
    d.update(kw)
    P, B, H, D = d["num_phys_blocks"], d["block_size"], d["num_kv_heads"], d["head_dim"]
    strides = d.pop("strides", (P * B * H * D, B * H * D, H * D, D))
    return kka.c_kpool(d["k"], d["num_layers"], d["num_kv_heads"], d["head_dim"], d["block_size"],
                       d["num_phys_blocks"], *strides)


def seqs(**kw):
    d = dict(num_seqs=2, total_blocks=64, seq_len=FAKE, block_offsets=FAKE, block_table=FAKE)
    d.update(kw)
    return kka.c_seqs(d["num_seqs"], d["total_blocks"], d["seq_len"], d["block_offsets"], d["block_table"])


def pool(L, kp, sq, blocks=None, nb=0, mode=0, hw=FAKE, out=FAKE, stride=0, ws=None, wsb=0):
    return L.kka_pool_blocks(ctypes.byref(kp), ctypes.byref(sq), blocks, nb, mode, hw, out, stride, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1),
    (dict(head_dim=12), 2),
    (dict(head_dim=2048), 2),
    (dict(num_layers=0), 2),
    (dict(block_size=0), 2),
    (dict(num_phys_blocks=0), 2),
    (dict(num_kv_heads=128, head_dim=128), 2),      # H*D/8 > 1024 threads
    (dict(num_layers=2048, num_kv_heads=4), 2),     # L*H > 4096 weights
    (dict(k=FAKE_ODD), 3),
    (dict(strides=(8, 8, 8, 4)), 3),
    (dict(strides=(8, -8, 8, 8)), 2),
])
def test_pool_rejects_bad_kpool(L, kw, code):
    assert pool(L, kpool(**kw), seqs()) == code


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=-1), 2),
    (dict(total_blocks=-3), 2),
    (dict(seq_len=None), 1),
    (dict(block_offsets=None), 1),
    (dict(block_table=None), 1),
    (dict(num_seqs=0, total_blocks=5), 2),
])
def test_pool_rejects_bad_seqs(L, kw, code):
    assert pool(L, kpool(), seqs(**kw)) == code


def test_pool_rejects_bad_call_arguments(L):
    kp, sq = kpool(), seqs()
    assert pool(L, kp, sq, mode=3) == 2
    assert pool(L, kp, sq, blocks=FAKE, nb=-1) == 2
    assert pool(L, kp, sq, blocks=FAKE, nb=4, mode=1) == 2          # variance needs every block
    assert pool(L, kp, sq, mode=2, hw=None) == 1                    # given weights missing
    assert pool(L, kp, sq, mode=1, hw=None) == 1
    assert pool(L, kp, sq, stride=-1) == 2
    assert pool(L, kp, sq, out=None) == 1
    assert pool(L, kp, sq, out=FAKE_ODD) == 3
    assert pool(L, kp, seqs(num_seqs=1, total_blocks=0, block_table=None), blocks=FAKE, nb=2) == 2
    # variance mode needs a workspace
    need = L.kka_pool_blocks_workspace(ctypes.byref(kp), ctypes.byref(sq), None, 0, 1)
    assert need > 0
    assert pool(L, kp, sq, mode=1) == 4
    assert pool(L, kp, sq, mode=1, ws=FAKE, wsb=need - 1) == 4
    assert pool(L, kp, sq, mode=1, ws=FAKE_ODD, wsb=need) == 3


def test_workspace_sizes(L):
    kp = kpool(num_phys_blocks=8192)
    big = seqs(num_seqs=1, total_blocks=8192)
    small = seqs(num_seqs=1, total_blocks=256)
    # enough blocks to fill the chip: one pass, no partials
    assert L.kka_pool_blocks_workspace(ctypes.byref(kp), ctypes.byref(big), None, 0, 0) == 0
    # few blocks: split over layers; one arrival counter per block (rounded
    # up to 256 bytes), then D floats per (block, split): 256 blocks want 8
    # splits of 28 layers, but a share keeps at least 128 KiB of keys (8
    # layers of 16 KiB), which makes 4 splits
    n = L.kka_pool_blocks_workspace(ctypes.byref(kp), ctypes.byref(small), None, 0, 0)
    assert n == 256 * 4 + 256 * 4 * 128 * 4
    # blocks of 96 KiB (0.5B shape) are not split at all: no workspace
    kp_small = kpool(num_layers=24, num_kv_heads=2, head_dim=64, block_size=16, num_phys_blocks=256)
    assert L.kka_pool_blocks_workspace(ctypes.byref(kp_small), ctypes.byref(small), None, 0, 0) == 0
    # variance: per-(block, layer, head) sums + squares + per-(seq, head) fp64 variances
    v = L.kka_pool_blocks_workspace(ctypes.byref(kp), ctypes.byref(big), None, 0, 1)
    assert v >= 8192 * 112 * 129 * 4 + 112 * 8
    a = L.kka_pool_anchor_workspace(ctypes.byref(kp), ctypes.byref(big), 16)
    assert a == 256 + 28 * 128 * 4  # one sequence split over every layer: its counter, then 28 partials
    # 32 sequences: one share per layer would take 896 work-groups, so shares
    # of 4 layers (7 per sequence, 224 work-groups) are taken instead
    s32 = seqs(num_seqs=32, total_blocks=32 * 256)
    assert L.kka_pool_anchor_workspace(ctypes.byref(kp), ctypes.byref(s32), 16) == 256 + 32 * 7 * 128 * 4
    # 64 sequences would need shares of 7 layers: one share per layer stays
    s64 = seqs(num_seqs=64, total_blocks=64 * 128)
    assert L.kka_pool_anchor_workspace(ctypes.byref(kp), ctypes.byref(s64), 16) == 256 + 64 * 28 * 128 * 4


def test_level_rows_and_score_validation(L):
    lay = kka.c_level_layout(64, 8192, 128, 1, 16, 16)
    assert L.kka_level_rows(ctypes.byref(lay)) == 8192 + 512 + 32
    flat = kka.c_level_layout(4, 1025, 128, 0, 16, 16)
    assert L.kka_level_rows(ctypes.byref(flat)) == 1025
    for bad in (kka.c_level_layout(1, 100, 12, 1, 16, 16), kka.c_level_layout(1, 100, 128, 1, 0, 16),
                kka.c_level_layout(1, 16 * 16385, 128, 1, 16, 16), kka.c_level_layout(1, 100, 1024, 1, 16, 17),
                kka.c_level_layout(-1, 100, 128, 0, 16, 16), kka.c_level_layout(1, (1 << 30) + 1, 128, 0, 16, 16),
                kka.c_level_layout(1, 1 << 30, 128, 1, (1 << 29) + 1, 16)):
        assert L.kka_level_rows(ctypes.byref(bad)) == -1
    # page counts up to 2^30, also once rounded up to whole chunks
    assert L.kka_level_rows(ctypes.byref(kka.c_level_layout(1, 1 << 30, 128, 0, 16, 16))) == 1 << 30
    assert L.kka_level_rows(ctypes.byref(kka.c_level_layout(1, 1 << 30, 128, 1, 1 << 16, 16))) == (1 << 30) + 16384 + 1024
    sel = kka.c_select(4, 16, 64)
    ws = L.kka_score_topk_workspace(ctypes.byref(lay), ctypes.byref(sel), 0)
    assert ws >= 256 + 64 * 8736 * 4  # per-sequence tile counters, then scratch affinities
    assert L.kka_score_topk_workspace(ctypes.byref(lay), ctypes.byref(sel), 1) == 256  # counters only
    assert L.kka_score_topk_workspace(ctypes.byref(kka.c_level_layout(0, 100, 128, 1, 16, 16)),
                                      ctypes.byref(sel), 1) == 0

    def score(lay_, sel_, lvl=FAKE, npg=FAKE, anc=FAKE, idx=FAKE, w=FAKE, wb=ws):
        return L.kka_score_topk(ctypes.byref(lay_), lvl, npg, anc, ctypes.byref(sel_), None, idx, None, None, w,
                                wb, None)

    assert score(lay, kka.c_select(4, 16, 1025)) == 2
    assert score(lay, kka.c_select(-1, 16, 64)) == 2
    assert score(lay, sel, lvl=None) == 1
    assert score(lay, sel, idx=None) == 1
    assert score(lay, sel, anc=FAKE_ODD) == 3
    assert score(lay, sel, w=None) == 4
    assert score(lay, sel, wb=ws - 4) == 4
    assert score(kka.c_level_layout(1, 100, 12, 1, 16, 16), sel) == 2
    assert L.kka_build_levels(ctypes.byref(kka.c_level_layout(1, 100, 12, 1, 16, 16)), FAKE, FAKE, None,
                              None) == 2
    # the lazy entry point validates exactly like kka_score_topk
    def lazy(lay_, sel_, lvl=FAKE, npg=FAKE, anc=FAKE, idx=FAKE, w=FAKE, wb=ws):
        return L.kka_score_topk_lazy(ctypes.byref(lay_), lvl, npg, anc, ctypes.byref(sel_), None, idx, None, None,
                                     w, wb, None)

    assert lazy(lay, kka.c_select(4, 16, 1025)) == 2
    assert lazy(lay, kka.c_select(4, -1, 64)) == 2
    assert lazy(lay, sel, npg=None) == 1
    assert lazy(lay, sel, lvl=FAKE_ODD) == 3
    assert lazy(lay, sel, wb=ws - 4) == 4
    assert lazy(flat, kka.c_select(0, 0, 1025)) == 2
    assert lazy(kka.c_level_layout(0, 100, 128, 1, 16, 16), sel, lvl=None, npg=None, anc=None, idx=None,
                w=None, wb=0) == 0
    # the stability variant: kka_score_topk's rules plus its own
    def stable(st, lay_=lay, sel_=sel, anc=FAKE):
        return L.kka_score_topk_stable(ctypes.byref(lay_), FAKE, FAKE, anc, ctypes.byref(sel_),
                                       None if st is None else ctypes.byref(st), None, FAKE, None, None, FAKE, ws,
                                       None)

    st = lambda h=FAKE, so=None, W=20, th=0.5: kka.c_stability(h, so, W, th)
    assert stable(None) == 1
    assert stable(st(W=0)) == 2
    assert stable(st(W=33)) == 2
    assert stable(st(th=float("nan"))) == 2
    assert stable(st(th=float("inf"))) == 2
    assert stable(st(h=None)) == 1
    assert stable(st(h=FAKE + 2)) == 3
    assert stable(st(so=FAKE + 1)) == 3
    assert stable(st(), sel_=kka.c_select(4, 16, 1025)) == 2
    assert stable(st(), anc=FAKE_ODD) == 3
    assert stable(st(), lay_=kka.c_level_layout(0, 100, 128, 1, 16, 16)) == 0
    assert L.kka_build_levels(ctypes.byref(lay), None, FAKE, None, None) == 1
    assert L.kka_build_levels(ctypes.byref(lay), FAKE_ODD, FAKE, None, None) == 3


def test_pool_on_write_validation(L):
    kp, sq = kpool(), seqs()

    def f(kp_=kp, sq_=sq, nk=FAKE, mode=0, hw=None, run=FAKE, out=FAKE, stride=0):
        return L.kka_pool_on_write(ctypes.byref(kp_), ctypes.byref(sq_), nk, mode, hw, run, 0, out, stride, None)

    assert f(mode=1) == 2            # variance weights are computed by kka_pool_blocks, then frozen
    assert f(mode=7) == 2
    assert f(mode=2) == 1            # given weights need head_weight
    assert f(run=None) == 1
    assert f(out=None) == 1
    assert f(out=FAKE_ODD) == 3
    assert f(nk=FAKE_ODD) == 3
    assert f(stride=-1) == 2
    assert f(kp_=kpool(head_dim=12)) == 2
    assert f(kp_=kpool(block_size=1 << 20, num_layers=64, num_kv_heads=16)) == 2
    assert f(sq_=seqs(num_seqs=0, total_blocks=0), run=None, out=None) == 0
    assert L.kka_pool_on_write(None, ctypes.byref(sq), FAKE, 0, None, FAKE, 0, FAKE, 0, None) == 1


def test_attention_topk_validation(L):
    kp, sq = kpool(), seqs()  # 28 layers, 4 KV heads, head_dim 128, blocks of 16
    ws = L.kka_attention_topk_workspace(ctypes.byref(kp), ctypes.byref(sq), 28)
    # block partials and tile max/sum of 28 x 28 (layer, query head) pairs
    assert ws >= 784 * 64 * 4 + 2 * 784 * 4

    def f(kp_=kp, sq_=sq, q=FAKE, hq=28, scale=0.1, k=8, out=FAKE, stride=64, idx=FAKE, w=FAKE, wb=ws):
        return L.kka_attention_topk(ctypes.byref(kp_), ctypes.byref(sq_), q, hq, scale, k, out, stride, idx, None,
                                    None, w, wb, None)

    assert f(hq=6) == 2                 # not a multiple of the KV heads
    assert f(hq=68) == 2                # 17 query heads per KV head
    assert f(kp_=kpool(head_dim=96), hq=40) == 2  # vector path: 10 query heads per KV head
    assert f(kp_=kpool(head_dim=96)) == 2
    assert f(kp_=kpool(head_dim=1024, num_kv_heads=1)) == 2
    assert f(scale=float("nan")) == 2
    assert f(k=1025) == 2
    assert f(stride=0) == 2
    assert f(q=None) == 1
    assert f(idx=None) == 1
    assert f(out=FAKE_ODD) == 3
    assert f(w=None) == 4
    assert f(wb=ws - 1) == 4
    assert f(sq_=seqs(num_seqs=0, total_blocks=0), q=None, out=None, idx=None, w=None, wb=0) == 0
    assert L.kka_attention_topk_workspace(ctypes.byref(kp), ctypes.byref(sq), 6) == 0


def test_anchor_validation(L):
    kp, sq = kpool(), seqs()
    f = lambda kp_, sq_, W=16, out=FAKE, ws=FAKE, wb=1 << 20: L.kka_pool_anchor(
        ctypes.byref(kp_), ctypes.byref(sq_), W, None, out, ws, wb, None)
    assert f(kp, sq, W=-1) == 2
    assert f(kp, sq, out=None) == 1
    assert f(kp, sq, out=FAKE_ODD) == 3
    assert f(kp, sq, ws=None) == 4
    assert f(kpool(head_dim=7), sq) == 2


def test_anchor_noalloc_validation_and_scratch_limit(L):
    """The allocation-free anchor validates like kka_pool_anchor and refuses,
    before anything is enqueued, a call whose partial sums exceed its fixed
    4 MiB scratch (KKA_ERR_SCRATCH)."""
    kp, sq = kpool(), seqs()
    f = lambda kp_, sq_, W=16, out=FAKE: L.kka_pool_anchor_noalloc(ctypes.byref(kp_), ctypes.byref(sq_), W, None,
                                                                   out, None)
    assert f(kp, sq, W=-1) == 2
    assert f(kp, sq, out=None) == 1
    assert f(kp, sq, out=FAKE_ODD) == 3
    assert f(kpool(head_dim=7), sq) == 2
    scratch = lambda kp_, sq_: L.kka_pool_anchor_noalloc_scratch(ctypes.byref(kp_), ctypes.byref(sq_))
    assert scratch(kp, sq) == 2 * 28 * 128 * 4          # 2 sequences, one share per layer
    assert scratch(kp, seqs(num_seqs=4096, total_blocks=4096)) == 0  # one work-group per sequence
    wide = kpool(num_kv_heads=1, head_dim=1024)
    many = seqs(num_seqs=300, total_blocks=300)
    assert scratch(wide, many) == 300 * 7 * 1024 * 4 > 4 << 20
    assert f(wide, many) == 6
    assert f(kp, seqs(num_seqs=0, total_blocks=0), out=None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    if not os.path.exists(kka.LIB_PATH):
        pytest.skip("libkka.so not built")
    k = torch.zeros(16 * 4 * 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kka.KPool(k, 1, 4, 128, 16, 1)
