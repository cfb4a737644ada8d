"""Benchmark of the Key-Key Semantic Affinity path on one MI355X.

Timed step = the whole path over one batch of the 128K-context 7B-shape
workload (28 layers x 4 KV heads x head_dim 128, 131072 tokens in blocks of
16 = 8192 blocks behind a permuted block table, 3.76 GB of bf16 keys):
block pooling -> anchor pooling -> grid/chunk vectors -> affinity of all
8736 level rows + Grid->Chunk->Page top-4/16/64.  Inputs are resident in
HBM before timing starts.  Also measured: the serving-scale decode step
(score + top-K for 64 sequences x 8192 block vectors, rotating three
buffer sets so no step finds its rows in the 256 MB last-level cache) and
the CPU oracle on the same workload.

Prints one JSON line.  Algorithmic bytes are counted once per launch:
  K-pool   = sum(n_b * L * H * D * 2) + n_blocks * D * 4 + n_blocks * 4
  anchor   = W * L * H * D * 2 + D * 4
  levels   = n_pages * D * 4 + (n_chunks + n_grids) * D * 4
  score    = rows * D * 4 + S * D * 4 + rows * 4 + S * k_page * 8
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "K-pool HBM GB/s (% peak); score+top-K µs/decode step, 7B shape @128K ctx"
COUNTERS = os.path.join(ROOT, "profiles", "kpool_7b_128k_hbm_counters.json")
SCORE_COUNTERS = os.path.join(ROOT, "profiles", "score_topk_64seq_decode_hbm_counters.json")


def kernel_source_hash(name: str) -> str:
    with open(os.path.join(ROOT, "kv_cache_block_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kpool_bytes(w) -> int:
    import numpy as np
    B = w.B
    n_tok = 0
    for s in range(w.S):
        n_tok += int(w.seq_len[s])
    nb = w.total_blocks
    return n_tok * w.L * w.H * w.D * 2 + nb * w.D * 4 + nb * 4


def score_bytes(S, rows, D, k_page) -> int:
    return S * rows * D * 4 + S * D * 4 + S * rows * 4 + S * k_page * 8


def score_traffic_from_counters():
    """HBM bytes per serving-batch kka_score_topk call (scoring launch plus
    selection launch) from the committed counter runs, if they were taken on
    the current scoring source; else None."""
    try:
        with open(SCORE_COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash("kka_score.hip"):
        return None
    return c.get("traffic_bytes_per_call")


def host_info() -> dict:
    """CPU model and the cores this process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "usable_cores": usable, "os_cpu_count": os.cpu_count()}


def traffic_from_counters(algo_bytes_unused=None):
    """HBM bytes per K-pool launch from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256_16") != kernel_source_hash("kka_pool.hip"):
        return None
    return c.get("traffic_bytes_per_launch")


_HIP = None


def _hip_runtime():
    """The HIP runtime library this process has loaded (torch's), so that
    its events and torch's streams belong to one runtime."""
    global _HIP
    if _HIP is None:
        import ctypes
        with open("/proc/self/maps") as f:
            paths = [ln.split()[-1] for ln in f if "libamdhip64" in ln]
        if not paths:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        H = ctypes.CDLL(paths[0])
        H.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        H.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        H.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = H
    return _HIP


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it skips the system-scope cache write-back and invalidate that
    a default event (torch.cuda.Event) performs, which adds about 2 us to
    every interval such events bracket.  Its timestamp is still taken once
    the work queued before it on the stream has completed.  Same interface
    as torch.cuda.Event for record() and elapsed_time() (milliseconds)."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self._H = _hip_runtime()
        self._ev = ctypes.c_void_p()
        rc = self._H.hipEventCreateWithFlags(ctypes.byref(self._ev), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        import ctypes
        rc = self._H.hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self._H.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "_ev", None) is not None and self._ev.value:
            self._H.hipEventDestroy(self._ev)
            self._ev = None


def run(args):
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- c3 step
    t_gen = time.perf_counter()
    w = synth.config3(args.seed)
    gen_s = time.perf_counter() - t_gen
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                    torch.from_numpy(w.block_table).to(dev), w.total_blocks)
    sel = Selector(kp, seqs, w.select, max_pages=w.total_blocks, window=w.window, device=dev)
    npg = torch.tensor([w.total_blocks], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        sel.pool()
        if evs is not None:
            evs[1].record(stream)
        sel.anchor()
        if evs is not None:
            evs[2].record(stream)
        sel.levels(npg)
        if evs is not None:
            evs[3].record(stream)
        sel.score(npg)
        if evs is not None:
            evs[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[TimingEvent() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if kka.kka_device_error() != 0:
        raise RuntimeError("device error flag raised during the benchmark")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    pool_ms = [e[0].elapsed_time(e[1]) for e in events]
    anchor_ms = [e[1].elapsed_time(e[2]) for e in events]
    levels_ms = [e[2].elapsed_time(e[3]) for e in events]
    score_ms = [e[3].elapsed_time(e[4]) for e in events]
    anchor_us = 1e3 * float(np.mean(anchor_ms))
    anchor_med_us = 1e3 * float(np.median(anchor_ms))
    levels_us = 1e3 * float(np.mean(levels_ms))
    pool_us = 1e3 * float(np.mean(pool_ms))
    c3_score_us = 1e3 * float(np.mean(score_ms))
    pool_med_us = 1e3 * float(np.median(pool_ms))
    c3_score_med_us = 1e3 * float(np.median(score_ms))

    n_p = w.total_blocks
    n_c = -(-n_p // w.select["pages_per_chunk"])
    n_g = -(-n_c // w.select["chunks_per_grid"])
    rows = n_p + n_c + n_g
    b_pool = kpool_bytes(w)
    b_anchor = w.window * w.L * w.H * w.D * 2 + w.D * 4
    b_levels = n_p * w.D * 4 + (n_c + n_g) * w.D * 4
    b_score = score_bytes(1, rows, w.D, w.select["k_page"])
    step_bytes = b_pool + b_anchor + b_levels + b_score
    kpool_gbps = b_pool / (pool_us * 1e-6) / 1e9
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the timed steps must still find the planted anchor run (parity itself is the tests' job)
    run = w.extra["anchor_run"]
    if not set(range(run * 32, run * 32 + 32)) <= set(sel.page_idx[0].cpu().numpy().tolist()):
        raise RuntimeError("benchmark selection lost the planted anchor run")

    # c3 lazy (coarse-to-fine) scoring of the same levels: must select the same pages
    full_idx = sel.page_idx.clone()
    def lazy3(i):
        sel.score(npg, lazy=True)
    c3_lazy_us = time_calls(lazy3, args.steps, max(3, args.warmup), stream)
    if not torch.equal(sel.page_idx, full_idx):
        raise RuntimeError("lazy scoring selected different pages than the full pass")
    c3_lazy_rows = lazy_rows(n_g, w.select)
    # the launch floor of this stream: a one-element torch add, event-timed
    # like the calls above (what any launch costs before it does any work)
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    def tiny_add(i):
        tiny.add_(1.0)
    floor_us = time_calls(tiny_add, args.steps, max(3, args.warmup), stream)
    # the score call and the floor again between torch's default events
    # (a system-scope fence at each record), for comparison with timings
    # taken that way
    def torch_event():
        return torch.cuda.Event(enable_timing=True)
    def score3_torch(i):
        sel.score(npg)
    def tiny_add_torch(i):
        tiny.add_(1.0)
    c3_score_torch_us = time_calls(score3_torch, args.steps, max(3, args.warmup), stream, event=torch_event)
    floor_torch_us = time_calls(tiny_add_torch, args.steps, max(3, args.warmup), stream, event=torch_event)

    # c3 attention reference (QK^T softmax averaged over layers and query
    # heads, per block) for one planted decode query with 28 query heads, and
    # the overlap of its top-64 with the key-key top-64
    Hq = 28
    q3 = torch.from_numpy(synth.planted_queries(w, Hq, 12.0, 1.0, seed=args.seed)[None].copy()).to(dev)
    att3 = torch.zeros((1, w.total_blocks), dtype=torch.float32, device=dev)
    aidx3 = torch.zeros((1, 64), dtype=torch.int32, device=dev)
    ws_att = kka.new_workspace(kka.kka_attention_topk_workspace(kp, seqs, Hq), dev)

    def attn3(i):
        kka.kka_attention_topk(kp, seqs, q3, Hq, att3, w.total_blocks, k=64, idx_out=aidx3, workspace=ws_att)

    attn_us = time_calls(attn3, min(args.steps, 20), 2, stream)
    attn_bytes = w.L * w.H * w.D * 2 * int(w.seq_len[0]) + w.L * Hq * w.D * 4 + w.total_blocks * 4 + 64 * 8
    c3_overlap = overlap(sel.page_idx[0, :64].cpu().numpy(), aidx3[0].cpu().numpy(), 64)

    # ---------------------------------------------------------------- pool-on-write decode step
    # 64 sequences of the same 7B key shape, each owning 128 blocks of this
    # pool; every step appends one token per sequence (its keys stored into
    # the pool, its block's vector brought up to date).
    S_w, nb_w = 64, 128
    len_w = torch.full((S_w,), 1990, dtype=torch.int32, device=dev)
    offs_w = torch.arange(0, (S_w + 1) * nb_w, nb_w, dtype=torch.int32, device=dev)
    seqs_w = kka.Seqs(len_w, offs_w, torch.from_numpy(w.block_table[:S_w * nb_w].copy()).to(dev), S_w * nb_w)
    vb_w = torch.zeros((S_w, nb_w, w.D), dtype=torch.float32, device=dev)
    run_w = torch.zeros((S_w, w.D), dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    new_k = (torch.randn((S_w, w.L, w.H, w.D), generator=g, device=dev)).to(torch.bfloat16)
    kka.kka_pool_on_write(kp, seqs_w, vb_w, run_w, new_k=new_k, seed=True, vb_seq_stride=nb_w)

    def write_step(i):
        len_w.add_(1)
        kka.kka_pool_on_write(kp, seqs_w, vb_w, run_w, new_k=new_k, vb_seq_stride=nb_w)

    # time only the library launch: the length update sits outside the events
    n_w = min(args.steps, 2040 - 1991 - max(3, args.warmup))
    for _ in range(max(3, args.warmup)):
        write_step(0)
    torch.cuda.synchronize()
    ev_w = [[TimingEvent() for _ in range(2)] for _ in range(n_w)]
    if hasattr(torch.cuda, "_sleep"):
        # the host queues every timed call while the device spins (see time_calls)
        torch.cuda._sleep(int(n_w * 100e-6 * 2.4e9))
    for i in range(n_w):
        len_w.add_(1)
        ev_w[i][0].record(stream)
        kka.kka_pool_on_write(kp, seqs_w, vb_w, run_w, new_k=new_k, vb_seq_stride=nb_w)
        ev_w[i][1].record(stream)
    torch.cuda.synchronize()
    write_us = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in ev_w]))
    write_bytes = S_w * (2 * w.L * w.H * w.D * 2 + 3 * w.D * 4)
    if kka.kka_device_error() != 0:
        raise RuntimeError("device error flag raised by pool-on-write")

    del sel, k, kp
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- c4 decode step
    v = synth.config4(args.seed)
    S, NP, D = v.vb.shape
    lay4 = kka.LevelLayout(S, NP, D, True, 16, 16)
    npg4 = torch.full((S,), NP, dtype=torch.int32, device=dev)
    n_sets = 3
    levels = []
    base = lay4.new_buffer(dev)
    base[:, :NP] = torch.from_numpy(v.vb).to(dev)
    kka.kka_build_levels(lay4, base, npg4)
    levels.append(base)
    for _ in range(n_sets - 1):
        levels.append(base.clone())
    anchors = torch.from_numpy(v.anchors).to(dev)
    kp4 = v.select["k_page"]
    idx4 = torch.zeros((S, kp4), dtype=torch.int32, device=dev)
    sc4 = torch.zeros((S, kp4), dtype=torch.float32, device=dev)
    cnt4 = torch.zeros(S, dtype=torch.int32, device=dev)
    affs = [torch.zeros((S, lay4.rows_per_seq), dtype=torch.float32, device=dev) for _ in range(n_sets)]
    ws4 = kka.new_workspace(kka.kka_score_topk_workspace(lay4, True), dev)

    def score4(i):
        kka.kka_score_topk(lay4, levels[i % n_sets], npg4, anchors, k_page=kp4, k_grid=v.select["k_grid"],
                           k_chunk=v.select["k_chunk"], page_idx_out=idx4, page_score_out=sc4, n_selected_out=cnt4,
                           affinity_out=affs[i % n_sets], workspace=ws4)

    for i in range(max(3, args.warmup)):
        score4(i)
    torch.cuda.synchronize()
    ev4 = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    if hasattr(torch.cuda, "_sleep"):
        # the host queues every timed call while the device spins (see time_calls)
        torch.cuda._sleep(int(args.steps * 100e-6 * 2.4e9))
    for i in range(args.steps):
        ev4[i][0].record(stream)
        score4(i)
        ev4[i][1].record(stream)
    torch.cuda.synchronize()
    c4_ms = [e[0].elapsed_time(e[1]) for e in ev4]
    c4_us = 1e3 * float(np.mean(c4_ms))
    c4_med_us = 1e3 * float(np.median(c4_ms))
    # the same calls on one buffer set: the level rows stay in the last-level cache
    def score4_warm(i):
        score4(0)
    c4_warm_us = time_calls(score4_warm, args.steps, args.warmup, stream)
    rows4 = lay4.rows_per_seq
    b4 = score_bytes(S, rows4, D, kp4)
    c4_gbps = b4 / (c4_us * 1e-6) / 1e9
    # every sequence must select its planted topic
    got = idx4.cpu().numpy()
    recovered = int(sum((v.page_topic[s][got[s]] == v.anchor_topic[s]).all() for s in range(S)))
    if recovered != S:
        raise RuntimeError(f"serving selection lost the planted topic in {S - recovered} of {S} sequences")

    # lazy (coarse-to-fine) scoring of the same batch: same selection, fewer rows read
    def lazy4(i):
        kka.kka_score_topk_lazy(lay4, levels[i % n_sets], npg4, anchors, k_page=kp4, k_grid=v.select["k_grid"],
                                k_chunk=v.select["k_chunk"], page_idx_out=idx4, page_score_out=sc4,
                                n_selected_out=cnt4, affinity_out=affs[i % n_sets], workspace=ws4)

    c4_lazy_us = time_calls(lazy4, args.steps, max(3, args.warmup), stream)
    if not np.array_equal(idx4.cpu().numpy(), got):
        raise RuntimeError("lazy scoring selected different pages than the full pass (serving batch)")
    n_c4 = -(-NP // 16)
    n_g4 = -(-n_c4 // 16)
    c4_lazy_rows = lazy_rows(n_g4, v.select)

    # single pass with the stability filter fused in (window 20, theta 0.5)
    hist4 = torch.zeros((S, NP), dtype=torch.int32, device=dev)
    stab4 = torch.zeros((S, NP), dtype=torch.float32, device=dev)

    def stable4(i):
        kka.kka_score_topk_stable(lay4, levels[i % n_sets], npg4, anchors, history=hist4, stability_out=stab4,
                                  window=20, theta=0.5, k_page=kp4, k_grid=v.select["k_grid"],
                                  k_chunk=v.select["k_chunk"], page_idx_out=idx4, page_score_out=sc4,
                                  n_selected_out=cnt4, affinity_out=affs[i % n_sets], workspace=ws4)

    c4_stable_us = time_calls(stable4, args.steps, max(3, args.warmup), stream)
    if not np.array_equal(idx4.cpu().numpy(), got):
        raise RuntimeError("scoring with the stability filter selected different pages (serving batch)")

    del levels, affs, ws4, hist4, stab4
    torch.cuda.empty_cache()
    others = reported_configs(args, dev, stream)

    quality = quality_overlaps(args, dev)
    quality["7B_128K_b16_uniform_hier_top64"] = {"overlap": c3_overlap}

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, step_bytes, args.cpu_seconds)
        cpu_all = cpu_baseline_all_cores(w, step_bytes, args.cpu_seconds)

    traffic = traffic_from_counters()
    out = {
        "metric": METRIC,
        "value": round(kpool_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "7B key shape (28 layers x 4 KV heads x head_dim 128), 131072-token context, "
                        "block 16 = 8192 blocks behind a permuted block table, bf16 keys, 256 planted topics; "
                        "uniform pooling, anchor = last 16 tokens, grid/chunk/page 16x16, top 4/16/64",
            "step": "pool all blocks + anchor + build levels + score all 8736 rows + hierarchical top-K",
            "key_dtype": "bf16",
            "accumulate_dtype": "f32",
            "step_algorithmic_bytes": step_bytes,
        },
        "value_is": "K-pool GB/s: algorithmic bytes of one kka_pool_blocks launch over the 8192 blocks / its mean "
                    "event-timed duration",
        "step_GBps": round(step_gbps, 2),
        "anchor_us": round(anchor_us, 2),
        "anchor_median_us": round(anchor_med_us, 2),
        "anchor_algorithmic_bytes": b_anchor,
        "anchor_GBps": round(b_anchor / (anchor_us * 1e-6) / 1e9, 2),
        "levels_us": round(levels_us, 2),
        "levels_algorithmic_bytes": b_levels,
        "kpool_GBps": round(kpool_gbps, 2),
        "kpool_frac_of_peak": round(kpool_gbps / PEAK_HBM_GBPS, 4),
        "kpool_us": round(pool_us, 2),
        "kpool_median_us": round(pool_med_us, 2),
        "kpool_algorithmic_bytes": b_pool,
        "score_topk_us_per_step": round(c3_score_us, 2),
        "score_topk_median_us": round(c3_score_med_us, 2),
        "score_topk_launches": "one (score_select_kernel): 69 work-groups score every row; the one that "
                               "finishes the sequence's last tile selects it (lean selection)",
        "serving_score_topk_launches": "one (score_topk_kernel): a selecting work-group per sequence "
                                       "(coarse-to-fine, re-scoring its candidate rows) beside the work-groups "
                                       "that score every row",
        "serving_score_topk_us_per_step": round(c4_us, 2),
        "serving_score_topk_median_us": round(c4_med_us, 2),
        "serving_score_topk_warm_cache_us": round(c4_warm_us, 2),
        "serving_score_topk_warm_cache_median_us": median_of(score4_warm),
        "serving_score_topk_GBps": round(c4_gbps, 2),
        "serving_score_topk_frac_of_peak": round(c4_gbps / PEAK_HBM_GBPS, 4),
        "serving_workload": "64 sequences x 8192 fp32 block vectors (D=128) + 512 chunk + 32 grid rows each, "
                            "top 4/16/64, three rotating buffer sets (cold last-level cache)",
        "serving_algorithmic_bytes": b4,
        "lazy_score_topk_us_per_step": round(c3_lazy_us, 2),
        "lazy_score_topk_median_us": median_of(lazy3),
        "launch_floor_us": round(floor_us, 2),
        "launch_floor_median_us": median_of(tiny_add),
        "launch_floor": "one-element torch add_ on the same stream, event-timed like the score calls",
        "event_timing": "HIP events created with hipEventDisableSystemFence (timing only) around each call; the "
                        "*_torch_event_* fields time the same calls between torch.cuda.Event pairs",
        "score_topk_torch_event_us": round(c3_score_torch_us, 2),
        "score_topk_torch_event_median_us": median_of(score3_torch),
        "launch_floor_torch_event_us": round(floor_torch_us, 2),
        "lazy_rows_scored_per_seq": c3_lazy_rows,
        "serving_lazy_score_topk_us_per_step": round(c4_lazy_us, 2),
        "serving_lazy_score_topk_median_us": median_of(lazy4),
        "serving_lazy_rows_scored_per_seq": c4_lazy_rows,
        "serving_stable_score_topk_us_per_step": round(c4_stable_us, 2),
        "serving_stable_score_topk_median_us": median_of(stable4),
        "pool_on_write_us_per_step": round(write_us, 2),
        "pool_on_write_workload": "64 sequences x 7B key shape, one token appended per sequence (keys stored into "
                                  "the paged pool, open block's vector updated)",
        "pool_on_write_algorithmic_bytes": write_bytes,
        "attention_reference_us": round(attn_us, 2),
        "attention_reference_GBps": round(attn_bytes / (attn_us * 1e-6) / 1e9, 2),
        "attention_reference_workload": "one decode query, 28 query heads over the 7B 128K pool: QK^T softmax "
                                        "averaged over layers and heads per block, top-64",
        "attention_reference_algorithmic_bytes": attn_bytes,
        "qk_overlap": quality,
        "reported_configs": others,
        "serving_topic_recovered_seqs": recovered,
        "roofline": {
            "bound": "hbm",
            "kernel": "pool_kernel<uniform> (kka_pool_blocks)",
            "achieved": round(kpool_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(kpool_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
        "roofline_serving_score": {
            "bound": "hbm",
            "kernel": "kka_score_topk: score_topk_kernel, one launch (whole call, event-timed)",
            "achieved": round(c4_gbps, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(c4_gbps / PEAK_HBM_GBPS, 4),
            "traffic": score_traffic_from_counters(),
        },
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "generation_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)


def quality_overlaps(args, dev):
    """The page's quality metric on planted workloads: overlap of the key-key
    top-k with the attention top-k (one planted decode query), uniform and
    variance-weighted pooling, plus the share of planted anchor-topic blocks
    in each top-k."""
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    res = {}
    for name, w, Hq, amp, noise in (("0.5B_4K_b16", synth.config1(args.seed), 14, 8.0, 0.5),
                                    ("7B_32K_b128_bias_heads", synth.config2(args.seed), 28, 12.0, 1.0)):
        k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
        kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
        seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                        torch.from_numpy(w.block_table).to(dev), w.total_blocks)
        kq = w.select["k_page"]
        q = torch.from_numpy(synth.planted_queries(w, Hq, amp, noise, seed=args.seed)[None].copy()).to(dev)
        att = torch.zeros((1, w.total_blocks), dtype=torch.float32, device=dev)
        aidx = torch.zeros((1, kq), dtype=torch.int32, device=dev)
        kka.kka_attention_topk(kp, seqs, q, Hq, att, w.total_blocks, k=kq, idx_out=aidx)
        a_idx = aidx[0].cpu().numpy()
        topic = w.block_topic[0]
        entry = {"k": kq, "attention_topic_share": float((topic[a_idx] == w.anchor_topic[0]).mean())}
        # also at k = the number of planted anchor-topic blocks, where both
        # methods should pick exactly the relevant set
        kt = int((topic == w.anchor_topic[0]).sum())
        aidx_t = torch.zeros((1, kt), dtype=torch.int32, device=dev)
        kka.kka_attention_topk(kp, seqs, q, Hq, att, w.total_blocks, k=kt, idx_out=aidx_t)
        a_idx_t = aidx_t[0].cpu().numpy()
        entry["k_topic"] = kt
        npg = torch.tensor([w.total_blocks], dtype=torch.int32, device=dev)
        for mode_name, mode in (("uniform", kka.WEIGHT_UNIFORM), ("variance", kka.WEIGHT_VARIANCE)):
            sel = Selector(kp, seqs, w.select, max_pages=w.total_blocks, window=w.window, mode=mode, device=dev)
            sel.step(npg)
            s_idx = sel.page_idx[0, :kq].cpu().numpy()
            sel_t = Selector(kp, seqs, dict(w.select, k_page=kt), max_pages=w.total_blocks, window=w.window,
                             mode=mode, device=dev)
            sel_t.step(npg)
            entry[mode_name] = {"overlap": overlap(s_idx, a_idx, kq),
                                "topic_share": float((topic[s_idx] == w.anchor_topic[0]).mean()),
                                "overlap_at_k_topic": overlap(sel_t.page_idx[0, :kt].cpu().numpy(), a_idx_t, kt)}
        torch.cuda.synchronize()
        res[name] = entry
        del k, kp, seqs
        torch.cuda.empty_cache()
    # positional heads (shared drift with position, small spread) beside topic
    # heads of graded relevance (large spread): the case variance weighting is for
    w, q_np, rel, role = synth.positional_heads_workload(args.seed)
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                    torch.from_numpy(w.block_table).to(dev), w.total_blocks)
    kq, Hq = w.select["k_page"], q_np.shape[1]
    att = torch.zeros((1, w.total_blocks), dtype=torch.float32, device=dev)
    aidx = torch.zeros((1, kq), dtype=torch.int32, device=dev)
    kka.kka_attention_topk(kp, seqs, torch.from_numpy(q_np[None].copy()).to(dev), Hq, att, w.total_blocks, k=kq,
                           idx_out=aidx)
    a_idx = aidx[0].cpu().numpy()
    entry = {"k": kq, "attention_mean_relevance": round(float(rel[a_idx].mean()), 4),
             "workload": "0.5B key shape, 4096 tokens, 16 topic heads of graded relevance r ~ U(0, 1) and 32 "
                         "positional heads (a drift with position shared by all of them); the query attends "
                         "through the topic heads"}
    npg = torch.tensor([w.total_blocks], dtype=torch.int32, device=dev)
    for mode_name, mode in (("uniform", kka.WEIGHT_UNIFORM), ("variance", kka.WEIGHT_VARIANCE)):
        sel = Selector(kp, seqs, w.select, max_pages=w.total_blocks, window=w.window, mode=mode, device=dev)
        sel.step(npg)
        s_idx = sel.page_idx[0, :kq].cpu().numpy()
        entry[mode_name] = {"overlap": overlap(s_idx, a_idx, kq),
                            "mean_relevance": round(float(rel[s_idx].mean()), 4)}
    torch.cuda.synchronize()
    res["0.5B_positional_heads"] = entry
    del k, kp, seqs
    torch.cuda.empty_cache()
    return res


def overlap(a, b, k):
    """Share of the top-k set a that is also in the top-k set b."""
    return len(set(list(a)[:k]) & set(list(b)[:k])) / k if k else 0.0


def time_calls(fn, steps, warmup, stream, event=None):
    """Mean device time (us) of fn(i), bracketed by timing events (or
    `event()` instances) on `stream`.  A spinning kernel queued first keeps
    the device busy while the host queues every timed call, so no host-side
    gap falls between an event and its call."""
    import numpy as np
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    make = event or TimingEvent
    ev = [[make() for _ in range(2)] for _ in range(steps)]
    if hasattr(torch.cuda, "_sleep"):
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(steps * 100e-6 * 2.4e9))  # about 100 us of device time per call queued
    for i in range(steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    _MEDIANS[fn] = 1e3 * float(np.median(ms))
    return 1e3 * float(np.mean(ms))


# median (us) of the last time_calls of each function: one stalled call moves
# a mean of 50 by microseconds, a median not at all
_MEDIANS = {}


def median_of(fn) -> float:
    return round(_MEDIANS.get(fn, float("nan")), 2)


def reported_configs(args, dev, stream):
    """K-pool GB/s of the 0.5B and 7B/32K workloads, and for the ragged
    variance-weighted batch the weighted K-pool GB/s (one-pass algorithmic
    bytes) and one decode step (re-pool of each sequence's newest block with
    the frozen weights, anchor, score, flat top-48).  Reported, not gated.
    Each timed call follows an untimed 1 GiB write, so no input is served
    from the last-level cache."""
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def cold_us(fn, steps):
        ev = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            flush.zero_()
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
        return float(np.mean(t)), float(np.median(t))

    def upload(w):
        k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
        kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
        seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                        torch.from_numpy(w.block_table).to(dev), w.total_blocks)
        return k, kp, seqs

    out = {}
    for name, w in (("0.5B_4K_b16", synth.config1(args.seed)), ("7B_32K_b128", synth.config2(args.seed))):
        k, kp, seqs = upload(w)
        sel = Selector(kp, seqs, w.select, max_pages=w.total_blocks, window=w.window, device=dev)
        for _ in range(args.warmup):
            sel.pool()
        mean_us, med_us = cold_us(sel.pool, args.steps)
        b = kpool_bytes(w)
        out[name] = {"kpool_us": round(mean_us, 2), "kpool_median_us": round(med_us, 2),
                     "kpool_algorithmic_bytes": b, "kpool_GBps": round(b / (mean_us * 1e-6) / 1e9, 2),
                     "kpool_frac_of_peak": round(b / (mean_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        del sel, kp, seqs, k
    torch.cuda.empty_cache()

    w = synth.config5(args.seed)
    after = w.extra["after"]
    k, kp, seqs = upload(w)
    max_pages = int(np.max(np.diff(after["block_offsets"])))
    sel = Selector(kp, seqs, w.select, max_pages=max_pages, window=w.window, mode=kka.WEIGHT_VARIANCE, device=dev)
    steps5 = max(5, args.steps // 5)
    for _ in range(2):
        sel.pool()
    pool_mean, pool_med = cold_us(sel.pool, steps5)
    b5 = kpool_bytes(w)
    npg = torch.from_numpy(np.diff(w.block_offsets).astype(np.int32)).to(dev)
    sel.anchor()
    sel.score(npg)
    # the decode step: one token more per sequence, newest block re-pooled with the frozen weights
    sel.seqs = kka.Seqs(torch.from_numpy(after["seq_len"]).to(dev), torch.from_numpy(after["block_offsets"]).to(dev),
                        torch.from_numpy(after["block_table"]).to(dev), int(after["block_offsets"][-1]))
    newest = torch.from_numpy((after["block_offsets"][1:] - 1).astype(np.int32)).to(dev)
    npg_after = torch.from_numpy(np.diff(after["block_offsets"]).astype(np.int32)).to(dev)
    ws_re = kka.new_workspace(kka.kka_pool_blocks_workspace(kp, sel.seqs, kka.WEIGHT_GIVEN, newest), dev)

    def decode():
        sel.decode_step(newest, npg_after, workspace=ws_re)

    for _ in range(args.warmup):
        decode()
    dec_mean, dec_med = cold_us(decode, args.steps)
    if kka.kka_device_error() != 0:
        raise RuntimeError("device error flag raised on the ragged batch")
    out["ragged32_b64_variance"] = {
        "sequences": int(w.S), "tokens": int(w.seq_len.sum()), "blocks": int(w.total_blocks),
        "weighted_kpool_us": round(pool_mean, 2), "weighted_kpool_median_us": round(pool_med, 2),
        "kpool_algorithmic_bytes": b5, "weighted_kpool_GBps": round(b5 / (pool_mean * 1e-6) / 1e9, 2),
        "weighted_kpool_frac_of_peak": round(b5 / (pool_mean * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "decode_step_us": round(dec_mean, 2), "decode_step_median_us": round(dec_med, 2),
        "decode_step": "re-pool the newest block of each sequence (frozen weights) + anchor + score + flat top-48",
    }
    del sel, kp, seqs, k, flush
    torch.cuda.empty_cache()
    return out


def lazy_rows(n_g, select):
    """Rows the coarse-to-fine pass scores per sequence (full-length levels):
    every grid, the chunks of the kept grids, the pages of the kept chunks."""
    return n_g + min(select["k_grid"], n_g) * select["chunks_per_grid"] + select["k_chunk"] * select["pages_per_chunk"]


def cpu_baseline(w, step_bytes, seconds):
    """The oracle as it stands (single-threaded C) over the same workload:
    whole steps (pool every block, anchor, levels, affinity, selection)
    repeated until `seconds` have passed; GB/s on the step's algorithmic
    bytes."""
    import numpy as np
    import oracle

    kp = oracle.KPool.of(w)
    reps = 0
    t0 = time.perf_counter()
    while True:
        vb = oracle.pool_blocks(kp, w.seq_len, w.block_offsets, w.block_table)
        pages = np.stack([vb[b] for b in range(w.total_blocks)])
        a = oracle.pool_anchor(kp, w.block_table, int(w.seq_len[0]), w.window)
        oracle.score_select(pages, a, w.select)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    gbps = reps * step_bytes / el / 1e9
    # the per-decode-step part alone (chunk and grid vectors, affinities, hierarchical top-K)
    n_sel = 0
    t1 = time.perf_counter()
    while True:
        oracle.score_select(pages, a, w.select)
        n_sel += 1
        el_sel = time.perf_counter() - t1
        if el_sel >= min(2.0, seconds) or n_sel >= 200:
            break
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole step(s) of the same 131072-token workload ({reps * step_bytes / 1e9:.2f} GB "
                      f"of algorithmic bytes) in {el:.1f} s on one host core",
            "ms_per_step": round(el * 1e3 / reps, 1),
            "levels_score_topk_ms_per_step": round(el_sel * 1e3 / n_sel, 3),
            "levels_score_topk_sample": f"{n_sel} decode step(s) of the same sequence: chunk and grid vectors, "
                                        "affinity of every row, hierarchical top-K",
            "host": host_info()}


def cpu_baseline_all_cores(w, step_bytes, seconds):
    """The same oracle steps with the per-block pooling partitioned over
    every usable host core (threads calling the unchanged single-threaded C
    oracle on disjoint block ranges; the C calls run without the GIL); the
    anchor, levels, affinity and selection of the one sequence stay on one
    thread."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    kp = oracle.KPool.of(w)
    n = max(1, host_info()["usable_cores"])
    nb = w.total_blocks
    ranges = [(i * nb // n, (i + 1) * nb // n) for i in range(n)]
    pages = np.empty((nb, w.D), dtype=np.float32)

    def pool_range(r):
        lo, hi = r
        for b in range(lo, hi):
            s = 0  # one sequence: block b is logical block b of sequence 0
            pages[b] = oracle.pool_block(kp, int(w.block_table[b]), oracle.n_valid(w.seq_len, kp.B, b, s))

    reps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        while True:
            list(ex.map(pool_range, ranges))
            a = oracle.pool_anchor(kp, w.block_table, int(w.seq_len[0]), w.window)
            oracle.score_select(pages, a, w.select)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 200:
                break
    gbps = reps * step_bytes / el / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"{reps} whole step(s) of the same 131072-token workload ({reps * step_bytes / 1e9:.2f} GB "
                      f"of algorithmic bytes) in {el:.1f} s, block pooling split over {n} threads",
            "ms_per_step": round(el * 1e3 / reps, 1)}


def oracle_table(args):
    """The oracle as it stands, timed on the host over each workload (bounded
    samples), on one core and split over every usable core (threads calling
    the unchanged single-threaded C oracle on disjoint items): the CPU
    columns of the results table.  GB/s on the algorithmic bytes of what was
    timed."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    n = max(1, host_info()["usable_cores"])

    def timed(fn, items, threads, budget_s=2.0):
        """Mean seconds of one pass of fn over items, passes repeated until
        budget_s has gone by (one pass at least), one untimed pass first when
        a pass is short."""
        items = list(items)
        slices = [items[i::threads] for i in range(threads)]

        def run(part):
            for x in part:
                fn(x)

        def one_pass(ex):
            if ex is None:
                run(items)
            else:
                list(ex.map(run, slices))
        ex = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None
        try:
            t0 = time.perf_counter()
            one_pass(ex)
            first = time.perf_counter() - t0
            if first >= budget_s:
                return first
            reps, t0 = 0, time.perf_counter()
            while reps == 0 or time.perf_counter() - t0 < budget_s:
                one_pass(ex)
                reps += 1
            return (time.perf_counter() - t0) / reps
        finally:
            if ex is not None:
                ex.shutdown()

    out = {"host": host_info()}
    for name, w in (("0.5B_4K_b16", synth.config1(args.seed)), ("7B_32K_b128", synth.config2(args.seed)),
                    ("7B_128K_b16", synth.config3(args.seed))):
        kp = oracle.KPool.of(w)
        blocks = list(range(w.total_blocks))

        def pool(b):
            oracle.pool_block(kp, int(w.block_table[b]), oracle.n_valid(w.seq_len, kp.B, b, 0))
        b_all = kpool_bytes(w)
        t1 = timed(pool, blocks, 1)
        tn = timed(pool, blocks, n)
        out[name] = {"stage": "K-pool (every block)", "bytes": b_all, "oracle_1core_ms": round(t1 * 1e3, 1),
                     "oracle_1core_GBps": round(b_all / t1 / 1e9, 3), "oracle_allcore_ms": round(tn * 1e3, 1),
                     "oracle_allcore_GBps": round(b_all / tn / 1e9, 3)}
    v = synth.config4(args.seed)
    S, NP, D = v.vb.shape

    def step(s):
        oracle.score_select(v.vb[s], v.anchors[s], v.select)
    b4 = score_bytes(S, NP + 512 + 32, D, v.select["k_page"])
    t1 = timed(step, range(8), 1) * S / 8
    tn = timed(step, range(S), n)
    out["serving_64x8192"] = {"stage": "levels + affinity + top-K, 64 sequences (one core: 8 of them, scaled)",
                              "bytes": b4, "oracle_1core_ms": round(t1 * 1e3, 1),
                              "oracle_1core_GBps": round(b4 / t1 / 1e9, 3), "oracle_allcore_ms": round(tn * 1e3, 1),
                              "oracle_allcore_GBps": round(b4 / tn / 1e9, 3)}
    w = synth.config5(args.seed)
    kp = oracle.KPool.of(w)

    def seq_pool(s):
        tab = oracle.seq_table(w.block_offsets, w.block_table, s)
        wts = oracle.head_weights(kp, tab, int(w.seq_len[s]))
        for i in range(len(tab)):
            oracle.pool_block(kp, int(tab[i]), oracle.n_valid(w.seq_len, kp.B, i, s), wts)
    order = np.argsort(w.seq_len)
    sample = [int(order[k]) for k in (0, 8, 16, 24)]
    tok_sample = sum(int(w.seq_len[s]) for s in sample)
    t1 = timed(seq_pool, sample, 1) * int(w.seq_len.sum()) / tok_sample
    tn = timed(seq_pool, [int(x) for x in order[::-1]], n)
    b5 = kpool_bytes(w)
    out["ragged32_b64_variance"] = {"stage": "weights + weighted K-pool (one core: 4 sequences, scaled by tokens)",
                                    "bytes": b5, "oracle_1core_ms": round(t1 * 1e3, 1),
                                    "oracle_1core_GBps": round(b5 / t1 / 1e9, 3),
                                    "oracle_allcore_ms": round(tn * 1e3, 1),
                                    "oracle_allcore_GBps": round(b5 / tn / 1e9, 3), "threads": n}
    print(json.dumps(out), flush=True)


def profile_pass(args):
    """Short run for hardware-counter passes: a plain 1 GiB device copy
    (calibrates FETCH_SIZE / WRITE_SIZE against known bytes), then a few
    K-pool and score launches on the same workload as the benchmark."""
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    dev = "cuda:0"
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = synth.config3(args.seed)
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                    torch.from_numpy(w.block_table).to(dev), w.total_blocks)
    sel = Selector(kp, seqs, w.select, max_pages=w.total_blocks, window=w.window, device=dev)
    npg = torch.tensor([w.total_blocks], dtype=torch.int32, device=dev)
    for _ in range(3):
        sel.step(npg)
    torch.cuda.synchronize()
    del sel, kp, k
    torch.cuda.empty_cache()
    # the serving decode step: 64 sequences, scoring launch then selection launch
    v = synth.config4(args.seed)
    S, NP, D = v.vb.shape
    lay4 = kka.LevelLayout(S, NP, D, True, 16, 16)
    npg4 = torch.full((S,), NP, dtype=torch.int32, device=dev)
    lvl4 = lay4.new_buffer(dev)
    lvl4[:, :NP] = torch.from_numpy(v.vb).to(dev)
    kka.kka_build_levels(lay4, lvl4, npg4)
    anchors = torch.from_numpy(v.anchors).to(dev)
    idx4 = torch.zeros((S, v.select["k_page"]), dtype=torch.int32, device=dev)
    sc4 = torch.zeros((S, v.select["k_page"]), dtype=torch.float32, device=dev)
    aff4 = torch.zeros((S, lay4.rows_per_seq), dtype=torch.float32, device=dev)
    ws4 = kka.new_workspace(kka.kka_score_topk_workspace(lay4, True), dev)
    for _ in range(3):
        kka.kka_score_topk(lay4, lvl4, npg4, anchors, k_page=v.select["k_page"], k_grid=v.select["k_grid"],
                           k_chunk=v.select["k_chunk"], page_idx_out=idx4, page_score_out=sc4, affinity_out=aff4,
                           workspace=ws4)
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": "done", "copy_bytes": (1 << 28) * 4, "kpool_algorithmic_bytes":
                      kpool_bytes(w), "serving_score_algorithmic_bytes": score_bytes(S, lay4.rows_per_seq, D,
                                                                                     v.select["k_page"]),
                      "kernel_source_sha256_16": kernel_source_hash("kka_pool.hip"),
                      "score_source_sha256_16": kernel_source_hash("kka_score.hip")}), flush=True)


def profile_pass_ragged(args):
    """Short run for hardware-counter passes over the variance-weighted
    K-pool of the ragged batch (32 sequences of 4096-65536 tokens, 7B key
    shape, blocks of 64): a plain 1 GiB device copy for calibration, then
    three kka_pool_blocks calls in variance mode."""
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    dev = "cuda:0"
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = synth.config5(args.seed)
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                    torch.from_numpy(w.block_table).to(dev), w.total_blocks)
    sel = Selector(kp, seqs, w.select, max_pages=int(np.max(np.diff(w.block_offsets))), window=w.window,
                   mode=kka.WEIGHT_VARIANCE, device=dev)
    for _ in range(3):
        sel.pool()
    torch.cuda.synchronize()
    if kka.kka_device_error() != 0:
        raise RuntimeError("device error flag raised on the ragged batch")
    print(json.dumps({"profile_pass": "ragged", "copy_bytes": (1 << 28) * 4, "kpool_algorithmic_bytes": kpool_bytes(w),
                      "blocks": int(w.total_blocks), "tokens": int(w.seq_len.sum()),
                      "kernel_source_sha256_16": kernel_source_hash("kka_pool.hip")}), flush=True)


_POOL_PASSES = {
    "ragged": ("kka_pool_blocks, variance mode (all kernels of one call)",
               "32 sequences, lengths uniform in [4096, 65536], 7B key shape (28 x 4 x 128), blocks of 64, "
               "permuted shared pool, head-variance weights"),
    "c1": ("kka_pool_blocks, uniform (one call)",
           "0.5B key shape (24 x 2 x 64), 4096 tokens, block 16 (256 blocks), permuted shared pool"),
    "c2": ("kka_pool_blocks, uniform (one call)",
           "7B key shape (28 x 4 x 128), 32768 tokens, block 128 (256 blocks), permuted shared pool"),
}


def profile_pass_pool(args, which: str):
    """Short run for hardware-counter passes over one K-pool workload (the
    0.5B or 7B/32K uniform pool): a plain 1 GiB device copy for
    calibration, then three kka_pool_blocks calls."""
    import numpy as np
    import torch

    import kv_cache_block_amd as kka
    import synth
    from kv_cache_block_amd.pipeline import Selector

    dev = "cuda:0"
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = synth.config1(args.seed) if which == "c1" else synth.config2(args.seed)
    k = torch.from_numpy(w.k.reshape(-1).view(np.int16)).to(dev)
    kp = kka.KPool(k, w.L, w.H, w.D, w.B, w.P)
    seqs = kka.Seqs(torch.from_numpy(w.seq_len).to(dev), torch.from_numpy(w.block_offsets).to(dev),
                    torch.from_numpy(w.block_table).to(dev), w.total_blocks)
    sel = Selector(kp, seqs, w.select, max_pages=int(np.max(np.diff(w.block_offsets))), window=w.window,
                   mode=kka.WEIGHT_UNIFORM, device=dev)
    for _ in range(3):
        sel.pool()
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": which, "copy_bytes": (1 << 28) * 4, "kpool_algorithmic_bytes": kpool_bytes(w),
                      "kernel_source_sha256_16": kernel_source_hash("kka_pool.hip")}), flush=True)


def write_ragged_counter_summary(fetch_csv: str, write_csv: str, stall_csv: str, out_json: str, command: str,
                                 which: str = "ragged"):
    """Per-kernel HBM bytes of the variance-weighted K-pool of the ragged batch
    from --pmc runs of --profile-pass ragged: FETCH_SIZE, WRITE_SIZE (each
    scaled by what it reads for the 1 GiB copy) and the write-path counters
    of a third run (raw sums per dispatch)."""
    import csv
    import statistics

    def per_kernel(path):
        out = {}
        for r in csv.DictReader(open(path)):
            out.setdefault((r["Kernel_Name"], r["Grid_Size"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        return out

    f = per_kernel(fetch_csv)
    w = per_kernel(write_csv)
    st = per_kernel(stall_csv) if stall_csv != "-" else {}
    copy_bytes = float(1 << 30)
    ck = [k for k in f if "copyBuffer" in k[0] and k[2] == "FETCH_SIZE" and max(f[k]) > 4e5]
    if not ck:
        raise SystemExit("no 1 GiB copy dispatch found in the counter run")
    fetch_factor = copy_bytes / (statistics.median(f[ck[0]]) * 1024.0)
    wk_copy = (ck[0][0], ck[0][1], "WRITE_SIZE")
    write_factor = copy_bytes / (statistics.median(w[wk_copy]) * 1024.0)
    kernels = {}
    total = 0.0
    for k in f:
        if "kka::" not in k[0] or k[2] != "FETCH_SIZE":
            continue
        fb = statistics.mean(f[k]) * 1024.0 * fetch_factor
        wb = statistics.mean(w.get((k[0], k[1], "WRITE_SIZE"), [0.0])) * 1024.0 * write_factor
        entry = {"fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": len(f[k])}
        for sk, v in st.items():
            if sk[0] == k[0] and sk[1] == k[1]:
                entry[sk[2]] = round(statistics.mean(v))
        kernels[f"{_short(k[0])} grid={k[1]}"] = entry
        total += fb + wb
    call, workload = _POOL_PASSES[which]
    summary = {
        "call": call,
        "workload": workload,
        "kernel_source_sha256_16": kernel_source_hash("kka_pool.hip"),
        "fetch_factor": round(fetch_factor, 5),
        "write_factor": round(write_factor, 5),
        "traffic_bytes_per_call": round(total),
        "per_kernel": kernels,
        "commands": command,
    }
    if which != "ragged":
        import synth
        w = synth.config1(0) if which == "c1" else synth.config2(0)
        summary["kpool_algorithmic_bytes"] = kpool_bytes(w)
        summary["traffic_over_algorithmic"] = round(total / kpool_bytes(w), 5)
    with open(out_json, "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps({"traffic_bytes_per_call": summary["traffic_bytes_per_call"]}))


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("kka::(anonymous namespace)::", "")
    return name.split("(kka::")[0] if "(kka::" in name else name[:60]


def write_counter_summary(fetch_csv: str, write_csv: str, out_dir: str, command: str):
    """Per-dispatch HBM bytes of the K-pool kernel and of the serving-batch
    scoring call (scoring launch plus selection launch) from two rocprofv3
    --pmc runs of --profile-pass (FETCH_SIZE, then WRITE_SIZE, in KiB), each
    scaled by what the same counter reads for the plain 1 GiB device copy that
    the profile pass runs first (known bytes: 1 GiB read and 1 GiB written).
    Writes the two summaries into out_dir."""
    import csv
    import statistics

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault((r["Kernel_Name"], r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = float(1 << 30)
    copy_key = [k for k in f if "copyBuffer" in k[0] and max(f[k]) > 4e5]
    if not copy_key:
        raise SystemExit("no 1 GiB copy dispatch found in the counter run")
    fetch_factor = copy_bytes / (statistics.median(f[copy_key[0]]) * 1024.0)
    write_factor = copy_bytes / (statistics.median(w[copy_key[0]]) * 1024.0)
    pool = [k for k in f if "pool_kernel" in k[0]]
    kernels = {}
    for k in f:
        if "kka::" not in k[0]:
            continue
        fk = statistics.mean(f[k]) * 1024.0 * fetch_factor
        wk = statistics.mean(w.get(k, [0.0])) * 1024.0 * write_factor
        kernels[f"{_short(k[0])} grid={k[1]}"] = {"fetch_bytes": round(fk), "write_bytes": round(wk),
                                                  "dispatches": len(f[k])}
    pk = pool[0]
    traffic = statistics.mean(f[pk]) * 1024.0 * fetch_factor + statistics.mean(w[pk]) * 1024.0 * write_factor
    summary = {
        "kernel": _short(pk[0]),
        "workload": "7B key shape, 131072 tokens, block 16 (8192 blocks), uniform pooling",
        "kernel_source_sha256_16": kernel_source_hash("kka_pool.hip"),
        "fetch_factor": round(fetch_factor, 5),
        "write_factor": round(write_factor, 5),
        "traffic_bytes_per_launch": round(traffic),
        "kpool_algorithmic_bytes": 3762323456,
        "traffic_over_algorithmic": round(traffic / 3762323456, 5),
        "per_kernel": kernels,
        "commands": command,
    }
    with open(os.path.join(out_dir, os.path.basename(COUNTERS)), "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps({"traffic_bytes_per_launch": summary["traffic_bytes_per_launch"],
                      "fetch_factor": summary["fetch_factor"], "write_factor": summary["write_factor"]}))
    # serving batch: the one-launch scoring call (grid of 64 selecting groups plus the scoring tiles)
    sk = [k for k in f if "score_topk_kernel" in k[0] and int(k[1]) > 64 * 256 * 64]
    if sk:
        parts = {}
        for k in sk[:1]:
            parts[_short(k[0])] = {"fetch_bytes": round(statistics.mean(f[k]) * 1024.0 * fetch_factor),
                                   "write_bytes": round(statistics.mean(w[k]) * 1024.0 * write_factor),
                                   "dispatches": len(f[k])}
        call = sum(v["fetch_bytes"] + v["write_bytes"] for v in parts.values())
        algo = 288563200
        score = {
            "call": "kka_score_topk on the serving batch: score_topk_kernel (one launch)",
            "workload": "64 sequences x 8192 fp32 block vectors (D = 128) + 512 chunk + 32 grid rows, top 4/16/64",
            "kernel_source_sha256_16": kernel_source_hash("kka_score.hip"),
            "fetch_factor": round(fetch_factor, 5),
            "write_factor": round(write_factor, 5),
            "traffic_bytes_per_call": call,
            "score_algorithmic_bytes": algo,
            "traffic_over_algorithmic": round(call / algo, 5),
            "per_kernel": parts,
            "commands": command,
        }
        with open(os.path.join(out_dir, os.path.basename(SCORE_COUNTERS)), "w") as fh:
            json.dump(score, fh, indent=1)
        print(json.dumps({"traffic_bytes_per_call": call, "over_algorithmic": score["traffic_over_algorithmic"]}))


def write_stats_summary(stats_csv: str, out_md: str, title: str, command: str = ""):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel summary."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", command, "```",
             "", "| kernel | calls | average us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if trace_csv != stats_csv and os.path.exists(trace_csv):
        # the same kernel launched on different workloads, told apart by grid size
        per = {}
        for r in csv.DictReader(open(trace_csv)):
            if "kka::" not in r["Kernel_Name"]:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            per.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "Per launch shape (from the kernel trace of the same run; grid in work-items):", "",
                  "| kernel | grid | work-group | calls | average us | median us | min us |",
                  "|---|---:|---:|---:|---:|---:|---:|"]
        for (name, grid, wg), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            v.sort()
            lines.append(f"| `{name}` | {grid} | {wg} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | "
                         f"{v[0]:.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the oracle on every workload, one core and all cores (no GPU needed)")
    ap.add_argument("--profile-pass", nargs="?", const="c3", choices=["c3", "ragged", "c1", "c2"],
                    help="short run for rocprofv3 counter passes: the 128K workload and the serving batch (c3), or "
                         "the variance-weighted K-pool of the ragged batch (ragged)")
    ap.add_argument("--write-pool-counter-summary", nargs=4, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "OUT"),
                    help="summarise --pmc runs of --profile-pass c1 or c2 (no GPU needed)")
    ap.add_argument("--write-ragged-counter-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "STALL_CSV", "OUT"),
                    help="summarise --pmc runs of --profile-pass ragged (no GPU needed; STALL_CSV may be -)")
    ap.add_argument("--write-counter-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --profile-pass (no GPU needed)")
    ap.add_argument("--write-stats-summary", nargs=3, metavar=("STATS_CSV", "OUT_MD", "TITLE"),
                    help="summarise a rocprofv3 --kernel-trace --stats run (no GPU needed)")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()
    if args.write_counter_summary:
        write_counter_summary(*args.write_counter_summary, command=args.command)
        return
    if args.write_stats_summary:
        write_stats_summary(*args.write_stats_summary, command=args.command)
        return
    if args.write_pool_counter_summary:
        which, fetch_csv, write_csv, out_json = args.write_pool_counter_summary
        if which not in ("c1", "c2"):
            raise SystemExit("--write-pool-counter-summary: WORKLOAD is c1 or c2")
        write_ragged_counter_summary(fetch_csv, write_csv, "-", out_json, command=args.command, which=which)
        return
    if args.write_ragged_counter_summary:
        write_ragged_counter_summary(*args.write_ragged_counter_summary, command=args.command)
        return
    if args.oracle_table:
        oracle_table(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the selection path is independent per sequence and per block, "
              "and this library runs it on a single MI355X; shard sequences or blocks across processes for more GPUs. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.profile_pass == "ragged":
        profile_pass_ragged(args)
    elif args.profile_pass in ("c1", "c2"):
        profile_pass_pool(args, args.profile_pass)
    elif args.profile_pass:
        profile_pass(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
