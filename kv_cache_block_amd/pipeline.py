"""Buffer plumbing for one batch: owns the level buffer, anchors, outputs and
workspaces (torch allocations) and calls the four library entry points in
the order the page "Key-Key Semantic Affinity: Key vectors replace
attention scores for KV-cache importance" (10100.com) gives in section 5.2:
block vectors once when blocks are written, then per decode step anchor ->
(levels) -> affinity + top-K.  No arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (WEIGHT_GIVEN, WEIGHT_UNIFORM, WEIGHT_VARIANCE, KPool, LevelLayout, Seqs, _torch_stream,
               kka_build_levels, kka_pool_anchor, kka_pool_anchor_workspace, kka_pool_blocks,
               kka_pool_blocks_workspace, kka_pool_on_write, kka_score_topk, kka_score_topk_workspace, new_workspace,
               order_after_current)


class Selector:
    """One batch of sequences over one key pool.

    select: dict with hierarchical, k_grid, k_chunk, k_page, pages_per_chunk,
    chunks_per_grid.  max_pages bounds the pages of any sequence (rows per
    sequence in the level buffer).
    """

    def __init__(self, kp: KPool, seqs: Seqs, select: dict, max_pages: int, window: int, mode: int = WEIGHT_UNIFORM,
                 keep_affinity: bool = True, device="cuda", stability_window: int = 0, stability_theta: float = 0.5):
        self.kp, self.seqs, self.sel, self.window, self.mode = kp, seqs, dict(select), window, mode
        S = seqs.num_seqs
        self.lay = LevelLayout(S, max_pages, kp.head_dim, bool(select["hierarchical"]),
                               select.get("pages_per_chunk", 16), select.get("chunks_per_grid", 16))
        self.level = self.lay.new_buffer(device)
        self.anchors = torch.zeros((S, kp.head_dim), dtype=torch.float32, device=device)
        k_page = select["k_page"]
        self.page_idx = torch.full((S, max(1, k_page)), -1, dtype=torch.int32, device=device)
        self.page_score = torch.zeros((S, max(1, k_page)), dtype=torch.float32, device=device)
        self.n_selected = torch.zeros(S, dtype=torch.int32, device=device)
        self.affinity = (torch.zeros((S, self.lay.rows_per_seq), dtype=torch.float32, device=device)
                         if keep_affinity else None)
        LH = kp.num_layers * kp.num_kv_heads
        self.head_weight = torch.zeros((S, LH), dtype=torch.float32, device=device) if mode != WEIGHT_UNIFORM else None
        self.ws_pool = new_workspace(kka_pool_blocks_workspace(kp, seqs, mode), device)
        self.ws_anchor = new_workspace(kka_pool_anchor_workspace(kp, seqs, window), device)
        self.ws_score = new_workspace(kka_score_topk_workspace(self.lay, keep_affinity, k_page,
                                                               select.get("k_grid", 0), select.get("k_chunk", 0)),
                                      device)
        # stability filter state (section 5.3): window words and scores per page
        self.stability_window, self.stability_theta = stability_window, stability_theta
        self.history = self.stability = None
        if stability_window:
            self.history = torch.zeros((S, max_pages), dtype=torch.int32, device=device)
            self.stability = torch.zeros((S, max_pages), dtype=torch.float32, device=device)
        self._streams_seen = set()

    def _on(self, stream):
        """Before the first launch on a stream other than torch's current one:
        order it after the current stream's work (the zero fills of this
        object's buffers and workspaces) and mark the buffers as used there."""
        st = _torch_stream(stream, self.level.device)
        if st is None or st.cuda_stream in self._streams_seen:
            return
        order_after_current(st, self.level.device, self.level, self.anchors, self.page_idx, self.page_score,
                            self.n_selected, self.affinity, self.head_weight, self.ws_pool, self.ws_anchor,
                            self.ws_score, self.history, self.stability, getattr(self, "running", None))
        self._streams_seen.add(st.cuda_stream)

    @property
    def anchor_weights(self) -> Optional[torch.Tensor]:
        return self.head_weight

    def pool(self, stream=None):
        """Block vectors of every block into the page rows of the level buffer
        (variance mode also computes and freezes the head weights)."""
        self._on(stream)
        kka_pool_blocks(self.kp, self.seqs, self.level, mode=self.mode, head_weight=self.head_weight,
                        vb_seq_stride=self.lay.rows_per_seq, workspace=self.ws_pool, stream=stream)

    def repool(self, blocks: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None):
        """Re-pool a subset of blocks with the frozen weights (incremental update).
        Without a workspace the binding allocates a zero-filled one ordered
        before the launch on `stream` and kept alive until it ends."""
        mode = WEIGHT_GIVEN if self.mode != WEIGHT_UNIFORM else WEIGHT_UNIFORM
        self._on(stream)
        kka_pool_blocks(self.kp, self.seqs, self.level, mode=mode, head_weight=self.head_weight, blocks=blocks,
                        vb_seq_stride=self.lay.rows_per_seq, workspace=workspace, stream=stream)

    def append(self, new_k: Optional[torch.Tensor] = None, seed: bool = False, stream=None):
        """Pool-on-write for one decode step (seq_len already counts the new
        token of each sequence): stores new_k into the pool when given and
        brings the open block's page row up to date."""
        if getattr(self, "running", None) is None:
            self.running = torch.zeros((self.seqs.num_seqs, self.kp.head_dim), dtype=torch.float32,
                                       device=self.level.device)
            seed = True
            self._streams_seen.clear()  # a new buffer: order it on every stream again
        self._on(stream)
        mode = WEIGHT_GIVEN if self.mode != WEIGHT_UNIFORM else WEIGHT_UNIFORM
        kka_pool_on_write(self.kp, self.seqs, self.level, self.running, new_k=new_k, mode=mode,
                          head_weight=self.head_weight, seed=seed, vb_seq_stride=self.lay.rows_per_seq,
                          stream=stream)

    def anchor(self, stream=None):
        self._on(stream)
        kka_pool_anchor(self.kp, self.seqs, self.window, self.anchors, head_weight=self.head_weight,
                        workspace=self.ws_anchor, stream=stream)

    def levels(self, n_pages: torch.Tensor, first_dirty_page: Optional[torch.Tensor] = None, stream=None):
        self._on(stream)
        kka_build_levels(self.lay, self.level, n_pages, first_dirty_page, stream=stream)

    def score(self, n_pages: torch.Tensor, anchors: Optional[torch.Tensor] = None, stream=None, lazy: bool = False):
        """Affinity + top-K; lazy=True scores only children of kept parents.
        With a stability window the single pass also advances every page's
        window word and stability score."""
        self._on(stream)
        stab = {}
        if getattr(self, "history", None) is not None and not lazy:
            stab = dict(history=self.history, stability_out=self.stability, window=self.stability_window,
                        theta=self.stability_theta)
        kka_score_topk(self.lay, self.level, n_pages, self.anchors if anchors is None else anchors,
                       k_page=self.sel["k_page"], k_grid=self.sel.get("k_grid", 0),
                       k_chunk=self.sel.get("k_chunk", 0), page_idx_out=self.page_idx,
                       page_score_out=self.page_score, n_selected_out=self.n_selected,
                       affinity_out=self.affinity, workspace=self.ws_score, stream=stream, lazy=lazy, **stab)

    def step(self, n_pages: torch.Tensor, stream=None):
        """Whole path over the batch: pool, anchor, levels, score + top-K."""
        self.pool(stream)
        self.anchor(stream)
        self.levels(n_pages, stream=stream)
        self.score(n_pages, stream=stream)

    def decode_step(self, blocks: torch.Tensor, n_pages: torch.Tensor, first_dirty_page: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None, lazy: bool = False):
        """One decode step once the new tokens are in the pool (section 5.2:
        the block vectors of the written blocks, then anchor -> levels ->
        affinity + top-K): re-pool `blocks` with the frozen weights, pool the
        anchor, rebuild the levels above each sequence's first dirty page
        (hierarchical layouts; all of them without first_dirty_page), then
        score and select, all on `stream`."""
        self.repool(blocks, workspace=workspace, stream=stream)
        self.anchor(stream)
        if self.lay.hierarchical:
            self.levels(n_pages, first_dirty_page, stream=stream)
        self.score(n_pages, stream=stream, lazy=lazy)

    # views of the level buffer
    def pages(self, s: int, n: int) -> torch.Tensor:
        return self.level[s, :n]

    def chunks(self, s: int, n_c: int) -> torch.Tensor:
        return self.level[s, self.lay.chunk_row0:self.lay.chunk_row0 + n_c]

    def grids(self, s: int, n_g: int) -> torch.Tensor:
        return self.level[s, self.lay.grid_row0:self.lay.grid_row0 + n_g]


__all__ = ["Selector", "WEIGHT_UNIFORM", "WEIGHT_VARIANCE", "WEIGHT_GIVEN"]
