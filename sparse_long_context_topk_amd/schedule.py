"""Static per-layer CSA2 schedules and a decode-step driver.

Every CSA2 layer has a fixed mode: Full (own main KV, fresh Top-512),
Reindex (re-scores the last Full layer's keys with its own indexer query) or
Reuse (takes the group head's Top-K list, no indexer).  The decoder's 20
layers form 5 groups of 4: Full + 3 Reuse, then 4 x (Reindex + 3 Reuse); the
encoder's CSA2 layers form groups of 1 Full + 5 Reuse.  Source: "DeepSeek AI
выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4 ..."
(wire.sakhanda.co), section "Сжатое разреженное внимание 2 (CSA2)".

The driver only sequences the C-ABI calls of one decode step; all arithmetic
runs in libcsa2.so.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (block_keys, index_topk, index_topk_chunk, index_topk_fp8, quant_append, reindex_topk,
               reindex_topk_fp8, sparse_attn, Workspace)

FULL, REINDEX, REUSE = "full", "reindex", "reuse"


def decoder_schedule() -> list[str]:
    """The 20 decoder layers: [Full, Reuse x3] + 4 x [Reindex, Reuse x3]."""
    return [FULL, REUSE, REUSE, REUSE] + [REINDEX, REUSE, REUSE, REUSE] * 4


def encoder_group() -> list[str]:
    """One encoder group: 1 Full + 5 Reuse."""
    return [FULL] + [REUSE] * 5


@dataclass
class LayerInputs:
    """Per-layer tensors: each layer owns its main query and its window rows;
    Full/Reindex layers also own an indexer query and head weights."""
    mode: str
    q: torch.Tensor                       # [n_q, h, 512] fp32 | bf16
    swa: torch.Tensor                     # [rows, 512] bf16
    swa_row0: torch.Tensor                # [n_q] int64
    swa_len: torch.Tensor                 # [n_q] int32
    iq: torch.Tensor | None = None        # [n_q, h_i, d_i] bf16
    w: torch.Tensor | None = None         # [n_q, h_i] f32
    swa_new: torch.Tensor | None = None   # [n_q, 512] this step's window row of each query's sequence
    swa_dst: torch.Tensor | None = None   # [n_q] int64 its row in swa (ring row: newest position mod 128)


@dataclass
class DecodeState:
    """Shared tensors of one decode batch: the FP4 main KV and the indexer keys
    written by the Full layer, and the per-query sequence bookkeeping."""
    cache: torch.Tensor                   # [rows, 288] uint8
    ik: torch.Tensor                      # [rows, d_i] bf16
    seq_base: torch.Tensor                # [n_seq] int64
    q_seq: torch.Tensor                   # [n_q] int32
    q_nvis: torch.Tensor                  # [n_q] int32
    max_nvis: int
    k: int = 512
    keep_blocks: int = 2048               # pool size built by the Full layer (0: none)
    w_max: int = 128
    softmax_scale: float = 512 ** -0.5
    chunk_base: int | None = None         # all queries in one sequence whose keys start at this row (no pool)
    # pool-based Full variant: the Full layer picks its Top-K inside its own pool,
    # scanning stored block keys (kbar) instead of every token key
    pool_full: bool = False
    kbar: torch.Tensor | None = None      # [block rows, d_i] bf16, block b of sequence s at kbar_base[s] + b
    kbar_base: torch.Tensor | None = None # [n_seq] int64
    q_nblk: torch.Tensor | None = None    # [n_q] int32: ceil(q_nvis / 8), the blocks each query sees
    max_nblk: int = 0
    seq_len: torch.Tensor | None = None   # [n_seq] int32 positions per sequence
    blk_last: torch.Tensor | None = None  # [n_seq] int32: block of each sequence's newest position
    # FP8 indexer keys (the low-precision indexer-key variant): the Full and
    # Reindex layers read ik8/ik8_exp (csa2_index_keys_fp8 of ik) instead of ik
    fp8_keys: bool = False
    ik8: torch.Tensor | None = None       # [rows, d_i] uint8 E4M3 codes
    ik8_exp: torch.Tensor | None = None   # [rows] uint8 exponent bytes
    ws_index: Workspace = field(default_factory=Workspace)
    ws_attn: Workspace = field(default_factory=Workspace)


def decode_step(st: DecodeState, layers: list[LayerInputs], append_x=None, append_rows=None,
                scan_events=None, keep_outputs=True):
    """Run one decode step over `layers`.  append_x/append_rows: new main-KV
    rows quantised into the cache before the Full layer indexes; each layer's
    new window rows (swa_new) go into its ring before its attention.  Returns a
    list of (idx, out, lse) per layer (idx shared by a group's Reuse layers)."""
    from . import record_scan_events
    if append_x is not None:
        quant_append(append_x, append_rows, st.cache)
    results = []
    idx = pool = None
    for lay in layers:
        if lay.mode == FULL:
            if scan_events is not None:
                record_scan_events(*scan_events)
            if st.fp8_keys and (st.chunk_base is not None or st.pool_full):
                raise ValueError("FP8 indexer keys serve the decode Full and Reindex calls only")
            if st.chunk_base is not None:
                if st.keep_blocks:
                    raise ValueError("a chunk of one sequence's queries builds no pool")
                idx, pool = index_topk_chunk(lay.iq, lay.w, st.q_nvis, st.max_nvis, st.ik, st.chunk_base, k=st.k,
                                             ws=st.ws_index), None
            elif st.pool_full:
                if not st.keep_blocks:
                    raise ValueError("the pool-based Full variant needs keep_blocks > 0")
                if append_x is not None:
                    # the appended position's block key changes with it
                    block_keys(st.ik, st.seq_base, st.seq_len, st.kbar, st.kbar_base, 1, blk_from=st.blk_last)
                pool = index_topk(lay.iq, lay.w, st.q_seq, st.q_nblk, st.max_nblk, st.kbar, st.kbar_base,
                                  k=st.keep_blocks, ws=st.ws_index)
                idx = reindex_topk(lay.iq, lay.w, st.q_seq, st.q_nvis, st.ik, st.seq_base, pool, k=st.k,
                                   ws=st.ws_index)
            elif st.fp8_keys:
                r = index_topk_fp8(lay.iq, lay.w, st.q_seq, st.q_nvis, st.max_nvis, st.ik8, st.ik8_exp, st.seq_base,
                                   k=st.k, keep_blocks=st.keep_blocks, ws=st.ws_index)
                idx, pool = (r if st.keep_blocks else (r, None))
            else:
                r = index_topk(lay.iq, lay.w, st.q_seq, st.q_nvis, st.max_nvis, st.ik, st.seq_base, k=st.k,
                               keep_blocks=st.keep_blocks, ws=st.ws_index)
                idx, pool = (r if st.keep_blocks else (r, None))
        elif lay.mode == REINDEX:
            if pool is None:
                raise ValueError("a Reindex layer needs a preceding Full layer that built a pool")
            if st.fp8_keys:
                idx = reindex_topk_fp8(lay.iq, lay.w, st.q_seq, st.q_nvis, st.ik8, st.ik8_exp, st.seq_base, pool,
                                       k=st.k, ws=st.ws_index)
            else:
                idx = reindex_topk(lay.iq, lay.w, st.q_seq, st.q_nvis, st.ik, st.seq_base, pool, k=st.k,
                                   ws=st.ws_index)
        elif lay.mode != REUSE:
            raise ValueError(f"unknown layer mode {lay.mode}")
        if idx is None:
            raise ValueError("a Reuse layer needs a preceding Full or Reindex layer")
        # the layer's new window row enters its ring in the attention call itself
        out, lse = sparse_attn(lay.q, st.q_seq, st.cache, st.seq_base, idx, lay.swa, lay.swa_row0,
                               lay.swa_len, st.w_max, st.softmax_scale, ws=st.ws_attn, swa_new=lay.swa_new,
                               swa_dst=lay.swa_dst)
        if keep_outputs:
            results.append((idx, out, lse))
    return results, pool


class StepGraph:
    """One decode step captured as a HIP graph and replayed.

    Every kernel launch of the step becomes a node of one graph, so a replay
    costs the host a single launch and the GPU runs the nodes back to back.
    The graph reads the tensors it was captured with (the state, the layers'
    queries and window rows, the appended rows): update them in place between
    replays.  Its outputs (per layer idx, out, lse, and the pool) live in the
    graph's own memory and each replay overwrites them.  The library itself
    allocates nothing and issues no memset, so the captured launches are the
    eager ones."""

    def __init__(self, st: DecodeState, layers: list[LayerInputs], append_x=None, append_rows=None):
        # an eager step first, so every workspace has its final size before capture
        decode_step(st, layers, append_x=append_x, append_rows=append_rows, keep_outputs=False)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.results, self.pool = decode_step(st, layers, append_x=append_x, append_rows=append_rows,
                                                  keep_outputs=True)

    def replay(self):
        """Enqueue one step on the current stream; returns the (overwritten) outputs."""
        self.graph.replay()
        return self.results, self.pool
