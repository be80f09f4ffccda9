"""One CSA2 decode step run by the oracle, layer by layer, on host arrays.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the bench).
It sequences the oracle calls in schedule order -- Full: index (+pool),
Reindex: re-score the pool, Reuse: the group head's list -- and attends each
layer with its own query and window rows, as CSA2 prescribes ("DeepSeek AI
выпустила DeepSeek-V4.1-Flash ..." (wire.sakhanda.co), section "Сжатое
разреженное внимание 2 (CSA2)").

The FP4 records the attention reads are quantised here by the oracle from the
raw rows (callers pass a function that draws raw rows from the seeded input
generator), so no oracle input comes from the GPU path.
"""
from __future__ import annotations

import time

import numpy as np

from . import block_keys, index_topk, pool_full_topk, quantize_rows, reindex_topk, sparse_attn


def decode_step(layers, ik, seq_base, q_seq, q_nvis, k, keep_blocks, block, raw_rows_fn, append_x,
                scale, n_threads=0, pool_full=False):
    """layers: list of dicts of host arrays: mode, q (float32 or uint16 bf16 bits),
    swa (uint16), swa_row0, swa_len, optionally swa_new (uint16 [n_q, 512]) and
    swa_dst (the step's new window rows and their rows in swa) and, for
    full/reindex, iq (uint16) and w.
    raw_rows_fn(rows) -> raw main-KV rows (float32 or uint16) of global cache rows.
    Returns (results, pool, seconds): results = [(idx, out, lse)] per layer and
    the time spent inside the oracle's decode-step calls (input plumbing excluded).
    pool_full: the Full layer picks its Top-K inside its own pool, built from
    stored block keys (computed here for every query's visible prefix, outside
    the timed calls, as they are resident before a decode step)."""
    secs = 0.0
    if pool_full:
        qbase = np.asarray(seq_base, np.int64)[np.asarray(q_seq)]
        nblk = (np.asarray(q_nvis, np.int64) + block - 1) // block
        kb_base = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
        kbar = np.zeros((max(int(nblk.sum()), 1), ik.shape[1]), np.uint16)
        block_keys(ik, qbase, q_nvis, kbar, kb_base, block=block)
    t0 = time.perf_counter()
    if append_x is not None:
        quantize_rows(append_x)            # a1: the new token of every sequence
    secs += time.perf_counter() - t0
    idx = pool = None
    results = []
    for lay in layers:
        mode = lay["mode"]
        t0 = time.perf_counter()
        if mode == "full" and pool_full:
            idx, pool = pool_full_topk(lay["iq"], lay["w"], np.arange(len(q_seq), dtype=np.int32), q_nvis, ik,
                                       qbase, kbar, kb_base, k, keep_blocks, block=block, n_threads=n_threads)
        elif mode == "full":
            r = index_topk(lay["iq"], lay["w"], q_seq, q_nvis, ik, seq_base, k, block=block,
                           keep_blocks=keep_blocks, n_threads=n_threads)
            idx, pool = r if keep_blocks else (r, None)
        elif mode == "reindex":
            idx = reindex_topk(lay["iq"], lay["w"], q_seq, q_nvis, ik, seq_base, pool, k, block=block,
                               n_threads=n_threads)
        secs += time.perf_counter() - t0
        # records of the selected entries, quantised by the oracle
        rows = np.where(idx >= 0, seq_base[q_seq][:, None] + idx, -1)
        uniq = np.unique(rows[rows >= 0])
        recs = quantize_rows(raw_rows_fn(uniq)) if len(uniq) else np.zeros((1, 288), np.uint8)
        cidx = np.where(rows >= 0, np.searchsorted(uniq, rows), -1).astype(np.int32)
        zq = np.zeros(len(q_seq), np.int32)
        swa = lay["swa"]
        if lay.get("swa_new") is not None:
            # this step's window rows enter the layer's ring (bf16 rows: a copy)
            swa = np.array(swa, copy=True)
            swa[np.asarray(lay["swa_dst"], np.int64)] = lay["swa_new"]
        t0 = time.perf_counter()
        out, lse = sparse_attn(lay["q"], zq, recs, np.zeros(1, np.int64), cidx, swa, lay["swa_row0"],
                               lay["swa_len"], scale, n_threads=n_threads)
        secs += time.perf_counter() - t0
        results.append((idx, out, lse))
    return results, pool, secs
