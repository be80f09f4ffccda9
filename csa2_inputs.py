"""Seeded synthetic inputs for the CSA2 decode path.

This module is shared by the tests and the benchmark and feeds both the HIP
library and the CPU oracle.  It holds none of the method's arithmetic: it only
draws seeded random tensors (torch generators, on the CPU or on the GPU) with
the shapes and value distributions of the workloads, rounds them to the
storage dtype (bf16 by torch's own conversion) and lays them out.

Every tensor is addressed by (seed, tag[, chunk]) so that any part of a large
input can be drawn again on the same device without keeping it in memory.
"""
from __future__ import annotations

import math
import zlib

import numpy as np
import torch

ROW_CHUNK = 1 << 16          # rows per generator chunk for large row-major tensors


def _sub_seed(seed: int, tag: str, chunk: int = 0) -> int:
    return (int(seed) * 0x9E3779B1 + zlib.crc32(tag.encode()) * 0x85EBCA77 + int(chunk) * 0xC2B2AE3D) & (
        (1 << 63) - 1)


def _gen(device, seed, tag, chunk=0):
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, tag, chunk))
    return g


def normal(shape, seed, tag, device="cpu", dtype=torch.float32, outlier_p=0.0, outlier_mult=20.0):
    """N(0,1) draws; with outlier_p > 0 each element is independently scaled by
    outlier_mult with probability outlier_p.  Rounded to `dtype` at the end."""
    g = _gen(device, seed, tag)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if outlier_p > 0:
        m = torch.rand(shape, generator=g, device=device) < outlier_p
        x = torch.where(m, x * outlier_mult, x)
    return x.to(dtype)


def uniform(shape, seed, tag, device="cpu"):
    """U(0,1) float32 draws."""
    g = _gen(device, seed, tag)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def normal_rows(seed, tag, row0, nrows, ncols, device="cpu", dtype=torch.bfloat16,
                outlier_p=0.0, outlier_mult=20.0):
    """Rows [row0, row0+nrows) of a conceptually huge N(0,1) matrix with `ncols`
    columns.  Chunks of ROW_CHUNK rows have their own generator, so a row range
    can be drawn again without drawing the rest."""
    out = torch.empty((nrows, ncols), dtype=dtype, device=device)
    r = row0
    while r < row0 + nrows:
        c = r // ROW_CHUNK
        c0 = c * ROW_CHUNK
        c1 = min(c0 + ROW_CHUNK, row0 + nrows)
        g = _gen(device, seed, tag, c)
        blk = torch.randn((ROW_CHUNK, ncols), generator=g, device=device, dtype=torch.float32)
        if outlier_p > 0:
            m = torch.rand((ROW_CHUNK, ncols), generator=g, device=device) < outlier_p
            blk = torch.where(m, blk * outlier_mult, blk)
        out[r - row0:c1 - row0] = blk[r - c0:c1 - c0].to(dtype)
        r = c1
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def log_uniform_lengths(n, lo, hi, seed, tag="lengths"):
    """Sequence lengths floor(exp(U(ln lo, ln hi))), a mixed-length batch."""
    u = uniform((n,), seed, tag).double()
    v = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return [int(min(hi, max(lo, math.floor(x)))) for x in v.tolist()]


# ---------------------------------------------------------------------------
# Decode workloads (shapes and distributions of the CSA2 configurations).
# A workload is a plain dict; the tensors are drawn on demand.
# ---------------------------------------------------------------------------
def _decoder_layers():
    return ["full", "reuse", "reuse", "reuse"] + ["reindex", "reuse", "reuse", "reuse"] * 4


def workload(name: str, seed: int | None = None, length_div: int = 1) -> dict:
    """Named decode workload.  length_div > 1 shrinks every context length
    (for oracle-sized parity runs) and keeps everything else."""
    base = {"k": 512, "w": 128, "outlier_p": 0.0, "block": 8}
    if name == "c1":
        wl = dict(base, desc="single Full layer, batch 1, context 4096, 16 heads fp32 query, "
                             "indexer 4x64", lengths=[4096], h=16, q_dtype="f32", kv_dtype="f32",
                  h_i=4, d_i=64, layers=["full"], keep_blocks=0, append=True)
    elif name == "c2":
        wl = dict(base, desc="decoder group 1 (Full + 3 Reuse), batch 8, context 131072",
                  lengths=[131072] * 8, h=64, q_dtype="bf16", kv_dtype="bf16", h_i=64, d_i=128,
                  layers=["full", "reuse", "reuse", "reuse"], keep_blocks=0, append=True)
    elif name == "c3":
        wl = dict(base, desc="Reindex group at 1M context, batch 4: Full + pool (2048 blocks of 8), "
                             "then Reindex; 64 heads, FP4 512-ch KV, indexer 64x128, Top-512, SWA-128",
                  lengths=[1 << 20] * 4, h=64, q_dtype="bf16", kv_dtype="bf16", h_i=64, d_i=128,
                  layers=["full", "reindex"], keep_blocks=2048, append=True)
    elif name == "c4":
        # Encoder-side chunk at compression ratio 2: 1,048,576 tokens held as
        # 524,288 compressed entries (entry j covers tokens 2j, 2j + 1); 4096
        # causal queries at tokens t0 .. t0 + 4095, each seeing the entries j
        # with 2j + 1 <= t, and its own window of tokens t - 127 .. t (rows of
        # one window tensor shared by the chunk).  1 Full + 5 Reuse layers;
        # every tensor N(0,1) with 1% of the values scaled by 20.
        n_ent, n_chunk = 1 << 19, 4096
        t0 = (1 << 20) - n_chunk
        wl = dict(base, desc="encoder-side chunk at compression ratio 2: 524288 FP4 entries of a 1M-token "
                             "context, 4096 causal queries, Full + 5 Reuse",
                  lengths=[n_ent], h=64, q_dtype="bf16", kv_dtype="bf16", h_i=64, d_i=128,
                  layers=["full"] + ["reuse"] * 5, keep_blocks=0, append=False, outlier_p=0.01,
                  q_seq=[0] * n_chunk, q_nvis=[(t + 1) // 2 for t in range(t0, t0 + n_chunk)],
                  swa_shared=True, chunk=True)
    elif name == "c5":
        s = 0xC5A20005 if seed is None else seed
        wl = dict(base, desc="20-layer decoder schedule, 64 sequences, lengths log-uniform in "
                             "[4096, 1048576]", lengths=log_uniform_lengths(64, 4096, 1 << 20, s),
                  h=64, q_dtype="bf16", kv_dtype="bf16", h_i=64, d_i=128, layers=_decoder_layers(),
                  keep_blocks=2048, append=True)
    else:
        raise ValueError(f"unknown workload {name}")
    wl["name"] = name
    wl["seed"] = (0xC5A20000 + int(name[1:])) if seed is None else seed
    if length_div > 1:
        if "q_seq" in wl:
            raise ValueError("length_div applies to decode workloads only")
        wl["lengths"] = [max(1, L // length_div) for L in wl["lengths"]]
        wl["name"] = f"{name}/{length_div}"
    # decode workloads: one query per sequence, seeing the whole sequence
    wl.setdefault("q_seq", list(range(len(wl["lengths"]))))
    wl.setdefault("q_nvis", list(wl["lengths"]))
    wl.setdefault("swa_shared", False)
    wl["n_q"] = len(wl["q_seq"])
    wl["rows"] = int(sum(wl["lengths"]))
    wl["seq_base"] = [0] + [int(v) for v in np.cumsum(wl["lengths"])[:-1]]
    return wl


def _tdtype(s):
    return torch.float32 if s == "f32" else torch.bfloat16


def kv_rows(wl, row0, nrows, device="cpu"):
    """Raw (unquantised) main-KV rows [row0, row0+nrows) of the whole batch."""
    return normal_rows(wl["seed"], "main-kv", row0, nrows, 512, device=device, dtype=_tdtype(wl["kv_dtype"]),
                       outlier_p=wl["outlier_p"])


def index_keys(wl, device="cpu", row0=0, nrows=None):
    nrows = wl["rows"] - row0 if nrows is None else nrows
    return normal_rows(wl["seed"], "index-k", row0, nrows, wl["d_i"], device=device, dtype=torch.bfloat16,
                       outlier_p=wl["outlier_p"])


def seq_tensors(wl, device="cpu"):
    return dict(seq_base=torch.tensor(wl["seq_base"], dtype=torch.int64, device=device),
                q_seq=torch.tensor(wl["q_seq"], dtype=torch.int32, device=device),
                q_nvis=torch.tensor(wl["q_nvis"], dtype=torch.int32, device=device))


def layer_tensors(wl, layer, device="cpu"):
    """Layer `layer`'s own main query, window rows and (Full/Reindex) indexer query."""
    n_q, h, W = wl["n_q"], wl["h"], wl["w"]
    s, tag = wl["seed"], f"layer{layer}"
    if wl["swa_shared"]:
        # consecutive queries of one chunk: query i's window is rows i .. i + W - 1
        swa = normal((n_q + W - 1, 512), s, tag + "-swa", device=device, dtype=torch.bfloat16,
                     outlier_p=wl["outlier_p"])
        row0 = torch.arange(n_q, dtype=torch.int64, device=device)
        wlen = torch.full((n_q,), W, dtype=torch.int32, device=device)
    else:
        swa = normal((n_q * W, 512), s, tag + "-swa", device=device, dtype=torch.bfloat16,
                     outlier_p=wl["outlier_p"])
        row0 = torch.arange(n_q, dtype=torch.int64, device=device) * W
        wlen = torch.tensor([min(W, L) for L in wl["lengths"]], dtype=torch.int32, device=device)
    d = dict(mode=wl["layers"][layer],
             q=normal((n_q, h, 512), s, tag + "-q", device=device, dtype=_tdtype(wl["q_dtype"]),
                      outlier_p=wl["outlier_p"]),
             swa=swa, swa_row0=row0, swa_len=wlen)
    if wl.get("append", True) and not wl["swa_shared"]:
        # the decode step's new window row of every sequence (its newest
        # position L - 1), written into its 128-row ring at row (L - 1) mod W
        d["swa_new"] = normal((n_q, 512), s, tag + "-swa-new", device=device, dtype=torch.bfloat16,
                              outlier_p=wl["outlier_p"])
        d["swa_dst"] = torch.tensor([i * W + (L - 1) % W for i, L in enumerate(wl["lengths"])],
                                    dtype=torch.int64, device=device)
    if d["mode"] in ("full", "reindex"):
        d["iq"] = normal((n_q, wl["h_i"], wl["d_i"]), s, tag + "-iq", device=device, dtype=torch.bfloat16,
                         outlier_p=wl["outlier_p"])
        d["w"] = uniform((n_q, wl["h_i"]), s, tag + "-w", device=device)
    return d


def append_rows(wl, device="cpu"):
    """The new token of every sequence (its last position): raw row and cache
    row; (None, None) for a workload without appends."""
    if not wl.get("append", True):
        return None, None
    rows = [wl["seq_base"][i] + wl["lengths"][i] - 1 for i in range(wl["n_q"])]
    x = torch.cat([kv_rows(wl, r, 1, device) for r in rows])
    return x, torch.tensor(rows, dtype=torch.int64, device=device)


def kv_rows_at(wl, rows, device="cpu"):
    """Raw main-KV rows at arbitrary global row indices (sorted or not),
    drawing each generator chunk once."""
    rows = np.asarray(rows, dtype=np.int64)
    out = torch.empty((len(rows), 512), dtype=_tdtype(wl["kv_dtype"]), device=device)
    if len(rows) == 0:
        return out
    chunks = rows // ROW_CHUNK
    for c in np.unique(chunks):
        sel = np.nonzero(chunks == c)[0]
        c0 = int(c) * ROW_CHUNK
        n = min(ROW_CHUNK, wl["rows"] - c0)
        blk = kv_rows(wl, c0, n, device)
        out[torch.from_numpy(sel).to(device)] = blk[torch.from_numpy(rows[sel] - c0).to(device)]
    return out
