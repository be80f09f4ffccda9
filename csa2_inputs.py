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
    return (int(seed) * 0x9E3779B1 + zlib.crc32(tag.encode()) * 0x85EBCA77 + chunk * 0xC2B2AE3D) & (
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
