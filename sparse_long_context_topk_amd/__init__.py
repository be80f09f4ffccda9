"""CSA2 decode hot path for AMD MI355X (gfx950): Python binding of libcsa2.so.

The calls below are the C-ABI entry points of ``include/csa2.h`` with the
same names; this module only marshals torch tensors (device memory) and the
current HIP stream into them and turns a non-OK status into an exception.
Every step runs in the library's HIP kernels.  There is no fallback: if the
library is missing or cannot be loaded, every call raises.

The method (CSA2 as described on the page "DeepSeek AI выпустила
DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4 ..."
(wire.sakhanda.co), section "Сжатое разреженное внимание 2 (CSA2)"):
  Full layer:    quant_append (new rows) -> index_topk -> sparse_attn
  Reindex layer: reindex_topk -> sparse_attn
  Reuse layer:   sparse_attn with the group head's idx
  pool-based Full variant: block_keys (appended block) -> index_topk over the
                 block keys (the pool) -> reindex_topk with the Full query
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

KV_CH = 512
KV_RECORD_BYTES = 288
F32, BF16 = 0, 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace too small",
           4: "HIP launch failed"}

_lib = None


class Csa2Error(RuntimeError):
    pass


def lib():
    """Load libcsa2.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Csa2Error(f"{LIB_PATH} is missing: build the HIP library first "
                            "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.csa2_quant_append.restype = i32
        L.csa2_quant_append.argtypes = [vp, i32, i64, vp, vp, i64, vp]
        L.csa2_index_topk.restype = i32
        L.csa2_index_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, ctypes.c_int32, vp, vp, i32, vp,
                                      i32, i32, vp, vp, sz, vp]
        L.csa2_index_topk_ws_bytes.restype = sz
        L.csa2_index_topk_ws_bytes.argtypes = [i32, ctypes.c_int32, i32, i32, i32, i32, i32]
        L.csa2_index_keys_fp8.restype = i32
        L.csa2_index_keys_fp8.argtypes = [vp, i32, i64, vp, vp, vp]
        L.csa2_index_topk_fp8.restype = i32
        L.csa2_index_topk_fp8.argtypes = [vp, vp, i32, i32, i32, vp, vp, ctypes.c_int32, vp, vp, vp, i32, vp,
                                          i32, i32, vp, vp, sz, vp]
        L.csa2_reindex_topk_fp8.restype = i32
        L.csa2_reindex_topk_fp8.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp,
                                            vp, sz, vp]
        L.csa2_index_topk_chunk.restype = i32
        L.csa2_index_topk_chunk.argtypes = [vp, vp, i32, i32, i32, vp, ctypes.c_int32, vp, i64, i32, vp, vp,
                                            ctypes.c_size_t, vp]
        L.csa2_reindex_topk.restype = i32
        L.csa2_reindex_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp,
                                        vp, sz, vp]
        L.csa2_reindex_topk_ws_bytes.restype = sz
        L.csa2_reindex_topk_ws_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.csa2_reindex_topk_noalloc.restype = i32
        L.csa2_reindex_topk_noalloc.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
        L.csa2_sparse_attn.restype = i32
        L.csa2_sparse_attn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, i32,
                                       f32, vp, vp, vp, sz, vp]
        L.csa2_sparse_attn_append.restype = i32
        L.csa2_sparse_attn_append.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, i64, vp, vp, i32,
                                              vp, vp, f32, vp, vp, vp, sz, vp]
        L.csa2_sparse_attn_ws_bytes.restype = sz
        L.csa2_sparse_attn_ws_bytes.argtypes = [i32, i32, i32, i32]
        L.csa2_topk_merge.restype = i32
        L.csa2_topk_merge.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
        L.csa2_topk_merge_ws_bytes.restype = sz
        L.csa2_topk_merge_ws_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.csa2_window_append.restype = i32
        L.csa2_window_append.argtypes = [vp, i32, i64, vp, vp, i64, vp]
        L.csa2_block_keys.restype = i32
        L.csa2_block_keys.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, vp, vp]
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_status_string.argtypes = [i32]
        L.csa2_last_hip_error.restype = i32
        L.csa2_last_hip_error.argtypes = []
        L.csa2_record_scan_events.restype = None
        L.csa2_record_scan_events.argtypes = [vp, vp]
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        extra = ""
        if status == 4:
            extra = f" (hipError {lib().csa2_last_hip_error()})"
        raise Csa2Error(f"{what}: {_STATUS.get(status, status)}{extra}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Workspace:
    """Caller-owned scratch buffer for the index/attention calls, grown on demand."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _ws(device, nbytes, ws):
    if ws is None:
        key = torch.device(device)
        ws = _default_ws.setdefault(key, Workspace())
    return ws.get(nbytes, device)


def record_scan_events(start, stop) -> None:
    """Have the next index/reindex call record these torch.cuda.Event objects
    around its scan kernel (each event must have been recorded once already so
    that its HIP handle exists)."""
    lib().csa2_record_scan_events(ctypes.c_void_p(start.cuda_event) if start is not None else None,
                                  ctypes.c_void_p(stop.cuda_event) if stop is not None else None)


# ------------------------------------------------------------------ calls
def quant_append(x: torch.Tensor, dst_row: torch.Tensor, cache: torch.Tensor) -> None:
    """Quantise rows x[n,512] (fp32 or bf16) into cache[rows,288] (uint8) at dst_row[n] (int64)."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, x.dtype, "x")
    _need(dst_row, torch.int64, "dst_row")
    _need(cache, torch.uint8, "cache")
    if x.dim() != 2 or x.shape[1] != KV_CH or cache.dim() != 2 or cache.shape[1] != KV_RECORD_BYTES:
        raise ValueError("x must be [n,512] and cache [rows,288]")
    if dst_row.numel() != x.shape[0]:
        raise ValueError("dst_row must have one entry per row of x")
    st = lib().csa2_quant_append(_ptr(x), F32 if x.dtype == torch.float32 else BF16, x.shape[0],
                                 _ptr(dst_row), _ptr(cache), cache.shape[0], _stream(x.device))
    _check(st, "csa2_quant_append")


def window_append(x: torch.Tensor, dst_row: torch.Tensor, swa: torch.Tensor) -> None:
    """Write rows x[n,512] (fp32, rounded to bf16, or bf16) into a layer's window
    rows swa[rows,512] (bf16) at dst_row[n] (int64); a ring of 128 rows per
    sequence takes position p at ring row p mod 128."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, x.dtype, "x")
    _need(dst_row, torch.int64, "dst_row")
    _need(swa, torch.bfloat16, "swa")
    if x.dim() != 2 or x.shape[1] != KV_CH or swa.dim() != 2 or swa.shape[1] != KV_CH:
        raise ValueError("x must be [n,512] and swa [rows,512]")
    if dst_row.numel() != x.shape[0]:
        raise ValueError("dst_row must have one entry per row of x")
    st = lib().csa2_window_append(_ptr(x), F32 if x.dtype == torch.float32 else BF16, x.shape[0], _ptr(dst_row),
                                  _ptr(swa), swa.shape[0], _stream(x.device))
    _check(st, "csa2_window_append")


def index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block=8, keep_blocks=0) -> int:
    return lib().csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks)


def index_topk(iq, w, q_seq, q_nvis, max_nvis, ik, seq_base, k=512, block=8, keep_blocks=0,
               idx_out=None, pool_out=None, ws=None):
    """Full layer.  iq [n_q,h_i,d_i] bf16, w [n_q,h_i] f32, q_seq/q_nvis [n_q] int32,
    ik [rows,d_i] bf16, seq_base [n_seq] int64.  Returns idx [n_q,k] int32 (and the
    pool [n_q,keep_blocks] int32 when keep_blocks > 0)."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik, torch.bfloat16, "ik")
    _need(seq_base, torch.int64, "seq_base")
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    if keep_blocks and pool_out is None:
        pool_out = torch.empty((n_q, keep_blocks), dtype=torch.int32, device=dev)
    nbytes = index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks)
    buf = _ws(dev, nbytes, ws)
    st = lib().csa2_index_topk(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(q_nvis), int(max_nvis),
                               _ptr(ik), _ptr(seq_base), k, _ptr(idx_out), block, keep_blocks,
                               _ptr(pool_out) if keep_blocks else None, _ptr(buf), buf.numel(),
                               _stream(dev))
    _check(st, "csa2_index_topk")
    return (idx_out, pool_out) if keep_blocks else idx_out


def index_keys_fp8(ik, codes=None, exps=None):
    """Quantise bf16 key rows ik [rows, d_i] to FP8 (E4M3FN codes uint8 [rows, d_i]
    and one exponent byte per row, uint8 [rows]; the stored key is
    code * 2^(exp - 127)).  Returns (codes, exps)."""
    _need(ik, torch.bfloat16, "ik")
    rows, d_i = ik.shape
    dev = ik.device
    if codes is None:
        codes = torch.empty((rows, d_i), dtype=torch.uint8, device=dev)
    if exps is None:
        exps = torch.empty((rows,), dtype=torch.uint8, device=dev)
    _need(codes, torch.uint8, "codes")
    _need(exps, torch.uint8, "exps")
    st = lib().csa2_index_keys_fp8(_ptr(ik), d_i, rows, _ptr(codes), _ptr(exps), _stream(dev))
    _check(st, "csa2_index_keys_fp8")
    return codes, exps


def index_topk_fp8(iq, w, q_seq, q_nvis, max_nvis, ik8, ik8_exp, seq_base, k=512, block=8, keep_blocks=0,
                   idx_out=None, pool_out=None, ws=None):
    """index_topk over FP8 keys (ik8 [rows, 128] uint8 codes, ik8_exp [rows] uint8)."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik8, torch.uint8, "ik8")
    _need(ik8_exp, torch.uint8, "ik8_exp")
    _need(seq_base, torch.int64, "seq_base")
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    if keep_blocks and pool_out is None:
        pool_out = torch.empty((n_q, keep_blocks), dtype=torch.int32, device=dev)
    buf = _ws(dev, index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks), ws)
    st = lib().csa2_index_topk_fp8(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(q_nvis), int(max_nvis),
                                   _ptr(ik8), _ptr(ik8_exp), _ptr(seq_base), k, _ptr(idx_out), block, keep_blocks,
                                   _ptr(pool_out) if keep_blocks else None, _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "csa2_index_topk_fp8")
    return (idx_out, pool_out) if keep_blocks else idx_out


def reindex_topk_fp8(iq, w, q_seq, q_nvis, ik8, ik8_exp, seq_base, pool_blocks, k=512, block=8, idx_out=None,
                     ws=None):
    """reindex_topk over FP8 keys."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik8, torch.uint8, "ik8")
    _need(ik8_exp, torch.uint8, "ik8_exp")
    _need(seq_base, torch.int64, "seq_base")
    _need(pool_blocks, torch.int32, "pool_blocks")
    keep_blocks = pool_blocks.shape[1]
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    buf = _ws(dev, reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks), ws)
    st = lib().csa2_reindex_topk_fp8(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(q_nvis), _ptr(ik8),
                                     _ptr(ik8_exp), _ptr(seq_base), _ptr(pool_blocks), block, keep_blocks, k,
                                     _ptr(idx_out), _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "csa2_reindex_topk_fp8")
    return idx_out


def index_topk_chunk(iq, w, q_nvis, max_nvis, ik, ik_base=0, k=512, idx_out=None, ws=None):
    """Full layer for a chunk of queries of one sequence (encoder side): query
    i sees key rows ik_base .. ik_base + q_nvis[i] - 1.  iq [n_q,h_i,d_i] bf16,
    w [n_q,h_i] f32, q_nvis [n_q] int32, ik [rows,d_i] bf16.  Returns idx
    [n_q,k] int32 (same result as index_topk with one shared sequence)."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik, torch.bfloat16, "ik")
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    nbytes = index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, 8, 0)
    buf = _ws(dev, nbytes, ws)
    st = lib().csa2_index_topk_chunk(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_nvis), int(max_nvis), _ptr(ik),
                                     int(ik_base), k, _ptr(idx_out), _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "csa2_index_topk_chunk")
    return idx_out


def topk_merge(iq, w, q_seq, ik, seq_base, cand, k=512, idx_out=None, ws=None):
    """Exact Top-K of each query among candidate positions cand [n_q,n_cand] int32
    (ascending, distinct, -1 padded at the end), e.g. the concatenated local Top-K
    lists of a context's shards.  Returns idx [n_q,k] int32."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(ik, torch.bfloat16, "ik")
    _need(seq_base, torch.int64, "seq_base")
    _need(cand, torch.int32, "cand")
    n_cand = cand.shape[1] if cand.dim() == 2 else 0
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    buf = _ws(dev, lib().csa2_topk_merge_ws_bytes(n_q, max(n_cand, 1), h_i, d_i, k), ws)
    st = lib().csa2_topk_merge(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(ik), _ptr(seq_base), _ptr(cand),
                               n_cand, k, _ptr(idx_out), _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "csa2_topk_merge")
    return idx_out


def reindex_topk_ws_bytes(n_q, h_i, d_i, k, block=8, keep_blocks=2048) -> int:
    return lib().csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks)


def reindex_topk(iq, w, q_seq, q_nvis, ik, seq_base, pool_blocks, k=512, block=8, idx_out=None, ws=None):
    """Reindex layer: re-score the positions of pool_blocks [n_q,keep_blocks] int32."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik, torch.bfloat16, "ik")
    _need(seq_base, torch.int64, "seq_base")
    _need(pool_blocks, torch.int32, "pool_blocks")
    keep_blocks = pool_blocks.shape[1]
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    nbytes = reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks)
    buf = _ws(dev, nbytes, ws)
    st = lib().csa2_reindex_topk(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(q_nvis), _ptr(ik),
                                 _ptr(seq_base), _ptr(pool_blocks), block, keep_blocks, k, _ptr(idx_out),
                                 _ptr(buf), buf.numel(), _stream(dev))
    _check(st, "csa2_reindex_topk")
    return idx_out


NOALLOC_SCRATCH_BYTES = 32 << 20


def reindex_topk_noalloc(iq, w, q_seq, q_nvis, ik, seq_base, pool_blocks, k=512, block=8, idx_out=None):
    """reindex_topk without a caller workspace (csa2_reindex_topk_noalloc): the
    library's fixed per-GPU scratch array serves as the workspace, so the call
    allocates nothing when idx_out is given.  Calls overlapping on one GPU race."""
    _need(iq, torch.bfloat16, "iq")
    n_q, h_i, d_i = iq.shape
    _need(w, torch.float32, "w")
    _need(q_seq, torch.int32, "q_seq")
    _need(q_nvis, torch.int32, "q_nvis")
    _need(ik, torch.bfloat16, "ik")
    _need(seq_base, torch.int64, "seq_base")
    _need(pool_blocks, torch.int32, "pool_blocks")
    keep_blocks = pool_blocks.shape[1]
    dev = iq.device
    if idx_out is None:
        idx_out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    st = lib().csa2_reindex_topk_noalloc(_ptr(iq), _ptr(w), n_q, h_i, d_i, _ptr(q_seq), _ptr(q_nvis), _ptr(ik),
                                         _ptr(seq_base), _ptr(pool_blocks), block, keep_blocks, k, _ptr(idx_out),
                                         _stream(dev))
    _check(st, "csa2_reindex_topk_noalloc")
    return idx_out


def block_keys(ik, seq_base, seq_len, kbar, kbar_base, max_blocks, blk_from=None) -> None:
    """Pool-based Full variant: write the bf16 mean keys of blocks of 8 positions
    into kbar [rows,d_i] bf16 at kbar_base[s] + b, for blocks blk_from[s] (0 if
    None) .. +max_blocks-1 that lie inside seq_len[s].  ik [rows,d_i] bf16,
    seq_base/kbar_base [n_seq] int64, seq_len/blk_from [n_seq] int32."""
    _need(ik, torch.bfloat16, "ik")
    _need(seq_base, torch.int64, "seq_base")
    _need(seq_len, torch.int32, "seq_len")
    _need(kbar, torch.bfloat16, "kbar")
    _need(kbar_base, torch.int64, "kbar_base")
    if blk_from is not None:
        _need(blk_from, torch.int32, "blk_from")
    if ik.dim() != 2 or kbar.dim() != 2 or kbar.shape[1] != ik.shape[1]:
        raise ValueError("ik and kbar must be [rows, d_i] with the same d_i")
    st = lib().csa2_block_keys(_ptr(ik), ik.shape[1], _ptr(seq_base), _ptr(seq_len), _ptr(blk_from),
                               seq_len.numel(), int(max_blocks), _ptr(kbar), _ptr(kbar_base), _stream(ik.device))
    _check(st, "csa2_block_keys")


def sparse_attn_ws_bytes(n_q, h, k, w_max) -> int:
    return lib().csa2_sparse_attn_ws_bytes(n_q, h, k, w_max)


def sparse_attn(q, q_seq, cache, seq_base, idx, swa, swa_row0, swa_len, w_max, softmax_scale,
                out=None, lse=None, want_lse=True, ws=None, swa_new=None, swa_dst=None):
    """q [n_q,h,512] fp32|bf16; idx [n_q,k] int32 (-1 skipped); swa [rows,512] bf16 with
    per-query rows swa_row0[i] .. + swa_len[i]-1.  Returns (out [n_q,h,512] f32, lse [n_q,h] f32).
    swa_new [n_q,512] bf16 / swa_dst [n_q] int64: this step's window rows, written into swa at
    swa_dst in the same call (csa2_sparse_attn_append)."""
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, q.dtype, "q")
    n_q, h, d = q.shape
    _need(q_seq, torch.int32, "q_seq")
    _need(cache, torch.uint8, "cache")
    _need(seq_base, torch.int64, "seq_base")
    _need(idx, torch.int32, "idx")
    k = idx.shape[1]
    if w_max > 0:
        _need(swa, torch.bfloat16, "swa")
        _need(swa_row0, torch.int64, "swa_row0")
        _need(swa_len, torch.int32, "swa_len")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, h, d), dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((n_q, h), dtype=torch.float32, device=dev)
    nbytes = sparse_attn_ws_bytes(n_q, h, k, w_max)
    buf = _ws(dev, nbytes, ws)
    if swa_new is not None:
        _need(swa_new, torch.bfloat16, "swa_new")
        _need(swa_dst, torch.int64, "swa_dst")
        if swa_new.shape != (n_q, KV_CH) or swa_dst.numel() != n_q or w_max <= 0:
            raise ValueError("swa_new must be [n_q,512] with one swa_dst per query, and a window given")
        st = lib().csa2_sparse_attn_append(_ptr(q), F32 if q.dtype == torch.float32 else BF16, n_q, h, d,
                                           _ptr(q_seq), _ptr(cache), _ptr(seq_base), _ptr(idx), k, _ptr(swa),
                                           swa.shape[0], _ptr(swa_row0), _ptr(swa_len), int(w_max),
                                           _ptr(swa_new), _ptr(swa_dst), float(softmax_scale), _ptr(out),
                                           _ptr(lse) if want_lse else None, _ptr(buf), buf.numel(), _stream(dev))
        _check(st, "csa2_sparse_attn_append")
        return out, lse
    st = lib().csa2_sparse_attn(_ptr(q), F32 if q.dtype == torch.float32 else BF16, n_q, h, d, _ptr(q_seq),
                                _ptr(cache), _ptr(seq_base), _ptr(idx), k,
                                _ptr(swa) if w_max > 0 else None, _ptr(swa_row0) if w_max > 0 else None,
                                _ptr(swa_len) if w_max > 0 else None, int(w_max), float(softmax_scale),
                                _ptr(out), _ptr(lse) if want_lse else None, _ptr(buf), buf.numel(),
                                _stream(dev))
    _check(st, "csa2_sparse_attn")
    return out, lse
