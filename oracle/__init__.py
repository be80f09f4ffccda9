"""Plain CPU oracle of the CSA2 decode hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library in
``sparse_long_context_topk_amd``) never imports it, and the two share no code.

The arithmetic lives in ``csa2_ref.cpp`` (plain C++, built with
``g++ -O2 -ffp-contract=off -fno-fast-math -fopenmp``); this module only builds
and loads that library and marshals numpy arrays into it.  Every function
takes and returns host numpy arrays.

Sources (page title and section):
  [W1] "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн токенов,
       KV-кэшем FP4 и повторным использованием внимания между слоями"
       (wire.sakhanda.co) -- sections on CSA2, on FP4 KV and on the
       encoder-decoder.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa2_ref.cpp")
LIB = os.path.join(HERE, "libcsa2_ref.so")

CH = 512
RECORD = 288

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no GPU code involved)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        cmd = ["g++", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-std=c++17", "-shared", "-fPIC", "-Wall", "-o", tmp, SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.csa2_ref_e2m1_value.restype = ctypes.c_double
        L.csa2_ref_e2m1_value.argtypes = [i32]
        L.csa2_ref_e4m3_value.restype = ctypes.c_double
        L.csa2_ref_e4m3_value.argtypes = [i32]
        L.csa2_ref_bf16_bits.restype = ctypes.c_uint16
        L.csa2_ref_bf16_bits.argtypes = [f32]
        L.csa2_ref_e4m3_round_scale.restype = i32
        L.csa2_ref_e4m3_round_scale.argtypes = [f32]
        L.csa2_ref_e2m1_round_mag.restype = i32
        L.csa2_ref_e2m1_round_mag.argtypes = [f32, i32]
        L.csa2_ref_quant_append.restype = i32
        L.csa2_ref_quant_append.argtypes = [vp, i32, i64, vp, vp, i64]
        L.csa2_ref_dequant_record.restype = None
        L.csa2_ref_dequant_record.argtypes = [vp, vp]
        L.csa2_ref_index_score.restype = f32
        L.csa2_ref_index_score.argtypes = [vp, vp, i32, i32, vp]
        L.csa2_ref_block_score.restype = f32
        L.csa2_ref_block_score.argtypes = [vp, vp, i32, i32, vp, i32]
        L.csa2_ref_topk.restype = None
        L.csa2_ref_topk.argtypes = [vp, vp, i64, i32, vp]
        L.csa2_ref_index_topk.restype = i32
        L.csa2_ref_index_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, i32, vp,
                                          i32, i32, vp, i32]
        L.csa2_ref_reindex_topk.restype = i32
        L.csa2_ref_reindex_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32,
                                            i32, i32, vp, i32]
        L.csa2_ref_block_keys.restype = i32
        L.csa2_ref_block_keys.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]
        L.csa2_ref_index_keys_fp8.restype = i32
        L.csa2_ref_index_keys_fp8.argtypes = [vp, i64, i32, vp, vp]
        L.csa2_ref_dequant_keys_fp8.restype = None
        L.csa2_ref_dequant_keys_fp8.argtypes = [vp, vp, i64, i32, vp]
        L.csa2_ref_sparse_attn.restype = i32
        L.csa2_ref_sparse_attn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32,
                                           vp, vp, vp, f32, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return lib().csa2_ref_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().csa2_ref_e4m3_value(int(code))


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), nearest-even."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().csa2_ref_bf16_bits
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def e4m3_round_scale(amax: float) -> int:
    return lib().csa2_ref_e4m3_round_scale(float(amax))


def e2m1_round_mag(ax: float, scale_code: int) -> int:
    return lib().csa2_ref_e2m1_round_mag(float(ax), int(scale_code))


# ---------------------------------------------------------------- a1 / a6
def quant_append(x: np.ndarray, dst_row: np.ndarray, cache: np.ndarray) -> None:
    """x: float32 [n,512] or uint16 (bf16 bits) [n,512]; cache: uint8 [rows,288] (in place)."""
    if x.dtype == np.float32:
        dt = 0
    elif x.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    x = np.ascontiguousarray(x)
    dst = _c(dst_row, np.int64)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.shape[1] == RECORD
    rc = lib().csa2_ref_quant_append(_p(x), dt, x.shape[0], _p(dst), _p(cache), cache.shape[0])
    if rc:
        raise ValueError("csa2_ref_quant_append: invalid arguments")


def quantize_rows(x: np.ndarray) -> np.ndarray:
    n = x.shape[0]
    cache = np.zeros((n, RECORD), dtype=np.uint8)
    quant_append(x, np.arange(n, dtype=np.int64), cache)
    return cache


def dequant_records(recs: np.ndarray) -> np.ndarray:
    recs = _c(recs, np.uint8).reshape(-1, RECORD)
    out = np.empty((recs.shape[0], CH), dtype=np.float32)
    f = lib().csa2_ref_dequant_record
    for i in range(recs.shape[0]):
        f(_p(recs[i]), _p(out[i]))
    return out


# ---------------------------------------------------------------- a2 / a4
def index_score(iq: np.ndarray, w: np.ndarray, key: np.ndarray) -> float:
    """iq: uint16 [h_i,d_i] (bf16 bits), w: float32 [h_i], key: uint16 [d_i]."""
    iq = _c(iq, np.uint16)
    w = _c(w, np.float32)
    key = _c(key, np.uint16)
    h_i, d_i = iq.shape
    return lib().csa2_ref_index_score(_p(iq), _p(w), h_i, d_i, _p(key))


def block_score(iq: np.ndarray, w: np.ndarray, keys: np.ndarray) -> float:
    """Score of one pool block whose members are the rows of keys (uint16
    [n_members, d_i]): the mean of the members' per-head dots (fp32 sum in row
    order, IEEE division), then ReLU and the head chain as for a token."""
    iq = _c(iq, np.uint16)
    w = _c(w, np.float32)
    keys = _c(keys, np.uint16)
    h_i, d_i = iq.shape
    return lib().csa2_ref_block_score(_p(iq), _p(w), h_i, d_i, _p(keys), keys.shape[0])


def topk(scores: np.ndarray, k: int, pos: np.ndarray | None = None) -> np.ndarray:
    s = _c(scores, np.float32)
    p = None if pos is None else _c(pos, np.int32)
    out = np.empty(k, dtype=np.int32)
    lib().csa2_ref_topk(_p(s), _p(p), s.shape[0], k, _p(out))
    return out


def index_topk(iq, w, q_seq, q_nvis, ik, seq_base, k, block=8, keep_blocks=0, n_threads=0):
    """Full layer.  Returns idx [n_q,k] (and pool blocks [n_q,keep_blocks] if keep_blocks)."""
    iq = _c(iq, np.uint16)
    n_q, h_i, d_i = iq.shape
    w = _c(w, np.float32)
    q_seq = _c(q_seq, np.int32)
    q_nvis = _c(q_nvis, np.int32)
    ik = _c(ik, np.uint16)
    seq_base = _c(seq_base, np.int64)
    idx = np.empty((n_q, k), dtype=np.int32)
    pool = np.empty((n_q, keep_blocks), dtype=np.int32) if keep_blocks else None
    rc = lib().csa2_ref_index_topk(_p(iq), _p(w), n_q, h_i, d_i, _p(q_seq), _p(q_nvis),
                                   _p(ik), _p(seq_base), k, _p(idx), block, keep_blocks,
                                   _p(pool), n_threads)
    if rc:
        raise ValueError("csa2_ref_index_topk: invalid arguments")
    return (idx, pool) if keep_blocks else idx


def reindex_topk(iq, w, q_seq, q_nvis, ik, seq_base, pool_blocks, k, block=8, n_threads=0):
    iq = _c(iq, np.uint16)
    n_q, h_i, d_i = iq.shape
    pool_blocks = _c(pool_blocks, np.int32)
    keep_blocks = pool_blocks.shape[1]
    idx = np.empty((n_q, k), dtype=np.int32)
    rc = lib().csa2_ref_reindex_topk(_p(iq), _p(_c(w, np.float32)), n_q, h_i, d_i,
                                     _p(_c(q_seq, np.int32)), _p(_c(q_nvis, np.int32)),
                                     _p(_c(ik, np.uint16)), _p(_c(seq_base, np.int64)),
                                     _p(pool_blocks), block, keep_blocks, k, _p(idx), n_threads)
    if rc:
        raise ValueError("csa2_ref_reindex_topk: invalid arguments")
    return idx


# ---------------------------------------------------------------- pool-based Full
def block_keys(ik, seq_base, seq_len, kbar, kbar_base, blk_from=None, block=8, max_blocks=None):
    """Write the bf16 mean keys of blocks into kbar (uint16 [rows, d_i], updated in
    place): for sequence s, blocks blk_from[s] <= b < ceil(seq_len[s]/block), at most
    max_blocks of them, go to row kbar_base[s] + b.  Defaults: every block."""
    ik = _c(ik, np.uint16)
    d_i = ik.shape[1]
    seq_len = _c(seq_len, np.int32)
    n_seq = seq_len.shape[0]
    blk_from = np.zeros(n_seq, np.int32) if blk_from is None else _c(blk_from, np.int32)
    if max_blocks is None:
        max_blocks = int(((seq_len.astype(np.int64) + block - 1) // block).max(initial=0))
    if kbar.dtype != np.uint16 or not kbar.flags["C_CONTIGUOUS"]:
        raise TypeError("kbar must be a contiguous uint16 array")
    rc = lib().csa2_ref_block_keys(_p(ik), d_i, _p(_c(seq_base, np.int64)), _p(seq_len), _p(blk_from),
                                   n_seq, block, int(max_blocks), _p(kbar), _p(_c(kbar_base, np.int64)))
    if rc:
        raise ValueError("csa2_ref_block_keys: invalid arguments")
    return kbar


def pool_full_topk(iq, w, q_seq, q_nvis, ik, seq_base, kbar, kbar_base, k, keep_blocks, block=8,
                   n_threads=0):
    """Full layer of the pool-based variant: the Top-keep_blocks blocks by the
    token score of their stored keys (kbar), then the Top-K positions of that
    pool re-scored with the same query.  Returns (idx [n_q,k], pool [n_q,keep_blocks])."""
    q_nvis = _c(q_nvis, np.int32)
    q_nblk = ((q_nvis.astype(np.int64) + block - 1) // block).astype(np.int32)
    pool = index_topk(iq, w, q_seq, q_nblk, kbar, kbar_base, keep_blocks, n_threads=n_threads)
    idx = reindex_topk(iq, w, q_seq, q_nvis, ik, seq_base, pool, k, block=block, n_threads=n_threads)
    return idx, pool


# ---------------------------------------------------------------- FP8 indexer keys (variant)
def index_keys_fp8(ik):
    """bf16 key rows (uint16 [rows, d_i]) -> (E4M3 codes uint8 [rows, d_i],
    exponent bytes uint8 [rows]): one power-of-two scale 2^(exps - 127) per row."""
    ik = _c(ik, np.uint16)
    rows, d_i = ik.shape
    codes = np.empty((rows, d_i), np.uint8)
    exps = np.empty(rows, np.uint8)
    if lib().csa2_ref_index_keys_fp8(_p(ik), rows, d_i, _p(codes), _p(exps)):
        raise ValueError("csa2_ref_index_keys_fp8: invalid arguments")
    return codes, exps


def dequant_keys_fp8(codes, exps):
    """The stored keys code * 2^(exps - 127) as bf16 bits (exact)."""
    codes = _c(codes, np.uint8)
    exps = _c(exps, np.uint8)
    rows, d_i = codes.shape
    out = np.empty((rows, d_i), np.uint16)
    lib().csa2_ref_dequant_keys_fp8(_p(codes), _p(exps), rows, d_i, _p(out))
    return out


# ---------------------------------------------------------------- a7
def sparse_attn(q, q_seq, cache, seq_base, idx, swa, swa_row0, swa_len, softmax_scale,
                n_threads=0):
    """q: float32 or uint16(bf16) [n_q,h,512]; returns (out [n_q,h,512] f32, lse [n_q,h] f32)."""
    q = np.ascontiguousarray(q)
    if q.dtype == np.float32:
        qdt = 0
    elif q.dtype == np.uint16:
        qdt = 1
    else:
        raise TypeError("q must be float32 or uint16 (bf16 bits)")
    n_q, h, d = q.shape
    idx = _c(idx, np.int32)
    k = idx.shape[1] if idx.ndim == 2 else 0
    out = np.empty((n_q, h, d), dtype=np.float32)
    lse = np.empty((n_q, h), dtype=np.float32)
    swa = _c(swa, np.uint16) if swa is not None else np.zeros((1, CH), np.uint16)
    rc = lib().csa2_ref_sparse_attn(_p(q), qdt, n_q, h, d, _p(_c(q_seq, np.int32)),
                                    _p(_c(cache, np.uint8)), _p(_c(seq_base, np.int64)),
                                    _p(idx), k, _p(swa), _p(_c(swa_row0, np.int64)),
                                    _p(_c(swa_len, np.int32)), float(softmax_scale),
                                    _p(out), _p(lse), n_threads)
    if rc:
        raise ValueError("csa2_ref_sparse_attn: invalid arguments")
    return out, lse
