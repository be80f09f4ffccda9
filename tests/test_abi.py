"""The C-ABI library loads on a machine without a GPU, exports every symbol its
header declares, and rejects bad arguments on the host before enqueueing
anything (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import sparse_long_context_topk_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(csa2.LIB_PATH), reason="libcsa2.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"csa2_quant_append", "csa2_index_topk", "csa2_reindex_topk", "csa2_sparse_attn"} <= set(names)
    L = ctypes.CDLL(csa2.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    L = csa2.lib()
    assert L.csa2_status_string(0) == b"ok"
    assert L.csa2_status_string(3) == b"workspace too small"
    assert L.csa2_last_hip_error() == 0


FAKE = ctypes.c_void_p(1 << 20)    # aligned, never dereferenced: checks fail first


def test_index_topk_argument_checks():
    L = csa2.lib()
    args = dict(iq=FAKE, w=FAKE, n_q=2, h_i=64, d_i=128, q_seq=FAKE, q_nvis=FAKE, max_nvis=1000,
                ik=FAKE, seq_base=FAKE, k=512, idx=FAKE, block=8, keep=0, pool=None, ws=FAKE,
                ws_bytes=1, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.csa2_index_topk(a["iq"], a["w"], a["n_q"], a["h_i"], a["d_i"], a["q_seq"], a["q_nvis"],
                                 a["max_nvis"], a["ik"], a["seq_base"], a["k"], a["idx"], a["block"],
                                 a["keep"], a["pool"], a["ws"], a["ws_bytes"], a["stream"])
    assert call(k=0) == 1 and call(k=4096) == 1 and call(n_q=-1) == 1
    assert call(d_i=96) == 2 and call(h_i=65) == 2
    assert call(keep=2048, block=4, pool=FAKE) == 2
    assert call(keep=2048, pool=None) == 1
    assert call(iq=ctypes.c_void_p((1 << 20) + 2)) == 1           # unaligned
    assert call() == 3                                             # workspace too small
    assert call(n_q=0) == 0                                        # nothing to do
    need = L.csa2_index_topk_ws_bytes(2, 1000, 64, 128, 512, 8, 0)
    need_pool = L.csa2_index_topk_ws_bytes(2, 1000, 64, 128, 512, 8, 2048)
    assert 0 < need < need_pool


def test_index_topk_chunk_argument_checks():
    L = csa2.lib()
    args = dict(iq=FAKE, w=FAKE, n_q=2, h_i=64, d_i=128, q_nvis=FAKE, max_nvis=1000, ik=FAKE, base=0, k=512,
                idx=FAKE, ws=FAKE, ws_bytes=1, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.csa2_index_topk_chunk(a["iq"], a["w"], a["n_q"], a["h_i"], a["d_i"], a["q_nvis"], a["max_nvis"],
                                       a["ik"], a["base"], a["k"], a["idx"], a["ws"], a["ws_bytes"], a["stream"])
    assert call(k=0) == 1 and call(k=4096) == 1 and call(n_q=-1) == 1 and call(base=-5) == 1
    assert call(d_i=96) == 2 and call(h_i=65) == 2
    assert call(ik=None) == 1 and call(q_nvis=None) == 1
    assert call(ik=ctypes.c_void_p((1 << 20) + 2)) == 1           # unaligned
    assert call() == 3                                             # workspace too small
    assert call(n_q=0) == 0                                        # nothing to do


def test_attn_and_quant_argument_checks():
    L = csa2.lib()
    sp = lambda **kw: L.csa2_sparse_attn(FAKE, kw.get("qdt", 1), 2, kw.get("h", 64), kw.get("d", 512),
                                         FAKE, FAKE, FAKE, FAKE, kw.get("k", 512), FAKE, FAKE, FAKE,
                                         kw.get("w", 128), ctypes.c_float(0.04), FAKE, None, FAKE,
                                         kw.get("ws", 0), None)
    assert sp(d=256) == 2 and sp(h=24) == 2 and sp(h=80) == 2
    assert sp(qdt=5) == 1 and sp(k=-1) == 1
    assert sp() == 3
    assert L.csa2_quant_append(FAKE, 1, -1, FAKE, FAKE, 10, None) == 1
    assert L.csa2_quant_append(FAKE, 7, 1, FAKE, FAKE, 10, None) == 1
    assert L.csa2_quant_append(None, 1, 0, None, None, 0, None) == 0


def test_workspace_sizes_grow_with_inputs():
    L = csa2.lib()
    a = L.csa2_index_topk_ws_bytes(4, 1 << 20, 64, 128, 512, 8, 2048)
    b = L.csa2_index_topk_ws_bytes(8, 1 << 20, 64, 128, 512, 8, 2048)
    assert b > a > 0
    assert L.csa2_reindex_topk_ws_bytes(4, 64, 128, 512, 8, 2048) > 0
    assert L.csa2_sparse_attn_ws_bytes(64, 64, 512, 128) >= L.csa2_sparse_attn_ws_bytes(1, 64, 512, 128)


def test_block_keys_argument_checks():
    L = csa2.lib()
    bk = lambda **kw: L.csa2_block_keys(kw.get("ik", FAKE), kw.get("d", 128), FAKE, FAKE, kw.get("frm", None),
                                        kw.get("n_seq", 2), kw.get("mb", 4), kw.get("kbar", FAKE), FAKE, None)
    assert bk(d=100) == 2 and bk(d=0) == 2 and bk(d=2048) == 2
    assert bk(n_seq=-1) == 1 and bk(mb=-1) == 1
    assert bk(ik=None) == 1 and bk(kbar=None) == 1
    assert bk(ik=ctypes.c_void_p((1 << 20) + 8)) == 1 and bk(frm=ctypes.c_void_p((1 << 20) + 2)) == 1
    assert bk(n_seq=0) == 0 and bk(mb=0) == 0 and bk(ik=None, mb=0) == 0   # nothing to do, nothing enqueued


def test_window_append_argument_checks():
    L = csa2.lib()
    wa = lambda **kw: L.csa2_window_append(kw.get("x", FAKE), kw.get("dt", 1), kw.get("n", 4), kw.get("dst", FAKE),
                                           kw.get("swa", FAKE), kw.get("rows", 10), None)
    assert wa(n=-1) == 1 and wa(rows=-1) == 1 and wa(dt=3) == 1
    assert wa(x=None) == 1 and wa(dst=None) == 1 and wa(swa=None) == 1
    assert wa(x=ctypes.c_void_p((1 << 20) + 4)) == 1 and wa(dst=ctypes.c_void_p((1 << 20) + 4)) == 1
    assert wa(n=0) == 0 and wa(x=None, n=0) == 0


def test_attention_append_argument_checks():
    L = csa2.lib()
    ap = lambda **kw: L.csa2_sparse_attn_append(FAKE, 1, 2, 64, 512, FAKE, FAKE, FAKE, FAKE, 512, kw.get("swa", FAKE),
                                                kw.get("rows", 256), FAKE, FAKE, 128, kw.get("new", FAKE),
                                                kw.get("dst", FAKE), ctypes.c_float(0.04), FAKE, None, FAKE,
                                                kw.get("ws", 0), None)
    assert ap(new=None) == 1 and ap(dst=None) == 1 and ap(swa=None) == 1 and ap(rows=-1) == 1
    assert ap(new=ctypes.c_void_p((1 << 20) + 8)) == 1 and ap(dst=ctypes.c_void_p((1 << 20) + 4)) == 1
    assert ap() == 3   # every check passes but the (zero) workspace: nothing is enqueued


def test_topk_merge_argument_checks():
    L = csa2.lib()
    mg = lambda **kw: L.csa2_topk_merge(FAKE, FAKE, kw.get("n_q", 2), 64, kw.get("d", 128), FAKE, kw.get("ik", FAKE),
                                        FAKE, kw.get("cand", FAKE), kw.get("nc", 1024), kw.get("k", 512), FAKE,
                                        FAKE, kw.get("ws", 0), None)
    assert mg(d=100) == 2 and mg(nc=(1 << 25) + 1) == 2
    assert mg(k=0) == 1 and mg(k=4096) == 1 and mg(nc=-1) == 1 and mg(cand=None) == 1
    assert mg(ik=ctypes.c_void_p((1 << 20) + 8)) == 1
    assert mg() == 3 and mg(n_q=0) == 0
    assert L.csa2_topk_merge_ws_bytes(2, 1024, 64, 128, 512) > 2 * 1024 * 128 * 2
