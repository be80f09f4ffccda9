"""csa2_reindex_topk_noalloc -- the Reindex call for callers that cannot
allocate -- against csa2_reindex_topk (the same kernels with a caller
workspace): identical indices on two calls in a row, the second smaller than
the first, both through the raw C ABI; calls beyond the fixed scratch are
refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, index_inputs, note, to_dev


def _raw_noalloc(d, iq, pool, k, idx_out, dev):
    L = csa2.lib()
    n_q, h_i, d_i = iq.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return L.csa2_reindex_topk_noalloc(p(iq), p(d["w"]), n_q, h_i, d_i, p(d["q_seq"]), p(d["nvis"]), p(d["ik"]),
                                       p(d["seq_base"]), p(pool), 8, pool.shape[1], k, p(idx_out),
                                       ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))


def _case(lengths, keep, k, seed):
    dev = device()
    inp = index_inputs(lengths, 64, 128, seed=seed)
    _, pool = oracle.index_topk(bits(inp["iq"]), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(),
                                bits(inp["ik"]), inp["seq_base"].numpy(), k, block=8, keep_blocks=keep)
    d = to_dev(inp, dev)
    iq2 = torch.flip(inp["iq"], dims=[1]).contiguous().to(dev)       # the Reindex layer's own query
    pool_d = torch.from_numpy(pool).to(dev)
    ref = csa2.reindex_topk(iq2, d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"], pool_d, k=k)
    out = torch.full((len(lengths), k), -7, dtype=torch.int32, device=dev)
    st = _raw_noalloc(d, iq2, pool_d, k, out, dev)
    assert st == 0, csa2.lib().csa2_status_string(st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@gpu
def test_noalloc_reindex_equals_workspace_reindex_twice_second_smaller():
    note("no-alloc reindex: 40 queries, 2048-block pools")
    lengths = [20000 - 311 * i for i in range(40)]
    got, ref = _case(lengths, 2048, 512, seed=900)
    assert np.array_equal(got, ref)
    note("no-alloc reindex: 3 queries, 300-block pools (smaller, same scratch)")
    got2, ref2 = _case([5000, 2401, 16391], 300, 64, seed=901)
    assert np.array_equal(got2, ref2)


@gpu
def test_noalloc_reindex_multi_kernel_pool():
    # a 4096-block pool (32,768 slots) takes the multi-kernel selection, whose
    # first launch clears its histograms in the shared scratch
    note("no-alloc reindex: 4096-block pools")
    got, ref = _case([40000, 33000, 700], 4096, 512, seed=902)
    assert np.array_equal(got, ref)


@gpu
def test_noalloc_reindex_refuses_calls_beyond_its_scratch():
    dev = device()
    n_q = 200                                             # 200 queries x 2048-block pools > 32 MiB
    assert csa2.reindex_topk_ws_bytes(n_q, 64, 128, 512, 8, 2048) > csa2.NOALLOC_SCRATCH_BYTES
    iq = torch.zeros((n_q, 64, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((n_q, 64), dtype=torch.float32, device=dev)
    z32 = torch.zeros(n_q, dtype=torch.int32, device=dev)
    ik = torch.zeros((8, 128), dtype=torch.bfloat16, device=dev)
    sb = torch.zeros(n_q, dtype=torch.int64, device=dev)
    pool = torch.full((n_q, 2048), -1, dtype=torch.int32, device=dev)
    with pytest.raises(csa2.Csa2Error, match="workspace too small"):
        csa2.reindex_topk_noalloc(iq, w, z32, z32, ik, sb, pool, k=512)
