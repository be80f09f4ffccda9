"""The pool-based Full variant on the GPU: csa2_block_keys bit-exact against
the oracle (ragged sequences, partial last blocks, range refreshes that leave
other rows alone, outliers, signed zeros and subnormal means), and the
variant's Full layer (block scan over the stored keys, then the pool
re-scored with the same query) bit-exact on indices and pools."""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, index_inputs, note, to_dev

LENGTHS = [1, 7, 8, 9, 63, 64, 65, 1000, 4093, 16384, 16391, 70001]


def _layout(lengths):
    nblk = [(L + 7) // 8 for L in lengths]
    seq_base = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    kb_base = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    return nblk, seq_base, kb_base


def _keys(lengths, d_i, seed):
    ik = index_inputs(lengths, 1, d_i, seed)["ik"]
    x = ik.float()
    g = torch.Generator().manual_seed(seed)
    r = torch.rand(x.shape, generator=g)
    x = torch.where(r < 0.01, x * 20, x)                        # 1% outliers x20
    x = torch.where((r > 0.5) & (r < 0.502), torch.zeros_like(x) * -1.0, x)   # some -0
    x = torch.where((r > 0.6) & (r < 0.601), x * 2.0 ** -128, x)  # means in the subnormal range
    return x.to(torch.bfloat16)


@gpu
@pytest.mark.parametrize("d_i", [64, 128])
def test_block_keys_bitexact(d_i):
    dev = device()
    note(f"block keys d_i={d_i}")
    ik = _keys(LENGTHS, d_i, seed=300 + d_i)
    nblk, sb, kbb = _layout(LENGTHS)
    kbar = torch.full((sum(nblk), d_i), 7.0, dtype=torch.bfloat16, device=dev)
    lens = torch.tensor(LENGTHS, dtype=torch.int32)
    csa2.block_keys(ik.to(dev), torch.from_numpy(sb).to(dev), lens.to(dev), kbar, torch.from_numpy(kbb).to(dev),
                    max(nblk))
    torch.cuda.synchronize()
    ref = np.zeros((sum(nblk), d_i), np.uint16)
    oracle.block_keys(bits(ik), sb, lens.numpy(), ref, kbb)
    assert np.array_equal(bits(kbar.cpu()), ref)


@gpu
def test_block_keys_range_refresh_touches_only_named_blocks():
    dev = device()
    note("block keys range refresh")
    d_i = 128
    ik = _keys(LENGTHS, d_i, seed=310)
    nblk, sb, kbb = _layout(LENGTHS)
    lens = torch.tensor(LENGTHS, dtype=torch.int32)
    rng = np.random.default_rng(311)
    frm = np.array([rng.integers(-1, n + 2) for n in nblk], np.int32)   # some before the first, some past the last
    for mb in (1, 3):
        sentinel = torch.full((sum(nblk), d_i), 7.0, dtype=torch.bfloat16)
        kbar = sentinel.to(dev)
        csa2.block_keys(ik.to(dev), torch.from_numpy(sb).to(dev), lens.to(dev), kbar, torch.from_numpy(kbb).to(dev),
                        mb, blk_from=torch.from_numpy(frm).to(dev))
        torch.cuda.synchronize()
        ref = bits(sentinel).copy()
        oracle.block_keys(bits(ik), sb, lens.numpy(), ref, kbb, blk_from=frm, max_blocks=mb)
        assert np.array_equal(bits(kbar.cpu()), ref), f"max_blocks={mb}"


def _variant(inp, k, keep, dev):
    lens = inp["nvis"].numpy()
    nblk, sb, kbb = _layout(lens)
    d = to_dev(inp, dev)
    kbar = torch.empty((max(sum(nblk), 1), inp["ik"].shape[1]), dtype=torch.bfloat16, device=dev)
    kb_base = torch.from_numpy(kbb).to(dev)
    csa2.block_keys(d["ik"], d["seq_base"], d["nvis"], kbar, kb_base, max(nblk))
    q_nblk = torch.tensor(nblk, dtype=torch.int32, device=dev)
    pool = csa2.index_topk(d["iq"], d["w"], d["q_seq"], q_nblk, max(nblk), kbar, kb_base, k=keep)
    idx = csa2.reindex_topk(d["iq"], d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"], pool, k=k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), pool.cpu().numpy()


@gpu
@pytest.mark.parametrize("h_i,d_i,k,keep", [(64, 128, 512, 2048), (4, 64, 512, 256), (20, 128, 64, 100)])
def test_pool_based_full_layer(h_i, d_i, k, keep):
    dev = device()
    note(f"pool-based full h_i={h_i} d_i={d_i} k={k} keep={keep}")
    lengths = [1, 9, 512, 513, 4096, 16384, 16391, 40000]
    inp = index_inputs(lengths, h_i, d_i, seed=320 + h_i)
    got_idx, got_pool = _variant(inp, k, keep, dev)
    nblk, sb, kbb = _layout(lengths)
    kbar = np.zeros((sum(nblk), d_i), np.uint16)
    oracle.block_keys(bits(inp["ik"]), sb, inp["nvis"].numpy(), kbar, kbb)
    ref_idx, ref_pool = oracle.pool_full_topk(bits(inp["iq"]), inp["w"].numpy(), inp["q_seq"].numpy(),
                                              inp["nvis"].numpy(), bits(inp["ik"]), sb, kbar, kbb, k, keep)
    assert np.array_equal(got_pool, ref_pool)
    assert np.array_equal(got_idx, ref_idx)
