"""The low-precision indexer-key variant on the GPU: csa2_index_keys_fp8 codes
and exponent bytes bit-exact against the oracle's quantiser, and the Full and
Reindex selections over FP8 keys bit-exact against the oracle's selections
over the stored keys (which the oracle quantises itself from the same bf16
keys)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, index_inputs, note, to_dev


def _quant_gpu(ik_host):
    dev = device()
    codes, exps = csa2.index_keys_fp8(ik_host.to(dev))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), exps.cpu().numpy()


@gpu
@pytest.mark.parametrize("d_i", [64, 128])
def test_quantiser_random_rows_bitexact(d_i):
    note(f"fp8 keys quantiser d_i={d_i}")
    g = torch.Generator().manual_seed(700 + d_i)
    rows = 5000
    x = torch.randn((rows, d_i), generator=g) * torch.exp2(torch.randint(-140, 120, (rows, 1), generator=g).float())
    x[::7] *= torch.where(torch.rand((rows // 7 + 1, d_i), generator=g) < 0.05, 20.0, 1.0)[: x[::7].shape[0]]
    x[3] = 0.0
    x[4, :5] = -0.0
    x[5] = 448.0 * torch.sign(torch.randn(d_i, generator=g))
    ik = x.to(torch.bfloat16)
    gc, ge = _quant_gpu(ik)
    rc, re = oracle.index_keys_fp8(bits(ik))
    assert np.array_equal(ge, re)
    assert np.array_equal(gc, rc)


@gpu
def test_quantiser_every_bf16_value():
    # every finite bf16 value of magnitude <= 448, 127 per row beside a 448 (E = 0)
    note("fp8 keys quantiser: every bf16 value")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = (b.astype(np.uint32) << 16).view(np.float32)
    vals = b[np.isfinite(f) & (np.abs(f) <= 448)]
    pad = (-len(vals)) % 127
    vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 127)
    head = np.full((vals.shape[0], 1), 0x43E0, np.uint16)   # 448
    rows = np.concatenate([head, vals], axis=1)
    ik = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16)
    gc, ge = _quant_gpu(ik)
    rc, re = oracle.index_keys_fp8(rows)
    assert np.all(re == 127)
    assert np.array_equal(ge, re) and np.array_equal(gc, rc)


def _fp8_inputs(lengths, seed):
    inp = index_inputs(lengths, 64, 128, seed=seed)
    ik8, ik8e = oracle.index_keys_fp8(bits(inp["ik"]))        # the oracle's own quantisation
    return inp, oracle.dequant_keys_fp8(ik8, ik8e)


@gpu
@pytest.mark.parametrize("lengths,keep", [([20003, 17001, 3000, 1], 2048), ([9000, 4097, 0], 0),
                                          ([40000, 12000], 512)])
def test_full_and_reindex_over_fp8_keys(lengths, keep):
    note(f"fp8 keys full/reindex {lengths} keep={keep}")
    inp, kq = _fp8_inputs(lengths, 710 + len(lengths))
    dev = device()
    d = to_dev(inp, dev)
    ik8, ik8e = csa2.index_keys_fp8(d["ik"])
    max_nvis = int(max(lengths))
    r = csa2.index_topk_fp8(d["iq"], d["w"], d["q_seq"], d["nvis"], max_nvis, ik8, ik8e, d["seq_base"], k=512,
                            keep_blocks=keep)
    torch.cuda.synchronize()
    ref = oracle.index_topk(bits(inp["iq"]), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(), kq,
                            inp["seq_base"].numpy(), 512, block=8, keep_blocks=keep)
    if keep:
        g_idx, g_pool = r[0].cpu().numpy(), r[1].cpu().numpy()
        r_idx, r_pool = ref
        assert np.array_equal(g_pool, r_pool)
        assert np.array_equal(g_idx, r_idx)
        # Reindex with another query over that pool, FP8 keys
        iq2 = torch.flip(inp["iq"], dims=[1]).contiguous()
        gr = csa2.reindex_topk_fp8(iq2.to(dev), d["w"], d["q_seq"], d["nvis"], ik8, ik8e, d["seq_base"],
                                   torch.from_numpy(r_pool).to(dev), k=512)
        torch.cuda.synchronize()
        rr = oracle.reindex_topk(bits(iq2), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(), kq,
                                 inp["seq_base"].numpy(), r_pool, 512, block=8)
        assert np.array_equal(gr.cpu().numpy(), rr)
    else:
        assert np.array_equal(r.cpu().numpy(), ref)
