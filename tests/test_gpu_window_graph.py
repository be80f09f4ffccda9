"""Window rows and the captured decode step on the GPU.

csa2_window_append: rows land bit-exactly (bf16 copies, fp32 rounded to the
nearest bf16 as the oracle's conversion does) at their ring rows, rows outside
the buffer are skipped, nothing else changes.  StepGraph: a decode step
captured as a HIP graph and replayed several times, with eager steps and
synchronisations between the replays, gives bit-identical indices, pools and
attention outputs to the eager step every time."""
import numpy as np
import pytest
import torch

import bench
import csa2_inputs as gen
import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, note
from sparse_long_context_topk_amd.schedule import StepGraph, decode_step


@gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_window_append_rows(dtype):
    dev = device()
    note(f"window append {dtype}")
    g = torch.Generator().manual_seed(401)
    n, rows = 37, 300
    x = (torch.randn((n, 512), generator=g) * torch.exp2(torch.randint(-20, 20, (n, 1), generator=g).float()))
    x[3, :7] = -0.0
    x = x.to(dtype)
    dst = torch.randperm(rows, generator=g)[:n].to(torch.int64)
    dst[5], dst[9] = -1, rows            # skipped
    base = torch.randn((rows, 512), generator=g).to(torch.bfloat16)
    swa = base.to(dev)
    csa2.window_append(x.to(dev), dst.to(dev), swa)
    torch.cuda.synchronize()
    exp = bits(base).copy()
    xv = x.numpy() if dtype == torch.float32 else None
    for i in range(n):
        d = int(dst[i])
        if 0 <= d < rows:
            exp[d] = oracle.bf16_bits(xv[i]) if xv is not None else bits(x[i:i + 1])[0]
    assert np.array_equal(bits(swa.cpu()), exp)


@gpu
@pytest.mark.parametrize("name,div,pool_full", [("c1", 1, False), ("c3", 16, False), ("c3", 16, True),
                                                ("c5", 64, False)])
def test_captured_step_replays_equal_eager(name, div, pool_full):
    dev = device()
    note(f"graph capture {name}/{div} pool_full={pool_full}")
    wl = gen.workload(name, length_div=div)
    if pool_full:
        wl["pool_full"] = True
    st, layers, app_x, app_rows = bench.build_state(wl, dev)
    ref, rpool = decode_step(st, layers, append_x=app_x, append_rows=app_rows, keep_outputs=True)
    torch.cuda.synchronize()
    ref = [(i.cpu().numpy(), o.cpu().numpy(), l.cpu().numpy()) for i, o, l in ref]
    rpool = rpool.cpu().numpy() if rpool is not None else None
    gr = StepGraph(st, layers, append_x=app_x, append_rows=app_rows)
    for rep in range(3):
        res, pool = gr.replay()
        torch.cuda.synchronize()
        for li, ((gi, go, gl), (ri, ro, rl)) in enumerate(zip(res, ref)):
            assert np.array_equal(gi.cpu().numpy(), ri), f"replay {rep} layer {li}: indices"
            assert np.array_equal(go.cpu().numpy(), ro), f"replay {rep} layer {li}: output"
            assert np.array_equal(gl.cpu().numpy(), rl), f"replay {rep} layer {li}: lse"
        if rpool is not None:
            assert np.array_equal(pool.cpu().numpy(), rpool), f"replay {rep}: pool"
        # eager work between replays
        decode_step(st, layers, append_x=app_x, append_rows=app_rows, keep_outputs=False)
        torch.cuda.synchronize()


@gpu
@pytest.mark.parametrize("qdt,lens", [(torch.bfloat16, [1, 77, 128, 5000]), (torch.float32, [300, 128, 2])])
def test_attention_with_window_append_equals_two_calls(qdt, lens):
    # csa2_sparse_attn_append must give the window rows and the outputs of
    # csa2_window_append followed by csa2_sparse_attn, bit for bit
    dev = device()
    note(f"attention + window append {qdt} {lens}")
    g = torch.Generator().manual_seed(411)
    n_q, W, h = len(lens), 128, 64
    L = max(lens)
    raw = torch.randn((n_q * L, 512), generator=g)
    cache = torch.empty((n_q * L, 288), dtype=torch.uint8, device=dev)
    csa2.quant_append(raw.to(dev), torch.arange(n_q * L, dtype=torch.int64, device=dev), cache)
    idx = torch.full((n_q, 512), -1, dtype=torch.int32)
    for i, n in enumerate(lens):
        sel = torch.randperm(n, generator=g)[:min(512, n)].sort().values
        idx[i, :len(sel)] = sel.to(torch.int32)
    q = torch.randn((n_q, h, 512), generator=g).to(qdt)
    swa0 = torch.randn((n_q * W, 512), generator=g).to(torch.bfloat16)
    new = torch.randn((n_q, 512), generator=g).to(torch.bfloat16)
    row0 = torch.arange(n_q, dtype=torch.int64) * W
    wlen = torch.tensor([min(W, n) for n in lens], dtype=torch.int32)
    dst = torch.tensor([i * W + (n - 1) % W for i, n in enumerate(lens)], dtype=torch.int64)
    sb = torch.arange(n_q, dtype=torch.int64) * L
    qs = torch.arange(n_q, dtype=torch.int32)
    d = lambda t: t.to(dev)
    sa, sb_ = d(swa0), d(swa0)
    csa2.window_append(d(new), d(dst), sa)
    o1, l1 = csa2.sparse_attn(d(q), d(qs), cache, d(sb), d(idx), sa, d(row0), d(wlen), W, 0.044)
    o2, l2 = csa2.sparse_attn(d(q), d(qs), cache, d(sb), d(idx), sb_, d(row0), d(wlen), W, 0.044,
                              swa_new=d(new), swa_dst=d(dst))
    torch.cuda.synchronize()
    assert torch.equal(sa.cpu(), sb_.cpu())
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(l1.cpu(), l2.cpu())
