"""csa2_sparse_attn on the GPU versus the oracle (fp64): normwise error per
(query, head) row within 2e-3, for fp32 and bf16 queries, window-only,
selection-only, padded selections, empty rows, many and few splits."""
import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, normwise_err, note

TOL = 2e-3


def _case(n_q, h, L, k, nswa, qdtype, seed, idx_fn=None, outliers=0.0):
    raw = gen.normal((n_q * L, 512), seed, "kv", dtype=torch.bfloat16, outlier_p=outliers)
    cache = oracle.quantize_rows(bits(raw))
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(L, min(k, L), replace=False)) for _ in range(n_q)]).astype(np.int32)
    if idx.shape[1] < k:
        idx = np.concatenate([idx, -np.ones((n_q, k - idx.shape[1]), np.int32)], axis=1)
    if idx_fn is not None:
        idx = idx_fn(idx)
    q = gen.normal((n_q, h, 512), seed, "q", dtype=qdtype, outlier_p=outliers)
    swa = gen.normal((n_q * max(nswa, 1), 512), seed, "swa", dtype=torch.bfloat16, outlier_p=outliers)
    seq_base = np.arange(n_q, dtype=np.int64) * L
    q_seq = np.arange(n_q, dtype=np.int32)[::-1].copy()          # queries read other sequences
    swa_row0 = np.arange(n_q, dtype=np.int64) * max(nswa, 1)
    swa_len = np.array([max(0, nswa - (i % 3)) for i in range(n_q)], np.int32) if nswa else np.zeros(n_q, np.int32)
    return dict(cache=cache, idx=idx, q=q, swa=swa, seq_base=seq_base, q_seq=q_seq, swa_row0=swa_row0,
                swa_len=swa_len, nswa=nswa)


def _run(c, scale=512 ** -0.5):
    dev = device()
    w_max = c["nswa"]
    out, lse = csa2.sparse_attn(c["q"].to(dev), torch.from_numpy(c["q_seq"]).to(dev),
                                torch.from_numpy(c["cache"]).to(dev), torch.from_numpy(c["seq_base"]).to(dev),
                                torch.from_numpy(c["idx"]).to(dev), c["swa"].to(dev),
                                torch.from_numpy(c["swa_row0"]).to(dev), torch.from_numpy(c["swa_len"]).to(dev),
                                w_max, scale)
    torch.cuda.synchronize()
    qn = c["q"].numpy() if c["q"].dtype == torch.float32 else bits(c["q"])
    ro, rl = oracle.sparse_attn(qn, c["q_seq"], c["cache"], c["seq_base"], c["idx"], bits(c["swa"]),
                                c["swa_row0"], c["swa_len"], scale)
    return out.cpu().numpy(), lse.cpu().numpy(), ro, rl


@gpu
@pytest.mark.parametrize("n_q,h,qdt", [(3, 64, torch.bfloat16), (1, 16, torch.float32), (64, 64, torch.bfloat16),
                                       (5, 32, torch.float32), (2, 48, torch.bfloat16)])
def test_topk_plus_window(n_q, h, qdt):
    note(f"attn n_q={n_q} h={h} {qdt}")
    c = _case(n_q, h, 4096, 512, 128, qdt, seed=n_q * 7 + h)
    o, l, ro, rl = _run(c)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
    assert np.allclose(l, rl, rtol=1e-4, atol=1e-4)


@gpu
def test_outliers_and_large_scores():
    note("attn outliers")
    c = _case(4, 64, 8192, 512, 128, torch.bfloat16, seed=3, outliers=0.01)
    o, l, ro, rl = _run(c, scale=0.08)
    assert normwise_err(o, ro) <= TOL


@gpu
def test_window_only_and_selection_only():
    note("attn window only")
    c = _case(4, 64, 600, 512, 128, torch.bfloat16, seed=4, idx_fn=lambda i: -np.ones_like(i))
    o, l, ro, rl = _run(c)
    assert normwise_err(o, ro) <= TOL
    note("attn selection only")
    c = _case(4, 64, 600, 512, 0, torch.bfloat16, seed=5)
    o, l, ro, rl = _run(c)
    assert normwise_err(o, ro) <= TOL


@gpu
def test_padded_and_short_selections_and_empty_rows():
    note("attn padded")

    def pad(i):
        i = i.copy()
        i[0, 100:] = -1          # 100 entries
        i[1, :] = -1             # window only
        i[2, ::3] = -1
        return i
    c = _case(4, 64, 3000, 512, 17, torch.bfloat16, seed=6, idx_fn=pad)
    c["swa_len"][1] = 0          # query 1: no key at all
    o, l, ro, rl = _run(c)
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))
    keep = [0, 2, 3]
    assert normwise_err(o[keep], ro[keep]) <= TOL


@gpu
def test_short_context_and_odd_k():
    note("attn short")
    c = _case(6, 64, 40, 37, 5, torch.float32, seed=8)
    o, l, ro, rl = _run(c)
    assert normwise_err(o, ro) <= TOL


@gpu
def test_reuse_layers_share_indices():
    """Reuse: the group's idx with each layer's own q and window rows."""
    note("attn reuse")
    base = _case(8, 64, 4096, 512, 128, torch.bfloat16, seed=9)
    for layer in range(3):
        c = dict(base)
        c["q"] = gen.normal((8, 64, 512), 50 + layer, "q", dtype=torch.bfloat16)
        c["swa"] = gen.normal((8 * 128, 512), 50 + layer, "swa", dtype=torch.bfloat16)
        o, l, ro, rl = _run(c)
        assert normwise_err(o, ro) <= TOL


@gpu
def test_deterministic():
    note("attn determinism")
    c = _case(3, 64, 2048, 512, 128, torch.bfloat16, seed=10)
    a = _run(c)[0]
    b = _run(c)[0]
    assert np.array_equal(a, b)


@gpu
@pytest.mark.parametrize("n_q,h,k,nswa", [(128, 64, 500, 128), (300, 32, 512, 100)])
def test_many_queries_long_splits(n_q, h, k, nswa):
    """Calls with few splits per query (128 queries: 2 splits of 10 sub-tiles;
    300: 1 split of 20), where the bf16 kernel's decode runs its selected-only
    loop for most sub-tiles; k = 500 leaves a sub-tile that straddles the
    window, h = 32 leaves two multiply waves idle, and a tenth of the selected
    entries are padding (-1) scattered through the lists."""
    note(f"attn many queries n_q={n_q} h={h} k={k} nswa={nswa}")

    def pad(i):
        i = i.copy()
        rng = np.random.default_rng(n_q)
        i[rng.random(i.shape) < 0.1] = -1
        return i
    c = _case(n_q, h, 640, k, nswa, torch.bfloat16, seed=n_q + k, idx_fn=pad)
    o, l, ro, rl = _run(c)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
    assert np.allclose(l, rl, rtol=1e-4, atol=1e-4)


@gpu
@pytest.mark.parametrize("n_q,k,nswa,L", [(16, 512, 128, 4096), (64, 512, 128, 2048), (128, 500, 128, 640),
                                          (300, 512, 100, 640), (8, 2048, 1024, 4096)])
def test_partial_head_groups(n_q, k, nswa, L):
    """48 heads (three 16-head tiles) where the bf16 kernel's work-groups take
    two or four tiles each, so that one head group is partly past h: two-tile
    groups with 7 and with 1 split(s) per query (16 and 128 queries), four-tile
    groups with 4, 1 and 32 splits (64, 300 and 8 queries, the last at the
    largest lists); padding (-1) scattered through the selections."""
    note(f"attn h=48 n_q={n_q} k={k} nswa={nswa}")

    def pad(i):
        i = i.copy()
        rng = np.random.default_rng(n_q + 1)
        i[rng.random(i.shape) < 0.05] = -1
        return i
    c = _case(n_q, 48, L, k, nswa, torch.bfloat16, seed=90 + n_q, idx_fn=pad)
    o, l, ro, rl = _run(c)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
    assert np.allclose(l, rl, rtol=1e-4, atol=1e-4)


@gpu
@pytest.mark.parametrize("n_q,h,qdt", [(3, 64, torch.bfloat16), (2, 16, torch.float32), (40, 64, torch.bfloat16)])
def test_largest_selection_and_window(n_q, h, qdt):
    """The largest supported lists: k = 2048 selected entries and windows of up
    to w_max = 1024 rows (3072 keys per query)."""
    note(f"attn k=2048 w_max=1024 n_q={n_q} h={h} {qdt}")
    c = _case(n_q, h, 4096, 2048, 1024, qdt, seed=70 + n_q)
    o, l, ro, rl = _run(c)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
    assert np.allclose(l, rl, rtol=1e-4, atol=1e-4)


def _scaled_rows(n, seed, group_scale):
    """N(0,1) rows whose 16-channel groups are multiplied by group_scale[row, group]."""
    x = gen.normal((n, 512), seed, "kv-small", dtype=torch.float32)
    return (x.view(n, 32, 16) * torch.from_numpy(group_scale)[:, :, None]).view(n, 512).to(torch.bfloat16)


@gpu
def test_subnormal_and_zero_scales():
    """FP4 records whose E4M3 scales are subnormal (groups scaled by 2^-7 and
    2^-8: amax / 6 falls in [2^-9, 2^-6)) or zero (groups scaled by 2^-12, and
    all-zero groups), gathered with k = 2048 and a 1024-row window of the same
    magnitude, so that the decoded values of these groups carry the output."""
    note("attn subnormal and zero scales")
    n_q, L, k = 4, 4096, 2048
    rng = np.random.default_rng(77)
    fac = rng.choice([2.0 ** -7, 2.0 ** -8, 2.0 ** -12, 0.0], size=(n_q * L, 32), p=[0.45, 0.35, 0.1, 0.1])
    raw = _scaled_rows(n_q * L, 77, fac.astype(np.float32))
    cache = oracle.quantize_rows(bits(raw))
    sc = cache[:, 256:288]
    subn = ((sc & 0x78) == 0) & ((sc & 0x07) != 0)
    print(f"scales: {subn.mean():.2f} subnormal, {(sc == 0).mean():.2f} zero")
    assert subn.mean() > 0.5 and (sc == 0).mean() > 0.1
    c = _case(n_q, 64, L, k, 1024, torch.bfloat16, seed=78)
    c["cache"] = cache
    c["swa"] = (c["swa"].float() * 2.0 ** -7).to(torch.bfloat16)
    o, l, ro, rl = _run(c, scale=8.0)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
    # window off: the output is made of the decoded FP4 values alone
    c["swa_len"][:] = 0
    o, l, ro, rl = _run(c, scale=8.0)
    assert normwise_err(o, ro) <= TOL


@gpu
def test_bf16_values_near_the_fp16_range_limit():
    """bf16 queries and window rows are converted to fp16 for the MFMA: values
    up to the documented limit (|x| < 65504) stay exact in range; elements of
    magnitude up to 60,000 in the query and in the window rows."""
    note("attn fp16 range edge")
    c = _case(3, 64, 2048, 512, 128, torch.bfloat16, seed=79)
    q = c["q"].float()
    q[:, :, ::37] = 60000.0 * torch.sign(q[:, :, ::37])
    c["q"] = q.to(torch.bfloat16)
    s = c["swa"].float()
    s[::5, ::41] = -59904.0
    c["swa"] = s.to(torch.bfloat16)
    o, l, ro, rl = _run(c, scale=2.0 ** -40)
    err = normwise_err(o, ro)
    print(f"normwise err {err:.3e}")
    assert err <= TOL
