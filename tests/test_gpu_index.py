"""csa2_index_topk / csa2_reindex_topk on the GPU: indices and pools bit-exact
versus the oracle at ragged lengths, ties, pools and both indexer shapes."""
import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, index_inputs, note, to_dev


def _gpu_full(inp, k, keep_blocks=0, ws=None):
    dev = device()
    d = to_dev(inp, dev)
    max_nvis = int(inp["nvis"].max()) if len(inp["nvis"]) else 0
    r = csa2.index_topk(d["iq"], d["w"], d["q_seq"], d["nvis"], max_nvis, d["ik"], d["seq_base"], k=k,
                        keep_blocks=keep_blocks, ws=ws)
    torch.cuda.synchronize()
    if keep_blocks:
        return r[0].cpu().numpy(), r[1].cpu().numpy()
    return r.cpu().numpy()


def _ref_full(inp, k, keep_blocks=0):
    return oracle.index_topk(bits(inp["iq"]), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(),
                             bits(inp["ik"]), inp["seq_base"].numpy(), k, block=8, keep_blocks=keep_blocks)


EDGE_LENGTHS = [1, 7, 8, 9, 127, 128, 129, 511, 512, 513, 4096, 16383, 16384, 16385, 16391, 20000]


@gpu
@pytest.mark.parametrize("h_i,d_i", [(4, 64), (64, 128), (20, 128), (33, 64)])
def test_full_ragged_lengths(h_i, d_i):
    note(f"full ragged h_i={h_i} d_i={d_i}")
    inp = index_inputs(EDGE_LENGTHS, h_i, d_i, seed=100 + h_i)
    got = _gpu_full(inp, 512)
    ref = _ref_full(inp, 512)
    assert np.array_equal(got, ref)


@gpu
@pytest.mark.parametrize("h_i,d_i", [(4, 64), (64, 128), (33, 64)])
def test_full_short_ragged_lengths(h_i, d_i):
    """Every context <= 16,384 and no pool: the call selects through the
    Reindex kernels over all blocks of each context.  The edge lengths, with
    an empty sequence last (its base row is the key array's end)."""
    note(f"full short ragged h_i={h_i} d_i={d_i}")
    inp = index_inputs([L for L in EDGE_LENGTHS if L <= 16384] + [0], h_i, d_i, seed=150 + h_i)
    got = _gpu_full(inp, 512)
    ref = _ref_full(inp, 512)
    assert np.array_equal(got, ref)
    assert np.all(got[-1] == -1)


@gpu
@pytest.mark.parametrize("lengths", [[20000, 3000, 1], [9000, 3000, 1]], ids=["multi_kernel", "short"])
@pytest.mark.parametrize("k", [1, 64, 512, 2048])
def test_full_k_values(k, lengths):
    # a context above 16,384 positions takes the multi-kernel selection (fine
    # histogram, compaction, rescoring, final select); all contexts at or below
    # it take the one-work-group select over every block of the context
    note(f"full k={k} lengths={lengths}")
    inp = index_inputs(lengths, 64, 128, seed=7 + k)
    assert np.array_equal(_gpu_full(inp, k), _ref_full(inp, k))


@gpu
@pytest.mark.parametrize("case", ["zero", "equal", "dup_blocks", "two_values"])
def test_full_ties(case):
    note(f"full ties {case}")

    def kf(ik):
        if case == "zero":
            return torch.zeros_like(ik)
        if case == "equal":
            return ik[:1].expand_as(ik).contiguous()
        if case == "dup_blocks":
            ik = ik.clone()
            ik[4096:8192] = ik[0:4096]
            return ik
        ik = ik.clone()
        ik[::2] = ik[0]
        ik[1::2] = ik[1]
        return ik
    inp = index_inputs([8192, 5000], 64, 128, seed=3, key_fn=kf)
    assert np.array_equal(_gpu_full(inp, 512), _ref_full(inp, 512))


@gpu
def test_full_ties_larger_than_lds_band():
    """All keys equal over 20000 positions: every candidate is in the band and
    uncertain, which takes the final selection's global-memory path."""
    note("full ties 20000 equal")
    inp = index_inputs([20000, 13000], 64, 128, seed=4, key_fn=lambda ik: ik[:1].expand_as(ik).contiguous())
    g_idx, g_pool = _gpu_full(inp, 512, 2048)
    r_idx, r_pool = _ref_full(inp, 512, 2048)
    assert np.array_equal(g_idx, r_idx) and np.array_equal(g_pool, r_pool)


@gpu
@pytest.mark.parametrize("lengths,keep", [([20000, 16391, 300], 2048), ([4096, 1000, 8], 64),
                                          ([16384, 16385], 2048), ([30000], 1024)])
def test_full_with_pool(lengths, keep):
    note(f"full+pool {lengths} keep={keep}")
    inp = index_inputs(lengths, 64, 128, seed=11)
    g_idx, g_pool = _gpu_full(inp, 512, keep)
    r_idx, r_pool = _ref_full(inp, 512, keep)
    assert np.array_equal(g_idx, r_idx)
    assert np.array_equal(g_pool, r_pool)


@gpu
def test_pool_with_block_constant_keys():
    note("pool block-constant keys")
    inp = index_inputs([24000], 64, 128, seed=12, key_fn=lambda ik: ik[::8].repeat_interleave(8, 0)[:ik.shape[0]].contiguous())
    g_idx, g_pool = _gpu_full(inp, 512, 512)
    r_idx, r_pool = _ref_full(inp, 512, 512)
    assert np.array_equal(g_idx, r_idx) and np.array_equal(g_pool, r_pool)


@gpu
@pytest.mark.parametrize("lengths,keep", [([20000, 16391, 300], 2048), ([40000, 9], 512),
                                          ([40000, 33000, 700], 4096)])   # 32,768 slots: the multi-kernel path
def test_reindex(lengths, keep):
    note(f"reindex {lengths} keep={keep}")
    inp = index_inputs(lengths, 64, 128, seed=21)
    _, r_pool = _ref_full(inp, 512, keep)
    iq2 = torch.flip(inp["iq"], dims=[1]).contiguous()       # the Reindex layer's own query
    dev = device()
    d = to_dev(inp, dev)
    got = csa2.reindex_topk(iq2.to(dev), d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"],
                            torch.from_numpy(r_pool).to(dev), k=512)
    torch.cuda.synchronize()
    ref = oracle.reindex_topk(bits(iq2), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(),
                              bits(inp["ik"]), inp["seq_base"].numpy(), r_pool, 512, block=8)
    assert np.array_equal(got.cpu().numpy(), ref)


@gpu
@pytest.mark.parametrize("case", ["equal", "two_values", "scaled_copies"])
def test_reindex_ties_and_narrow_ranges(case):
    """Degenerate score sets for the single-work-group Reindex select: every
    score equal, two distinct values, and many keys that are scaled copies of
    one row (scores on a few exact multiples)."""
    note(f"reindex ties {case}")

    def kf(ik):
        if case == "equal":
            return ik[:1].expand_as(ik).contiguous()
        if case == "two_values":
            ik = ik.clone()
            ik[::2] = ik[0]
            ik[1::2] = ik[1]
            return ik
        scale = (torch.arange(ik.shape[0]) % 5 + 1).to(torch.float32)[:, None]
        return (ik[:1].float() * scale).to(torch.bfloat16).expand_as(ik).contiguous()
    inp = index_inputs([20000, 9000], 64, 128, seed=23, key_fn=kf)
    _, r_pool = _ref_full(inp, 512, 2048)
    iq2 = torch.flip(inp["iq"], dims=[1]).contiguous()
    dev = device()
    d = to_dev(inp, dev)
    got = csa2.reindex_topk(iq2.to(dev), d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"],
                            torch.from_numpy(r_pool).to(dev), k=512)
    torch.cuda.synchronize()
    ref = oracle.reindex_topk(bits(iq2), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(),
                              bits(inp["ik"]), inp["seq_base"].numpy(), r_pool, 512, block=8)
    assert np.array_equal(got.cpu().numpy(), ref)


@gpu
@pytest.mark.parametrize("n_q,h_i,d_i", [(7, 64, 128), (6, 20, 128), (5, 33, 64), (1, 4, 64)])
def test_chunk_of_one_sequence(n_q, h_i, d_i):
    """Causal queries of one sequence (the encoder-side chunk path): each sees
    its own prefix of the keys; odd query counts leave the last work-group of
    the multi-query scan half empty."""
    note(f"chunk n_q={n_q} h_i={h_i} d_i={d_i}")
    L, base = 30000, 777
    inp = index_inputs([base + L], h_i, d_i, seed=31 + n_q)
    nvis = np.array([max(0, L - 4099 * i) for i in range(n_q)][::-1], np.int32)   # ragged, ascending
    nvis[0] = min(nvis[0], 300)                                                    # one short query
    iq = inp["iq"][:1].expand(n_q, h_i, d_i).contiguous()
    iq = (iq.float() * torch.linspace(0.5, 1.5, n_q)[:, None, None]).to(torch.bfloat16)
    w = inp["w"][:1].expand(n_q, h_i).contiguous()
    dev = device()
    got = csa2.index_topk_chunk(iq.to(dev), w.to(dev), torch.from_numpy(nvis).to(dev), int(nvis.max()),
                                inp["ik"].to(dev), ik_base=base, k=512)
    torch.cuda.synchronize()
    ref = oracle.index_topk(bits(iq), w.numpy(), np.zeros(n_q, np.int32), nvis, bits(inp["ik"]),
                            np.array([base], np.int64), 512, block=8, keep_blocks=0)
    assert np.array_equal(got.cpu().numpy(), ref)


@gpu
def test_reindex_with_full_query_equals_full_when_pool_covers_context():
    note("reindex == full")
    inp = index_inputs([16000, 7000], 64, 128, seed=22)
    g_idx, g_pool = _gpu_full(inp, 512, 2048)
    dev = device()
    d = to_dev(inp, dev)
    got = csa2.reindex_topk(d["iq"], d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"],
                            torch.from_numpy(g_pool).to(dev), k=512)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), g_idx)


@gpu
def test_deterministic_and_workspace_reuse():
    note("determinism")
    inp = index_inputs([20000, 512, 70000], 64, 128, seed=5)
    ws = csa2.Workspace()
    a = _gpu_full(inp, 512, 2048, ws=ws)
    small = index_inputs([600], 64, 128, seed=6)
    _gpu_full(small, 512, 2048, ws=ws)
    b = _gpu_full(inp, 512, 2048, ws=ws)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@gpu
def test_mfma_scores_within_proven_bound():
    """The scan's approximate scores (left in the workspace) never leave the
    rounding bound the selection relies on."""
    note("mfma bound")
    L, h_i, d_i = 6000, 64, 128
    inp = index_inputs([L], h_i, d_i, seed=9)
    inp["ik"] = (inp["ik"].float() * torch.where(torch.arange(L)[:, None] % 97 == 0, 20.0, 1.0)).to(torch.bfloat16)
    ws = csa2.Workspace()
    _gpu_full(inp, 512, ws=ws)
    approx = ws.buf[:L * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    iqb, ikb, w = bits(inp["iq"])[0], bits(inp["ik"]), inp["w"].numpy()[0]
    exact = np.array([oracle.index_score(iqb, w, ikb[t]) for t in range(L)])
    qf = inp["iq"][0].double().numpy()
    kf = inp["ik"].double().numpy()
    # t_k = sum_h |w_h| sum_d |q_hd| |k_d|, the key magnitude the kernels' bound uses
    t = np.abs(kf) @ (np.abs(w)[:, None] * np.abs(qf)).sum(axis=0)
    u, u2 = 2.0 ** -24, 2.0 ** -23
    gam = lambda n, uu: n * uu / (1 - n * uu)
    gd, gm, gh = gam(d_i, u), gam(d_i + 2, u2), gam(66, u)
    c = 2 * (gd + gm + gh * (2 + gd + gm))
    bound = c * t
    ratio = np.abs(approx - exact) / bound
    print(f"max |mfma - exact| / bound = {ratio.max():.3e}")
    assert np.all(np.abs(approx - exact) <= bound)


@gpu
@pytest.mark.parametrize("n_q,L,chunk", [(1, 3000, 1024), (8, 131072 // 16, 1024), (40, 30000, 2048),
                                         (64, 32768, 4096), (4, 1 << 20, 8192)])
def test_full_with_pool_at_every_scan_chunk_size(n_q, L, chunk):
    # the scan's keys per work-group follow the batch shape (8192 down to 1024,
    # keeping at least 512 work-groups); each shape here selects the size named,
    # with the pool and ragged lengths (every 3rd sequence is shorter)
    note(f"full + pool, scan chunk {chunk}: n_q={n_q} L={L}")
    lengths = [L if i % 3 else max(1, L - 4093 * (i + 1)) for i in range(n_q)]
    h_i, d_i = (4, 64) if L * n_q >= (1 << 20) else (64, 128)   # oracle work within seconds
    inp = index_inputs(lengths, h_i, d_i, seed=500 + n_q)
    keep = 2048 if L > 16384 else 256
    got_idx, got_pool = _gpu_full(inp, 512, keep_blocks=keep)
    ref_idx, ref_pool = _ref_full(inp, 512, keep_blocks=keep)
    assert np.array_equal(got_pool, ref_pool)
    assert np.array_equal(got_idx, ref_idx)


@gpu
@pytest.mark.parametrize("n_q,chunk", [(4, 256), (20, 512), (40, 1024), (80, 2048)])
def test_reindex_at_every_scan_chunk_size(n_q, chunk):
    # the Reindex scan's pool slots per work-group grow with the batch (256 up
    # to 2048 while at least 512 work-groups remain); each batch here selects
    # the size named (pools of 2048 blocks, ragged lengths)
    note(f"reindex, scan chunk {chunk}: n_q={n_q}")
    lengths = [20000 - 37 * i for i in range(n_q)]
    inp = index_inputs(lengths, 4, 64, seed=600 + n_q)
    _, pool = _ref_full(inp, 512, keep_blocks=2048)
    rng = np.random.default_rng(601)
    iq2 = torch.from_numpy(rng.standard_normal(inp["iq"].shape).astype(np.float32)).to(torch.bfloat16)
    w2 = torch.from_numpy(rng.uniform(0, 1, inp["w"].shape).astype(np.float32))
    dev = device()
    d = to_dev(inp, dev)
    got = csa2.reindex_topk(iq2.to(dev), w2.to(dev), d["q_seq"], d["nvis"], d["ik"], d["seq_base"],
                            torch.from_numpy(pool).to(dev), k=512)
    torch.cuda.synchronize()
    ref = oracle.reindex_topk(bits(iq2), w2.numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(), bits(inp["ik"]),
                              inp["seq_base"].numpy(), pool, 512, block=8)
    assert np.array_equal(got.cpu().numpy(), ref)


# ---------------------------------------------------------------- rounding bound of the MFMA scores
def _bound_consts(d_i):
    """The scan's rounding constants: per key, |approximate - exact fp32 chain|
    <= C * t_k with t_k = sum_h |w_h| sum_d |q_hd| |k_d| (tokens), and for a
    block <= C_blk * (its members' largest t_k)."""
    u, u2 = 2.0 ** -24, 2.0 ** -23
    gam = lambda n, uu: n * uu / (1 - n * uu)
    e = gam(d_i, u) + gam(d_i + 2, u2)
    eb = e + 2 * gam(8, u) + 8 * u
    gh = gam(66, u)
    return 2 * (e + gh * (2 + e)), 2 * (eb + gh * (2 + eb))


def _t_of(iq_bits, w, ik_bits):
    qf = (iq_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf = (ik_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.abs(kf) @ (np.abs(w.astype(np.float64))[:, None] * np.abs(qf)).sum(axis=0)


@gpu
def test_full_pool_scan_scores_within_proven_bound():
    """The 1M decode path's scan (Full layer with the pool): every token score
    and every block score it leaves in the workspace lies within the rounding
    bound the selection relies on, against the exact fp32 chains of the score
    definition -- contexts above 16,384 positions, a partial last block in both
    sequences, keys with 20x outliers.  Block scores include the partial
    blocks' mean (a reciprocal of the member count)."""
    note("mfma bound: full + pool scan")
    lengths, h_i, d_i, keep = [20003, 17001], 64, 128, 2048
    inp = index_inputs(lengths, h_i, d_i, seed=19)
    total = sum(lengths)
    inp["ik"] = (inp["ik"].float() * torch.where(torch.arange(total)[:, None] % 97 == 0, 20.0, 1.0)).to(torch.bfloat16)
    ws = csa2.Workspace()
    g_idx, g_pool = _gpu_full(inp, 512, keep, ws=ws)
    r_idx, r_pool = _ref_full(inp, 512, keep)
    assert np.array_equal(g_idx, r_idx) and np.array_equal(g_pool, r_pool)
    n_q = len(lengths)
    stride = (max(lengths) + 4095) // 4096 * 4096
    sc = ws.buf[:2 * n_q * stride * 4].view(torch.float32).cpu().numpy().astype(np.float64).reshape(2 * n_q, stride)
    c_tok, c_blk = _bound_consts(d_i)
    iqb, ikb, w, sb = bits(inp["iq"]), bits(inp["ik"]), inp["w"].numpy(), inp["seq_base"].numpy()
    worst_t = worst_b = 0.0
    for q, L in enumerate(lengths):
        keys = ikb[sb[q]:sb[q] + L]
        exact = np.array([oracle.index_score(iqb[q], w[q], keys[t]) for t in range(L)])
        t = _t_of(iqb[q], w[q], keys)
        err = np.abs(sc[q, :L] - exact)
        assert np.all(err <= c_tok * t), f"query {q}: token score outside the bound"
        worst_t = max(worst_t, float((err / (c_tok * t)).max()))
        nb = (L + 7) // 8
        bex = np.array([oracle.block_score(iqb[q], w[q], keys[8 * b:min(L, 8 * b + 8)]) for b in range(nb)])
        tb = np.array([t[8 * b:min(L, 8 * b + 8)].max() for b in range(nb)])
        errb = np.abs(sc[n_q + q, :nb] - bex)
        assert np.all(errb <= c_blk * tb), f"query {q}: block score outside the bound"
        worst_b = max(worst_b, float((errb / (c_blk * tb)).max()))
        assert L % 8 != 0                                   # the last block is partial
    print(f"max |mfma - exact| / bound: tokens {worst_t:.3e}, blocks {worst_b:.3e}")


@gpu
def test_chunk_scan_scores_within_proven_bound():
    """The encoder-chunk scan (several causal queries of one sequence per
    work-group, head sums in a different order): every score it leaves in the
    workspace lies within the rounding bound of the exact chain."""
    note("mfma bound: chunk scan")
    L, base, n_q, h_i, d_i = 12000, 100, 5, 64, 128
    inp = index_inputs([base + L], h_i, d_i, seed=41)
    inp["ik"] = (inp["ik"].float() * torch.where(torch.arange(base + L)[:, None] % 89 == 0, 20.0, 1.0)).to(torch.bfloat16)
    nvis = np.array([L - 2001 * i for i in range(n_q)][::-1], np.int32)
    rng = np.random.default_rng(41)
    iq = torch.from_numpy(rng.standard_normal((n_q, h_i, d_i)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.uniform(0, 1, (n_q, h_i)).astype(np.float32))
    dev = device()
    ws = csa2.Workspace()
    got = csa2.index_topk_chunk(iq.to(dev), w.to(dev), torch.from_numpy(nvis).to(dev), int(nvis.max()),
                                inp["ik"].to(dev), ik_base=base, k=512, ws=ws)
    torch.cuda.synchronize()
    iqb, ikb, wn = bits(iq), bits(inp["ik"]), w.numpy()
    ref = oracle.index_topk(iqb, wn, np.zeros(n_q, np.int32), nvis, ikb, np.array([base], np.int64), 512)
    assert np.array_equal(got.cpu().numpy(), ref)
    stride = (int(nvis.max()) + 4095) // 4096 * 4096
    sc = ws.buf[:n_q * stride * 4].view(torch.float32).cpu().numpy().astype(np.float64).reshape(n_q, stride)
    c_tok, _ = _bound_consts(d_i)
    worst = 0.0
    for q in range(n_q):
        keys = ikb[base:base + nvis[q]]
        exact = np.array([oracle.index_score(iqb[q], wn[q], keys[t]) for t in range(nvis[q])])
        t = _t_of(iqb[q], wn[q], keys)
        err = np.abs(sc[q, :nvis[q]] - exact)
        assert np.all(err <= c_tok * t), f"query {q}: chunk score outside the bound"
        worst = max(worst, float((err / (c_tok * t)).max()))
    print(f"max |mfma - exact| / bound (chunk scan) = {worst:.3e}")


# ---------------------------------------------------------------- bf16 subnormal inputs
def _subnormal_mix(t, frac, seed):
    """Replace a fraction of the elements with bf16 subnormals (|x| < 2^-126)."""
    g = torch.Generator().manual_seed(seed)
    m = torch.rand(t.shape, generator=g) < frac
    tiny = (torch.randn(t.shape, generator=g) * 2.0 ** -129).to(torch.bfloat16)
    return torch.where(m, tiny, t)


@gpu
def test_subnormal_keys_and_queries():
    """bf16-subnormal key and query elements: a sequence with 30 % subnormal key
    elements, one whose keys are all subnormal (every score is then a tiny fp32
    value, many of them subnormal, and the rounding bound's underflow term
    leaves every key undecided), and queries with 20 % subnormal elements;
    Full with the pool, Reindex over it, and the short no-pool path."""
    note("index subnormal inputs")
    lengths = [20000, 17000, 3000]
    inp = index_inputs(lengths, 64, 128, seed=43)
    ik = _subnormal_mix(inp["ik"], 0.3, 1)
    s1 = inp["seq_base"][1].item()
    ik[s1:s1 + lengths[1]] = (inp["ik"][s1:s1 + lengths[1]].float() * 2.0 ** -129).to(torch.bfloat16)
    inp["ik"] = ik
    inp["iq"] = _subnormal_mix(inp["iq"], 0.2, 2)
    kb = bits(inp["ik"])
    exp_field = (kb >> 7) & 0xFF
    assert np.mean((exp_field == 0) & ((kb & 0x7F) != 0)) > 0.2
    g_idx, g_pool = _gpu_full(inp, 512, 2048)
    r_idx, r_pool = _ref_full(inp, 512, 2048)
    assert np.array_equal(g_idx, r_idx) and np.array_equal(g_pool, r_pool)
    iq2 = torch.flip(inp["iq"], dims=[1]).contiguous()
    dev = device()
    d = to_dev(inp, dev)
    got = csa2.reindex_topk(iq2.to(dev), d["w"], d["q_seq"], d["nvis"], d["ik"], d["seq_base"],
                            torch.from_numpy(r_pool).to(dev), k=512)
    torch.cuda.synchronize()
    ref = oracle.reindex_topk(bits(iq2), inp["w"].numpy(), inp["q_seq"].numpy(), inp["nvis"].numpy(),
                              bits(inp["ik"]), inp["seq_base"].numpy(), r_pool, 512, block=8)
    assert np.array_equal(got.cpu().numpy(), ref)
    short = dict(inp)
    short["nvis"] = torch.tensor([9000, 9000, 3000], dtype=torch.int32)   # every context <= 16,384, no pool
    assert np.array_equal(_gpu_full(short, 512), _ref_full(short, 512))


@gpu
def test_pool_rescoring_beyond_shared_block_list():
    """More than 256 queries with a pool: their block work-groups rescore
    each query's own block band (the shared block list serves up to 256
    queries).  The 300-query call must equal three 100-query calls (which
    take the shared list), and both equal the oracle on a sample."""
    n_q = 300
    lengths = [17000 + (i * 7919) % 9000 for i in range(n_q)]
    note(f"full + pool, {n_q} queries over {sum(lengths)} positions")
    inp = index_inputs(lengths, 16, 64, seed=77)
    got_idx, got_pool = _gpu_full(inp, 512, keep_blocks=2048)
    for q0 in range(0, n_q, 100):
        part = dict(inp)
        part["iq"], part["w"] = inp["iq"][q0:q0 + 100], inp["w"][q0:q0 + 100]
        part["q_seq"], part["nvis"] = inp["q_seq"][q0:q0 + 100], inp["nvis"][q0:q0 + 100]
        p_idx, p_pool = _gpu_full(part, 512, keep_blocks=2048)
        assert np.array_equal(p_idx, got_idx[q0:q0 + 100]), f"indices of queries {q0}..{q0 + 99} differ"
        assert np.array_equal(p_pool, got_pool[q0:q0 + 100]), f"pools of queries {q0}..{q0 + 99} differ"
    sample = [0, 1, 150, 298, 299]
    sub = dict(inp)
    sub["iq"], sub["w"] = inp["iq"][sample], inp["w"][sample]
    sub["q_seq"], sub["nvis"] = inp["q_seq"][sample], inp["nvis"][sample]
    r_idx, r_pool = _ref_full(sub, 512, keep_blocks=2048)
    assert np.array_equal(got_idx[sample], r_idx)
    assert np.array_equal(got_pool[sample], r_pool)


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_large_mode_with_pool_equals_per_work_group_mode(fmt):
    """A Full call with a pool whose token scores pass 1 GB (300 queries over
    one 1M-position sequence: 1.2 GB) runs the large selection mode for both
    of its problems (token rows with group keys, block rows loading every
    group); three 100-query calls on the same queries (0.4 GB each) run the
    per-work-group mode.  Both are exact, so indices and pools must agree;
    with bf16 keys and with FP8 keys."""
    dev = device()
    n_q, L, h_i = 300, 1 << 20, 16
    d_i = 64 if fmt == "bf16" else 128
    note(f"large mode with a pool ({fmt} keys): {n_q} queries over one {L}-position sequence")
    ik = gen.normal((L, d_i), 91, "ik", dtype=torch.bfloat16).to(dev)
    iq = gen.normal((n_q, h_i, d_i), 91, "iq", dtype=torch.bfloat16).to(dev)
    w = gen.uniform((n_q, h_i), 91, "w").to(dev)
    nvis = torch.tensor([L - 4093 * (i % 7) for i in range(n_q)], dtype=torch.int32, device=dev)
    q_seq = torch.zeros(n_q, dtype=torch.int32, device=dev)
    seq_base = torch.zeros(1, dtype=torch.int64, device=dev)
    if fmt == "fp8":
        ik8, ik8e = csa2.index_keys_fp8(ik)

    def call(sl):
        args = (iq[sl].contiguous(), w[sl].contiguous(), q_seq[sl].contiguous(), nvis[sl].contiguous(), L)
        if fmt == "fp8":
            r = csa2.index_topk_fp8(*args, ik8, ik8e, seq_base, k=512, keep_blocks=2048)
        else:
            r = csa2.index_topk(*args, ik, seq_base, k=512, keep_blocks=2048)
        torch.cuda.synchronize()
        return r[0].cpu().numpy(), r[1].cpu().numpy()

    big_idx, big_pool = call(slice(0, n_q))
    for q0 in range(0, n_q, 100):
        sl = slice(q0, q0 + 100)
        i2, p2 = call(sl)
        assert np.array_equal(i2, big_idx[sl]), f"indices of queries {q0}..{q0 + 99} differ"
        assert np.array_equal(p2, big_pool[sl]), f"pools of queries {q0}..{q0 + 99} differ"
