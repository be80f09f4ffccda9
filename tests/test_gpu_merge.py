"""csa2_topk_merge on the GPU: the merge step of a context split over several
devices.  Each shard's local Top-K (csa2_index_topk on its position range),
offset to global positions and concatenated, merged on the GPU, equals the
oracle's Top-K over the whole context bit for bit; an arbitrary candidate set
gives the oracle's Top-K among those candidates; empty and short lists pad."""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, index_inputs, note, to_dev


def _shard_lists(d, L, G, k):
    """Local Top-K of every shard of one sequence of length L at global positions."""
    edges = np.linspace(0, L, G + 1).astype(np.int64)
    lists = []
    for a, b in zip(edges[:-1], edges[1:]):
        n_q = d["iq"].shape[0]
        loc = csa2.index_topk(d["iq"], d["w"], torch.zeros(n_q, dtype=torch.int32, device=d["iq"].device),
                              torch.full((n_q,), int(b - a), dtype=torch.int32, device=d["iq"].device), int(b - a),
                              d["ik"], torch.tensor([int(a)], dtype=torch.int64, device=d["iq"].device), k=k)
        lists.append(torch.where(loc >= 0, loc + int(a), loc))
    return lists


@gpu
@pytest.mark.parametrize("L,G,h_i,d_i", [(200000, 8, 64, 128), (70001, 3, 4, 64), (1500, 4, 64, 128)])
def test_sharded_context_merges_to_the_full_topk(L, G, h_i, d_i):
    dev = device()
    note(f"topk merge: L={L} G={G} h_i={h_i} d_i={d_i}")
    k = 512
    inp = index_inputs([L], h_i, d_i, seed=700 + G)
    # three queries over the same sequence
    inp["iq"] = torch.cat([inp["iq"], index_inputs([1], h_i, d_i, seed=701)["iq"],
                           index_inputs([1], h_i, d_i, seed=702)["iq"]])
    inp["w"] = torch.cat([inp["w"]] * 3)
    d = to_dev(inp, dev)
    lists = _shard_lists(d, L, G, k)
    # valid entries first (ascending: shards in order), then -1 padding
    cat = torch.cat(lists, dim=1).cpu().numpy()
    cand = np.full_like(cat, -1)
    for i in range(cat.shape[0]):
        v = cat[i][cat[i] >= 0]
        cand[i, :len(v)] = v
    q_seq = torch.zeros(3, dtype=torch.int32, device=dev)
    got = csa2.topk_merge(d["iq"], d["w"], q_seq, d["ik"], d["seq_base"][:1], torch.from_numpy(cand).to(dev), k=k)
    torch.cuda.synchronize()
    ref = oracle.index_topk(bits(inp["iq"]), inp["w"].numpy(), np.zeros(3, np.int32), np.full(3, L, np.int32),
                            bits(inp["ik"]), np.zeros(1, np.int64), k)
    assert np.array_equal(got.cpu().numpy(), ref)


@gpu
@pytest.mark.parametrize("n_cand", [2000, 20000])
def test_merge_of_arbitrary_candidates_ties_and_padding(n_cand):
    """2000 candidates take the one-work-group select, 20000 (over 16,384) the
    multi-kernel one; both must give the oracle's Top-K among the candidates."""
    dev = device()
    note(f"topk merge: arbitrary candidates n_cand={n_cand}")
    L, k = 30000, 300
    inp = index_inputs([L, L], 64, 128, seed=710)
    inp["ik"][5000:6000] = inp["ik"][9000:10000]        # equal keys: ties resolve by position
    rng = np.random.default_rng(711)
    cand = np.full((2, n_cand), -1, np.int32)
    cand[0] = np.sort(rng.choice(L, n_cand, replace=False))
    short = np.sort(rng.choice(np.arange(4000, 11000), 250, replace=False))   # fewer than k candidates
    cand[1, :250] = short
    d = to_dev(inp, dev)
    got = csa2.topk_merge(d["iq"], d["w"], d["q_seq"], d["ik"], d["seq_base"], torch.from_numpy(cand).to(dev), k=k)
    empty = csa2.topk_merge(d["iq"], d["w"], d["q_seq"], d["ik"], d["seq_base"],
                            torch.empty((2, 0), dtype=torch.int32, device=dev), k=k)
    torch.cuda.synchronize()
    ikb, iqb, w = bits(inp["ik"]), bits(inp["iq"]), inp["w"].numpy()
    for i in range(2):
        c = cand[i][cand[i] >= 0]
        sc = np.array([oracle.index_score(iqb[i], w[i], ikb[i * L + p]) for p in c], np.float32)
        assert np.array_equal(got[i].cpu().numpy(), oracle.topk(sc, k, c)), f"query {i}"
    assert np.all(empty.cpu().numpy() == -1)
