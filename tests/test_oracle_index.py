"""Pins of the oracle's indexer score, Top-K, hierarchical pool and Reindex
(CPU only).  Exact integer cases, an fp64 error bound, brute-force sorting,
tie rules and the mode equivalences the CSA2 description implies."""
import numpy as np
import pytest
import torch

import oracle


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_score_exact_on_integer_inputs():
    # integers in [-3,3] and weights in {0, .5, 1}: every product, sum and
    # weighted sum is exact in fp32, so the score is a hand-computable integer.
    rng = np.random.default_rng(10)
    for h_i, d_i in [(4, 64), (64, 128), (3, 5)]:
        for _ in range(20):
            q = rng.integers(-3, 4, (h_i, d_i))
            k = rng.integers(-3, 4, d_i)
            w = rng.choice([0.0, 0.5, 1.0], h_i)
            exp = sum(w[h] * max(0, int(q[h] @ k)) for h in range(h_i))
            got = oracle.index_score(bf16(q), w.astype(np.float32), bf16(k))
            assert got == exp


def test_score_within_rounding_bound_of_fp64():
    rng = np.random.default_rng(11)
    h_i, d_i = 64, 128
    u = 2.0 ** -24
    g = lambda n: n * u / (1 - n * u)
    for _ in range(200):
        q = bf16(rng.standard_normal((h_i, d_i)))
        k = bf16(rng.standard_normal(d_i))
        w = rng.uniform(0, 1, h_i).astype(np.float32)
        qf, kf = bf16f(q).astype(np.float64), bf16f(k).astype(np.float64)
        dots = qf @ kf
        exact = float(np.sum(w.astype(np.float64) * np.maximum(dots, 0)))
        absdots = np.abs(qf) @ np.abs(kf)
        bound = float(np.sum(w * (g(d_i) * absdots))) + g(h_i) * float(np.sum(w * (np.maximum(dots, 0) + g(d_i) * absdots)))
        got = oracle.index_score(q, w, k)
        assert abs(got - exact) <= bound


def _brute_topk(scores, k, pos=None):
    n = len(scores)
    pos = np.arange(n) if pos is None else np.asarray(pos)
    order = np.lexsort((pos, -np.asarray(scores, np.float64)))
    sel = np.sort(pos[order[:min(k, n)]])
    return np.concatenate([sel, -np.ones(k - len(sel), np.int64)]).astype(np.int32)


@pytest.mark.parametrize("n", [0, 1, 7, 511, 512, 513, 4096])
def test_topk_matches_full_sort(n):
    rng = np.random.default_rng(n)
    s = rng.standard_normal(n).astype(np.float32)
    s[rng.integers(0, max(n, 1), n // 3)] = 0.25        # plenty of exact ties
    got = oracle.topk(s, 512)
    assert np.array_equal(got, _brute_topk(s, 512))
    keep = min(512, n)
    assert np.all(got[keep:] == -1) and np.all(np.diff(got[:keep]) > 0)
    if 0 < keep < n:   # every kept score >= every dropped score
        mask = np.zeros(n, bool)
        mask[got[:keep]] = True
        assert s[mask].min() >= s[~mask].max()


def test_topk_ties_go_to_lower_position_and_minus_zero_equals_zero():
    assert np.array_equal(oracle.topk(np.full(2000, 3.0, np.float32), 512), np.arange(512))
    s = np.zeros(1000, np.float32)
    s[::2] = -0.0
    assert np.array_equal(oracle.topk(s, 512), np.arange(512))
    # explicit positions: ties resolved by the position, not the list order
    s = np.array([1, 1, 1, 2], np.float32)
    pos = np.array([40, 10, 30, 20], np.int32)
    assert list(oracle.topk(s, 2, pos)) == [10, 20]


def _inputs(n_q, L, h_i=4, d_i=64, seed=0):
    rng = np.random.default_rng(seed)
    iq = bf16(rng.standard_normal((n_q, h_i, d_i)))
    w = rng.uniform(0, 1, (n_q, h_i)).astype(np.float32)
    ik = bf16(rng.standard_normal((n_q * L, d_i)))
    seq_base = np.arange(n_q, dtype=np.int64) * L
    return iq, w, np.arange(n_q, dtype=np.int32), np.full(n_q, L, np.int32), ik, seq_base


def test_full_is_topk_of_scores_with_zero_keys_and_equal_keys():
    iq, w, qs, nv, ik, sb = _inputs(1, 3000)
    ik[:] = 0                                           # every score is +0
    assert np.array_equal(oracle.index_topk(iq, w, qs, nv, ik, sb, 512)[0], np.arange(512))
    ik[:] = bf16(np.ones(64))                           # every key equal
    assert np.array_equal(oracle.index_topk(iq, w, qs, nv, ik, sb, 512)[0], np.arange(512))


def test_full_short_context_selects_everything():
    for L in (1, 7, 300, 512):
        iq, w, qs, nv, ik, sb = _inputs(2, L, seed=L)
        idx = oracle.index_topk(iq, w, qs, nv, ik, sb, 512)
        ref = np.concatenate([np.arange(L), -np.ones(512 - L)]).astype(np.int32)
        assert np.array_equal(idx[0], ref) and np.array_equal(idx[1], ref)


def test_full_matches_brute_force_sort():
    iq, w, qs, nv, ik, sb = _inputs(2, 2500, seed=3)
    idx = oracle.index_topk(iq, w, qs, nv, ik, sb, 512)
    for q in range(2):
        sc = [oracle.index_score(iq[q], w[q], ik[sb[q] + t]) for t in range(2500)]
        assert np.array_equal(idx[q], _brute_topk(sc, 512))


def test_duplicated_blocks_prefer_lower_positions():
    iq, w, qs, nv, ik, sb = _inputs(1, 2048, seed=4)
    ik[1024:2048] = ik[0:1024]                          # second half repeats the first
    idx = oracle.index_topk(iq, w, qs, nv, ik, sb, 512)[0]
    # a copy in the second half can only be chosen together with its original
    hi = idx[idx >= 1024]
    assert np.all(np.isin(hi - 1024, idx))


def test_pool_takes_every_block_when_few():
    iq, w, qs, nv, ik, sb = _inputs(2, 1000, seed=5)
    idx, pool = oracle.index_topk(iq, w, qs, nv, ik, sb, 512, block=8, keep_blocks=2048)
    nb = (1000 + 7) // 8
    ref = np.concatenate([np.arange(nb), -np.ones(2048 - nb)]).astype(np.int32)
    assert np.array_equal(pool[0], ref) and np.array_equal(pool[1], ref)
    # the pool covers the whole context, so Reindex with the Full layer's own
    # query reproduces Full bit for bit
    r = oracle.reindex_topk(iq, w, qs, nv, ik, sb, pool, 512, block=8)
    assert np.array_equal(r, idx)


def test_block_constant_keys_make_reindex_equal_full():
    # every block of 8 holds one key repeated, and keys, queries and weights are
    # small integers / halves so every dot product, sum and mean is exact: a
    # block then scores exactly as its members, the Top-512 tokens are the
    # members of the Top-64 blocks, all inside a 128-block pool, and Reindex
    # with the Full query reproduces Full.
    L, keep = 4096, 128
    rng = np.random.default_rng(6)
    ik = bf16(np.repeat(rng.integers(-3, 4, (L // 8, 64)), 8, axis=0))
    iq = bf16(rng.integers(-3, 4, (1, 4, 64)))
    w = rng.choice([0.0, 0.5, 1.0], (1, 4)).astype(np.float32)
    w[0, 0] = 1.0
    qs, nv, sb = np.zeros(1, np.int32), np.array([L], np.int32), np.zeros(1, np.int64)
    idx, pool = oracle.index_topk(iq, w, qs, nv, ik, sb, 512, block=8, keep_blocks=keep)
    bsc = [oracle.index_score(iq[0], w[0], ik[8 * b]) for b in range(L // 8)]
    assert np.array_equal(pool[0], _brute_topk(bsc, keep))
    tsc = [oracle.index_score(iq[0], w[0], ik[t]) for t in range(L)]
    assert np.array_equal(idx[0], _brute_topk(tsc, 512))
    assert np.all(np.isin(idx[0] // 8, pool[0]))
    r = oracle.reindex_topk(iq, w, qs, nv, ik, sb, pool, 512, block=8)
    assert np.array_equal(r, idx)


def test_pool_block_mean_and_partial_last_block():
    # hand-made keys: block 0 = keys 1..8 times e_0 (mean 4.5), a partial last
    # block of 3 tokens (mean of 2, 4, 9 = 5).  With one head, q = e_0 and w = 1,
    # the block score is the mean itself.
    d_i = 64
    L = 8 * 3 + 3
    ik = np.zeros((L, d_i), np.float32)
    ik[0:8, 0] = np.arange(1, 9)
    ik[8:16, 0] = -1.0
    ik[16:24, 0] = 0.5
    ik[24:27, 0] = [2, 4, 9]
    iq = np.zeros((1, 1, d_i), np.float32)
    iq[0, 0, 0] = 1
    _, pool = oracle.index_topk(bf16(iq), np.ones((1, 1), np.float32), np.zeros(1, np.int32),
                                np.array([L], np.int32), bf16(ik), np.zeros(1, np.int64), 4,
                                block=8, keep_blocks=2)
    assert list(pool[0]) == [0, 3]     # scores 4.5, 0, 0.5, 5 -> blocks 3 and 0


def test_block_score_below_member_mean_jensen():
    # ReLU is convex and w >= 0, so a block's score (the score of its mean
    # key) is at most the mean of its members' scores, up to fp32 rounding.
    rng = np.random.default_rng(7)
    h_i, d_i = 8, 64
    for _ in range(50):
        iq = bf16(rng.standard_normal((1, h_i, d_i)))
        w = rng.uniform(0, 1, (1, h_i)).astype(np.float32)
        keys = bf16(rng.standard_normal((8, d_i)))
        member = [oracle.index_score(iq[0], w[0], keys[j]) for j in range(8)]
        _, pool = oracle.index_topk(iq, w, np.zeros(1, np.int32), np.array([8], np.int32), keys,
                                    np.zeros(1, np.int64), 1, block=8, keep_blocks=1)
        assert pool[0, 0] == 0
        # the block score itself, by the exact-arithmetic definition, in fp64
        qf, kf = bf16f(iq[0]).astype(np.float64), bf16f(keys).astype(np.float64)
        bs = float(np.sum(w[0] * np.maximum(qf @ kf.mean(axis=0), 0)))
        assert bs <= np.mean(member) + 1e-4


def test_block_score_is_mean_of_member_dots():
    # the oracle's block scores, read back through a pool of every block,
    # against the same definition evaluated in fp64: equal to rounding error
    rng = np.random.default_rng(17)
    h_i, d_i, L = 16, 64, 8 * 40 + 5
    iq = bf16(rng.standard_normal((1, h_i, d_i)))
    w = rng.uniform(0, 1, (1, h_i)).astype(np.float32)
    ik = bf16(rng.standard_normal((L, d_i)))
    qf, kf = bf16f(iq[0]).astype(np.float64), bf16f(ik).astype(np.float64)
    exact = []
    for b in range(41):
        blk = kf[8 * b:min(L, 8 * b + 8)]
        exact.append(float(np.sum(w[0] * np.maximum(qf @ blk.mean(axis=0), 0))))
    # order of the 41 blocks by the fp64 definition must match the oracle's
    # Top-k for every k (no near-ties at this seed)
    order = np.argsort(-np.array(exact), kind="stable")
    for k in (1, 5, 20, 40):
        _, pool = oracle.index_topk(iq, w, np.zeros(1, np.int32), np.array([L], np.int32), ik,
                                    np.zeros(1, np.int64), 1, block=8, keep_blocks=k)
        assert np.array_equal(pool[0], np.sort(order[:k]))


def test_reindex_uses_only_pool_positions_and_visibility():
    iq, w, qs, nv, ik, sb = _inputs(1, 200, seed=8)
    pool = np.array([[3, 7, 24, -1]], np.int32)          # block 24 = positions 192..199
    nv = np.array([197], np.int32)                       # 195 is the last visible position
    r = oracle.reindex_topk(iq, w, qs, nv, ik, sb, pool, 64, block=8)[0]
    cand = list(range(24, 32)) + list(range(56, 64)) + list(range(192, 197))
    assert np.array_equal(r, np.concatenate([cand, -np.ones(64 - len(cand))]).astype(np.int32))
    r = oracle.reindex_topk(iq, w, qs, nv, ik, sb, pool, 5, block=8)[0]
    sc = [oracle.index_score(iq[0], w[0], ik[p]) for p in cand]
    assert np.array_equal(r, _brute_topk(sc, 5, cand))


# ---------------------------------------------------------------- pool-based Full variant
def _kb(ik, lens, block=8, blk_from=None, max_blocks=None, kbar=None):
    lens = np.asarray(lens, np.int32)
    sb = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    nb = (lens.astype(np.int64) + block - 1) // block
    kbb = np.concatenate([[0], np.cumsum(nb)[:-1]]).astype(np.int64)
    if kbar is None:
        kbar = np.full((int(nb.sum()), ik.shape[1]), 0xFFFF, np.uint16)
    oracle.block_keys(ik, sb, lens, kbar, kbb, blk_from=blk_from, block=block, max_blocks=max_blocks)
    return kbar, kbb


def test_block_keys_hand_worked_rounding():
    # one dimension, one block of 8 (values exact in bf16):
    #   1..8                 -> 36/8 = 4.5 (exact)
    #   seven 1s and 2^-7    -> (7 + 2^-7)/8 = 0.8759765625: bf16 keeps 8 significant
    #                           bits, the rest 0.01b is below half -> 0.875
    #   seven 1s and 1+2^-5  -> 1 + 2^-8, halfway between 1 and 1 + 2^-7 -> even: 1
    #   seven 1s and 1+3*2^-5 -> 1 + 3*2^-8, halfway between 1 + 2^-7 and 1 + 2^-6 -> even: 1 + 2^-6
    cases = [(np.arange(1, 9), 4.5), ([1] * 7 + [2 ** -7], 0.875), ([1] * 7 + [1 + 2 ** -5], 1.0),
             ([1] * 7 + [1 + 3 * 2 ** -5], 1 + 2 ** -6)]
    for vals, exp in cases:
        ik = bf16(np.asarray(vals, np.float64)[:, None])
        kbar, _ = _kb(ik, [8])
        assert bf16f(kbar)[0, 0] == np.float32(exp)
    # a partial last block: 3 members, mean of 2, 4, 9 = 5; of 1, 1, 2 = 4/3 -> fp32 quotient, then bf16
    ik = bf16(np.array([[1.0]] * 8 + [[2.0], [4.0], [9.0]]))
    kbar, _ = _kb(ik, [11])
    assert bf16f(kbar)[1, 0] == 5.0
    ik = bf16(np.array([[1.0], [1.0], [2.0]]))
    kbar, _ = _kb(ik, [3])
    assert bf16f(kbar)[0, 0] == bf16f(bf16(np.float32(4.0) / np.float32(3.0)))[()]


def test_block_keys_match_exact_mean_when_sums_are_exact():
    # magnitudes in [2^-6, 8): eight bf16 values then sum exactly in fp32, so the
    # stored key must be the nearest-even bf16 of the exact mean (a single
    # rounding, done here by torch from the exact fp32 mean)
    rng = np.random.default_rng(20)
    lens = [8 * 37, 8 * 5 + 3, 1, 8]
    L = sum(lens)
    mag = np.exp2(rng.uniform(-6, 3, (L, 64)))
    ik = bf16(np.where(rng.random((L, 64)) < 0.5, -mag, mag))
    kbar, kbb = _kb(ik, lens)
    x = bf16f(ik).astype(np.float64)
    t0 = 0
    for s, n in enumerate(lens):
        for b in range((n + 7) // 8):
            rows = x[t0 + 8 * b: t0 + min(n, 8 * b + 8)]
            exact = rows.sum(axis=0) / len(rows)            # exact in fp64 for these inputs
            if len(rows) == 8:
                exp = bf16(exact.astype(np.float32))          # exact mean is an fp32 value: one rounding
            else:
                exp = bf16(rows.sum(axis=0).astype(np.float32) / np.float32(len(rows)))
            assert np.array_equal(kbar[kbb[s] + b], exp)
        t0 += n


def test_block_keys_range_updates_only_named_blocks():
    rng = np.random.default_rng(21)
    lens = [100, 37]
    ik = bf16(rng.standard_normal((sum(lens), 64)))
    full, kbb = _kb(ik, lens)
    part = np.full_like(full, 0x1234)
    _kb(ik, lens, blk_from=[12, 2], max_blocks=1, kbar=part)
    for s, b in [(0, 12), (1, 2)]:
        assert np.array_equal(part[kbb[s] + b], full[kbb[s] + b])
    touched = {int(kbb[0] + 12), int(kbb[1] + 2)}
    for r in range(len(part)):
        if r not in touched:
            assert np.all(part[r] == 0x1234)
    # blocks past a sequence's end are never written
    part2 = np.full_like(full, 0x1234)
    _kb(ik, lens, blk_from=[13, 5], max_blocks=4, kbar=part2)
    assert np.all(part2 == 0x1234)


def _pool_inputs(n_q, L, seed, h_i=4, d_i=64):
    iq, w, qs, nv, ik, sb = _inputs(n_q, L, h_i, d_i, seed)
    kbar, kbb = _kb(ik, [L] * n_q)
    return iq, w, qs, nv, ik, sb, kbar, kbb


def test_pool_full_equals_full_when_pool_covers_context():
    for L in (1, 500, 4096):
        iq, w, qs, nv, ik, sb, kbar, kbb = _pool_inputs(2, L, seed=L)
        idx, pool = oracle.pool_full_topk(iq, w, qs, nv, ik, sb, kbar, kbb, 512, 512)
        nb = (L + 7) // 8
        assert np.array_equal(pool[0], np.concatenate([np.arange(nb), -np.ones(512 - nb)]).astype(np.int32))
        assert np.array_equal(idx, oracle.index_topk(iq, w, qs, nv, ik, sb, 512))


def test_pool_full_equals_full_with_block_constant_keys():
    # a block's stored key is then its members' key, so the block scores as its
    # members; the Top-512 tokens fill the Top-64 blocks, which every pool of
    # at least 64 blocks contains
    L, keep = 6000, 100
    rng = np.random.default_rng(22)
    ik = bf16(np.repeat(rng.standard_normal((L // 8, 64)), 8, axis=0))
    iq = bf16(rng.standard_normal((2, 4, 64)))
    w = rng.uniform(0, 1, (2, 4)).astype(np.float32)
    qs, nv, sb = np.zeros(2, np.int32), np.full(2, L, np.int32), np.zeros(1, np.int64)
    kbar, kbb = _kb(ik, [L])
    assert np.array_equal(kbar, ik[::8])
    idx, pool = oracle.pool_full_topk(iq, w, qs, nv, ik, sb, kbar, kbb, 512, keep)
    assert np.array_equal(idx, oracle.index_topk(iq, w, qs, nv, ik, sb, 512))


def test_pool_full_matches_brute_force():
    L, keep, k = 1003, 40, 64
    iq, w, qs, nv, ik, sb, kbar, kbb = _pool_inputs(2, L, seed=23)
    nv = np.array([L, 777], np.int32)          # the second query sees a shorter prefix
    # the second query's blocks: its own prefix of 777 positions (a partial block at the end)
    kbar2, kbb2 = _kb(ik[sb[1]:sb[1] + 777], [777])
    idx, pool = oracle.pool_full_topk(iq[1:], w[1:], np.zeros(1, np.int32), nv[1:], ik[sb[1]:], np.zeros(1, np.int64),
                                      kbar2, kbb2, k, keep)
    # block keys are pinned by the tests above; this checks the selection built on them
    bsc = [oracle.index_score(iq[1], w[1], kbar2[b]) for b in range(98)]
    ref_pool = _brute_topk(bsc, keep)
    assert np.array_equal(pool[0], ref_pool)
    pos = np.array([8 * b + o for b in ref_pool if b >= 0 for o in range(8) if 8 * b + o < 777])
    tsc = [oracle.index_score(iq[1], w[1], ik[sb[1] + p]) for p in pos]
    assert np.array_equal(idx[0], _brute_topk(tsc, k, pos))


def test_sharded_topk_merge_equals_full_context():
    # a context split into position ranges: the Top-K among the union of the
    # shards' local Top-Ks (rescored, positions kept) is the whole context's
    # Top-K, ties included (the score of a position does not depend on the
    # shard).  Brute-force merge over the oracle's own per-shard selections.
    iq, w, qs, nv, ik, sb = _inputs(1, 5000, seed=24)
    ik[1000:1500] = ik[3000:3500]                       # ties across shards
    full = oracle.index_topk(iq, w, qs, nv, ik, sb, 512)[0]
    for G in (2, 3, 7):
        edges = np.linspace(0, 5000, G + 1).astype(int)
        cand = []
        for a, b in zip(edges[:-1], edges[1:]):
            loc = oracle.index_topk(iq, w, np.zeros(1, np.int32), np.array([b - a], np.int32), ik[a:b],
                                    np.zeros(1, np.int64), 512)[0]
            cand.extend(int(a + p) for p in loc if p >= 0)
        cand = np.array(cand, np.int32)
        sc = [oracle.index_score(iq[0], w[0], ik[p]) for p in cand]
        assert np.array_equal(oracle.topk(np.array(sc, np.float32), 512, cand), full)


def test_block_score_function_special_cases():
    # a block of one member scores exactly as that member (sum from +0 of one
    # dot, divided by 1); a block of n equal integer-valued members scores as
    # each member (the sum and the division by n are exact); random blocks lie
    # within the fp32 rounding bound of the fp64 mean-of-dots definition
    rng = np.random.default_rng(25)
    h_i, d_i = 8, 64
    for _ in range(20):
        iq = bf16(rng.standard_normal((h_i, d_i)))
        w = rng.uniform(0, 1, h_i).astype(np.float32)
        k1 = bf16(rng.standard_normal((1, d_i)))
        assert oracle.block_score(iq, w, k1) == oracle.index_score(iq, w, k1[0])
        qi = bf16(rng.integers(-3, 4, (h_i, d_i)))
        wi = rng.choice([0.0, 0.5, 1.0], h_i).astype(np.float32)
        ki = bf16(rng.integers(-3, 4, (1, d_i)))
        for n in (2, 3, 5, 8):
            assert oracle.block_score(qi, wi, np.repeat(ki, n, axis=0)) == oracle.index_score(qi, wi, ki[0])
        keys = bf16(rng.standard_normal((8, d_i)))
        qf, kf = bf16f(iq).astype(np.float64), bf16f(keys).astype(np.float64)
        dots = qf @ kf.T                                 # [h_i, 8]
        exact = float(np.sum(w * np.maximum(dots.mean(axis=1), 0)))
        u = 2.0 ** -24
        g = lambda m: m * u / (1 - m * u)
        absdots = (np.abs(qf) @ np.abs(kf).T).mean(axis=1)
        bound = float(np.sum(w * ((g(d_i) + g(8) + u) * absdots))) * (1 + g(h_i)) + g(h_i) * exact
        assert abs(oracle.block_score(iq, w, keys) - exact) <= bound
