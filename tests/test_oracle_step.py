"""Pins of the oracle's decode-step sequencing and of the score's summation
order (CPU only).

A CSA2 decoder step runs its layers in a fixed order: the Full layer indexes
the whole context and builds the block pool, a Reindex layer re-scores that
pool with its own indexer query, and every Reuse layer takes the Top-K list
of its group's head (Full or Reindex) and attends with its own query and
window rows (page "DeepSeek AI выпустила DeepSeek-V4.1-Flash ..."
(wire.sakhanda.co), section "Сжатое разреженное внимание 2 (CSA2)").  The
step driver ``oracle.step.decode_step`` is checked here layer by layer
against direct calls of the oracle's single-layer functions over a whole,
uncompacted cache, on a schedule where each mode gives a different list.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle.step import decode_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    x = np.ascontiguousarray(x, np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16           # nearest-even (finite inputs)
    return b.astype(np.uint16)


def _decoder_schedule():
    return ["full", "reuse", "reuse", "reuse"] + ["reindex", "reuse", "reuse", "reuse"] * 4


def _step_inputs(seed, lengths, h_i=4, d_i=64, h=2, W=16, block_constant=False, shared_iq=False):
    rng = np.random.default_rng(seed)
    rows = int(sum(lengths))
    seq_base = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    n_q = len(lengths)
    if block_constant:
        ik = _bf16(np.repeat(rng.standard_normal(((rows + 7) // 8, d_i)), 8, axis=0)[:rows])
        # every sequence starts on a block boundary for this layout
        assert all(b % 8 == 0 for b in seq_base)
    else:
        ik = _bf16(rng.standard_normal((rows, d_i)))
    raw = _bf16(rng.standard_normal((rows, 512)))
    layers = []
    iq0 = w0 = None
    for li, mode in enumerate(_decoder_schedule()):
        lay = dict(mode=mode, q=_bf16(rng.standard_normal((n_q, h, 512))),
                   swa=_bf16(rng.standard_normal((n_q * W, 512))),
                   swa_row0=np.arange(n_q, dtype=np.int64) * W,
                   swa_len=np.array([min(W, L) for L in lengths], np.int32))
        if li % 3 == 1:
            # this step's new window row of every sequence enters its ring
            lay["swa_new"] = _bf16(rng.standard_normal((n_q, 512)))
            lay["swa_dst"] = np.array([i * W + (L - 1) % W for i, L in enumerate(lengths)], np.int64)
        if mode in ("full", "reindex"):
            if shared_iq and mode == "reindex":
                lay["iq"], lay["w"] = iq0, w0
            else:
                lay["iq"] = _bf16(rng.standard_normal((n_q, h_i, d_i)))
                lay["w"] = rng.uniform(0, 1, (n_q, h_i)).astype(np.float32)
            if mode == "full":
                iq0, w0 = lay["iq"], lay["w"]
        layers.append(lay)
    return dict(ik=ik, raw=raw, seq_base=seq_base, q_seq=np.arange(n_q, dtype=np.int32),
                q_nvis=np.asarray(lengths, np.int32), layers=layers)


def _run_step(inp, k, keep_blocks):
    return decode_step(inp["layers"], inp["ik"], inp["seq_base"], inp["q_seq"], inp["q_nvis"], k, keep_blocks, 8,
                       lambda r: inp["raw"][np.asarray(r, np.int64)], None, 512 ** -0.5)


def test_decode_step_full_reindex_reuse_sequencing():
    # 2 sequences of about 3000 positions, a 64-block pool (512 positions) and
    # Top-100, so the pool is a strict subset of the context and a Reindex
    # layer's choice inside it differs from the Full layer's
    lengths, k, keep = [3001, 2777], 100, 64
    inp = _step_inputs(31, lengths)
    res, pool, _ = _run_step(inp, k, keep)
    assert len(res) == 20
    lay, ik, sb, qs, nv = inp["layers"], inp["ik"], inp["seq_base"], inp["q_seq"], inp["q_nvis"]
    # Full: the whole context, and the pool it builds
    full_idx, full_pool = oracle.index_topk(lay[0]["iq"], lay[0]["w"], qs, nv, ik, sb, k, block=8,
                                            keep_blocks=keep)
    assert np.array_equal(res[0][0], full_idx)
    assert np.array_equal(pool, full_pool)
    cache = oracle.quantize_rows(inp["raw"])           # the whole FP4 cache, uncompacted
    heads = {}
    for li, (idx, out, lse) in enumerate(res):
        mode = lay[li]["mode"]
        if mode == "reindex":
            # its own indexer query over the Full layer's pool (read from the
            # Full layer, not from the previous Reindex layer)
            ref = oracle.reindex_topk(lay[li]["iq"], lay[li]["w"], qs, nv, ik, sb, full_pool, k, block=8)
            assert np.array_equal(idx, ref), f"layer {li}"
            assert not np.array_equal(idx, full_idx), "schedule not discriminating"
            for prev in heads.values():
                assert not np.array_equal(idx, prev), "schedule not discriminating"
            # every chosen position lies in a pool block
            for q in range(len(lengths)):
                sel = idx[q][idx[q] >= 0]
                assert np.all(np.isin(sel // 8, full_pool[q]))
        group_head = 4 * (li // 4)
        if mode in ("full", "reindex"):
            heads[li] = idx
        else:
            # a Reuse layer takes its own group head's list
            assert np.array_equal(idx, heads[group_head]), f"layer {li}"
        # every layer attends with its own query and window over the list it holds
        swa = lay[li]["swa"]
        if "swa_new" in lay[li]:
            swa = swa.copy()
            swa[lay[li]["swa_dst"]] = lay[li]["swa_new"]
        ro, rl = oracle.sparse_attn(lay[li]["q"], qs, cache, sb, heads[group_head], swa, lay[li]["swa_row0"],
                                    lay[li]["swa_len"], 512 ** -0.5)
        assert np.array_equal(out, ro) and np.array_equal(lse, rl), f"layer {li}"


def test_decode_step_reindex_with_full_query_on_block_constant_keys_repeats_full():
    # keys constant over each block of 8: a block scores as its members, the
    # Top-k positions fill the best k/8 blocks, which the pool holds; so a
    # Reindex layer that uses the Full layer's own indexer query reproduces
    # the Full list, and every layer of the step holds the same list
    lengths, k, keep = [4096, 2048], 64, 32
    inp = _step_inputs(32, lengths, block_constant=True, shared_iq=True)
    res, pool, _ = _run_step(inp, k, keep)
    for li, (idx, _, _) in enumerate(res):
        assert np.array_equal(idx, res[0][0]), f"layer {li}"
    assert np.all(np.isin(res[0][0][0] // 8, pool[0]))


def _golden_scores():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "score_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            v = val.split()
            if key == "case":
                cur = dict(name=v[0], h_i=int(v[1]), d_i=int(v[2]))
                cases.append(cur)
            elif key in ("q", "k"):
                cur[key] = np.array([int(x, 16) for x in v], np.uint16)
            elif key == "w":
                cur["w"] = np.array([int(x, 16) for x in v], np.uint32).view(np.float32)
            elif key == "score":
                cur["score"] = int(v[0], 16)
    return cases


def _f(bits16):
    return (np.asarray(bits16, np.uint32) << 16).view(np.float32)


def _chain(terms):
    acc = np.float32(0.0)
    for t in terms:
        acc = np.float32(acc + np.float32(t))      # each product here is exact in fp32
    return acc


@pytest.mark.parametrize("case", _golden_scores(), ids=lambda c: c["name"])
def test_score_summation_order_hand_worked(case):
    q = case["q"].reshape(case["h_i"], case["d_i"])
    got = np.float32(oracle.index_score(q, case["w"], case["k"]))
    assert got.view(np.uint32) == case["score"]
    # the golden value discriminates the order: the reversed order of the
    # chain at fault, and the exact sum, give other bits
    qf, kf, w = _f(q), _f(case["k"]), case["w"]
    prods = qf * kf[None, :]
    if case["h_i"] == 1:
        orders = list(itertools.permutations(range(case["d_i"])))
        rev = _chain(prods[0][::-1]) * w[0]
        exact = np.float32(np.sum(prods[0].astype(np.float64)))
    else:
        relu = np.maximum(prods.sum(axis=1), 0) * w
        orders = list(itertools.permutations(range(case["h_i"])))
        rev = _chain(relu[::-1])
        exact = np.float32(np.sum(relu.astype(np.float64)))
    assert rev.view(np.uint32) != case["score"] and exact.view(np.uint32) != case["score"]
    terms = prods[0] if case["h_i"] == 1 else relu
    n_diff = sum(_chain(terms[list(o)]).view(np.uint32) != case["score"] for o in orders)
    assert n_diff > 0
