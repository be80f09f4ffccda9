"""Pins of the oracle's sparse attention (CPU only): equality with the textbook
dense softmax when every entry is selected, degenerate queries, permutation
invariance, the split-and-merge identity, and the Reuse plumbing."""
import numpy as np
import torch

import oracle


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _setup(L=40, h=3, nw=0, seed=0, qdt="f32"):
    rng = np.random.default_rng(seed)
    cache = oracle.quantize_rows(rng.standard_normal((L, 512)).astype(np.float32))
    q = rng.standard_normal((1, h, 512)).astype(np.float32)
    if qdt == "bf16":
        q = bf16(q)
    swa = bf16(rng.standard_normal((max(nw, 1), 512)))
    return cache, q, swa


def _textbook(qf, K, scale):
    """softmax(scale * q K^T) K in float64 (K = V)."""
    z = scale * (qf.astype(np.float64) @ K.T.astype(np.float64))
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ K.astype(np.float64)


def _call(q, cache, idx, swa, swa_len, scale=0.05):
    n_q = q.shape[0]
    return oracle.sparse_attn(q, np.zeros(n_q, np.int32), cache, np.zeros(1, np.int64),
                              np.atleast_2d(idx).astype(np.int32), swa, np.zeros(n_q, np.int64),
                              np.array([swa_len] * n_q, np.int32), scale)


def test_dense_equality_when_all_entries_selected():
    L = 40
    cache, q, swa = _setup(L)
    idx = np.concatenate([np.arange(L), -np.ones(24)])
    out, lse = _call(q, cache, idx, swa, 0)
    K = oracle.dequant_records(cache)
    ref = _textbook(q[0], K, 0.05)
    assert np.max(np.abs(out[0] - ref)) <= 1e-6 * np.max(np.abs(ref))
    z = 0.05 * (q[0].astype(np.float64) @ K.T.astype(np.float64))
    lse_ref = z.max(1) + np.log(np.exp(z - z.max(1, keepdims=True)).sum(1))
    assert np.allclose(lse[0], lse_ref, rtol=1e-6)


def test_window_rows_join_the_same_softmax():
    L, nw = 20, 7
    cache, q, swa = _setup(L, nw=nw, seed=1, qdt="bf16")
    out, _ = _call(q, cache, np.arange(L), swa, nw)
    K = np.concatenate([oracle.dequant_records(cache), bf16f(swa[:nw])])
    ref = _textbook(bf16f(q[0]), K, 0.05)
    assert np.max(np.abs(out[0] - ref)) <= 1e-6 * np.max(np.abs(ref))
    # window only (no main entry selected)
    out2, _ = _call(q, cache, -np.ones(8), swa, nw)
    ref2 = _textbook(bf16f(q[0]), bf16f(swa[:nw]), 0.05)
    assert np.max(np.abs(out2[0] - ref2)) <= 1e-6 * np.max(np.abs(ref2))


def test_zero_query_gives_mean_and_single_entry_gives_row():
    L = 30
    cache, q, swa = _setup(L, nw=4, seed=2)
    K = oracle.dequant_records(cache)
    sel = np.array([3, 9, 17, -1, 25])
    out, _ = _call(np.zeros_like(q), cache, sel, swa, 4)
    mean = np.concatenate([K[[3, 9, 17, 25]], bf16f(swa[:4])]).astype(np.float64).mean(0)
    assert np.allclose(out[0], mean[None, :], rtol=0, atol=1e-6 * np.abs(mean).max())
    out, lse = _call(q, cache, np.array([11, -1, -1]), swa, 0)
    assert np.array_equal(out[0], np.broadcast_to(K[11], out[0].shape))


def test_no_valid_key_gives_zero_and_minus_inf():
    cache, q, swa = _setup(5)
    out, lse = _call(q, cache, -np.ones(4), swa, 0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_permuting_selection_does_not_change_output():
    cache, q, swa = _setup(64, nw=5, seed=3)
    rng = np.random.default_rng(0)
    sel = rng.choice(64, 40, replace=False)
    a, la = _call(q, cache, sel, swa, 5)
    b, lb = _call(q, cache, rng.permutation(sel), swa, 5)
    assert np.max(np.abs(a - b)) <= 1e-6 * np.abs(a).max() and np.allclose(la, lb, rtol=1e-7)


def test_split_and_merge_equals_unsplit():
    cache, q, swa = _setup(64, nw=6, seed=4)
    sel = np.arange(0, 64, 2)
    full, lf = _call(q, cache, sel, swa, 6)
    o1, l1 = _call(q, cache, sel[:10], swa, 0)
    o2, l2 = _call(q, cache, sel[10:], swa, 6)
    m = np.maximum(l1, l2)[..., None].astype(np.float64)
    a1, a2 = np.exp(l1[..., None] - m), np.exp(l2[..., None] - m)
    merged = (a1 * o1 + a2 * o2) / (a1 + a2)
    assert np.max(np.abs(merged - full)) <= 1e-5 * np.abs(full).max()


def test_reuse_layer_is_the_same_call_with_inherited_indices():
    # A Reuse layer keeps its own q and window rows and takes the Top-K list of
    # its group's head layer: with the same q it reproduces that layer exactly.
    cache, q, swa = _setup(50, nw=3, seed=5)
    sel = np.array([1, 5, 8, 13, 40])
    a, la = _call(q, cache, sel, swa, 3)
    b, lb = _call(q, cache, sel.copy(), swa, 3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_sequences_and_rows_are_addressed_through_seq_base():
    rng = np.random.default_rng(6)
    cache = oracle.quantize_rows(rng.standard_normal((100, 512)).astype(np.float32))
    q = rng.standard_normal((2, 2, 512)).astype(np.float32)
    swa = bf16(rng.standard_normal((10, 512)))
    idx = np.array([[0, 1, 2], [0, 1, 2]], np.int32)
    out, _ = oracle.sparse_attn(q, np.array([1, 0], np.int32), cache, np.array([0, 60], np.int64),
                                idx, swa, np.array([4, 0], np.int64), np.array([2, 3], np.int32), 0.05)
    K = oracle.dequant_records(cache)
    r0 = _textbook(q[0], np.concatenate([K[60:63], bf16f(swa[4:6])]), 0.05)
    r1 = _textbook(q[1], np.concatenate([K[0:3], bf16f(swa[0:3])]), 0.05)
    assert np.allclose(out[0], r0, atol=1e-6) and np.allclose(out[1], r1, atol=1e-6)
