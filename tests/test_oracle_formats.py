"""Pins of the oracle's number formats and FP4 quantiser (CPU only).

Each test checks the oracle against something other than itself: hand-written
golden tables (tests/golden, each with its source), torch's own float8/bf16
conversions, exact rational brute force, and invariants of the format.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def test_e2m1_table_matches_golden():
    got = {}
    for line in _rows("e2m1_values.txt"):
        c, v = line.split()
        got[int(c)] = float(v)
    assert sorted(got) == list(range(16))
    for c, v in got.items():
        o = oracle.e2m1_value(c)
        assert o == v and math.copysign(1, o) == math.copysign(1, v), (c, o, v)
    mags = sorted({abs(oracle.e2m1_value(c)) for c in range(16)})
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_anchors_match_golden():
    for line in _rows("e4m3_anchors.txt"):
        c, v = line.split()
        o = oracle.e4m3_value(int(c, 16))
        if v == "nan":
            assert math.isnan(o)
        else:
            assert o == float(v) and math.copysign(1, o) == math.copysign(1, float(v)), (c, o, v)


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        o = oracle.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(o), c
        else:
            assert o == ref[c] and math.copysign(1, o) == math.copysign(1, ref[c]), c


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),        # subnormals
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half an ulp (low 16 bits = 0x8000)
        (rng.integers(0, 2**31, 3000, dtype=np.uint32) & 0xFFFF0000 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], dtype=np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits(x)
    assert np.array_equal(got, ref)


def _e4m3_pos_values():
    return [Fraction(oracle.e4m3_value(c)) for c in range(127)]


def _nearest_even(q, values):
    """Index of the value nearest to q; ties to the even index; saturate at the end."""
    best = None
    for i, v in enumerate(values):
        d = abs(q - v)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_scale_rounding_matches_torch_float8():
    # torch rounds fp32 -> float8_e4m3fn nearest-even; below 464 it does not
    # reach NaN, so it must agree with the oracle's scale rule on amax/6.
    rng = np.random.default_rng(2)
    amax = np.concatenate([
        np.abs(rng.standard_normal(20000)) * 10,
        np.abs(rng.standard_normal(5000)) * 1e-2,
        rng.uniform(0, 2780, 5000),
    ]).astype(np.float32)
    q = (torch.from_numpy(amax) / 6.0)
    keep = q < 464
    ref = q[keep].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_round_scale(a) for a in amax[keep.numpy()]], dtype=np.uint8)
    assert np.array_equal(got, ref)
    # beyond the largest finite value the scale saturates at 448
    for a in [2688.0, 2700.0, 2784.0, 1e6, 3e38]:
        assert oracle.e4m3_round_scale(a) == 0x7E


def test_scale_rounding_exact_rational():
    vals = _e4m3_pos_values()
    rng = np.random.default_rng(3)
    mids = [(vals[i] + vals[i + 1]) / 2 * 6 for i in range(126)]
    cand = [float(m) for m in mids] + list(np.abs(rng.standard_normal(3000)).astype(np.float32) * 50)
    for a in cand:
        a = float(np.float32(a))
        exp = _nearest_even(Fraction(a) / 6, vals)
        assert oracle.e4m3_round_scale(a) == exp, a


def test_single_element_groups_exhaustive_bf16():
    """Every finite bf16 value as the only non-zero element of a group: the
    oracle's scale and code must equal exact rational nearest-even rounding."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    ok = np.isfinite(f)
    bits = bits[ok].astype(np.uint16)
    n = bits.shape[0]
    rows = (n + 31) // 32
    x = np.zeros((rows, 512), dtype=np.uint16)
    for i in range(n):
        x[i // 32, (i % 32) * 16] = bits[i]
    recs = oracle.quantize_rows(x)
    e4 = _e4m3_pos_values()
    e2 = [Fraction(m) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for i in range(n):
        r, g = i // 32, i % 32
        v = float(f[ok][i])
        a = Fraction(abs(v))
        sc = _nearest_even(a / 6, e4) if a / 6 <= e4[-1] else 126
        assert recs[r, 256 + g] == sc, (v, recs[r, 256 + g], sc)
        s = e4[sc]
        mag = 0 if s == 0 else _nearest_even(a / s, e2) if a / s <= 6 else 7
        code = mag | (8 if math.copysign(1, v) < 0 else 0)
        byte = recs[r, g * 8]
        assert (byte & 15) == code, (v, byte & 15, code)


def test_quant_golden_examples():
    lines = list(_rows("quant_examples.txt"))
    assert len(lines) % 3 == 0
    for i in range(0, len(lines), 3):
        x = np.array([float(t) for t in lines[i].split(":")[1].split()], dtype=np.float32)
        sc = int(lines[i + 1].split(":")[1], 16)
        codes = [int(t, 16) for t in lines[i + 2].split(":")[1].split()]
        row = np.zeros((1, 512), dtype=np.float32)
        row[0, 32:48] = x          # group 2, so the layout offsets are exercised too
        rec = oracle.quantize_rows(row)[0]
        assert rec[256 + 2] == sc, (lines[i], rec[258], sc)
        got = [(rec[16 + j // 2] >> (4 * (j % 2))) & 15 for j in range(16)]
        assert got == codes, (lines[i], got, codes)
        assert all(rec[256 + g] == 0 for g in range(32) if g != 2)


def test_record_size_and_layout():
    assert oracle.RECORD == 288 == 512 // 2 + 512 // 16
    x = np.zeros((1, 512), np.float32)
    x[0, 0] = 6.0        # group 0, channel 0 -> low nibble of byte 0
    x[0, 1] = -6.0       # channel 1 -> high nibble of byte 0
    x[0, 511] = 1.0      # group 31: 1/6 -> 0.171875 (0x23); 1/0.171875 = 5.8 -> code 7
    rec = oracle.quantize_rows(x)[0]
    assert rec[0] == 0xF7 and rec[255] >> 4 == 7 and rec[256] == 0x38 and rec[287] == 0x23


def _random_rows(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 512)) * scale).astype(np.float32)


def test_quant_invariants():
    x = _random_rows(64, 4)
    recs = oracle.quantize_rows(x)
    dq = oracle.dequant_records(recs)
    sc = recs[:, 256:].astype(np.int64)
    s = np.array([[oracle.e4m3_value(c) for c in row] for row in sc])
    s_ch = np.repeat(s, 16, axis=1)
    # (1) every decoded value is an E2M1 value times its group scale
    ratio = np.abs(dq) / s_ch
    assert np.all(np.isin(ratio, [0, 0.5, 1, 1.5, 2, 3, 4, 6]))
    # (2) error at most half the local E2M1 gap times the scale (no saturation here)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    r = np.abs(x) / s_ch
    j = np.clip(np.searchsorted(grid, r) - 1, 0, 6)
    half_gap = (grid[j + 1] - grid[j]) / 2
    assert np.all(np.abs(x - dq) <= half_gap * s_ch + 0)
    # (3) idempotence: quantising the dequantised row gives the same record
    assert np.array_equal(oracle.quantize_rows(dq), recs)
    # (4) sign symmetry: -x flips every sign bit, scales unchanged
    rn = oracle.quantize_rows(-x)
    assert np.array_equal(rn[:, 256:], recs[:, 256:])
    assert np.array_equal(rn[:, :256], recs[:, :256] ^ 0x88)
    # (5) x * 2^k keeps the codes and moves the scale exponent by k
    for k in (-3, 2):
        rk = oracle.quantize_rows((x * 2.0 ** k).astype(np.float32))
        assert np.array_equal(rk[:, :256], recs[:, :256])
        sk = np.array([[oracle.e4m3_value(c) for c in row] for row in rk[:, 256:]])
        assert np.array_equal(sk, s * 2.0 ** k)
    # (6) the largest magnitude of every group maps to code 6 (value 6*s or 4*s
    #     is impossible: amax/s lies in [5.65, 6.4] for normal scales)
    amax = np.abs(x).reshape(64, 32, 16).max(axis=2)
    q = amax / s
    assert np.all((q > 5.6) & (q < 6.5))


def test_quant_special_groups():
    x = np.zeros((1, 512), np.float32)
    x[0, 16:32] = 5000.0                   # group 1 saturates
    x[0, 32:48] = 1e-4                     # group 2 underflows to scale 0
    x[0, 48] = -0.0                        # group 3 keeps the sign of -0
    rec = oracle.quantize_rows(x)[0]
    assert rec[256] == 0 and all(rec[j] == 0 for j in range(8))     # zero group
    assert rec[257] == 0x7E and all(rec[j] == 0x77 for j in range(8, 16))
    assert rec[258] == 0 and all(rec[j] == 0 for j in range(16, 24))
    assert rec[259] == 0 and rec[24] == 0x08


def test_bf16_and_fp32_inputs_agree():
    xb = torch.from_numpy(_random_rows(8, 5)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    a = oracle.quantize_rows(bits)
    b = oracle.quantize_rows(xb.float().numpy())
    assert np.array_equal(a, b)


def test_quant_append_places_rows_and_skips_out_of_range():
    x = _random_rows(4, 6)
    cache = np.full((10, 288), 0xAB, np.uint8)
    oracle.quant_append(x, np.array([7, -1, 2, 10]), cache)
    ref = oracle.quantize_rows(x)
    assert np.array_equal(cache[7], ref[0]) and np.array_equal(cache[2], ref[2])
    untouched = [i for i in range(10) if i not in (2, 7)]
    assert np.all(cache[untouched] == 0xAB)
