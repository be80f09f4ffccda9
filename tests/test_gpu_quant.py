"""csa2_quant_append on the GPU: bit-exact FP4 codes and scales versus the oracle."""
import numpy as np
import pytest
import torch

import csa2_inputs as gen
import oracle
import sparse_long_context_topk_amd as csa2
from gpu_common import bits, device, gpu, note


def _run(x, dst, rows):
    dev = device()
    cache = torch.full((rows, 288), 0xAB, dtype=torch.uint8, device=dev)
    csa2.quant_append(x.to(dev), dst.to(dev), cache)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_random_rows(dtype):
    note(f"quant random rows {dtype}")
    x = gen.normal((4099, 512), 1, "q-rows", dtype=dtype, outlier_p=0.01)
    x = x * torch.exp2(gen.normal((4099, 1), 1, "q-row-scale") * 6).to(dtype)   # many scale ranges
    got = _run(x, torch.arange(4099, dtype=torch.int64), 4099)
    src = bits(x) if dtype == torch.bfloat16 else x.numpy()
    assert np.array_equal(got, oracle.quantize_rows(src))


@gpu
def test_every_bf16_value_as_single_element_group():
    note("quant exhaustive bf16")
    allb = np.arange(65536, dtype=np.uint32)
    f = (allb << 16).view(np.float32)
    vals = allb[np.isfinite(f)].astype(np.uint16)
    rows = (len(vals) + 31) // 32
    x = np.zeros((rows, 512), np.uint16)
    for i, v in enumerate(vals):
        x[i // 32, (i % 32) * 16 + (i % 16)] = v
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    got = _run(xt, torch.arange(rows, dtype=torch.int64), rows)
    assert np.array_equal(got, oracle.quantize_rows(x))


@gpu
def test_special_groups_and_row_placement():
    note("quant special groups")
    x = np.zeros((3, 512), np.float32)
    x[0, 16:32] = 5000.0
    x[0, 32:48] = 1e-4
    x[0, 48] = -0.0
    x[0, 64:80] = np.linspace(-6, 6, 16)
    x[1] = np.float32(6.0) * (np.arange(512) % 7 - 3) / 3       # exact E2M1 midpoints and values
    x[2] = np.tile([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], 64)
    dst = torch.tensor([5, -3, 2], dtype=torch.int64)             # row 1 goes nowhere
    got = _run(torch.from_numpy(x), dst, 8)
    ref = np.full((8, 288), 0xAB, np.uint8)
    oracle.quant_append(x, dst.numpy(), ref)
    assert np.array_equal(got, ref)


@gpu
def test_idempotent_on_dequantised_rows():
    note("quant idempotence")
    x = gen.normal((256, 512), 2, "idem")
    rec = _run(x, torch.arange(256, dtype=torch.int64), 256)
    dq = oracle.dequant_records(rec)
    rec2 = _run(torch.from_numpy(dq), torch.arange(256, dtype=torch.int64), 256)
    assert np.array_equal(rec, rec2)
