"""Whole decode steps of the CSA2 workloads at their real sizes, launched
exactly as bench.py launches them (same input builder, same schedule driver,
same workspaces): every layer's indices and the pool bit-exact against the
oracle, every attention output within 2e-3 normwise per (query, head) row.

The 1M-context batch is checked on every sequence (the oracle needs about ten
seconds of host time for it).  The mixed 64-sequence batch runs its full
20-layer schedule (Full + 3 Reuse, then 4 x (Reindex + 3 Reuse)) with every
context shortened 16-fold, which keeps contexts above the 16,384-position pool
and the oracle within seconds."""
import os

import numpy as np
import pytest
import torch

import bench
import csa2_inputs as gen
from gpu_common import bits, device, gpu, normwise_err, note
from oracle.step import decode_step as oracle_step
from sparse_long_context_topk_amd.schedule import decode_step

TOL = 2e-3


def _host(t):
    return bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _check_workload(name, length_div=1):
    dev = device()
    wl = gen.workload(name, length_div=length_div)
    note(f"workload {wl['name']}: {len(wl['lengths'])} sequences, {wl['rows']} rows, layers {wl['layers']}")
    st, layers, app_x, app_rows = bench.build_state(wl, dev)
    res, pool = decode_step(st, layers, append_x=app_x, append_rows=app_rows, keep_outputs=True)
    torch.cuda.synchronize()
    got = [(i.cpu().numpy(), o.cpu().numpy().astype(np.float64), l.cpu().numpy()) for i, o, l in res]
    gpool = pool.cpu().numpy() if pool is not None else None

    def raw_rows(rows):
        x = gen.kv_rows_at(wl, rows, dev)
        return x.cpu().numpy() if x.dtype == torch.float32 else bits(x)

    hl = []
    for lay in layers:
        d = dict(mode=lay.mode, q=_host(lay.q), swa=bits(lay.swa), swa_row0=_host(lay.swa_row0),
                 swa_len=_host(lay.swa_len))
        if lay.iq is not None:
            d["iq"], d["w"] = bits(lay.iq), _host(lay.w)
        hl.append(d)
    n_q = wl["n_q"]
    ref, rpool, secs = oracle_step(hl, bits(st.ik), np.asarray(wl["seq_base"], np.int64),
                                   np.arange(n_q, dtype=np.int32), np.asarray(wl["lengths"], np.int32),
                                   wl["k"], wl["keep_blocks"], wl["block"], raw_rows, _host(app_x),
                                   st.softmax_scale, n_threads=min(16, os.cpu_count() or 1))
    print(f"oracle step {secs:.1f} s", flush=True)
    worst = 0.0
    for li, ((gi, go, gl), (ri, ro, rl)) in enumerate(zip(got, ref)):
        assert np.array_equal(gi, ri), f"layer {li} ({wl['layers'][li]}): indices differ"
        err = normwise_err(go, ro)
        worst = max(worst, err)
        assert err <= TOL, f"layer {li}: normwise error {err:.3e}"
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(gl)), f"layer {li}: lse finiteness differs"
        assert np.abs(gl[fin] - rl[fin]).max(initial=0.0) <= 1e-3, f"layer {li}: lse differs"
    if wl["keep_blocks"]:
        assert np.array_equal(gpool, rpool), "pool differs"
    print(f"{wl['name']}: {len(got)} layers, worst normwise error {worst:.2e}", flush=True)


@gpu
def test_c1_single_full_layer_4k():
    _check_workload("c1")


@gpu
def test_c2_full_plus_reuse_128k_batch8():
    _check_workload("c2")


@gpu
def test_c3_full_pool_reindex_1m_batch4():
    _check_workload("c3")


@gpu
def test_c5_twenty_layer_schedule_mixed_lengths():
    _check_workload("c5", length_div=16)
