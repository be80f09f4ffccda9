#!/usr/bin/env python3
"""CSA2 decode-step benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: FP4 append of each
sequence's new token, then every layer of the workload's schedule (Full:
index scan + Top-512 (+ block pool); Reindex: pool re-scoring + Top-512;
Reuse: nothing), each followed by its sparse attention over the selected FP4
entries and its 128-row window.  Inputs are synthetic and seeded, resident in
HBM before timing starts.  The default workload is the 1M-context Reindex
group (batch 4, Full + Reindex layers).

Prints one JSON line.  `value` is query-layers per second (one query attended
in one layer, including that layer's index/reindex/append work).  `roofline`
covers the dominant kernel, the indexer scan: algorithmic bytes per launch /
its mean launch time (HIP events recorded around that kernel inside the timed
steps).  `cpu_baseline` runs the plain CPU oracle on the same inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 decode attention queries·layers/sec at 1M ctx; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
SCAN_SRC = os.path.join(ROOT, "sparse_long_context_topk_amd", "csrc", "index_topk.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--full-from-pool", action="store_true",
                   help="the pool-based Full variant: the Full layer picks its Top-K inside its own pool, "
                        "scanning stored block keys instead of every token key (reported as its own workload)")
    p.add_argument("--fp8-keys", action="store_true",
                   help="the low-precision indexer-key variant: indexer keys stored as E4M3 codes with one "
                        "power-of-two scale per row (129 bytes per 128-dim key); the Full and Reindex layers score "
                        "the stored keys (reported as its own workload)")
    p.add_argument("--graph", action="store_true",
                   help="also capture the step as a HIP graph and report the replayed step's rate as `value` "
                        "(the eager steps still time the scan for `roofline`)")
    p.add_argument("--cpu-baseline", default="auto", choices=["auto", "off"])
    p.add_argument("--cpu-seqs", type=int, default=0, help="sequences in the oracle sample (0: workload default)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run only a plain device-to-device copy of MIB MiB, 5 times (scales HBM byte counters)")
    return p.parse_args()


def build_state(wl, dev):
    import numpy as np
    import torch

    import csa2_inputs as gen
    import sparse_long_context_topk_amd as csa2
    from sparse_long_context_topk_amd.schedule import DecodeState, LayerInputs

    rows = wl["rows"]
    cache = torch.empty((rows, 288), dtype=torch.uint8, device=dev)
    chunk = 1 << 20
    for r0 in range(0, rows, chunk):
        n = min(chunk, rows - r0)
        x = gen.kv_rows(wl, r0, n, dev)
        csa2.quant_append(x, torch.arange(r0, r0 + n, dtype=torch.int64, device=dev), cache)
        del x
    ik = gen.index_keys(wl, dev)
    s = gen.seq_tensors(wl, dev)
    st = DecodeState(cache=cache, ik=ik, seq_base=s["seq_base"], q_seq=s["q_seq"], q_nvis=s["q_nvis"],
                     max_nvis=max(wl["q_nvis"]), k=wl["k"], keep_blocks=wl["keep_blocks"], w_max=wl["w"],
                     softmax_scale=512 ** -0.5,
                     chunk_base=int(wl["seq_base"][wl["q_seq"][0]]) if wl.get("chunk") else None)
    if wl.get("pool_full"):
        # stored block keys of every sequence, built before timing (a step
        # refreshes only the block of the appended position)
        lens = torch.tensor(wl["lengths"], dtype=torch.int32, device=dev)
        nblk = [(L + 7) // 8 for L in wl["lengths"]]
        kb_base = torch.tensor(np.concatenate([[0], np.cumsum(nblk)[:-1]]), dtype=torch.int64, device=dev)
        st.pool_full = True
        st.kbar = torch.empty((max(sum(nblk), 1), wl["d_i"]), dtype=torch.bfloat16, device=dev)
        st.kbar_base, st.seq_len = kb_base, lens
        st.blk_last = torch.tensor([(L - 1) // 8 for L in wl["lengths"]], dtype=torch.int32, device=dev)
        st.q_nblk = torch.tensor([(n + 7) // 8 for n in wl["q_nvis"]], dtype=torch.int32, device=dev)
        st.max_nblk = max((n + 7) // 8 for n in wl["q_nvis"])
        csa2.block_keys(ik, st.seq_base, lens, st.kbar, kb_base, max(nblk))
    if wl.get("fp8_keys"):
        # the keys' FP8 copy, written before timing as a cache would hold it
        st.ik8, st.ik8_exp = csa2.index_keys_fp8(ik)
        st.fp8_keys = True
    layers = [LayerInputs(**gen.layer_tensors(wl, i, dev)) for i in range(len(wl["layers"]))]
    app_x, app_rows = gen.append_rows(wl, dev)
    torch.cuda.synchronize()
    return st, layers, app_x, app_rows


def chunk_flops(wl):
    """FLOPs of one encoder-chunk scan launch: every (query, visible key) pair
    costs 2 * h_i * d_i (the per-head dot products)."""
    return sum(wl["q_nvis"]) * 2 * wl["h_i"] * wl["d_i"]


PEAK_MFMA_BF16_TFLOPS = 2500.0


def scan_bytes(wl):
    """Algorithmic bytes of one Full-layer indexer-scan launch: every visible
    key (d_i bf16) once, plus each query's indexer query and head weights.  In
    the pool-based Full variant the scan reads the stored block keys instead
    (one per 8 visible positions)."""
    n_q, h_i, d_i = wl["n_q"], wl["h_i"], wl["d_i"]
    keys = sum((n + 7) // 8 for n in wl["q_nvis"]) if wl.get("pool_full") else sum(wl["q_nvis"])
    return keys * key_bytes(wl) + n_q * (h_i * d_i * 2 + h_i * 4)


def key_bytes(wl):
    """Bytes of one stored indexer key: bf16, or FP8 codes plus the row's exponent byte."""
    return wl["d_i"] + 1 if wl.get("fp8_keys") else 2 * wl["d_i"]


def step_bytes(wl):
    """Algorithmic bytes of one whole step (what the method must move): each
    key once per scanning query (once per chunk for the encoder chunk, whose
    queries share them), the pool's keys, the selected records and window
    rows each query attends over (a chunk's shared window rows once), queries
    in and outputs out, and the appended rows."""
    n_q, h_i, d_i, h, k, W = wl["n_q"], wl["h_i"], wl["d_i"], wl["h"], wl["k"], wl["w"]
    qb = 4 if wl["q_dtype"] == "f32" else 2
    nvis = wl["q_nvis"]
    b = 0
    if wl.get("append", True):
        b += len(wl["lengths"]) * (1024 + 288)               # append: read a bf16 row, write a record
    for mode in wl["layers"]:
        if mode == "full" and wl.get("chunk"):
            b += max(nvis) * d_i * 2 + n_q * (h_i * d_i * 2 + h_i * 4 + k * 4)
        elif mode == "full" and wl.get("pool_full"):
            b += n_q * 9 * d_i * 2                               # block-key refresh: 8 keys in, 1 out
            b += scan_bytes(wl) + n_q * wl["keep_blocks"] * 4    # block scan -> pool
            b += sum(min(L, 8 * wl["keep_blocks"]) for L in nvis) * d_i * 2
            b += n_q * (h_i * d_i * 2 + h_i * 4 + k * 4)         # pool re-scored with the Full query
        elif mode == "full":
            b += scan_bytes(wl) + n_q * k * 4 + (n_q * wl["keep_blocks"] * 4)
        elif mode == "reindex":
            b += sum(min(L, 8 * wl["keep_blocks"]) for L in nvis) * key_bytes(wl)
            b += n_q * (h_i * d_i * 2 + h_i * 4 + wl["keep_blocks"] * 4 + k * 4)
        # attention: selected records and window rows, q in, out
        b += sum(min(k, L) * 288 for L in nvis)
        b += (n_q + W - 1) * 1024 if wl.get("swa_shared") else sum(min(W, L) * 1024 for L in nvis)
        b += n_q * h * 512 * (qb + 4)
    return b


def traffic_from_profile(kernel_sha, key="traffic_bytes_per_launch"):
    """HBM bytes per scan launch measured with rocprofv3 counters (committed
    summary; `key` names the bf16 or the FP8-key figure), if it was taken on
    the current kernel source."""
    path = os.path.join(ROOT, "profiles", "index_scan_c3_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"^" + key + r":\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != kernel_sha:
        return None
    return float(m_b.group(1))


def chunk_counters_from_profile(kernel_sha):
    """Counter-based MFMA utilisation of the encoder-chunk scan (committed
    rocprofv3 summary: MFMA-busy cycles and the MOPS rate, each a fraction of
    the dense bf16 peak), if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "encoder_chunk_scan_c4_mfma_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_busy = re.search(r"^mfma_busy_frac:\s*([0-9.]+)", text, re.M)
    m_mops = re.search(r"^mops_frac:\s*([0-9.]+)", text, re.M)
    if not m_sha or not m_busy or not m_mops or m_sha.group(1) != kernel_sha:
        return None
    return {"mfma_busy_frac": float(m_busy.group(1)), "mops_frac": float(m_mops.group(1)),
            "profile": "profiles/encoder_chunk_scan_c4_mfma_counters.md"}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _oracle_threads(n_indep):
    """Threads for the oracle's multi-thread leg: one per independent query of
    the sample, at most the host's CPUs and at most 16 (a GPU machine's share)."""
    return max(1, min(n_indep, 16, os.cpu_count() or 1))


def _cpu_record(value, threads, sample, value_1t, sample_1t):
    return {"value": value, "unit": "query·layers/s", "cores": threads, "threads": threads, "kind": "oracle",
            "sample": sample, "cpu": _cpu_model(), "host_logical_cpus": os.cpu_count(),
            "one_thread": {"value": value_1t, "unit": "query·layers/s", "sample": sample_1t}}


def cpu_baseline_chunk(wl, st, layers, dev, nq, gpu_results):
    """Time the CPU oracle on `nq` queries spread over the encoder chunk (all
    its layers, the same inputs); the sample's indices and outputs are checked
    against the timed GPU step's."""
    import numpy as np
    import torch

    import csa2_inputs as gen
    import oracle
    from oracle.step import decode_step as oracle_step

    bits = gen.bf16_bits
    n = wl["n_q"]
    sel = np.unique(np.linspace(0, n - 1, nq).astype(np.int64))
    ts = torch.from_numpy(sel).to(dev)
    host = lambda t: t.cpu().numpy() if t.dtype != torch.bfloat16 else bits(t)
    hl = []
    for li, lay in enumerate(layers):
        hl.append(dict(mode=lay.mode, q=host(lay.q[ts]), swa=bits(lay.swa), swa_row0=host(lay.swa_row0[ts]),
                       swa_len=host(lay.swa_len[ts])))
        if lay.iq is not None:
            hl[-1]["iq"], hl[-1]["w"] = bits(lay.iq[ts]), host(lay.w[ts])
    threads = _oracle_threads(len(sel))
    oracle.lib()

    def raw_rows(rows):
        x = gen.kv_rows_at(wl, rows, dev)
        return x.cpu().numpy() if x.dtype == torch.float32 else bits(x)

    res, _, secs = oracle_step(hl, bits(st.ik), np.asarray(wl["seq_base"], np.int64),
                               np.asarray(wl["q_seq"], np.int32)[sel], np.asarray(wl["q_nvis"], np.int32)[sel],
                               wl["k"], 0, wl["block"], raw_rows, None, st.softmax_scale, n_threads=threads)
    idx_ok, err = True, 0.0
    for (gidx, gout, _), (ridx, rout, _) in zip(gpu_results, res):
        idx_ok &= bool(np.array_equal(gidx[ts].cpu().numpy(), ridx))
        o = gout[ts].cpu().numpy()
        den = np.abs(rout).max(axis=-1)
        den[den == 0] = 1
        err = max(err, float((np.abs(o - rout).max(axis=-1) / den).max()))
    ql = len(sel) * len(wl["layers"])
    # one thread on one of the sampled queries, all layers
    one = sel[len(sel) // 2:len(sel) // 2 + 1]
    _, _, secs1 = oracle_step([{**d, **{key: d[key][len(sel) // 2:len(sel) // 2 + 1]
                                         for key in ("q", "swa_row0", "swa_len", "iq", "w") if key in d}}
                               for d in hl], bits(st.ik), np.asarray(wl["seq_base"], np.int64),
                              np.asarray(wl["q_seq"], np.int32)[one], np.asarray(wl["q_nvis"], np.int32)[one],
                              wl["k"], 0, wl["block"], raw_rows, None, st.softmax_scale, n_threads=1)
    ql1 = len(wl["layers"])
    return (_cpu_record(ql / secs, threads,
                        f"{len(sel)} of {n} chunk queries (spread over the chunk), all {len(wl['layers'])} layers "
                        f"= {ql} query-layers in {secs:.2f} s on {threads} threads (OpenMP over queries)",
                        ql1 / secs1, f"chunk query {int(one[0])}, all {ql1} layers = {ql1} query-layers in "
                                     f"{secs1:.2f} s on 1 thread"),
            {"idx_bitexact": idx_ok, "attn_max_normwise_err": err, "queries": int(len(sel))})


def cpu_baseline(wl, st, layers, app_x, dev, nseq, gpu_results):
    """Time the CPU oracle on the first `nseq` sequences of the same inputs."""
    import numpy as np
    import torch

    import csa2_inputs as gen
    import oracle
    from oracle.step import decode_step as oracle_step

    bits = gen.bf16_bits
    sel = list(range(nseq))
    lens = [wl["lengths"][i] for i in sel]
    base = [int(wl["seq_base"][i]) for i in sel]
    cbase = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    ik = np.concatenate([bits(st.ik[b:b + L]) for b, L in zip(base, lens)])
    if wl.get("fp8_keys"):
        # the variant scores the stored FP8 keys: the oracle quantises the same bf16 keys itself
        ik = oracle.dequant_keys_fp8(*oracle.index_keys_fp8(ik))

    def raw_rows(crow):
        # compact row -> (sequence, position) -> global row of the generator
        s = np.searchsorted(cbase, crow, side="right") - 1
        g = np.asarray(base)[s] + (crow - cbase[s])
        x = gen.kv_rows_at(wl, g, dev)
        return x.cpu().numpy() if x.dtype == torch.float32 else bits(x)

    def host(t):
        return t.cpu().numpy() if t.dtype != torch.bfloat16 else bits(t)

    hl = []
    for li, lay in enumerate(layers):
        # the generated window rows (the timed steps have written their new rows into lay.swa)
        swa = bits(gen.layer_tensors(wl, li, dev)["swa"])
        d = dict(mode=lay.mode, q=host(lay.q[:nseq]), swa=swa, swa_row0=host(lay.swa_row0[:nseq]),
                 swa_len=host(lay.swa_len[:nseq]))
        if lay.iq is not None:
            d["iq"], d["w"] = bits(lay.iq[:nseq]), host(lay.w[:nseq])
        if lay.swa_new is not None:
            d["swa_new"], d["swa_dst"] = bits(lay.swa_new[:nseq]), host(lay.swa_dst[:nseq])
        hl.append(d)
    ax = host(app_x[:nseq])
    threads = _oracle_threads(nseq)
    oracle.lib()
    res, _, secs = oracle_step(hl, ik, cbase, np.arange(nseq, dtype=np.int32), np.array(lens, np.int32),
                               wl["k"], wl["keep_blocks"], wl["block"], raw_rows, ax, st.softmax_scale,
                               n_threads=threads, pool_full=bool(wl.get("pool_full")))
    # parity of the sample against the timed GPU step's outputs
    idx_ok, err = True, 0.0
    for (gidx, gout, _), (ridx, rout, _) in zip(gpu_results, res):
        idx_ok &= bool(np.array_equal(gidx[:nseq].cpu().numpy(), ridx))
        o = gout[:nseq].cpu().numpy()
        den = np.abs(rout).max(axis=-1)
        den[den == 0] = 1
        err = max(err, float((np.abs(o - rout).max(axis=-1) / den).max()))
    ql = nseq * len(wl["layers"])
    # one thread on the first sequence of the sample, the same step
    hl1 = [{key: (v[:1] if key in ("q", "swa_row0", "swa_len", "iq", "w", "swa_new", "swa_dst") else v)
            for key, v in d.items()} for d in hl]
    _, _, secs1 = oracle_step(hl1, ik[:lens[0]], cbase[:1], np.zeros(1, np.int32), np.array(lens[:1], np.int32),
                              wl["k"], wl["keep_blocks"], wl["block"], raw_rows, ax[:1], st.softmax_scale,
                              n_threads=1, pool_full=bool(wl.get("pool_full")))
    ql1 = len(wl["layers"])
    return (_cpu_record(ql / secs, threads,
                        f"{nseq} of {wl['n_q']} sequences (full contexts {sorted(set(lens))}), all "
                        f"{len(wl['layers'])} layers of one step = {ql} query-layers in {secs:.2f} s on {threads} "
                        f"threads (OpenMP over queries)",
                        ql1 / secs1, f"sequence 0 (context {lens[0]}), all {ql1} layers of one step = {ql1} "
                                     f"query-layers in {secs1:.2f} s on 1 thread"),
            {"idx_bitexact": idx_ok, "attn_max_normwise_err": err, "sequences": nseq})


def copy_calibration(mib, dev):
    """A copy of known size: each launch reads and writes exactly `mib` MiB,
    so a profiler's HBM byte counters for it give the counters' scale."""
    import torch

    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def attainable_copy(dev, mib=1024, reps=10):
    """The HBM bandwidth a plain device copy reaches on this part (1 GiB read +
    1 GiB written per launch), timed after the measured steps: the attainable
    ceiling beside the published peak."""
    import torch

    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) * 1e-3 / reps
    gbps = 2 * n / secs / 1e9
    del src, dst
    return {"kernel": "device copy, 1 GiB read + 1 GiB written per launch", "GB/s": round(gbps, 1),
            "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import csa2_inputs as gen
    from sparse_long_context_topk_amd.schedule import decode_step

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration, dev)
        return
    wl = gen.workload(a.workload)
    if a.fp8_keys:
        if a.full_from_pool or wl.get("chunk") or wl["d_i"] != 128:
            sys.exit("--fp8-keys serves the decode workloads with a 128-dim indexer (c2, c3, c5)")
        wl["fp8_keys"] = True
        wl["desc"] += "; FP8 indexer keys (E4M3 codes, one power-of-two scale per row)"
    if a.full_from_pool:
        if not wl["keep_blocks"] or "full" not in wl["layers"]:
            sys.exit(f"--full-from-pool needs a workload with a Full layer and a pool ({a.workload} has none)")
        wl["pool_full"] = True
        wl["desc"] += "; pool-based Full variant (Full picks its Top-K inside its own pool of stored block keys)"
    log(f"workload {wl['name']}: {wl['desc']}; building inputs")
    t0 = time.time()
    st, layers, app_x, app_rows = build_state(wl, dev)
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def step(ev=None, keep=False):
        return decode_step(st, layers, append_x=app_x, append_rows=app_rows, scan_events=ev, keep_outputs=keep)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    K = a.steps
    has_full = "full" in wl["layers"]
    evs = []
    for _ in range(K if has_full else 0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()
        evs.append((e0, e1))
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        step(evs[i] if has_full else None)
    t_stop.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_stop) / K
    log(f"timed {K} steps: {ms:.4f} ms/step")
    ql_per_step = wl["n_q"] * len(wl["layers"])
    eager_ms = ms
    if a.graph:
        from sparse_long_context_topk_amd.schedule import StepGraph
        gr = StepGraph(st, layers, append_x=app_x, append_rows=app_rows)
        for _ in range(a.warmup):
            gr.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(K):
            gr.replay()
        g1.record()
        torch.cuda.synchronize()
        ms = g0.elapsed_time(g1) / K
        log(f"timed {K} graph replays: {ms:.4f} ms/step (eager {eager_ms:.4f})")
    value = ql_per_step / (ms * 1e-3)

    roofline = None
    if has_full and wl.get("chunk"):
        # the encoder chunk's scan is a dense causal contraction: MFMA-bound
        scan_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / K
        fl = chunk_flops(wl)
        achieved = fl / (scan_ms * 1e-3) / 1e12
        sha = hashlib.sha256(open(SCAN_SRC, "rb").read()).hexdigest()
        counters = chunk_counters_from_profile(sha) if a.workload == "c4" else None
        roofline = {"bound": "mfma", "kernel": "k_scan_chunk (encoder-chunk indexer scan, bf16 MFMA)",
                    "achieved": round(achieved, 1), "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": None,
                    "algorithmic_flops_per_launch": fl, "launch_ms": round(scan_ms, 5),
                    "counters": counters}
    elif has_full:
        scan_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / K
        sb = scan_bytes(wl)
        achieved = sb / (scan_ms * 1e-3) / 1e9
        sha = hashlib.sha256(open(SCAN_SRC, "rb").read()).hexdigest()
        traffic = traffic_from_profile(sha, "fp8_traffic_bytes_per_launch" if wl.get("fp8_keys")
                                       else "traffic_bytes_per_launch")
        kname = "k_scan over block keys (pool-based Full)" if wl.get("pool_full") else "k_scan (indexer scan, Full layer)"
        if wl.get("fp8_keys"):
            kname = "k_scan over FP8 keys (indexer scan, Full layer)"
        if wl.get("pool_full") or a.workload != "c3":
            traffic = None   # the committed counters cover the 1M batch-4 token scans (bf16 and FP8 keys) only
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": traffic, "algorithmic_bytes_per_launch": sb, "launch_ms": round(scan_ms, 5)}
    sbytes = step_bytes(wl)

    cpu = None
    parity = None
    if a.cpu_baseline == "auto":
        nseq = a.cpu_seqs or {"c1": 1, "c2": 8, "c3": 4, "c4": 8, "c5": 2}[a.workload]
        log(f"cpu baseline: oracle on {nseq} sequence(s) or chunk queries")
        gres, _ = step(keep=True)
        torch.cuda.synchronize()
        if wl.get("chunk"):
            cpu, parity = cpu_baseline_chunk(wl, st, layers, dev, nseq, gres)
        else:
            cpu, parity = cpu_baseline(wl, st, layers, app_x, dev, nseq, gres)
        log(f"cpu baseline {cpu['value']:.3f} q.l/s; sample parity {parity}")

    attainable = attainable_copy(dev)
    log(f"attainable copy {attainable['GB/s']} GB/s")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "query·layers/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl['name']}: {wl['desc']}", "batch": wl["n_q"],
                   "context": max(wl["lengths"]), "context_total": wl["rows"], "layers": wl["layers"],
                   "query_layers_per_step": ql_per_step, "heads": wl["h"],
                   "indexer": f"{wl['h_i']}x{wl['d_i']}", "top_k": wl["k"], "swa": wl["w"],
                   "pool_blocks": wl["keep_blocks"], "parallelism": "none (1 GPU)"},
        "step_hbm": {"algorithmic_bytes": sbytes, "GB/s": round(sbytes / (ms * 1e-3) / 1e9, 1),
                     "frac": round(sbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        "roofline": roofline,
        "attainable_hbm": attainable,
        "step_launch": ({"mode": "hip_graph", "eager_ms_per_step": round(eager_ms, 5)} if a.graph
                        else {"mode": "eager"}),
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
