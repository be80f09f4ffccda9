"""Shared helpers of the GPU parity tests: seeded inputs on the host, copies to
the device, and the oracle calls on the same bytes."""
import sys

import numpy as np
import pytest
import torch

import csa2_inputs as gen

gpu = pytest.mark.gpu


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def note(msg):
    """Name the case before a GPU step so a failing run says what it was doing."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


bits = gen.bf16_bits


def index_inputs(lengths, h_i, d_i, seed, key_fn=None):
    """Per-sequence indexer keys laid out back to back, one query per sequence."""
    n_q = len(lengths)
    total = int(sum(lengths))
    ik = gen.normal((max(total, 1), d_i), seed, "ik", dtype=torch.bfloat16)
    if key_fn is not None:
        ik = key_fn(ik)
    iq = gen.normal((n_q, h_i, d_i), seed, "iq", dtype=torch.bfloat16)
    w = gen.uniform((n_q, h_i), seed, "w")
    seq_base = torch.tensor(np.concatenate([[0], np.cumsum(lengths)[:-1]]), dtype=torch.int64)
    q_seq = torch.arange(n_q, dtype=torch.int32)
    nvis = torch.tensor(lengths, dtype=torch.int32)
    return dict(ik=ik, iq=iq, w=w, seq_base=seq_base, q_seq=q_seq, nvis=nvis)


def to_dev(d, dev):
    return {k: v.to(dev) for k, v in d.items()}


def normwise_err(got, ref):
    """max over (query, head) rows of max|g - o| / max|o|."""
    den = np.abs(ref).max(axis=-1)
    num = np.abs(got - ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())
