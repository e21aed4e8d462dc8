"""Helpers shared by the GPU tests: run a workload through the C ABI and fetch rows."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_REPORT = os.environ.get("DSPARK_TEST_LOG", "")


def say(msg: str):
    """Name the case before each GPU step, flushed, so a crash still says where it
    was. Parity reports (near-tie counts, largest errors) are also appended to
    the file that DSPARK_TEST_LOG names, if it is set, since pytest keeps a
    passing test's output to itself."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()
    if _REPORT:
        with open(_REPORT, "a") as f:
            f.write(f"[gpu] {msg}\n")


def run_gpu(w, chunk_cols=None, packed=False):
    """Run one block on cuda:0 (W packed once when ``packed``); return the problem."""
    import torch
    from ancestral_draft_token_amd.device import DeviceProblem
    say(f"run {w.name} B={w.B} K={w.K} V={w.V} r={w.r} base={w.base_dtype} chunk={chunk_cols} packed={packed}")
    p = DeviceProblem(w, chunk_cols=chunk_cols, packed=packed)
    if packed:
        assert p.W_packed is not None, "no packed W for this workload"
    p.enqueue()
    torch.cuda.synchronize()
    return p


def rows_to_host(p, rows):
    rows = np.asarray(rows, dtype=np.int64)
    import torch
    idx = torch.from_numpy(rows).to(p.tokens.device)
    return (p.tokens.index_select(0, idx).cpu().numpy(),
            p.logits.index_select(0, idx).cpu().numpy(),
            p.q.index_select(0, idx).cpu().numpy())
