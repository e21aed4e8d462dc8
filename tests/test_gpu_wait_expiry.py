"""The resident plans' bounded device waits, forced to expire from the host.

The resident kernels exchange each position's argmax partials between
workgroups with bounded waits. ``dspark_set_wait_limit(0)`` makes every such
wait expire at once without reading (no workgroup waits on another), so every
kernel still runs to its end: the block must then report the failure through
``dspark_block_status``, leave token -1 at every position it could not draw,
and write NaN proposals there. The next call, with the default limit, must be
correct again: the exchange state the library keeps on the device recovers by
itself.
"""

from __future__ import annotations

import pytest

from ancestral_draft_token_amd import inputs
from oracle import parity

from gpu_util import require_gpu, rows_to_host, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def status_now():
    import torch
    from ancestral_draft_token_amd import dspark_block_status
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    dspark_block_status(st)
    torch.cuda.synchronize()
    return int(st.item())


CASES = {
    # the VALU resident kernel (B <= 2) and the MFMA resident kernel (2 < B <= 128)
    "b1": (inputs.single_request, [0]),
    "b8": (inputs.small_batch, [0, 3, 7]),
    "b44": (inputs.mixed_batch, [0, 1, 43]),
    # six N-tiles: with packed W the owners' reductions are pipelined
    "b88": (inputs.WORKLOADS["b88"], [0, 40, 87, 88, 95]),
}


@pytest.mark.parametrize("packed", [False, True], ids=["w", "w_packed"])
@pytest.mark.parametrize("name", list(CASES))
def test_expired_wait_is_reported_and_recovers(name, packed):
    from ancestral_draft_token_amd import dspark_launch_plan, dspark_set_wait_limit
    make, rows = CASES[name]
    w = make()
    assert 4 in dspark_launch_plan(w.B, w.K, w.V, w.r), "the workload must take a resident plan"
    prev = dspark_set_wait_limit(0)
    try:
        say(f"{name}: every device wait expires at once (packed W: {packed})")
        p = run_gpu(w, packed=packed)
    finally:
        dspark_set_wait_limit(prev)
    assert status_now() == 1
    assert bool((p.tokens == -1).all())
    assert bool(p.q.isnan().all())
    del p
    say(f"{name}: the next call with the default limit")
    p2 = run_gpu(w, packed=packed)
    assert status_now() == 0
    assert bool(((p2.tokens >= 0) & (p2.tokens < w.V)).all())
    sub, order = w.subset_rows(rows)
    t, l, q = rows_to_host(p2, order)
    rep = parity.check(sub, t, l, q)
    say(f"parity ok after recovery {name} {rep.as_dict()}")


def test_per_position_plan_leaves_status_alone():
    """A failed resident call stays reported across a later per-position call
    (which has no device waits), and the next resident call clears it."""
    from ancestral_draft_token_amd import dspark_set_wait_limit
    w = inputs.single_request()
    prev = dspark_set_wait_limit(0)
    try:
        run_gpu(w)
    finally:
        dspark_set_wait_limit(prev)
    assert status_now() == 1
    p = run_gpu(w, chunk_cols=128)
    assert bool((p.tokens >= 0).all())
    assert status_now() == 1
    run_gpu(w)
    assert status_now() == 0
