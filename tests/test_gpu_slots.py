"""Proposals written by slot (dspark_draft_block_slots) against the row-indexed block.

The slot entry runs the same launches as dspark_draft_block; only the
proposal pass stores row b's q into row slot_index[b] of a [n_slots, K, V]
buffer. Checked, as bit patterns: tokens and logits equal to the row-indexed
block's, each row's q in its slot, every other slot untouched, and a row
whose slot is out of range storing no proposal. Its token and logits are
still written, which matters for the one-row per-position plan, whose
proposal pass takes the last position's token. Covered: the one- and two-row
resident kernel, the MFMA resident kernel with W itself and packed, and
per-position plans (rank 288 rules the resident kernels out) with one and
three rows.
"""

from __future__ import annotations

import pytest
import torch

from ancestral_draft_token_amd import dspark_draft_block_slots, dspark_launch_plan, inputs
from ancestral_draft_token_amd.device import DeviceProblem

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

SENTINEL = -7.0

# name: (workload sizes, slot of each row, n_slots, packed W)
CASES = {
    "b1_resident": (dict(B=1, K=7, V=4096, r=32), [2], 3, False),
    "b1_per_position": (dict(B=1, K=3, V=4096, r=288), [0], 1, False),
    "b1_per_position_out_of_range": (dict(B=1, K=3, V=4096, r=288), [5], 2, False),
    "b2_resident_greedy_row": (dict(B=2, K=4, V=2056, r=96, temperature=lambda b: [1.0, 0.0][b]), [1, 0], 2, False),
    "b3_per_position": (dict(B=3, K=3, V=4096, r=288), [4, -1, 0], 5, False),
    "b5_mfma_padding_row": (dict(B=5, K=3, V=1000, r=64, n_real=4), [7, 2, 9, 0, 5], 10, False),
    "b6_mfma_packed": (dict(B=6, K=4, V=3320, r=32, base_dtype="bf16"), [5, 4, 3, 2, 1, 0], 6, True),
}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def bits(x):
    return x.view(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_slots_equal_rows(name):
    sizes, slots, n_slots, packed = CASES[name]
    w = inputs.tiny(fixed_seed=None, fixed_offset=None, data_seed=3, **sizes)
    say(f"slots {name}: B={w.B} K={w.K} V={w.V} r={w.r} plan={dspark_launch_plan(w.B, w.K, w.V, w.r)}")
    a = DeviceProblem(w, packed=packed)
    a.enqueue()
    b = DeviceProblem(w, packed=packed)
    if packed:
        assert a.W_packed is not None and b.W_packed is not None
    dev = b.tokens.device
    slot_index = torch.tensor(slots, dtype=torch.int32, device=dev)
    dp = torch.full((n_slots, w.K, w.V), SENTINEL, dtype=torch.float32, device=dev)
    dspark_draft_block_slots(b.base, b.base_dtype, b.E, b.W, b.prev, b.seed, b.offset, b.temperature,
                             b.n_real, slot_index, n_slots, w.B, w.K, w.V, w.r, b.tokens, b.logits, dp,
                             b.workspace, b.ws_bytes, W_packed=b.W_packed, packed_bytes=b.packed_bytes)
    torch.cuda.synchronize()
    assert torch.equal(a.tokens, b.tokens)
    assert torch.equal(bits(a.logits), bits(b.logits))
    sent = set()
    for row, s in enumerate(slots):
        if 0 <= s < n_slots:
            assert torch.equal(bits(dp[s]), bits(a.q[row])), (row, s)
            sent.add(s)
    for s in range(n_slots):
        if s not in sent:
            assert bool((dp[s] == SENTINEL).all()), s
    say(f"slots ok {name}: {len(sent)} of {n_slots} slots written")
