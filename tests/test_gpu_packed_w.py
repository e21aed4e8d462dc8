"""W packed once for the resident kernels (dspark_pack_w) against W itself.

The packed copy changes only the order in which the resident kernels' setup
reads W, so a block run with it must give bit-identical tokens, logits and
proposals to one run from W. Checked on the small-batch plan (B = 1, 2) and
the MFMA plan (B = 3 .. 128), with whole and ragged vocabularies (V % 16 = 8),
vocabularies that leave most workgroups without columns, ranks below 256, f32
and bf16 bases, greedy and padding rows, and the four full-size workloads; one
packed block is also compared with the oracle, and one is replayed from a
hipGraph.
"""

from __future__ import annotations

import pytest
import torch

from ancestral_draft_token_amd import dspark_launch_plan, dspark_packed_w_bytes, inputs
from ancestral_draft_token_amd.device import DeviceProblem
from oracle import parity

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _w(name, **kw):
    args = dict(base_dtype="f32", base_std=2.0, ew_std=0.05, data_seed=11, temperature=1.0)
    args.update(kw)
    return inputs.make_workload(name, **args)


def _both(w):
    say(f"packed vs W: {w.name} B={w.B} K={w.K} V={w.V} r={w.r} base={w.base_dtype} "
        f"plan={dspark_launch_plan(w.B, w.K, w.V, w.r)}")
    a = DeviceProblem(w)
    a.enqueue()
    b = DeviceProblem(w, packed=True)
    assert b.W_packed is not None and b.packed_bytes == dspark_packed_w_bytes(w.V, w.r) > 0
    b.enqueue()
    torch.cuda.synchronize()
    return a, b


def _identical(a, b):
    assert torch.equal(a.tokens, b.tokens)
    # as bit patterns: NaN logits of padding rows compare too
    assert torch.equal(a.logits.view(torch.int32), b.logits.view(torch.int32))
    assert torch.equal(a.q.view(torch.int32), b.q.view(torch.int32))


SMALL = {
    "b1_v4096_r32": dict(B=1, K=7, V=4096, r=32),
    "b2_v1000_r64_greedy": dict(B=2, K=3, V=1000, r=64, temperature=lambda b: [1.0, 0.0][b]),
    "b3_v2056_r96_bf16": dict(B=3, K=4, V=2056, r=96, base_dtype="bf16"),
    "b4_v200064_r256": dict(B=4, K=2, V=200064, r=256, base_std=3.0, ew_std=0.02),
    "b5_v1000_r64_pad": dict(B=5, K=3, V=1000, r=64, n_real=4,
                             temperature=lambda b: [1.0, 0.0, 0.7, 2.5, 0.0][b]),
    "b6_v3320_r32_ragged_bf16_nan": dict(B=6, K=4, V=3320, r=32, base_dtype="bf16", n_real=2, pad_base="nan"),
    "b17_v264_r128": dict(B=17, K=2, V=264, r=128, temperature=lambda b: 0.5 + 0.1 * (b % 3)),
    "b128_v8192_r256": dict(B=128, K=2, V=8192, r=256),
    "b40_v200056_r224_ragged": dict(B=40, K=2, V=200056, r=224, base_std=3.0, ew_std=0.02),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_packed_equals_unpacked(name):
    w = _w(name, **SMALL[name])
    a, b = _both(w)
    assert 4 in dspark_launch_plan(w.B, w.K, w.V, w.r), "a resident plan expected"
    _identical(a, b)


@pytest.mark.parametrize("name", ["b1", "b8", "b44", "b88"])
def test_packed_equals_unpacked_full_size(name):
    a, b = _both(inputs.WORKLOADS[name]())
    _identical(a, b)
    del a, b
    torch.cuda.empty_cache()


def test_packed_block_matches_the_oracle():
    w = inputs.tiny()
    p = DeviceProblem(w, packed=True)
    assert p.W_packed is not None
    say("packed tiny block against the oracle")
    t, l, q = p.run()
    say(f"parity ok {parity.check(w, t, l, q).as_dict()}")


def test_packing_twice_gives_the_same_bytes():
    from ancestral_draft_token_amd import dspark_pack_w
    w = inputs.tiny()
    p = DeviceProblem(w, packed=True)
    again = torch.full_like(p.W_packed, 0x5A)
    say("pack W again into a filled buffer")
    dspark_pack_w(p.W, w.V, w.r, again, p.packed_bytes)
    torch.cuda.synchronize()
    assert torch.equal(again, p.W_packed)


def test_packed_block_replays_from_a_graph():
    w = inputs.single_request()
    p = DeviceProblem(w, packed=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("packed b1 eager")
    with torch.cuda.stream(s):
        p.enqueue()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (p.tokens, p.logits, p.q)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        p.enqueue()
        g.capture_end()
    torch.cuda.synchronize()
    for i in range(3):
        for x in (p.tokens, p.logits, p.q):
            x.zero_()
        torch.cuda.synchronize()
        say(f"packed b1 replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip((p.tokens, p.logits, p.q), ref):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
