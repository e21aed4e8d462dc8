"""Graph capture of the verification and attention entry points (GPU).

Each is captured once into a graph and replayed several times, with eager
work between the replays that overwrites the outputs; every replay must
equal the eager call bit for bit. Then a device-resident input changes (the
Philox offset for verification, the context length for the attention) and
a replay must follow it, as the eager call on the new input does: the
parameters are read on the device, not baked into the graph.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from ancestral_draft_token_amd import (dspark_init, dspark_verify_block, dspark_verify_block_workspace_bytes,
                                       dspark_verify_standard, dspark_verify_workspace_bytes,
                                       dspark_window_attention_workspace_bytes, dspark_window_block_attention)

from gpu_util import require_gpu, say
from test_gpu_verify import _case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _replays_equal(g, outs, eager, clobber, n=3):
    import torch
    for i in range(n):
        clobber()
        torch.cuda.synchronize()
        say(f"replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"replay {i} differs from eager"


@pytest.mark.parametrize("rule", ["standard", "block"])
def test_verification_graph_replay(rule):
    import torch
    dspark_init()
    B, K, V = 12, 7, 20000
    d, q, p, sd, off = _case(B, K, V, seed=31, mix=0.8)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    dd, qq, pp, ss, oo = t(d), t(q), t(p), t(sd), t(off)
    n = torch.empty(B, dtype=torch.int32, device="cuda:0")
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda:0")
    fn, wsb = ((dspark_verify_standard, dspark_verify_workspace_bytes) if rule == "standard"
               else (dspark_verify_block, dspark_verify_block_workspace_bytes))
    wb = wsb(B, K, V)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    call = lambda: fn(dd, qq, pp, ss, oo, B, K, V, n, out, ws, wb)
    say(f"verify_{rule} eager")
    call()
    torch.cuda.synchronize()
    eager = [n.clone(), out.clone()]
    g = _capture(call)

    def clobber():
        n.fill_(-7)
        out.fill_(-7)
        ws.fill_(0xAB)

    _replays_equal(g, (n, out), eager, clobber)
    # a new slot offset: the replay draws new uniforms, as the eager call does
    oo.add_(1)
    g.replay()
    torch.cuda.synchronize()
    replayed = [n.clone(), out.clone()]
    # new uniforms and new Gumbel words over 20000 columns: some draw moves
    assert not (torch.equal(replayed[0], eager[0]) and torch.equal(replayed[1], eager[1]))
    call()
    torch.cuda.synchronize()
    assert torch.equal(replayed[0], n) and torch.equal(replayed[1], out)
    say(f"verify_{rule}: replays equal eager; new offset followed")


# (3 rows: the split form with its merge launch; 64 rows x 4 heads = 256
# pairs: the single launch, also with head-major caches)
@pytest.mark.parametrize("B,layout", [(3, None), (64, None), (64, 1)])
def test_window_attention_graph_replay(B, layout):
    import torch
    dspark_init()
    K, Hq, Hkv, D, W = 7, 64, 4, 128, 256
    L = 900
    g0 = torch.Generator(device="cuda:0").manual_seed(3)
    q = torch.randn((B, K, Hq, D), device="cuda:0", generator=g0).to(torch.bfloat16)
    shape = (B, Hkv, L, D) if layout == 1 else (B, L, Hkv, D)
    kc = torch.randn(shape, device="cuda:0", generator=g0).to(torch.bfloat16)
    vc = torch.randn(shape, device="cuda:0", generator=g0).to(torch.bfloat16)
    ctx = torch.tensor(([300, 500, 893] * 22)[:B], dtype=torch.int32, device="cuda:0")
    o = torch.empty((B, K, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, K, Hq), dtype=torch.float32, device="cuda:0")
    wb = dspark_window_attention_workspace_bytes(B, K, Hq, Hkv, D, L, W)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    scale = 1.0 / math.sqrt(D)
    call = lambda: dspark_window_block_attention(q, kc, vc, ctx, B, K, Hq, Hkv, D, L, W, scale, o, lse, ws, wb,
                                                 layout=layout)
    say(f"window attention eager B={B} layout={layout}")
    call()
    torch.cuda.synchronize()
    eager = [o.clone(), lse.clone()]
    g = _capture(call)

    def clobber():
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xCD)

    _replays_equal(g, (o, lse), eager, clobber)
    # a new context length: the replay attends the new key range
    ctx.sub_(37)
    g.replay()
    torch.cuda.synchronize()
    replayed = [o.clone(), lse.clone()]
    assert not torch.equal(replayed[1], eager[1])
    call()
    torch.cuda.synchronize()
    assert torch.equal(replayed[0], o) and torch.equal(replayed[1], lse)
    say("window attention: replays equal eager; new context length followed")
