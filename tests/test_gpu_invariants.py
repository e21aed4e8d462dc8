"""GPU properties the pages test: graph replay equals the eager call, a new offset
draws anew, identical inputs give identical outputs, and the base logits
buffer is never written ("brb-nv/TensorRT-LLM pull 27", section "Test Coverage")."""

from __future__ import annotations

import hashlib

import numpy as np
import pytest

from ancestral_draft_token_amd import inputs

from gpu_util import require_gpu, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _digest(t):
    return hashlib.sha256(t.contiguous().view(-1).view(__import__("torch").uint8).cpu().numpy()
                          .tobytes()).hexdigest()


@pytest.mark.parametrize("make", [inputs.tiny, inputs.small_batch])
def test_deterministic_and_base_untouched(make):
    import torch
    w = make()
    p = run_gpu(w)
    base_hash = _digest(p.base)
    first = [x.clone() for x in (p.tokens, p.logits, p.q)]
    for _ in range(3):
        p.enqueue()
    torch.cuda.synchronize()
    for a, b in zip(first, (p.tokens, p.logits, p.q)):
        assert torch.equal(a, b)
    assert _digest(p.base) == base_hash
    host = np.ascontiguousarray(w.base)
    got = p.base.cpu().numpy().view(host.dtype)
    assert np.array_equal(got.reshape(host.shape), host)


@pytest.mark.parametrize("make", [inputs.tiny, inputs.mixed_batch])
def test_graph_replay_equals_eager(make):
    import torch
    w = make()
    p = run_gpu(w)
    eager = [x.clone() for x in (p.tokens, p.logits, p.q)]
    say("capture")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            p.enqueue()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(4):
        # eager work between replays
        p.tokens.fill_(-1)
        p.q.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"replay {i}")
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (p.tokens, p.logits, p.q)):
            assert torch.equal(a, b), f"replay {i} differs from eager"


def test_graph_replay_sees_new_offset():
    """The slot offset is read on the device: a replay after advancing it draws anew."""
    import torch
    w = inputs.tiny(B=4, fixed_seed=None, fixed_offset=None)
    p = run_gpu(w)
    before = p.tokens.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            p.enqueue()
    torch.cuda.synchronize()
    p.offset.add_(1)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    after = p.tokens.clone()
    assert not torch.equal(before, after)
    # and the replay equals an eager call with the advanced offset
    p.enqueue()
    torch.cuda.synchronize()
    assert torch.equal(after, p.tokens)
