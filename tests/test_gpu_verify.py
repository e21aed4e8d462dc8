"""GPU standard token-level verification vs the CPU oracle, through the C ABI.

The acceptance decisions (float32 ratio against the Philox uniform) are taken
in the same precision on both sides, so the number of accepted drafts must
match exactly. The emitted token is a Gumbel-max draw: it must be the
oracle's, or, where the oracle's top-2 margin is within TIE_EPS, one of the
oracle's near-tied candidates. Cases: small and ragged vocabularies (one and
several 8192-column chunks, K = 0), equal distributions (every draft
accepted, the bonus draw), a one-hot target (rejection onto its token), and
the full-size B=88 draft block's own tokens and proposals against a target
mixed from them.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from ancestral_draft_token_amd import dspark_init, dspark_verify_standard, dspark_verify_workspace_bytes

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _softmax32(x):
    x = x.astype(np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def _draw(q, rng):
    c = np.cumsum(q.astype(np.float64), axis=-1)
    u = rng.random(c.shape[:-1])
    return (u[..., None] > c).sum(-1).clip(0, q.shape[-1] - 1).astype(np.int32)


def _case(B, K, V, seed=0, mix=0.6):
    rng = np.random.default_rng(seed)
    q = _softmax32(rng.normal(0, 2.0, size=(B, K, V)))
    other = _softmax32(rng.normal(0, 2.0, size=(B, K + 1, V)))
    p = other.copy()
    if K:
        p[:, :K] = (mix * q.astype(np.float64) + (1 - mix) * other[:, :K]).astype(np.float32)
    d = _draw(q, rng) if K else np.zeros((B, 0), np.int32)
    sd = rng.integers(0, 2**62, size=B, dtype=np.int64)
    off = rng.integers(0, 2**40, size=B, dtype=np.int64)
    return d, q, p, sd, off


def verify_gpu(d, q, p, sd, off):
    import torch
    dspark_init()
    B, K = d.shape
    V = p.shape[-1]
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dd, qq, pp, ss, oo = t(d), t(q) if K else None, t(p), t(sd), t(off)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    wb = dspark_verify_workspace_bytes(B, K, V)
    ws = torch.empty(max(wb, 256), dtype=torch.uint8, device=dev)
    say(f"verify B={B} K={K} V={V}")
    dspark_verify_standard(dd, qq, pp, ss, oo, B, K, V, n, out, ws, wb)
    torch.cuda.synchronize()
    return n.cpu().numpy(), out.cpu().numpy()


def check(d, q, p, sd, off, n_gpu, out_gpu):
    ref = oracle.verify_standard(d, q if q is not None else np.zeros(d.shape + (p.shape[-1],), np.float32),
                                 p, sd, off)
    assert (n_gpu == ref.n_accepted).all(), (n_gpu, ref.n_accepted)
    B, K = d.shape
    near = 0
    for b in range(B):
        n = int(ref.n_accepted[b])
        assert (out_gpu[b, :n] == ref.out_tokens[b, :n]).all()
        assert (out_gpu[b, n + 1:] == -1).all()
        tok, want = int(out_gpu[b, n]), int(ref.out_tokens[b, n])
        if tok != want:
            assert ref.margin[b] <= oracle.TIE_EPS, (b, tok, want, ref.margin[b])
            assert tok in set(ref.cand[b][: ref.ncand[b]].tolist()), (b, tok)
            near += 1
    say(f"verify parity ok: rows {B}, accepted {int(ref.n_accepted.sum())}, near-tie branches {near}")
    return ref


@pytest.mark.parametrize("B,K,V", [(6, 3, 1000), (3, 7, 8192), (4, 2, 20000), (2, 0, 4096), (5, 1, 16388),
                                   (17, 7, 2056)])
def test_verify_shapes(B, K, V):
    d, q, p, sd, off = _case(B, K, V, seed=B * 1000 + K * 10 + V % 97)
    n, out = verify_gpu(d, q, p, sd, off)
    check(d, q, p, sd, off, n, out)


def test_verify_equal_distributions_accept_everything():
    d, q, p, sd, off = _case(8, 5, 3000, seed=3, mix=1.0)
    p[:, :5] = q
    n, out = verify_gpu(d, q, p, sd, off)
    assert (n == 5).all()
    check(d, q, p, sd, off, n, out)


def test_verify_one_hot_target_rejects_onto_its_token():
    B, K, V = 6, 3, 5000
    d, q, p, sd, off = _case(B, K, V, seed=4)
    a = (d[:, 0] + 7) % V
    p[:, 0] = 0.0
    p[np.arange(B), 0, a] = 1.0
    n, out = verify_gpu(d, q, p, sd, off)
    assert (n == 0).all() and (out[:, 0] == a).all() and (out[:, 1:] == -1).all()
    check(d, q, p, sd, off, n, out)


def test_verify_zero_proposal_accepts():
    d, q, p, sd, off = _case(3, 2, 1024, seed=5)
    q[np.arange(3), 0, d[:, 0]] = 0.0
    n, out = verify_gpu(d, q, p, sd, off)
    assert (n >= 1).all()
    check(d, q, p, sd, off, n, out)


def test_verify_full_size_after_the_draft_block():
    """The B=88 (of 96) draft block's tokens and proposals, against targets
    p_k = 0.7 q_k + 0.3 softmax(noise) (p_K: softmax(noise)); every row runs on
    the GPU, rows 0, 40, 87, 88, 95 are checked against the oracle at full width."""
    import torch
    from ancestral_draft_token_amd import inputs
    from ancestral_draft_token_amd.device import DeviceProblem
    w = inputs.large_padded()
    say(f"draft {w.name}")
    prob = DeviceProblem(w)
    prob.enqueue()
    torch.cuda.synchronize()
    B, K, V = w.B, w.K, w.V
    g = torch.Generator(device="cuda:0").manual_seed(7)
    noise = torch.softmax(torch.randn((B, K + 1, V), device="cuda:0", generator=g) * 2.0, dim=-1)
    p = noise.clone()
    p[:, :K] = 0.7 * prob.q + 0.3 * noise[:, :K]
    p = p.contiguous()
    n = torch.empty(B, dtype=torch.int32, device="cuda:0")
    out = torch.empty((B, K + 1), dtype=torch.int32, device="cuda:0")
    wb = dspark_verify_workspace_bytes(B, K, V)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    seed = torch.from_numpy(np.ascontiguousarray(w.seed, np.int64)).to("cuda:0")
    off = torch.from_numpy(np.ascontiguousarray(w.offset, np.int64)).to("cuda:0")
    say("verify full size")
    dspark_verify_standard(prob.tokens, prob.q, p, seed, off, B, K, V, n, out, ws, wb)
    torch.cuda.synchronize()
    rows = np.array([0, 40, 87, 88, 95])
    idx = torch.from_numpy(rows).to("cuda:0")
    check(prob.tokens.index_select(0, idx).cpu().numpy(), prob.q.index_select(0, idx).cpu().numpy(),
          p.index_select(0, idx).cpu().numpy(), np.asarray(w.seed, np.int64)[rows],
          np.asarray(w.offset, np.int64)[rows], n.cpu().numpy()[rows], out.cpu().numpy()[rows])
    nn = n.cpu().numpy()
    assert ((nn >= 0) & (nn <= K)).all()
    say(f"accepted per row: mean {nn.mean():.2f}")


def test_verify_empty_residual_falls_back_to_the_target():
    """p_k = q_k / 2 (not normalised): the ratio is 1/2, so about half the
    positions reject, and max(0, p - q) is empty everywhere: both sides then
    draw the emitted token from p_k itself."""
    d, q, p, sd, off = _case(12, 3, 9000, seed=6)
    p[:, :3] = (0.5 * q.astype(np.float64)).astype(np.float32)
    n, out = verify_gpu(d, q, p, sd, off)
    assert (n < 3).any()
    check(d, q, p, sd, off, n, out)
