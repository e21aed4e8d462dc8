"""GPU block verification vs the CPU oracle, through the C ABI.

Weights, residual masses and thresholds are double on both sides and only
the order in which the GPU sums each residual mass differs, so the number of
accepted drafts must match exactly unless a uniform lies within 1e-9 of its
threshold (the oracle reports that margin; such rows are counted and their
draw is not compared). The emitted token is a Gumbel-max draw: the oracle's,
or one of its near-tied candidates. Cases: small and ragged vocabularies
(K = 0 and K = 1 among them), equal distributions, a one-hot target, a case
where the block rule keeps drafts past a failed test, an unnormalised target
whose residuals are all empty (the fallback), and the full-size B=88 draft
block's own tokens and proposals (2048-column chunks).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from ancestral_draft_token_amd import dspark_init, dspark_verify_block, dspark_verify_block_workspace_bytes

from gpu_util import require_gpu, say
from test_gpu_verify import _case

pytestmark = pytest.mark.gpu

TAU_EPS = 1e-9


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def verify_block_gpu(d, q, p, sd, off):
    import torch
    dspark_init()
    B, K = d.shape
    V = p.shape[-1]
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    dd, qq, pp, ss, oo = t(d), t(q) if K else None, t(p), t(sd), t(off)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    wb = dspark_verify_block_workspace_bytes(B, K, V)
    ws = torch.empty(max(wb, 256), dtype=torch.uint8, device=dev)
    say(f"verify_block B={B} K={K} V={V}")
    dspark_verify_block(dd, qq, pp, ss, oo, B, K, V, n, out, ws, wb)
    torch.cuda.synchronize()
    return n.cpu().numpy(), out.cpu().numpy()


def check_block(d, q, p, sd, off, n_gpu, out_gpu):
    qq = q if q is not None else np.zeros(d.shape + (p.shape[-1],), np.float32)
    ref = oracle.verify_block(d, qq, p, sd, off)
    B, K = d.shape
    near_tau = near = 0
    for b in range(B):
        n = int(ref.n_accepted[b])
        if int(n_gpu[b]) != n:
            assert ref.tau_margin[b] < TAU_EPS, (b, int(n_gpu[b]), n, ref.tau_margin[b])
            near_tau += 1
            continue
        assert (out_gpu[b, :n] == ref.out_tokens[b, :n]).all()
        assert (out_gpu[b, n + 1:] == -1).all()
        tok, want = int(out_gpu[b, n]), int(ref.out_tokens[b, n])
        if tok != want:
            assert ref.margin[b] <= oracle.TIE_EPS, (b, tok, want, ref.margin[b])
            assert tok in set(ref.cand[b][: ref.ncand[b]].tolist()), (b, tok)
            near += 1
    assert near_tau <= max(1, B // 100)
    say(f"block parity ok: rows {B}, accepted {int(ref.n_accepted.sum())}, near-threshold rows {near_tau}, "
        f"near-tie draws {near}")
    return ref


@pytest.mark.parametrize("B,K,V", [(6, 3, 1000), (3, 7, 8192), (4, 2, 20000), (2, 0, 4096), (5, 1, 16388),
                                   (17, 7, 2056), (9, 5, 12292)])
def test_verify_block_shapes(B, K, V):
    d, q, p, sd, off = _case(B, K, V, seed=B * 1000 + K * 10 + V % 89, mix=0.8)
    n, out = verify_block_gpu(d, q, p, sd, off)
    check_block(d, q, p, sd, off, n, out)


def test_verify_block_keeps_drafts_past_a_failed_test():
    """Many rows, target close to the draft: some row must keep a prefix whose
    earlier test failed (the token-level rule would have stopped there)."""
    B, K, V = 64, 7, 3000
    d, q, p, sd, off = _case(B, K, V, seed=21, mix=0.9)
    n, out = verify_block_gpu(d, q, p, sd, off)
    ref = check_block(d, q, p, sd, off, n, out)
    bw = oracle.verify_block_weights(d, q, p, want_resid=False)
    past = 0
    for b in range(B):
        eta = [oracle.verify_uniform(int(sd[b]), int(off[b]), j - 1) for j in range(1, int(ref.n_accepted[b]) + 1)]
        past += any(not (e < bw.h[b, j + 1]) for j, e in enumerate(eta))
    assert past > 0


def test_verify_block_equal_distributions_accept_everything():
    d, q, p, sd, off = _case(8, 5, 3000, seed=3, mix=1.0)
    p[:, :5] = q
    n, out = verify_block_gpu(d, q, p, sd, off)
    assert (n == 5).all()
    check_block(d, q, p, sd, off, n, out)


def test_verify_block_one_hot_target_rejects_onto_its_token():
    B, K, V = 6, 3, 5000
    d, q, p, sd, off = _case(B, K, V, seed=4)
    a = (d[:, 0] + 7) % V
    p[:, 0] = 0.0
    p[np.arange(B), 0, a] = 1.0
    n, out = verify_block_gpu(d, q, p, sd, off)
    assert (n == 0).all() and (out[:, 0] == a).all() and (out[:, 1:] == -1).all()
    check_block(d, q, p, sd, off, n, out)


def test_verify_block_empty_residual_falls_back_to_the_target():
    """p_k = q_k / 2: every residual max(w p - q, 0) is empty; rows that stop
    before K draw the emitted token from p_n itself."""
    d, q, p, sd, off = _case(12, 3, 9000, seed=6)
    p[:, :3] = (0.5 * q.astype(np.float64)).astype(np.float32)
    n, out = verify_block_gpu(d, q, p, sd, off)
    assert (n < 3).any()
    check_block(d, q, p, sd, off, n, out)


def test_verify_block_full_size_after_the_draft_block():
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
    wb = dspark_verify_block_workspace_bytes(B, K, V)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    seed = torch.from_numpy(np.ascontiguousarray(w.seed, np.int64)).to("cuda:0")
    off = torch.from_numpy(np.ascontiguousarray(w.offset, np.int64)).to("cuda:0")
    say("verify_block full size")
    dspark_verify_block(prob.tokens, prob.q, p, seed, off, B, K, V, n, out, ws, wb)
    torch.cuda.synchronize()
    rows = np.array([0, 40, 87, 88, 95])
    idx = torch.from_numpy(rows).to("cuda:0")
    check_block(prob.tokens.index_select(0, idx).cpu().numpy(), prob.q.index_select(0, idx).cpu().numpy(),
                p.index_select(0, idx).cpu().numpy(), np.asarray(w.seed, np.int64)[rows],
                np.asarray(w.offset, np.int64)[rows], n.cpu().numpy()[rows], out.cpu().numpy()[rows])
    nn = n.cpu().numpy()
    assert ((nn >= 0) & (nn <= K)).all()
    say(f"accepted per row: mean {nn.mean():.2f}")


@pytest.mark.parametrize("rule", ["standard", "block"])
def test_verification_clamps_draft_tokens(rule):
    """Draft tokens are device data: out-of-range ids are clamped into [0, V)
    by both rules, as the oracle does, and the emitted prefix holds the
    clamped ids."""
    from test_gpu_verify import verify_gpu, check
    B, K, V = 6, 4, 3000
    d, q, p, sd, off = _case(B, K, V, seed=41, mix=0.95)
    d[:, 0] = np.array([-5, V + 3, -1, V, 2 * V, -(2**31)], dtype=np.int32)
    if rule == "standard":
        n, out = verify_gpu(d, q, p, sd, off)
        ref = check(d, q, p, sd, off, n, out)
    else:
        n, out = verify_block_gpu(d, q, p, sd, off)
        ref = check_block(d, q, p, sd, off, n, out)
    clamped = np.clip(d[:, 0].astype(np.int64), 0, V - 1)
    for b in range(B):
        if n[b] >= 1:
            assert out[b, 0] == clamped[b]
