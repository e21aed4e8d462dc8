"""Pins of the oracle's standard token-level verification (CPU only).

The rule (accept d_k with probability min(1, p_k(d_k)/q_k(d_k)); at the first
rejection draw from max(0, p_k - q_k) normalised; a bonus draw from p_K when
every draft is accepted) is checked against what it guarantees, not against a
second copy of itself: every emitted token is distributed as the target p_k
whatever q is (Leviathan, Kalman and Matias, ICML 2023, section 2.3 and
appendix A.1), the acceptance probability at a position is sum_v min(p, q)
(same paper, section 3.1), and the special cases p = q and one-hot p. A wrong
ratio direction, a residual without max(0, .) or a bonus drawn from q all
fail one of these.
"""

from __future__ import annotations

import numpy as np
import pytest
from scipy import stats

import oracle


def _draws_from(q, rng, n):
    """n independent draws per row from the distributions q[..., V] (numpy's own generator)."""
    c = np.cumsum(q.astype(np.float64), axis=-1)
    u = rng.random(c.shape[:-1] + (n,)) if n > 1 else rng.random(c.shape[:-1])
    return (u[..., None] > c).sum(-1).clip(0, q.shape[-1] - 1)


@pytest.fixture(scope="module")
def lossless_run():
    rng = np.random.default_rng(2024)
    B, K, V = 40000, 2, 6
    p_rows = np.array([[0.05, 0.30, 0.10, 0.25, 0.20, 0.10],
                       [0.40, 0.05, 0.05, 0.20, 0.10, 0.20],
                       [0.10, 0.10, 0.30, 0.10, 0.30, 0.10]], dtype=np.float32)
    q_rows = np.array([[0.30, 0.05, 0.25, 0.10, 0.10, 0.20],
                       [0.10, 0.30, 0.20, 0.05, 0.30, 0.05]], dtype=np.float32)
    p = np.broadcast_to(p_rows, (B, K + 1, V)).copy()
    q = np.broadcast_to(q_rows, (B, K, V)).copy()
    d = np.stack([_draws_from(q_rows[k][None, :].repeat(B, 0), rng, 1) for k in range(K)], 1).astype(np.int32)
    seed = np.arange(B, dtype=np.int64) * 7919 + 11
    off = np.full(B, 3, dtype=np.int64)
    r = oracle.verify_standard(d, q, p, seed, off)
    return dict(B=B, K=K, V=V, p=p_rows, q=q_rows, r=r)


def _chi2_pvalue(samples, probs):
    counts = np.bincount(samples, minlength=len(probs)).astype(np.float64)
    p64 = probs.astype(np.float64)
    expected = p64 / p64.sum() * counts.sum()
    return stats.chisquare(counts, expected).pvalue


def test_first_emitted_token_follows_the_target(lossless_run):
    r = lossless_run["r"]
    assert _chi2_pvalue(r.out_tokens[:, 0], lossless_run["p"][0]) > 1e-4


def test_second_emitted_token_follows_the_target(lossless_run):
    r = lossless_run["r"]
    rows = r.n_accepted >= 1
    assert rows.sum() > 10000
    assert _chi2_pvalue(r.out_tokens[rows, 1], lossless_run["p"][1]) > 1e-4


def test_bonus_token_follows_the_last_target(lossless_run):
    r, K = lossless_run["r"], lossless_run["K"]
    rows = r.n_accepted == K
    assert rows.sum() > 3000
    assert _chi2_pvalue(r.out_tokens[rows, K], lossless_run["p"][K]) > 1e-4


def test_acceptance_rate_is_sum_of_minima(lossless_run):
    r, p, q, B = lossless_run["r"], lossless_run["p"], lossless_run["q"], lossless_run["B"]
    expect = float(np.minimum(p[0], q[0]).sum())
    got = float((r.n_accepted >= 1).mean())
    sigma = np.sqrt(expect * (1 - expect) / B)
    assert abs(got - expect) < 5 * sigma


def test_layout_of_the_outputs(lossless_run):
    r, K = lossless_run["r"], lossless_run["K"]
    for b in range(200):
        n = r.n_accepted[b]
        assert 0 <= n <= K
        assert (r.out_tokens[b, :n + 1] >= 0).all()
        assert (r.out_tokens[b, n + 1:] == -1).all()


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(5)
    B, K, V = 500, 4, 9
    p = rng.dirichlet(np.ones(V), size=(B, K + 1)).astype(np.float32)
    q = p[:, :K].copy()
    d = np.stack([_draws_from(q[:, k], rng, 1) for k in range(K)], 1).astype(np.int32)
    r = oracle.verify_standard(d, q, p, np.arange(B), np.zeros(B))
    assert (r.n_accepted == K).all()
    assert (r.out_tokens[:, :K] == d).all()


def test_one_hot_target_rejects_onto_its_token():
    B, K, V = 64, 3, 7
    rng = np.random.default_rng(9)
    a = rng.integers(0, V, size=B)
    p = np.zeros((B, K + 1, V), dtype=np.float32)
    p[np.arange(B), 0, a] = 1.0
    p[:, 1:, :] = 1.0 / V
    q = rng.dirichlet(np.ones(V), size=(B, K)).astype(np.float32)
    d = (a + 1 + rng.integers(0, V - 1, size=B)) % V      # never the target's token
    dd = np.stack([d] + [rng.integers(0, V, size=B)] * (K - 1), 1).astype(np.int32)
    r = oracle.verify_standard(dd, q, p, np.arange(B), np.zeros(B))
    assert (r.n_accepted == 0).all()
    assert (r.out_tokens[:, 0] == a).all()
    assert (r.out_tokens[:, 1:] == -1).all()


def test_zero_proposal_with_positive_target_accepts():
    V = 5
    p = np.full((1, 2, V), 0.2, dtype=np.float32)
    q = np.zeros((1, 1, V), dtype=np.float32)
    q[0, 0, 0] = 1.0
    r = oracle.verify_standard(np.array([[3]], np.int32), q, p, [1], [0])
    assert r.n_accepted[0] == 1 and r.out_tokens[0, 0] == 3


def test_uniforms_come_from_the_stated_counter():
    """The acceptance uniform of position k is word 0 of Philox4x32-10 at counter
    (0xFFFFFFFF, 256 + k, lo32(offset), hi32(offset)) under key (lo32, hi32)(seed)."""
    seed, off = 0x0123456789ABCDEF, 0x1122334455667788
    for k in (0, 1, 6):
        x = oracle.philox4x32_10([0xFFFFFFFF, 256 + k, off & 0xFFFFFFFF, off >> 32],
                                 [seed & 0xFFFFFFFF, seed >> 32])[0]
        assert oracle.verify_uniform(seed, off, k) == np.float32(((int(x) >> 9) + 0.5) / 2**23)
