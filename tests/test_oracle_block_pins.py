"""Pins of the oracle's block verification (CPU only).

Block verification (Sun et al., "Block Verification Accelerates Speculative
Decoding", 2024) is checked against what it guarantees, not against a second
copy of its formulas:
- losslessness, exactly: on tiny vocabularies with a target and a drafter
  that depend on the whole prefix, every draft path is enumerated with its
  probability, every stopping point with the probability the oracle's
  thresholds give it, and every emitted token with the oracle's emission
  weights; the output, continued by the target, must have exactly the
  target's joint distribution over K+1 tokens;
- its expected number of accepted drafts, which follows from the
  definitions as sum over j and prefixes x^j of
  min_i Ms(x^{i-1}) Mb(x_i .. x_j | x^{i-1}), and is at least the
  token-level rule's sum over j of prod_i min(q_i, p_i);
- losslessness of the sampled outputs by chi-square, the check the pages
  list for the rule;
- K = 1, where the rule is the token-level one;
- the stopping point is the last position whose uniform passes its
  threshold, and the special cases p = q and a one-hot target.
A threshold with a wrong denominator, an uncapped or shifted prefix weight,
or a residual taken at the wrong position fails the exact check.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest
from scipy import stats

import oracle


# ---- a tiny prefix-dependent target and drafter -----------------------------

def _tree(rng, V, K, zero_frac=0.0):
    """p(.|prefix) for prefixes of length 0..K and q(.|prefix) for 0..K-1, as
    float32 rows that sum to 1 (some q entries zero when zero_frac > 0)."""
    def dist(allow_zero):
        x = rng.gamma(0.6, size=V)
        if allow_zero:
            x[rng.random(V) < zero_frac] = 0.0
            if x.sum() == 0.0:
                x[rng.integers(V)] = 1.0
        x = (x / x.sum()).astype(np.float32)
        return x
    p, q = {}, {}
    for n in range(K + 1):
        for pre in itertools.product(range(V), repeat=n):
            p[pre] = dist(False)
            if n < K:
                q[pre] = dist(True)
    return p, q


def _joint(table, seq):
    """prod_i table[seq[:i]][seq[i]] in float64."""
    out = 1.0
    for i, x in enumerate(seq):
        out *= float(table[tuple(seq[:i])][x])
    return out


def _enumerate(p, q, V, K):
    """Exact distribution of the output continued by the target, and the
    expected number of accepted drafts, from the oracle's thresholds and
    emission weights."""
    paths = [x for x in itertools.product(range(V), repeat=K) if _joint(q, x) > 0.0]
    d = np.array(paths, dtype=np.int32).reshape(len(paths), K)
    qs = np.stack([np.stack([q[x[:j]] for j in range(K)]) for x in paths])
    ps = np.stack([np.stack([p[x[:j]] for j in range(K + 1)]) for x in paths])
    bw = oracle.verify_block_weights(d, qs, ps)
    full = {}
    e_tau = 0.0
    for r, x in enumerate(paths):
        ms = _joint(q, x)
        h = bw.h[r]
        for j in range(K + 1):
            p_tau = h[j] * np.prod(1.0 - h[j + 1:])        # stop at j: pass j, fail every later test
            if p_tau == 0.0:
                continue
            e_tau += ms * p_tau * j
            wts = bw.resid[r, j].astype(np.float64)
            if j < K and wts.sum() == 0.0:
                wts = ps[r, j].astype(np.float64)            # the empty-residual fallback
            wts = wts / wts.sum()
            for y in range(V):
                if wts[y] == 0.0:
                    continue
                head = tuple(x[:j]) + (y,)
                mass = ms * p_tau * wts[y]
                # continue the output with the target up to K+1 tokens
                for tail in itertools.product(range(V), repeat=K - j):
                    s = head + tail
                    cont = 1.0
                    for i in range(j + 1, K + 1):
                        cont *= float(p[s[:i]][s[i]])
                    full[s] = full.get(s, 0.0) + mass * cont
    return full, e_tau


@pytest.mark.parametrize("V,K,zero_frac,seed", [(3, 2, 0.0, 1), (3, 3, 0.0, 2), (4, 2, 0.3, 3),
                                               (2, 4, 0.0, 4), (3, 3, 0.34, 5)])
def test_block_verification_is_exactly_lossless(V, K, zero_frac, seed):
    rng = np.random.default_rng(seed)
    p, q = _tree(rng, V, K, zero_frac)
    full, _ = _enumerate(p, q, V, K)
    worst = 0.0
    for s in itertools.product(range(V), repeat=K + 1):
        worst = max(worst, abs(full.get(s, 0.0) - _joint(p, s)))
    assert worst < 2e-6, worst


@pytest.mark.parametrize("V,K,seed", [(3, 2, 11), (3, 3, 12), (4, 3, 13)])
def test_expected_accepted_drafts_closed_form(V, K, seed):
    rng = np.random.default_rng(seed)
    p, q = _tree(rng, V, K)
    _, e_tau = _enumerate(p, q, V, K)
    closed = 0.0
    token_level = 0.0
    for j in range(1, K + 1):
        for x in itertools.product(range(V), repeat=j):
            terms = []
            for i in range(1, j + 2):   # Ms of the first i-1 drafts, Mb of the rest
                ms = _joint(q, x[:i - 1])
                mb = 1.0
                for l in range(i - 1, j):
                    mb *= float(p[x[:l]][x[l]])
                terms.append(ms * mb)
            closed += min(terms)
            tl = 1.0
            for l in range(j):
                tl *= min(float(q[x[:l]][x[l]]), float(p[x[:l]][x[l]]))
            token_level += tl
    assert abs(e_tau - closed) < 1e-6, (e_tau, closed)
    assert e_tau >= token_level - 1e-9, (e_tau, token_level)


# ---- the sampler --------------------------------------------------------------

def _draws_from(q, rng):
    c = np.cumsum(q.astype(np.float64), axis=-1)
    u = rng.random(c.shape[:-1])
    return (u[..., None] > c).sum(-1).clip(0, q.shape[-1] - 1)


@pytest.fixture(scope="module")
def sampled_run():
    rng = np.random.default_rng(77)
    B, K, V = 40000, 3, 4
    p_rows = np.array([[0.10, 0.40, 0.20, 0.30],
                       [0.35, 0.15, 0.25, 0.25],
                       [0.05, 0.25, 0.45, 0.25],
                       [0.30, 0.30, 0.20, 0.20]], dtype=np.float32)
    q_rows = np.array([[0.40, 0.10, 0.25, 0.25],
                       [0.10, 0.40, 0.20, 0.30],
                       [0.25, 0.25, 0.25, 0.25]], dtype=np.float32)
    p = np.broadcast_to(p_rows, (B, K + 1, V)).copy()
    q = np.broadcast_to(q_rows, (B, K, V)).copy()
    d = np.stack([_draws_from(np.broadcast_to(q_rows[k], (B, V)), rng) for k in range(K)], 1).astype(np.int32)
    seed = np.arange(B, dtype=np.int64) * 104729 + 5
    off = np.full(B, 9, dtype=np.int64)
    r = oracle.verify_block(d, q, p, seed, off)
    # continue each output with the (prefix-free) target up to K+1 tokens
    ext = r.out_tokens.copy()
    for j in range(K + 1):
        short = ext[:, j] < 0
        ext[short, j] = _draws_from(np.broadcast_to(p_rows[j], (int(short.sum()), V)), rng)
    return dict(B=B, K=K, V=V, p=p_rows, q=q_rows, d=d, seed=seed, off=off, r=r, ext=ext,
                q_full=q, p_full=p)


def test_sampled_outputs_follow_the_target(sampled_run):
    ext, p = sampled_run["ext"], sampled_run["p"].astype(np.float64)
    V = sampled_run["V"]
    for j in range(sampled_run["K"] + 1):
        counts = np.bincount(ext[:, j], minlength=V).astype(np.float64)
        assert stats.chisquare(counts, p[j] / p[j].sum() * counts.sum()).pvalue > 1e-4, j
    pair = ext[:, 0] * V + ext[:, 1]
    counts = np.bincount(pair, minlength=V * V).astype(np.float64)
    expected = np.outer(p[0] / p[0].sum(), p[1] / p[1].sum()).ravel() * counts.sum()
    assert stats.chisquare(counts, expected).pvalue > 1e-4


def test_block_accepts_more_than_token_level_on_average(sampled_run):
    s = sampled_run
    tl = oracle.verify_standard(s["d"], s["q_full"], s["p_full"], s["seed"], s["off"])
    assert s["r"].n_accepted.mean() > tl.n_accepted.mean()


def test_stop_is_the_last_passing_position():
    rng = np.random.default_rng(8)
    B, K, V = 300, 5, 40
    q = rng.dirichlet(np.full(V, 0.5), size=(B, K)).astype(np.float32)
    p = np.concatenate([0.6 * q + 0.4 * rng.dirichlet(np.full(V, 0.5), size=(B, K)),
                        rng.dirichlet(np.full(V, 0.5), size=(B, 1))], 1).astype(np.float32)
    d = np.stack([_draws_from(q[:, k], rng) for k in range(K)], 1).astype(np.int32)
    seed = rng.integers(0, 2**62, size=B).astype(np.int64)
    off = rng.integers(0, 2**40, size=B).astype(np.int64)
    r = oracle.verify_block(d, q, p, seed, off)
    bw = oracle.verify_block_weights(d, q, p, want_resid=False)
    for b in range(B):
        eta = [oracle.verify_uniform(int(seed[b]), int(off[b]), j - 1) for j in range(1, K + 1)]
        passing = [j for j in range(1, K + 1) if eta[j - 1] < bw.h[b, j]]
        n = max(passing) if passing else 0
        assert r.n_accepted[b] == n
        assert list(r.out_tokens[b, :n]) == list(d[b, :n])
        assert np.all(r.out_tokens[b, n + 1:] == -1)
        assert 0 <= r.out_tokens[b, n] < V
    # the rule does use later positions: some row stops after a failed test
    fails_before = 0
    for b in range(B):
        n = r.n_accepted[b]
        eta = [oracle.verify_uniform(int(seed[b]), int(off[b]), j - 1) for j in range(1, n + 1)]
        fails_before += any(not (eta[j - 1] < bw.h[b, j]) for j in range(1, n + 1))
    assert fails_before > 0


def test_single_position_is_the_token_level_rule():
    rng = np.random.default_rng(9)
    B, K, V = 3000, 1, 64
    q = rng.dirichlet(np.full(V, 0.4), size=(B, K)).astype(np.float32)
    p = rng.dirichlet(np.full(V, 0.4), size=(B, K + 1)).astype(np.float32)
    d = np.stack([_draws_from(q[:, 0], rng)], 1).astype(np.int32)
    seed = np.arange(B, dtype=np.int64) + 100
    off = np.zeros(B, dtype=np.int64)
    rb = oracle.verify_block(d, q, p, seed, off)
    rs = oracle.verify_standard(d, q, p, seed, off)
    ratio = p[np.arange(B), 0, d[:, 0]].astype(np.float64) / q[np.arange(B), 0, d[:, 0]].astype(np.float64)
    eta = np.array([oracle.verify_uniform(int(s), 0, 0) for s in seed])
    clear = np.abs(eta - ratio) > 1e-6
    assert np.array_equal(rb.n_accepted[clear], rs.n_accepted[clear])
    same_n = clear & (rb.n_accepted == rs.n_accepted)
    # the emitted draws agree unless the residual's rounding moved a near-tie
    differ = same_n & np.any(rb.out_tokens != rs.out_tokens, axis=1)
    assert np.all(np.minimum(rb.margin[differ], rs.margin[differ]) < 1e-4)
    assert differ.sum() <= 2
    assert 0.2 < rb.n_accepted.mean() < 0.8


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(10)
    B, K, V = 200, 6, 50
    q = rng.dirichlet(np.ones(V), size=(B, K)).astype(np.float32)
    p = np.concatenate([q, rng.dirichlet(np.ones(V), size=(B, 1)).astype(np.float32)], 1)
    d = np.stack([_draws_from(q[:, k], rng) for k in range(K)], 1).astype(np.int32)
    r = oracle.verify_block(d, q, p, np.arange(B), np.zeros(B))
    assert np.all(r.n_accepted == K)


def test_one_hot_target_rejects_onto_its_token():
    rng = np.random.default_rng(12)
    B, K, V = 100, 4, 30
    q = rng.dirichlet(np.ones(V), size=(B, K)).astype(np.float32)
    q[:, 0, 7] = 0.0
    q /= q.sum(-1, keepdims=True)
    p = rng.dirichlet(np.ones(V), size=(B, K + 1)).astype(np.float32)
    p[:, 0] = 0.0
    p[:, 0, 7] = 1.0
    d = np.stack([_draws_from(q[:, k], rng) for k in range(K)], 1).astype(np.int32)
    r = oracle.verify_block(d, q, p, np.arange(B) * 3, np.ones(B))
    assert np.all(r.n_accepted == 0)
    assert np.all(r.out_tokens[:, 0] == 7)
