"""Pins of the windowed block-attention oracle (CPU only).

- With a window that covers every key, the result is plain non-causal
  attention: torch's scaled_dot_product_attention (float64, CPU, key/value
  heads repeated for GQA) and torch.logsumexp give o and the log-sum-exp.
- The pages' lowering, a causal sliding-window decode merged by log-sum-exp
  with the block keys after each query, equals the direct two-sided
  definition (both halves and the merge are separate code paths).
- The window edge: the key at distance W-1 from a query changes its output,
  the key at distance W does not.
- One key: o = v and lse = scale <q, k>; two keys: the closed form.
A window off by one, a log-sum-exp left in another base, a merge with the
wrong weights or a wrong GQA head map fails one of these.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import window_attn as wa


def _case(B, K, Hq, Hkv, D, L, P, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, size=(B, K, Hq, D))
    kc = rng.normal(0, 1, size=(B, L, Hkv, D))
    vc = rng.normal(0, 1, size=(B, L, Hkv, D))
    return q, kc, vc, np.asarray(P, dtype=np.int64)


@pytest.mark.parametrize("B,K,Hq,Hkv,D,P", [(2, 3, 4, 1, 16, [5, 9]), (1, 7, 8, 2, 8, [12]), (3, 1, 2, 2, 4, [0, 3, 6])])
def test_full_window_is_plain_attention(B, K, Hq, Hkv, D, P):
    L = max(P) + K
    q, kc, vc, P = _case(B, K, Hq, Hkv, D, L, P, seed=B * 10 + K)
    scale = 1.0 / math.sqrt(D)
    o, lse = wa.window_block_attention(q, kc, vc, P, window=10**6, scale=scale)
    G = Hq // Hkv
    for b in range(B):
        n = int(P[b]) + K
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)                                   # [Hq,K,D]
        kt = torch.from_numpy(kc[b, :n]).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq,n,D]
        vt = torch.from_numpy(vc[b, :n]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(o[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
        ref_lse = torch.logsumexp(scale * (qt @ kt.transpose(1, 2)), dim=-1)          # [Hq,K]
        np.testing.assert_allclose(lse[b], ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W,P", [(5, [0, 3, 4, 5, 11]), (9, [7, 8, 9, 20, 2]), (4, [1, 6, 30, 3, 4])])
def test_causal_decode_plus_later_keys_is_the_two_sided_window(W, P):
    B, K, Hq, Hkv, D = len(P), 4, 4, 2, 8
    L = max(P) + K + 3
    q, kc, vc, P = _case(B, K, Hq, Hkv, D, L, P, seed=W)
    scale = 0.3
    o, lse = wa.window_block_attention(q, kc, vc, P, W, scale)
    o1, l1 = wa.causal_window_decode(q, kc, vc, P, W, scale)
    o2, l2 = wa.later_block_keys(q, kc, vc, P, scale)
    assert np.isneginf(l2[:, K - 1]).all()          # the last query has no later block key
    om, lm = wa.lse_merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=1e-12, atol=1e-12)


def test_window_edge():
    B, K, Hq, Hkv, D, W = 1, 3, 2, 1, 8, 8
    P = [20]
    q, kc, vc, P = _case(B, K, Hq, Hkv, D, 30, P, seed=5)
    o, _ = wa.window_block_attention(q, kc, vc, P, W, 0.5)
    for k in range(K):
        i = 20 + k
        inside, outside = i - (W - 1), i - W
        v2 = vc.copy()
        v2[0, inside] += 3.0
        o_in, _ = wa.window_block_attention(q, kc, v2, P, W, 0.5)
        assert np.abs(o_in[0, k] - o[0, k]).max() > 1e-3
        v3 = vc.copy()
        v3[0, outside] += 3.0
        o_out, _ = wa.window_block_attention(q, kc, v3, P, W, 0.5)
        assert np.array_equal(o_out[0, k], o[0, k])
    # keys past the block do not exist for the attention
    v4 = vc.copy()
    v4[0, 23:] += 5.0
    o_past, _ = wa.window_block_attention(q, kc, v4, P, W, 0.5)
    assert np.array_equal(o_past, o)


def test_one_and_two_keys_closed_form():
    rng = np.random.default_rng(3)
    D = 6
    q = rng.normal(size=(1, 1, 1, D))
    kc = rng.normal(size=(1, 2, 1, D))
    vc = rng.normal(size=(1, 2, 1, D))
    o, lse = wa.window_block_attention(q, kc, vc, [0], 4, 0.7)
    assert np.allclose(o[0, 0, 0], vc[0, 0, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.7 * float(q[0, 0, 0] @ kc[0, 0, 0])) < 1e-14
    o, lse = wa.window_block_attention(q, kc, vc, [1], 4, 0.7)
    s1, s2 = (0.7 * float(q[0, 0, 0] @ kc[0, t, 0]) for t in (0, 1))
    assert abs(lse[0, 0, 0] - math.log(math.exp(s1) + math.exp(s2))) < 1e-14
    want = (math.exp(s1) * vc[0, 0, 0] + math.exp(s2) * vc[0, 1, 0]) / (math.exp(s1) + math.exp(s2))
    assert np.allclose(o[0, 0, 0], want, rtol=0, atol=1e-14)


def test_rows_match_the_batch_form():
    B, K, Hq, Hkv, D, W = 2, 3, 4, 2, 8, 6
    q, kc, vc, P = _case(B, K, Hq, Hkv, D, 20, [9, 14], seed=8)
    o, lse = wa.window_block_attention(q, kc, vc, P, W, 0.25)
    rows = [(0, 0, 0), (1, 2, 3), (0, 1, 2)]
    ro, rl = wa.window_block_attention_rows(q, kc, vc, P, W, 0.25, rows)
    for n, (b, k, h) in enumerate(rows):
        assert np.array_equal(ro[n], o[b, k, h]) and rl[n] == lse[b, k, h]
