"""CPU oracle for DSpark's non-causal windowed block attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does, and the two
share no code. Plain numpy in float64.

What it computes ("brb-nv/TensorRT-LLM pull 21", section "1. Non-causal
DSpark draft blocks on TRTLLM (default path)", and "Serve MiniMax-M3.1-Flash
with its bundled DSpark drafter", the modeling_dspark.py / modeling_dflash.py
note): the drafter's windowed GQA layers are non-causal inside the draft
block with a two-sided window (W-1, W-1). A draft block of K queries sits at
positions P .. P+K-1 after a context of P tokens; query i = P + k attends
every key t with |i - t| <= W - 1 among the P + K keys that exist (the
whole draft block, plus the context keys no more than W - 1 positions
back). Per query head h
(GQA: key/value head h // (Hq / Hkv)):
    s_t = scale * <q_h, k_t>,   lse = ln sum_t exp(s_t),
    o = sum_t exp(s_t - lse) v_t.
The pages serve it as a causal sliding-window decode (keys i-W+1 .. i) that
returns its log-sum-exp, merged with the block keys after the query
(i+1 .. P+K-1); ``causal_window_decode``, ``later_block_keys`` and
``lse_merge`` state that lowering, which the tests check against the direct
definition.

Readings (the pages leave them open; each is listed in the design notes):
- the log-sum-exp is returned in natural-log units (the pages convert the
  decode kernel's base-2 value);
- K <= W, so the upper side of the window never cuts the block.
"""

from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _attend(q, keys, vals, scale):
    """Softmax attention of one query over a key set: (o, lse); an empty set
    gives (0, -inf)."""
    if keys.shape[0] == 0:
        return np.zeros(vals.shape[-1]), -np.inf
    s = scale * (keys @ q)
    m = s.max()
    e = np.exp(s - m)
    tot = e.sum()
    return (e / tot) @ vals, m + np.log(tot)


def _check(q, k_cache, v_cache, ctx_len):
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, K, Hq, D = q.shape
    Bk, L, Hkv, Dk = kc.shape
    if Bk != B or Dk != D or vc.shape != kc.shape or Hq % Hkv:
        raise ValueError("shapes: q [B,K,Hq,D], k_cache and v_cache [B,L,Hkv,D], Hq a multiple of Hkv")
    P = np.asarray(ctx_len, dtype=np.int64).reshape(B)
    if (P < 0).any() or (P + K > L).any():
        raise ValueError("need 0 <= ctx_len and ctx_len + K <= L")
    return q, kc, vc, P, B, K, Hq, Hkv, D


def _by_range(q, k_cache, v_cache, ctx_len, scale, bounds):
    """Attention of every query over keys [lo, hi) given by bounds(P, K, k)."""
    q, kc, vc, P, B, K, Hq, Hkv, D = _check(q, k_cache, v_cache, ctx_len)
    G = Hq // Hkv
    o = np.zeros((B, K, Hq, D))
    lse = np.full((B, K, Hq), -np.inf)
    for b in range(B):
        for k in range(K):
            lo, hi = bounds(int(P[b]), K, k)
            for h in range(Hq):
                o[b, k, h], lse[b, k, h] = _attend(q[b, k, h], kc[b, lo:hi, h // G], vc[b, lo:hi, h // G], scale)
    return o, lse


def window_block_attention(q, k_cache, v_cache, ctx_len, window, scale):
    """The direct definition: query i = P + k attends keys t in
    [max(0, i - (W-1)), min(P + K, i + W)). Returns (o [B,K,Hq,D], lse [B,K,Hq])
    in float64."""
    W = int(window)
    return _by_range(q, k_cache, v_cache, ctx_len, scale,
                     lambda P, K, k: (max(0, P + k - (W - 1)), min(P + K, P + k + W)))


def causal_window_decode(q, k_cache, v_cache, ctx_len, window, scale):
    """The pages' first half: causal sliding-window decode, keys
    [max(0, i - (W-1)), i] for query i = P + k."""
    W = int(window)
    return _by_range(q, k_cache, v_cache, ctx_len, scale,
                     lambda P, K, k: (max(0, P + k - (W - 1)), P + k + 1))


def later_block_keys(q, k_cache, v_cache, ctx_len, scale):
    """The pages' second half: the block keys after each query, (i, P + K)."""
    return _by_range(q, k_cache, v_cache, ctx_len, scale, lambda P, K, k: (P + k + 1, P + K))


def lse_merge(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint key sets from each set's
    (o, lse): lse = ln(e^lse1 + e^lse2), o = e^(lse1-lse) o1 + e^(lse2-lse) o2.
    An empty set (lse = -inf) contributes nothing."""
    lse1, lse2 = _f64(lse1), _f64(lse2)
    lse = np.logaddexp(lse1, lse2)
    safe = np.where(np.isfinite(lse), lse, 0.0)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - safe), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - safe), 0.0)
    return w1[..., None] * _f64(o1) + w2[..., None] * _f64(o2), lse


def window_block_attention_rows(q, k_cache, v_cache, ctx_len, window, scale, rows):
    """The direct definition for selected (b, k, h) triples only (full-size
    checks): returns (o [n,D], lse [n])."""
    W = int(window)
    q = np.asarray(q)
    B, K, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    P = np.asarray(ctx_len, dtype=np.int64).reshape(B)
    o = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    for n, (b, k, h) in enumerate(rows):
        i = int(P[b]) + k
        lo, hi = max(0, i - (W - 1)), min(int(P[b]) + K, i + W)
        o[n], lse[n] = _attend(_f64(q[b, k, h]), _f64(k_cache[b, lo:hi, h // G]), _f64(v_cache[b, lo:hi, h // G]),
                               scale)
    return o, lse
