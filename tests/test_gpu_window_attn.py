"""GPU non-causal windowed block attention vs the float64 oracle, through the C ABI.

Tolerances follow from the arithmetic: scores are exact bf16 products summed
in float32 (an error far below 2e-4 in the log-sum-exp at these sizes), and
the probabilities are rounded to bf16 before the product with V while the
normaliser keeps them in float32. With w_t the exact attention weights, an
output component is o_d = sum_t w_t (1 + e_t) v_td with independent rounding
errors |e_t| <= 2^-8 of mean zero (round to nearest even of varied values),
so its error has standard deviation at most 2^-8 / sqrt(3) * sqrt(sum_t w_t^2
v_td^2); the test allows six of those, plus 1e-5 * sum_t w_t |v_td| for the
float32 scores and normaliser and 1e-6 absolute. At W = 4096 that is a few
1e-4 against outputs of ~0.03, so a missing or repeated key tile fails it.
Cases: a window over part of the context, contexts around the window
edge (P = 0, W-1, W, W+1), K = 1..8 and K = W, the pages' head layouts 16/1
and 64/4, the 4096-token window, both launch forms (below and from 256 (row,
key/value head) pairs), and the full-size benchmark shape (B=88, P=8192) on
sampled (row, position, head) triples.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import window_attn as wa
from ancestral_draft_token_amd import (DSPARK_KV_LAYOUT_BHLD, DSPARK_KV_LAYOUT_BLHD, dspark_init,
                                       dspark_window_attention_workspace_bytes, dspark_window_block_attention)

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _inputs(B, K, Hq, Hkv, L, seed):
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    q = torch.randn((B, K, Hq, D), device="cuda:0", generator=g).to(torch.bfloat16)
    kc = torch.randn((B, L, Hkv, D), device="cuda:0", generator=g).to(torch.bfloat16)
    vc = torch.randn((B, L, Hkv, D), device="cuda:0", generator=g).to(torch.bfloat16)
    return q, kc, vc


def run_gpu(q, kc, vc, P, W, scale, layout=None):
    """The attention on caches kc, vc given as [B, L, Hkv, D]; with layout
    DSPARK_KV_LAYOUT_BHLD they are passed head-major ([B, Hkv, L, D] copies)."""
    import torch
    dspark_init()
    B, K, Hq, _ = q.shape
    L, Hkv = kc.shape[1], kc.shape[2]
    if layout == DSPARK_KV_LAYOUT_BHLD:
        kc, vc = kc.permute(0, 2, 1, 3).contiguous(), vc.permute(0, 2, 1, 3).contiguous()
    ctx = torch.tensor(P, dtype=torch.int32, device="cuda:0")
    out = torch.empty((B, K, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, K, Hq), dtype=torch.float32, device="cuda:0")
    wb = dspark_window_attention_workspace_bytes(B, K, Hq, Hkv, D, L, W)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda:0")
    say(f"window attention B={B} K={K} Hq={Hq} Hkv={Hkv} L={L} W={W} P={list(P)[:8]} layout={layout}")
    dspark_window_block_attention(q, kc, vc, ctx, B, K, Hq, Hkv, D, L, W, scale, out, lse, ws, wb, layout=layout)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _f64(t):
    import torch
    return t.to(torch.float32).cpu().numpy().astype(np.float64)


def rounding_tolerance(qv, kv, vv, lse_ref, scale):
    """Per-component output tolerance for one (row, position, head): qv [D], kv
    and vv [n, D] the keys and values it attends (float64), lse_ref its exact
    log-sum-exp; see the module docstring."""
    w = np.exp(scale * (kv @ qv) - lse_ref)
    rms = np.sqrt((w[:, None] ** 2 * vv ** 2).sum(axis=0))
    tot = (w[:, None] * np.abs(vv)).sum(axis=0)
    return 6.0 * 2.0 ** -8 / math.sqrt(3.0) * rms + 1e-5 * tot + 1e-6


def window_tolerance(q, kc, vc, P, W, scale, lse_ref):
    """rounding_tolerance for every (row, position, head), the window of the
    direct definition."""
    B, K, Hq, _ = q.shape
    G = Hq // kc.shape[2]
    tol = np.zeros(q.shape)
    for b in range(B):
        for k in range(K):
            i = int(P[b]) + k
            lo, hi = max(0, i - (W - 1)), min(int(P[b]) + K, i + W)
            for h in range(Hq):
                tol[b, k, h] = rounding_tolerance(q[b, k, h], kc[b, lo:hi, h // G], vc[b, lo:hi, h // G],
                                                  lse_ref[b, k, h], scale)
    return tol


def check(o, lse, o_ref, lse_ref, tol_o):
    bad = np.argwhere(~(np.abs(lse - lse_ref) <= 2e-4))
    if len(bad):
        say(f"lse mismatches at {len(bad)} (row, position, head) triples, first: "
            f"{[(tuple(int(v) for v in t), float(lse[tuple(t)]), float(lse_ref[tuple(t)])) for t in bad[:6]]}")
    err_o = np.abs(o - o_ref)
    assert (err_o <= tol_o).all(), (float(err_o.max()), float(np.max(err_o / tol_o)))
    err_l = np.abs(lse - lse_ref)
    assert err_l.max() <= 2e-4, float(err_l.max())
    say(f"attention parity ok: max |do| {err_o.max():.2e}, max |do|/tol {np.max(err_o / tol_o):.3f}, "
        f"median tol {np.median(tol_o):.2e}, max |dlse| {err_l.max():.2e}")


@pytest.mark.parametrize("B,K,Hq,Hkv,L,W,P", [
    (2, 7, 16, 1, 200, 64, [100, 37]),
    (7, 3, 64, 4, 400, 128, [0, 1, 126, 127, 128, 129, 300]),
    (3, 8, 16, 1, 40, 8, [0, 7, 30]),
    (2, 7, 64, 4, 9100, 4096, [4095, 9000]),
    (1, 1, 16, 1, 5000, 4096, [4999]),
    (1, 7, 64, 4, 8200, 4096, [8192]),   # the benchmark's one-row shape: 33 splits of two tiles
])
def test_window_attention_parity(B, K, Hq, Hkv, L, W, P):
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=B * 100 + K + W)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, kc, vc, P, W, scale)
    vq, vk, vv = _f64(q), _f64(kc), _f64(vc)
    o_ref, lse_ref = wa.window_block_attention(vq, vk, vv, np.asarray(P), W, scale)
    check(o, lse, o_ref, lse_ref, window_tolerance(vq, vk, vv, np.asarray(P), W, scale, lse_ref))


def _ragged_contexts(B, K, L, W, seed):
    """Contexts for B rows: 0, 1, around the window edge (W - 2 .. W + 1) and
    the largest (L - K) where they fit, the rest drawn uniformly."""
    fixed = [p for p in (0, 1, W - 2, W - 1, W, W + 1, L - K) if 0 <= p <= L - K][:B]
    rng = np.random.default_rng(seed)
    return fixed + [int(x) for x in rng.integers(0, L - K + 1, size=B - len(fixed))]


# B * Hkv >= 256 (row, key/value head) pairs: the single-launch kernel, whose
# two waves split the K positions (ceil(K / 2) slots each, the spare slot of
# an odd K repeating the last position); every output compared.
@pytest.mark.parametrize("B,K,Hq,Hkv,L,W", [
    (64, 7, 64, 4, 700, 256),     # the pages' head layout, 4 + 3 positions
    (64, 8, 64, 4, 300, 100),     # K = 8, a window that is not a multiple of the tile
    (96, 5, 48, 3, 500, 200),     # 3 + 2 positions
    (256, 3, 16, 1, 200, 64),     # one key/value head
    (128, 2, 32, 2, 400, 33),     # one position per wave
    (300, 1, 16, 1, 150, 40),     # K = 1: the second wave repeats the first
    (256, 8, 16, 1, 60, 8),       # K = W: every key tile is an edge tile
])
def test_window_attention_single_launch_parity(B, K, Hq, Hkv, L, W):
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=B * 10 + K * 3 + W)
    P = _ragged_contexts(B, K, L, W, seed=B + W)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, kc, vc, P, W, scale)
    vq, vk, vv = _f64(q), _f64(kc), _f64(vc)
    o_ref, lse_ref = wa.window_block_attention(vq, vk, vv, np.asarray(P), W, scale)
    check(o, lse, o_ref, lse_ref, window_tolerance(vq, vk, vv, np.asarray(P), W, scale, lse_ref))


@pytest.mark.parametrize("layout", [None, DSPARK_KV_LAYOUT_BHLD])
def test_window_attention_full_size_sampled(layout):
    """The benchmark shape: B=88 rows, 64/4 heads, K=7, W=4096, P=8192 for every
    row, in both cache layouts; 48 sampled (row, position, head) triples
    against the oracle."""
    B, K, Hq, Hkv, W, P = 88, 7, 64, 4, 4096, 8192
    L = P + K
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=4242)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, kc, vc, [P] * B, W, scale, layout=layout)
    rng = np.random.default_rng(9)
    rows = [(int(rng.integers(B)), int(rng.integers(K)), int(rng.integers(Hq))) for _ in range(48)]
    rows += [(0, 0, 0), (B - 1, K - 1, Hq - 1)]
    qs = _f64(q)
    lo = P - (W - 1)
    for (b, k, h) in rows:
        kvh = h // (Hq // Hkv)
        kk = _f64(kc[b, lo:, kvh:kvh + 1])
        vv = _f64(vc[b, lo:, kvh:kvh + 1])
        # the same triple on a cache cut to the window: context P - lo
        ro, rl = wa.window_block_attention_rows(qs[b:b + 1, :, h:h + 1], kk[None], vv[None], [P - lo], W, scale,
                                                [(0, k, 0)])
        tol = rounding_tolerance(qs[b, k, h], kk[:, 0], vv[:, 0], rl[0], scale)
        assert (np.abs(o[b, k, h] - ro[0]) <= tol).all(), (b, k, h, float(np.max(np.abs(o[b, k, h] - ro[0]) / tol)))
        assert abs(lse[b, k, h] - rl[0]) <= 2e-4, (b, k, h)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    say(f"full-size attention: {len(rows)} sampled triples ok")


# the head-major cache layout, in both launch forms (split key range below
# 256 pairs, one launch from 256)
@pytest.mark.parametrize("B,K,Hq,Hkv,L,W", [
    (7, 3, 64, 4, 400, 128),
    (2, 7, 64, 4, 9100, 4096),
    (64, 7, 64, 4, 700, 256),
    (256, 8, 16, 1, 60, 8),
])
def test_window_attention_head_major_layout(B, K, Hq, Hkv, L, W):
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=B * 7 + K + W)
    P = _ragged_contexts(B, K, L, W, seed=B * 3 + W)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, kc, vc, P, W, scale, layout=DSPARK_KV_LAYOUT_BHLD)
    vq, vk, vv = _f64(q), _f64(kc), _f64(vc)
    o_ref, lse_ref = wa.window_block_attention(vq, vk, vv, np.asarray(P), W, scale)
    check(o, lse, o_ref, lse_ref, window_tolerance(vq, vk, vv, np.asarray(P), W, scale, lse_ref))


@pytest.mark.parametrize("B", [7, 64])
def test_window_attention_layout_entry_matches_default_entry(B):
    """dspark_window_block_attention_layout with [B, L, Hkv, D] runs the same
    kernels as dspark_window_block_attention: bit-identical outputs."""
    K, Hq, Hkv, L, W = 7, 64, 4, 500, 200
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=B + 1)
    P = _ragged_contexts(B, K, L, W, seed=B)
    o0, l0 = run_gpu(q, kc, vc, P, W, 0.1)
    o1, l1 = run_gpu(q, kc, vc, P, W, 0.1, layout=DSPARK_KV_LAYOUT_BLHD)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_attention_clamps_context_length():
    """ctx_len is device data: a value below 0 acts as 0 and one above L - K as
    L - K (the header's defined behaviour); the oracle is run on the clamped
    values."""
    B, K, Hq, Hkv, L, W = 3, 7, 16, 1, 300, 128
    q, kc, vc = _inputs(B, K, Hq, Hkv, L, seed=77)
    scale = 1.0 / math.sqrt(D)
    o, lse = run_gpu(q, kc, vc, [-40, 5000, L - K], W, scale)
    Pc = np.array([0, L - K, L - K])
    vq, vk, vv = _f64(q), _f64(kc), _f64(vc)
    o_ref, lse_ref = wa.window_block_attention(vq, vk, vv, Pc, W, scale)
    check(o, lse, o_ref, lse_ref, window_tolerance(vq, vk, vv, Pc, W, scale, lse_ref))
