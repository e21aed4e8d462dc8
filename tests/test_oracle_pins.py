"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these re-types the oracle's own code. Each pin comes from outside it:
an independent library (rocRAND's Philox engine, a float64 matmul), a
distribution law (Gumbel-max sampling, tested by chi-square at p = 1e-4 as
the pages do), an invariant, a closed form, or brute force on tiny inputs.
The negative controls show that the chi-square tests have the power to
reject the plausible mistakes (a dropped ancestry, an ignored temperature, a
noise word shared between positions).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from ancestral_draft_token_amd import inputs
from ancestral_draft_token_amd.inputs import Workload, bf16_bits_to_f32, f32_to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
P_THRESHOLD = 1e-4      # the pages' chi-square level


# ---------------------------------------------------------------------------
# Philox4x32-10 against rocRAND's independent engine
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    src = os.path.join(HERE, "pins", "rocrand_philox_words.cpp")
    hdr = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"
    if not os.path.exists(hdr) or shutil.which("g++") is None:
        pytest.skip("rocRAND headers or g++ not available")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_words")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src, "-o", exe],
                   check=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(x)) for x in row) for row in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)

    return run


def test_philox_block_matches_rocrand(rocrand_words):
    rng = np.random.default_rng(11)
    rows = [[0, 0, 0, 0, 0, 0], [0xFFFFFFFF] * 6, [1, 2, 3, 4, 5, 6]]
    rows += rng.integers(0, 2**32, size=(200, 6), dtype=np.uint64).tolist()
    ref = rocrand_words(rows)
    for row, want in zip(rows, ref):
        got = oracle.philox4x32_10(counter=row[2:], key=row[:2])
        np.testing.assert_array_equal(got, want, err_msg=f"key/counter {row}")


def test_noise_word_layout(rocrand_words):
    """Noise of entry v, position k, slot (seed, offset): word v&3 of the block at
    counter (v>>2, k, lo(offset), hi(offset)) under key (lo(seed), hi(seed))."""
    rng = np.random.default_rng(12)
    cases = []
    for _ in range(100):
        seed = int(rng.integers(0, 2**63))
        off = int(rng.integers(0, 2**63))
        k = int(rng.integers(0, 16))
        v = int(rng.integers(0, 200064))
        cases.append((seed, off, k, v))
    cases += [(0, 0, 0, 0), (2**64 - 1, 2**64 - 1, 15, 200063), (1234, 0, 6, 4095)]
    rows = [[s & 0xFFFFFFFF, s >> 32, v >> 2, k, o & 0xFFFFFFFF, o >> 32] for s, o, k, v in cases]
    ref = rocrand_words(rows)
    for (s, o, k, v), want in zip(cases, ref):
        assert oracle.noise_word(s, o, k, v) == int(want[v & 3]), (s, o, k, v)


# ---------------------------------------------------------------------------
# uniform and Gumbel transforms: exhaustive over the 2^23 grid
# ---------------------------------------------------------------------------

def test_uniform_grid_exhaustive():
    m = np.arange(1 << 23, dtype=np.uint32)
    u = oracle.uniform(m << np.uint32(9))
    assert u[0] == 2.0 ** -24 and u[-1] == 1.0 - 2.0 ** -24
    assert np.all(np.diff(u) > 0), "not strictly increasing"
    assert np.all(u.astype(np.float32).astype(np.float64) == u), "not exact in float32"
    # the low 9 bits of the word are ignored
    u_hi = oracle.uniform((m << np.uint32(9)) | np.uint32(0x1FF))
    assert np.array_equal(u, u_hi)
    # equal spacing 2^-23: the grid is the midpoint rule on (0,1)
    assert np.all(np.diff(u) == 2.0 ** -23)


def test_gumbel_transform_matches_gumbel_cdf():
    """Over the whole grid the transform must push the uniform midpoints to the
    standard Gumbel law: #(g <= t) / 2^23 = exp(-exp(-t)) up to grid and rounding."""
    m = np.arange(1 << 23, dtype=np.uint32)
    g = oracle.gumbel(m << np.uint32(9)).astype(np.float64)
    assert np.all(np.isfinite(g))
    assert np.all(np.diff(g) >= 0), "g must be nondecreasing in u"
    t = np.linspace(-2.5, 12.0, 301)
    ecdf = np.searchsorted(g, t, side="right") / float(1 << 23)
    cdf = scipy.stats.gumbel_r.cdf(t)
    assert np.max(np.abs(ecdf - cdf)) < 3.0 / (1 << 23)
    # extremes of the grid: u = 2^-24 and 1 - 2^-24
    assert -2.9 < g[0] < -2.7 and 16.5 < g[-1] < 16.7


# ---------------------------------------------------------------------------
# helpers: an independent expected law from first principles
# ---------------------------------------------------------------------------

def _bias64(w: Workload, d: int) -> np.ndarray:
    """E[d] . W as a float64 library matmul over the widened bf16 values."""
    e = torch.from_numpy(bf16_bits_to_f32(w.E[d]).astype(np.float64))
    W = torch.from_numpy(bf16_bits_to_f32(w.W).astype(np.float64))
    return torch.matmul(e, W).numpy()


def _logits32(w: Workload, b: int, k: int, d: int, pad: bool = False) -> np.ndarray:
    base = np.zeros(w.V, np.float32) if pad else w.base_f32()[b, k]
    return (base + _bias64(w, d).astype(np.float32)).astype(np.float32)


def _softmax_law(logits32: np.ndarray, T: float) -> np.ndarray:
    s = (logits32 * np.float32(np.float32(1.0) / np.float32(T))).astype(np.float64)
    return scipy.special.softmax(s)


def _chi2_p(counts: np.ndarray, probs: np.ndarray) -> float:
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    exp = probs * n
    keep = exp > 0
    stat = float(np.sum((counts[keep] - exp[keep]) ** 2 / exp[keep]))
    dof = int(keep.sum()) - 1
    return float(scipy.stats.chi2.sf(stat, dof))


def _chi2_grouped_p(groups) -> float:
    """Sum chi-square statistics over independent groups [(counts, probs), ...]."""
    stat, dof = 0.0, 0
    for counts, probs in groups:
        counts = np.asarray(counts, np.float64)
        n = counts.sum()
        if n == 0:
            continue
        exp = probs * n
        keep = exp > 0
        stat += float(np.sum((counts[keep] - exp[keep]) ** 2 / exp[keep]))
        dof += int(keep.sum()) - 1
    return float(scipy.stats.chi2.sf(stat, dof))


def _law_workload(N, V, r, T, *, base_dtype="f32", same_seed=True, zero_w=False,
                  same_base_per_position=False, data_seed=5) -> Workload:
    """N independent rows of one small problem: shared base/E/W/prev, distinct slots."""
    rng = np.random.default_rng(data_seed)
    base_row = rng.standard_normal((2, V)).astype(np.float32)
    if same_base_per_position:
        base_row[1] = base_row[0]
    E = f32_to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * np.float32(0.5))
    W = f32_to_bf16_bits(rng.standard_normal((r, V)).astype(np.float32) * np.float32(0.5))
    if zero_w:
        W[:] = 0
    base = np.broadcast_to(base_row, (N, 2, V)).copy()
    if base_dtype == "bf16":
        base = f32_to_bf16_bits(base)
    prev = np.full(N, 3, np.int32)
    if same_seed:
        seed = np.full(N, 0x5EED5EED12345678, np.int64)
        off = np.arange(N, dtype=np.int64) * 977 + 5
    else:
        seed = rng.integers(0, 2**63, size=N, dtype=np.int64)
        off = np.full(N, 42, np.int64)
    return Workload(name="law", B=N, K=2, V=V, r=r, base_dtype=base_dtype, base=base, E=E, W=W,
                    prev_token=prev, seed=seed, offset=off,
                    temperature=np.full(N, T, np.float32), n_real=None)


# ---------------------------------------------------------------------------
# the sampling law (chi-square at p = 1e-4, as the pages test it)
# ---------------------------------------------------------------------------

N_LAW = 200_000


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("V", [8, 16])
@pytest.mark.parametrize("same_seed", [True, False])
def test_gumbel_max_law_and_ancestry(T, V, same_seed):
    w = _law_workload(N_LAW, V, 4, T, same_seed=same_seed)
    res = oracle.draft_block(w, want_logits=False, want_q=False)
    d0, d1 = res.tokens[:, 0], res.tokens[:, 1]
    lg0 = _logits32(w, 0, 0, 3)
    p0 = _softmax_law(lg0, T)
    assert _chi2_p(np.bincount(d0, minlength=V), p0) > P_THRESHOLD
    # position 1 given the drawn position 0
    cond = {t: _softmax_law(_logits32(w, 0, 1, t), T) for t in range(V)}
    groups = [(np.bincount(d1[d0 == t], minlength=V), cond[t]) for t in range(V)]
    assert _chi2_grouped_p(groups) > P_THRESHOLD
    # joint (d0, d1) against p(d0) p(d1 | d0), enumerated
    joint = np.concatenate([p0[t] * cond[t] for t in range(V)])
    assert _chi2_p(np.bincount(d0 * V + d1, minlength=V * V), joint) > P_THRESHOLD

    # negative control (i): no ancestry -- position 1 conditioned on prev_token
    no_anc = _softmax_law(_logits32(w, 0, 1, 3), T)
    assert _chi2_p(np.bincount(d1, minlength=V),
                   np.sum([p0[t] * cond[t] for t in range(V)], axis=0)) > P_THRESHOLD
    assert _chi2_p(np.bincount(d1, minlength=V), no_anc) < P_THRESHOLD
    # negative control (ii): temperature ignored
    if T != 1.0:
        assert _chi2_p(np.bincount(d0, minlength=V), _softmax_law(lg0, 1.0)) < P_THRESHOLD


def test_gumbel_max_law_bf16_base():
    w = _law_workload(N_LAW, 16, 4, 1.0, base_dtype="bf16", data_seed=9)
    res = oracle.draft_block(w, want_logits=False, want_q=False)
    p0 = _softmax_law(_logits32(w, 0, 0, 3), 1.0)
    assert _chi2_p(np.bincount(res.tokens[:, 0], minlength=16), p0) > P_THRESHOLD


def test_zero_bias_positions_independent():
    """W = 0 and the same base at both positions: the draws must be independent
    and identically distributed (a noise word shared across k would make d0 == d1)."""
    V = 8
    w = _law_workload(N_LAW, V, 4, 1.0, zero_w=True, same_base_per_position=True)
    res = oracle.draft_block(w, want_logits=False, want_q=False)
    d0, d1 = res.tokens[:, 0], res.tokens[:, 1]
    p = scipy.special.softmax(w.base_f32()[0, 0].astype(np.float64))
    assert _chi2_p(np.bincount(d0 * V + d1, minlength=V * V), np.outer(p, p).ravel()) > P_THRESHOLD
    assert np.mean(d0 == d1) < 0.5


def test_zero_bias_ignores_prev_token():
    w = inputs.tiny(B=3, K=4, fixed_seed=None, fixed_offset=None)
    w.W[:] = 0
    a = oracle.draft_block(w)
    w.prev_token[:] = (w.prev_token + 1234) % w.V
    b = oracle.draft_block(w)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.logits, b.logits)
    np.testing.assert_array_equal(a.logits, w.base_f32())


def test_new_offset_draws_anew():
    w = inputs.tiny(B=1, K=7)
    a = oracle.draft_block(w, want_q=False)
    w.offset[:] += 1
    b = oracle.draft_block(w, want_q=False)
    assert not np.array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.logits[:, 0], b.logits[:, 0])


# ---------------------------------------------------------------------------
# greedy rows, padding rows, bias, normalisation
# ---------------------------------------------------------------------------

def test_greedy_is_argmax_chain_with_one_hot_q():
    w = inputs.tiny(B=4, K=7, temperature=0.0, fixed_seed=None, fixed_offset=None)
    res = oracle.draft_block(w)
    for b in range(w.B):
        d = int(w.prev_token[b])
        for k in range(w.K):
            lg = _logits32(w, b, k, d)
            d = int(np.argmax(lg))               # first maximum = lowest index
            assert res.tokens[b, k] == d
            onehot = np.zeros(w.V)
            onehot[d] = 1.0
            np.testing.assert_array_equal(res.q[b, k], onehot)


def test_negative_temperature_and_nan_are_greedy():
    w = inputs.tiny(B=3, K=3, fixed_seed=None, fixed_offset=None)
    w.temperature[:] = [0.0, -1.0, np.nan]
    res = oracle.draft_block(w)
    w2 = inputs.tiny(B=3, K=3, fixed_seed=None, fixed_offset=None, temperature=0.0)
    ref = oracle.draft_block(w2)
    np.testing.assert_array_equal(res.tokens, ref.tokens)


def test_bias_matches_float64_matmul():
    w = inputs.tiny(B=2, K=7, fixed_seed=None, fixed_offset=None)
    res = oracle.draft_block(w)
    worst = 0.0
    for b in range(w.B):
        d = int(w.prev_token[b])
        for k in range(w.K):
            want = _logits32(w, b, k, d)
            diff = np.abs(res.logits[b, k].astype(np.float64) - want.astype(np.float64))
            ulp = np.spacing(np.abs(want)).astype(np.float64)
            assert np.all(diff <= ulp), (b, k)
            worst = max(worst, float(np.mean(diff > 0)))
            d = int(res.tokens[b, k])
    assert worst < 1e-3


def test_padding_rows_draw_from_bias_alone():
    w = inputs.tiny(B=6, K=5, n_real=3, pad_base="nan", fixed_seed=None, fixed_offset=None)
    assert np.isnan(w.base_f32()[3:]).all()
    res = oracle.draft_block(w)
    assert np.all((res.tokens >= 0) & (res.tokens < w.V))
    assert np.all(np.isfinite(res.q)) and np.all(np.isfinite(res.logits))
    for b in range(3, 6):
        d = int(w.prev_token[b])
        for k in range(w.K):
            bias32 = _bias64(w, d).astype(np.float32)
            assert np.max(np.abs(res.logits[b, k] - bias32) / np.spacing(np.abs(bias32))) <= 1
            np.testing.assert_allclose(res.q[b, k], _softmax_law(res.logits[b, k], 1.0),
                                       rtol=0, atol=1e-15)
            d = int(res.tokens[b, k])
    # a padding row draws exactly what a real row with base 0 in the same slot draws
    w0 = inputs.tiny(B=6, K=5, n_real=None, fixed_seed=None, fixed_offset=None)
    w0.base[3:] = 0.0
    ref = oracle.draft_block(w0)
    np.testing.assert_array_equal(res.tokens[3:], ref.tokens[3:])
    np.testing.assert_array_equal(res.tokens[:3], ref.tokens[:3])


@pytest.mark.parametrize("make", [inputs.tiny, lambda: inputs.tiny(B=5, n_real=2, temperature=0.4,
                                                                  fixed_seed=None, fixed_offset=None)])
def test_q_rows_sum_to_one(make):
    w = make()
    res = oracle.draft_block(w)
    np.testing.assert_allclose(res.q.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(res.q >= 0)


def test_q_is_softmax_of_scaled_float32_logits():
    w = inputs.tiny(B=2, K=7, temperature=0.7, fixed_seed=None, fixed_offset=None)
    res = oracle.draft_block(w)
    for b in range(2):
        for k in range(7):
            np.testing.assert_allclose(res.q[b, k], _softmax_law(res.logits[b, k], 0.7),
                                       rtol=1e-12, atol=1e-18)


# ---------------------------------------------------------------------------
# tie-breaking, NaN, clamping, forcing: brute force on tiny inputs
# ---------------------------------------------------------------------------

def _flat_workload(V=16, r=4, K=2, B=1, T=0.0):
    w = _law_workload(B, V, r, 1.0)
    w.K = K
    w.base = np.zeros((B, K, V), np.float32)
    w.W[:] = 0
    w.temperature[:] = T
    return w


def test_greedy_ties_go_to_lowest_index_and_are_reported():
    w = _flat_workload()
    w.base[0, 0, [5, 9, 12]] = 3.0
    w.base[0, 1, [2, 7]] = 1.0
    res = oracle.draft_block(w)
    assert res.tokens[0, 0] == 5 and res.tokens[0, 1] == 2
    assert res.margin[0, 0] == 0.0 and res.ncand[0, 0] == 3
    assert list(res.cand[0, 0, :3]) == [5, 9, 12]


def test_nan_never_wins():
    w = _flat_workload()
    w.base[0, 0, :] = np.nan
    w.base[0, 0, 11] = -50.0
    w.base[0, 1, :] = np.nan
    res = oracle.draft_block(w, want_q=False)
    assert res.tokens[0, 0] == 11
    assert res.tokens[0, 1] == 0     # every score NaN: token 0
    # sampling row: a NaN entry never wins
    w = _flat_workload(T=1.0)
    w.base[0, 0, :8] = np.nan
    res = oracle.draft_block(w, want_q=False)
    assert res.tokens[0, 0] >= 8


def test_prev_token_is_clamped():
    w = inputs.tiny(B=2, K=3, fixed_seed=None, fixed_offset=None)
    w.prev_token[:] = [-5, w.V + 10]
    a = oracle.draft_block(w)
    w.prev_token[:] = [0, w.V - 1]
    b = oracle.draft_block(w)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.logits, b.logits)


def test_forcing_conditions_the_next_position():
    w = inputs.tiny(B=1, K=3, fixed_seed=None, fixed_offset=None)
    free = oracle.draft_block(w)
    forced = np.full((1, 3), -1, np.int32)
    forced[0, 0] = free.tokens[0, 0]
    same = oracle.draft_block(w, forced=forced)
    np.testing.assert_array_equal(same.tokens, free.tokens)
    np.testing.assert_array_equal(same.logits, free.logits)
    t = (int(free.tokens[0, 0]) + 777) % w.V
    forced[0, 0] = t
    alt = oracle.draft_block(w, forced=forced)
    assert alt.tokens[0, 0] == t and alt.own_tokens[0, 0] == free.tokens[0, 0]
    np.testing.assert_array_equal(alt.logits[0, 0], free.logits[0, 0])
    want = _logits32(w, 0, 1, t)
    assert np.max(np.abs(alt.logits[0, 1] - want) / np.spacing(np.abs(want))) <= 1


def test_empty_batch_and_bad_arguments():
    w = inputs.tiny(B=1, K=7)
    w0 = inputs.tiny(B=1, K=7)
    w0.B = 0
    res = oracle.draft_block(w0, want_q=False)
    assert res.tokens.shape == (0, 7)
    w.V = 0
    with pytest.raises(RuntimeError):
        oracle.draft_block(w, want_q=False, want_logits=False)


def test_oracle_regression_record():
    """The tiny workload's outputs as recorded by tests/golden/make_golden.py."""
    import hashlib
    import json
    with open(os.path.join(HERE, "golden", "tiny_b1_v4096_r32.json")) as f:
        g = json.load(f)
    res = oracle.draft_block(inputs.tiny())
    assert res.tokens.tolist() == g["tokens"]
    assert hashlib.sha256(res.logits.tobytes()).hexdigest() == g["logits_sha256"]
    np.testing.assert_allclose(res.q[0][:, g["sample_v"]], g["q_sample"], rtol=1e-14, atol=0)
