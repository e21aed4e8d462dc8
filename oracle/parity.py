"""Parity check of a draft block against the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Criteria (the sampler's stated pass bar):
  * float32 logits within 2e-3 absolute of the oracle's, every entry;
  * q within 1e-6 absolute of the oracle's q (check A) and of the double
    softmax of the checked path's own float32 logits scaled by float32(1/T)
    (check B: the pages test that the proposal is exactly the softmax of the
    float32 biased logits, "brb-nv/TensorRT-LLM pull 27", section "Test
    Coverage");
    greedy rows must be exactly one-hot at their token;
  * tokens identical wherever the oracle's top-2 score margin exceeds 1e-4.

Several tokens are correct at a near-tie (two scores within 1e-4, which the
two float32 paths may order differently). The oracle runs free; where the
checked token differs from the oracle's, it must be one of the oracle's
near-tied candidates at that position, and the oracle is then continued
along that candidate (the branch it itself declared valid), so a single
near-tie cannot cascade into later positions. Any other difference fails.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from . import MAX_CAND, TIE_EPS, draft_block

LOGIT_ATOL = 2e-3
Q_ATOL = 1e-6
Q_SUM_ATOL = 1e-5


@dataclasses.dataclass
class ParityReport:
    rows: int
    positions: int
    near_ties: int              # oracle margins <= TIE_EPS
    branched: int               # positions where the checked token took another near-tied candidate
    max_logit_err: float
    max_q_err_oracle: float
    max_q_err_self: float
    max_q_sum_err: float
    min_margin: float

    def as_dict(self):
        return dataclasses.asdict(self)


class ParityError(AssertionError):
    pass


def _softmax64(s32: np.ndarray) -> np.ndarray:
    s = s32.astype(np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def check(w, tokens: np.ndarray, logits: np.ndarray, q: np.ndarray, *, num_threads: int = 0,
          logit_atol: float = LOGIT_ATOL, q_atol: float = Q_ATOL) -> ParityReport:
    """Compare outputs (host arrays for every row of ``w``) with the oracle; raise on failure."""
    B, K, V = w.B, w.K, w.V
    tokens = np.asarray(tokens)
    if tokens.shape != (B, K) or logits.shape != (B, K, V) or q.shape != (B, K, V):
        raise ParityError(f"shape mismatch: {tokens.shape} {logits.shape} {q.shape} vs {(B, K, V)}")
    if np.any((tokens < 0) | (tokens >= V)):
        raise ParityError("token out of range")

    forced = np.full((B, K), -1, np.int32)
    branched = 0
    for _ in range(K + 1):
        res = draft_block(w, forced=forced, num_threads=num_threads)
        diff = np.argwhere(res.tokens != tokens)
        if diff.size == 0:
            break
        # the first differing position of each row
        first = {}
        for b, k in diff:
            first.setdefault(int(b), int(k))
        for b, k in first.items():
            n = int(res.ncand[b, k])
            cands = res.cand[b, k, :min(n, MAX_CAND)]
            if n < 2 or int(tokens[b, k]) not in set(int(c) for c in cands):
                raise ParityError(
                    f"token mismatch at row {b} position {k}: got {int(tokens[b, k])}, oracle "
                    f"{int(res.tokens[b, k])}, margin {res.margin[b, k]:.3g}, near-tied {list(cands)}")
            forced[b, k] = tokens[b, k]
            branched += 1
    else:
        raise ParityError("branching did not converge")

    lerr = np.abs(logits.astype(np.float64) - res.logits.astype(np.float64))
    max_lerr = float(np.nanmax(lerr)) if lerr.size else 0.0
    if not np.all(lerr <= logit_atol):
        b, k, v = np.unravel_index(int(np.nanargmax(np.where(np.isnan(lerr), np.inf, lerr))), lerr.shape)
        raise ParityError(f"logits differ by {lerr[b, k, v]:.3g} at {(b, k, v)}: "
                          f"{logits[b, k, v]} vs oracle {res.logits[b, k, v]}")

    qerr = np.abs(q.astype(np.float64) - res.q)
    max_qerr = float(np.max(qerr)) if qerr.size else 0.0
    if not np.all(qerr <= q_atol):
        b, k, v = np.unravel_index(int(np.argmax(np.where(np.isnan(qerr), np.inf, qerr))), qerr.shape)
        raise ParityError(f"q differs from the oracle by {qerr[b, k, v]:.3g} at {(b, k, v)}")

    # check B: q against the softmax of the checked path's own logits
    max_self = 0.0
    T = np.asarray(w.temperature, np.float32)
    for b in range(B):
        if T[b] > 0:
            invT = np.float32(np.float32(1.0) / T[b])
            ref = _softmax64((logits[b] * invT).astype(np.float32))
        else:
            ref = np.zeros((K, V))
            ref[np.arange(K), tokens[b]] = 1.0
            if not np.array_equal(q[b].astype(np.float64), ref):
                raise ParityError(f"greedy row {b}: q is not one-hot at its tokens")
        e = float(np.max(np.abs(q[b].astype(np.float64) - ref)))
        max_self = max(max_self, e)
    if max_self > q_atol:
        raise ParityError(f"q differs from softmax(logits/T) by {max_self:.3g}")

    sums = q.astype(np.float64).sum(axis=-1)
    max_sum = float(np.max(np.abs(sums - 1.0))) if sums.size else 0.0
    if max_sum > Q_SUM_ATOL:
        raise ParityError(f"a row of q sums to 1 +- {max_sum:.3g}")

    return ParityReport(rows=B, positions=K, near_ties=int(np.sum(res.margin <= TIE_EPS)),
                        branched=branched, max_logit_err=max_lerr, max_q_err_oracle=max_qerr,
                        max_q_err_self=max_self, max_q_sum_err=max_sum,
                        min_margin=float(np.min(res.margin)) if res.margin.size else float("inf"))
