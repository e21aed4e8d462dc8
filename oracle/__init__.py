"""CPU oracle for the DSpark ancestral draft-block sampler -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never does, and the two
share no code.

The arithmetic lives in ``dspark_oracle.c`` (plain C, built with gcc, no
fast-math, FMA contraction off). This module only builds and loads it and
marshals numpy arrays. What it computes, and the passages it follows, are
stated in the header of ``dspark_oracle.c``.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libdspark_oracle.so")
_lock = threading.Lock()
_lib = None

TIE_EPS = 1e-4          # margin under which a draw counts as a near-tie
MAX_CAND = 16           # near-tie candidates reported per position


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.dspark_oracle_philox4x32_10.argtypes = [P, P, P]
        lib.dspark_oracle_philox4x32_10.restype = None
        lib.dspark_oracle_noise_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        lib.dspark_oracle_noise_word.restype = ctypes.c_uint32
        lib.dspark_oracle_uniform.argtypes = [ctypes.c_uint32]
        lib.dspark_oracle_uniform.restype = ctypes.c_double
        lib.dspark_oracle_gumbel.argtypes = [ctypes.c_uint32]
        lib.dspark_oracle_gumbel.restype = ctypes.c_float
        lib.dspark_oracle_uniform_batch.argtypes = [P, P, ctypes.c_int64]
        lib.dspark_oracle_uniform_batch.restype = None
        lib.dspark_oracle_gumbel_batch.argtypes = [P, P, ctypes.c_int64]
        lib.dspark_oracle_gumbel_batch.restype = None
        lib.dspark_oracle_max_threads.argtypes = []
        lib.dspark_oracle_max_threads.restype = ctypes.c_int
        lib.dspark_oracle_draft_block.argtypes = [
            P, ctypes.c_int, P, P, P, P, P, P, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, ctypes.c_double, ctypes.c_int,
            P, P, P, P, P, P, P, ctypes.c_int]
        lib.dspark_oracle_draft_block.restype = ctypes.c_int
        lib.dspark_oracle_verify_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32]
        lib.dspark_oracle_verify_uniform.restype = ctypes.c_float
        lib.dspark_oracle_verify_gumbel.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32]
        lib.dspark_oracle_verify_gumbel.restype = ctypes.c_float
        lib.dspark_oracle_verify_standard.argtypes = [
            P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
            P, P, P, P, P, P]
        lib.dspark_oracle_verify_standard.restype = ctypes.c_int
        lib.dspark_oracle_verify_block_weights.argtypes = [
            P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P]
        lib.dspark_oracle_verify_block_weights.restype = ctypes.c_int
        lib.dspark_oracle_verify_block.argtypes = [
            P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
            P, P, P, P, P, P]
        lib.dspark_oracle_verify_block.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def philox4x32_10(counter, key) -> np.ndarray:
    """One Philox4x32-10 block: four 32-bit counter words, two key words -> four words."""
    lib = _load()
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.dspark_oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def noise_word(seed: int, offset: int, k: int, v: int) -> int:
    return int(_load().dspark_oracle_noise_word(seed & (2**64 - 1), offset & (2**64 - 1), k, v))


def uniform(x: np.ndarray) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint32)
    u = np.empty(x.shape, dtype=np.float64)
    lib.dspark_oracle_uniform_batch(_ptr(x), _ptr(u), x.size)
    return u


def gumbel(x: np.ndarray) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint32)
    g = np.empty(x.shape, dtype=np.float32)
    lib.dspark_oracle_gumbel_batch(_ptr(x), _ptr(g), x.size)
    return g


def max_threads() -> int:
    return int(_load().dspark_oracle_max_threads())


@dataclasses.dataclass
class OracleResult:
    tokens: np.ndarray          # [B,K] int32: the token each position carries
    own_tokens: np.ndarray      # [B,K] int32: the oracle's own draw
    logits: Optional[np.ndarray]  # [B,K,V] float32
    q: Optional[np.ndarray]     # [B,K,V] float64
    margin: np.ndarray          # [B,K] float64: best minus runner-up score
    ncand: np.ndarray           # [B,K] int32: scores within TIE_EPS of the best
    cand: np.ndarray            # [B,K,MAX_CAND] int32: those indices, ascending


def draft_block(w, *, forced: Optional[np.ndarray] = None, want_logits: bool = True,
                want_q: bool = True, num_threads: int = 0, tie_eps: float = TIE_EPS) -> OracleResult:
    """Run the oracle on a workload (``ancestral_draft_token_amd.inputs.Workload``).

    ``forced`` ([B,K] int32, -1 = free) replaces the token a position carries
    into the next one; the position's own draw is still reported.
    """
    lib = _load()
    B, K, V, r = w.B, w.K, w.V, w.r
    base = np.ascontiguousarray(w.base)
    is_bf16 = 1 if w.base_dtype == "bf16" else 0
    E = np.ascontiguousarray(w.E, dtype=np.uint16)
    W = np.ascontiguousarray(w.W, dtype=np.uint16)
    prev = np.ascontiguousarray(w.prev_token, dtype=np.int32)
    seed = np.ascontiguousarray(w.seed, dtype=np.int64)
    off = np.ascontiguousarray(w.offset, dtype=np.int64)
    T = np.ascontiguousarray(w.temperature, dtype=np.float32)
    n_real = -1 if w.n_real is None else int(w.n_real)
    f = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    tokens = np.zeros((B, K), dtype=np.int32)
    own = np.zeros((B, K), dtype=np.int32)
    logits = np.empty((B, K, V), dtype=np.float32) if want_logits else None
    q = np.empty((B, K, V), dtype=np.float64) if want_q else None
    margin = np.zeros((B, K), dtype=np.float64)
    ncand = np.zeros((B, K), dtype=np.int32)
    cand = np.full((B, K, MAX_CAND), -1, dtype=np.int32)
    rc = lib.dspark_oracle_draft_block(
        _ptr(base), is_bf16, _ptr(E), _ptr(W), _ptr(prev), _ptr(seed), _ptr(off), _ptr(T),
        n_real, B, K, V, r, _ptr(f), float(tie_eps), MAX_CAND,
        _ptr(tokens), _ptr(own), _ptr(logits), _ptr(q), _ptr(margin), _ptr(ncand), _ptr(cand),
        int(num_threads))
    if rc != 0:
        raise RuntimeError(f"oracle draft_block failed with {rc}")
    return OracleResult(tokens=tokens, own_tokens=own, logits=logits, q=q, margin=margin,
                        ncand=ncand, cand=cand)


@dataclasses.dataclass
class VerifyResult:
    n_accepted: np.ndarray      # [B] int32: drafts accepted
    out_tokens: np.ndarray      # [B,K+1] int32: accepted drafts, the emitted token, then -1
    margin: np.ndarray          # [B] float64: best minus runner-up score of the emitted draw
    ncand: np.ndarray           # [B] int32: scores within tie_eps of the best
    cand: np.ndarray            # [B,MAX_CAND] int32: those indices, ascending


def verify_uniform(seed: int, offset: int, k: int) -> float:
    return float(_load().dspark_oracle_verify_uniform(seed & (2**64 - 1), offset & (2**64 - 1), k))


def verify_gumbel(seed: int, offset: int, v: int) -> float:
    return float(_load().dspark_oracle_verify_gumbel(seed & (2**64 - 1), offset & (2**64 - 1), v))


def verify_standard(draft_tokens, q, p, seed, offset, tie_eps: float = TIE_EPS) -> VerifyResult:
    """Standard token-level verification of a draft block (rules and readings in
    the header section of ``dspark_oracle.c``). ``q`` [B,K,V] and ``p``
    [B,K+1,V] are float32 (other float types are rounded to float32 first)."""
    lib = _load()
    d = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    B, K = d.shape
    q = np.ascontiguousarray(q, dtype=np.float32)
    p = np.ascontiguousarray(p, dtype=np.float32)
    V = p.shape[-1]
    if q.shape != (B, K, V) or p.shape != (B, K + 1, V):
        raise ValueError("shapes: q [B,K,V], p [B,K+1,V]")
    sd = np.ascontiguousarray(seed, dtype=np.int64)
    off = np.ascontiguousarray(offset, dtype=np.int64)
    n = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, K + 1), dtype=np.int32)
    margin = np.zeros(B, dtype=np.float64)
    ncand = np.zeros(B, dtype=np.int32)
    cand = np.full((B, MAX_CAND), -1, dtype=np.int32)
    rc = lib.dspark_oracle_verify_standard(_ptr(q), _ptr(p), _ptr(d), _ptr(sd), _ptr(off), B, K, V,
                                           float(tie_eps), MAX_CAND, _ptr(n), _ptr(out), None,
                                           _ptr(margin), _ptr(ncand), _ptr(cand))
    if rc != 0:
        raise RuntimeError(f"oracle verify_standard failed with {rc}")
    return VerifyResult(n_accepted=n, out_tokens=out, margin=margin, ncand=ncand, cand=cand)


def _verify_inputs(draft_tokens, q, p):
    d = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    B, K = d.shape
    q = np.ascontiguousarray(q, dtype=np.float32)
    p = np.ascontiguousarray(p, dtype=np.float32)
    V = p.shape[-1]
    if q.shape != (B, K, V) or p.shape != (B, K + 1, V):
        raise ValueError("shapes: q [B,K,V], p [B,K+1,V]")
    return d, q, p, B, K, V


@dataclasses.dataclass
class BlockWeights:
    w: np.ndarray               # [B,K+1] float64: prefix weights w_0 .. w_K
    S: np.ndarray               # [B,K+1] float64: residual masses S_0 .. S_{K-1} (S_K = 0)
    h: np.ndarray               # [B,K+1] float64: thresholds (h_0 = 1)
    resid: Optional[np.ndarray]  # [B,K+1,V] float32: weights of each position's emission


def verify_block_weights(draft_tokens, q, p, want_resid: bool = True) -> BlockWeights:
    """Prefix weights, residual masses and thresholds of block verification
    (rule and readings in the block-verification section of
    ``dspark_oracle.c``)."""
    lib = _load()
    d, q, p, B, K, V = _verify_inputs(draft_tokens, q, p)
    w = np.zeros((B, K + 1), dtype=np.float64)
    S = np.zeros((B, K + 1), dtype=np.float64)
    h = np.zeros((B, K + 1), dtype=np.float64)
    resid = np.zeros((B, K + 1, V), dtype=np.float32) if want_resid else None
    rc = lib.dspark_oracle_verify_block_weights(_ptr(q), _ptr(p), _ptr(d), B, K, V, _ptr(w), _ptr(S),
                                                _ptr(h), _ptr(resid))
    if rc != 0:
        raise RuntimeError(f"oracle verify_block_weights failed with {rc}")
    return BlockWeights(w=w, S=S, h=h, resid=resid)


@dataclasses.dataclass
class BlockVerifyResult(VerifyResult):
    tau_margin: np.ndarray = None   # [B] float64: min over j of |eta_j - h_j|


def verify_block(draft_tokens, q, p, seed, offset, tie_eps: float = TIE_EPS) -> BlockVerifyResult:
    """Block verification of a draft block (Sun et al., 2024; rule and
    readings in the block-verification section of ``dspark_oracle.c``)."""
    lib = _load()
    d, q, p, B, K, V = _verify_inputs(draft_tokens, q, p)
    sd = np.ascontiguousarray(seed, dtype=np.int64)
    off = np.ascontiguousarray(offset, dtype=np.int64)
    n = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, K + 1), dtype=np.int32)
    tm = np.zeros(B, dtype=np.float64)
    margin = np.zeros(B, dtype=np.float64)
    ncand = np.zeros(B, dtype=np.int32)
    cand = np.full((B, MAX_CAND), -1, dtype=np.int32)
    rc = lib.dspark_oracle_verify_block(_ptr(q), _ptr(p), _ptr(d), _ptr(sd), _ptr(off), B, K, V,
                                        float(tie_eps), MAX_CAND, _ptr(n), _ptr(out), _ptr(tm),
                                        _ptr(margin), _ptr(ncand), _ptr(cand))
    if rc != 0:
        raise RuntimeError(f"oracle verify_block failed with {rc}")
    return BlockVerifyResult(n_accepted=n, out_tokens=out, margin=margin, ncand=ncand, cand=cand,
                             tau_margin=tm)
