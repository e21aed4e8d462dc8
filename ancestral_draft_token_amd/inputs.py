"""Seeded synthetic workloads for the DSpark ancestral draft-block sampler.

This module only draws random inputs. It holds none of the sampler's
arithmetic, so both the CPU oracle's tests and the GPU path's tests and
benchmark can use it without sharing any part of the method.

The workloads stand in for the drafting-alone measurement of the pages
(batches of seven draft positions over a 200064-token vocabulary with a
rank-256 Markov head; page "brb-nv/TensorRT-LLM pull 27", section "Commits
1-2: fixed-shape decode", drafting-alone table). No dataset or trained weight is needed: the
sampler moves the same bytes whatever the values are.

Draw order inside one workload (one ``numpy.random.default_rng(data_seed)``):
base logits -> hot-token indices -> E -> W -> prev tokens -> Philox seeds ->
Philox offsets. bf16 tensors are made from float32 by round-to-nearest-even
and are held as ``uint16`` bit patterns.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb can wrap only for NaN bit patterns, which are replaced below
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One draft-block problem: every input of one sampler call, on the host."""

    name: str
    B: int
    K: int
    V: int
    r: int
    base_dtype: str                 # "f32" or "bf16"
    base: np.ndarray                # [B,K,V] float32, or uint16 bf16 bits
    E: np.ndarray                   # [V,r] uint16 (bf16 bits)
    W: np.ndarray                   # [r,V] uint16 (bf16 bits)
    prev_token: np.ndarray          # [B] int32
    seed: np.ndarray                # [B] int64 (bit pattern of the 64-bit key)
    offset: np.ndarray              # [B] int64
    temperature: np.ndarray         # [B] float32; !(T > 0) marks a greedy row
    n_real: Optional[int]           # rows b >= n_real are graph padding; None = all real

    @property
    def n_real_rows(self) -> int:
        return self.B if self.n_real is None else self.n_real

    def base_f32(self) -> np.ndarray:
        if self.base_dtype == F32:
            return self.base
        return bf16_bits_to_f32(self.base)

    def subset_rows(self, rows) -> "Workload":
        """The same problem restricted to some rows (rows are independent)."""
        rows = np.asarray(rows, dtype=np.int64)
        n_real = None
        if self.n_real is not None:
            # keep each row's padding status: real rows first, padding rows after
            real = rows[rows < self.n_real]
            pad = rows[rows >= self.n_real]
            rows = np.concatenate([real, pad])
            n_real = int(real.size)
        return dataclasses.replace(
            self,
            name=f"{self.name}[rows]",
            B=int(rows.size),
            base=np.ascontiguousarray(self.base[rows]),
            prev_token=np.ascontiguousarray(self.prev_token[rows]),
            seed=np.ascontiguousarray(self.seed[rows]),
            offset=np.ascontiguousarray(self.offset[rows]),
            temperature=np.ascontiguousarray(self.temperature[rows]),
            n_real=n_real,
        ), rows


def _normal_f32(rng, shape, std):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def make_workload(
    name: str,
    *,
    B: int,
    K: int,
    V: int,
    r: int,
    base_dtype: str,
    base_std: float,
    ew_std: float,
    data_seed: int,
    temperature,
    hot_per_position: int = 0,
    hot_boost: float = 8.0,
    n_real: Optional[int] = None,
    pad_base: str = "zero",
    fixed_seed: Optional[int] = None,
    fixed_offset: Optional[int] = None,
) -> Workload:
    """Draw one seeded workload.

    ``temperature`` is a scalar or a callable ``b -> T``. Padding rows
    (``b >= n_real``) get base 0 (``pad_base="zero"``) or NaN (``"nan"``);
    the sampler never reads them either way.
    """
    rng = np.random.default_rng(data_seed)
    base = _normal_f32(rng, (B, K, V), base_std)
    if hot_per_position:
        for b in range(B):
            for k in range(K):
                hot = rng.choice(V, size=hot_per_position, replace=False)
                base[b, k, hot] += np.float32(hot_boost)
    if n_real is not None and n_real < B:
        base[n_real:] = np.float32(0.0) if pad_base == "zero" else np.float32(np.nan)
    E = f32_to_bf16_bits(_normal_f32(rng, (V, r), ew_std))
    W = f32_to_bf16_bits(_normal_f32(rng, (r, V), ew_std))
    prev = rng.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    seeds = rng.integers(0, np.iinfo(np.int64).max, size=B, dtype=np.int64)
    offsets = rng.integers(0, 1 << 40, size=B, dtype=np.int64)
    if fixed_seed is not None:
        seeds[:] = fixed_seed
    if fixed_offset is not None:
        offsets[:] = fixed_offset
    if callable(temperature):
        T = np.array([temperature(b) for b in range(B)], dtype=np.float32)
    else:
        T = np.full(B, temperature, dtype=np.float32)
    if base_dtype == BF16:
        base = f32_to_bf16_bits(base)
    elif base_dtype != F32:
        raise ValueError(f"base_dtype must be 'f32' or 'bf16', got {base_dtype!r}")
    return Workload(
        name=name, B=B, K=K, V=V, r=r, base_dtype=base_dtype, base=np.ascontiguousarray(base),
        E=E, W=W, prev_token=prev, seed=seeds, offset=offsets, temperature=T, n_real=n_real,
    )


# The five workloads: a tiny reference case and the drafting-alone batch sizes
# B = 1 / 8 / 44 / 88 (padded to 96) at V = 200064, K = 7, r = 256.
VOCAB = 200064
RANK = 256
DRAFT_LEN = 7


def tiny(**kw) -> Workload:
    """B=1, K=7, V=4096, r=32; f32 base ~N(0,2^2); E,W ~N(0,0.05^2); T=1; seed 1234, offset 0."""
    args = dict(B=1, K=7, V=4096, r=32, base_dtype=F32, base_std=2.0, ew_std=0.05,
                data_seed=1234, temperature=1.0, fixed_seed=1234, fixed_offset=0)
    args.update(kw)
    return make_workload("tiny_b1_v4096_r32", **args)


def single_request(**kw) -> Workload:
    """B=1 decode: bf16 base ~N(0,3^2) with 16 hot tokens (+8) per position; T=1."""
    args = dict(B=1, K=DRAFT_LEN, V=VOCAB, r=RANK, base_dtype=BF16, base_std=3.0, ew_std=0.02,
                data_seed=7, temperature=1.0, hot_per_position=16)
    args.update(kw)
    return make_workload("decode_b1_v200064_r256_bf16", **args)


def small_batch(**kw) -> Workload:
    """B=8: f32 base ~N(0,3^2) + hot tokens; T=1; distinct (seed, offset) per row."""
    args = dict(B=8, K=DRAFT_LEN, V=VOCAB, r=RANK, base_dtype=F32, base_std=3.0, ew_std=0.02,
                data_seed=7, temperature=1.0, hot_per_position=16)
    args.update(kw)
    return make_workload("batch_b8_v200064_r256_f32", **args)


def mixed_batch(**kw) -> Workload:
    """B=44: bf16 base ~N(0,3^2); even rows sample at T=0.7, odd rows are greedy (T=0)."""
    args = dict(B=44, K=DRAFT_LEN, V=VOCAB, r=RANK, base_dtype=BF16, base_std=3.0, ew_std=0.02,
                data_seed=7, temperature=lambda b: 0.7 if b % 2 == 0 else 0.0)
    args.update(kw)
    return make_workload("mixed_b44_v200064_r256_bf16", **args)


def large_padded(**kw) -> Workload:
    """B=96 launched, 88 real: f32 base ~N(0,3^2); padding rows sample from the Markov bias only; T=1."""
    args = dict(B=96, K=DRAFT_LEN, V=VOCAB, r=RANK, base_dtype=F32, base_std=3.0, ew_std=0.02,
                data_seed=7, temperature=1.0, n_real=88)
    args.update(kw)
    return make_workload("padded_b88of96_v200064_r256_f32", **args)


WORKLOADS = {
    "tiny": tiny,
    "b1": single_request,
    "b8": small_batch,
    "b44": mixed_batch,
    "b88": large_padded,
}
