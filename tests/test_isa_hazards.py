"""Checks on the gfx950 assembly of the large-batch (MFMA) kernel.

The kernel keeps W resident in registers: 62 of its 64 A-operand fragments
per lane live in AGPRs for the whole launch, read there by the matrix
instructions. A build in which the register allocator spilled some of those
fragments to scratch memory gave bias values that changed from run to run.
There the spill store of an AGPR tuple was followed two instructions later by
an AGPR write of the same registers, and the fragments were reloaded inside
the N-tile loop. This test keeps that configuration out:

* no AGPR is spilled (no scratch store with AGPR data) anywhere in the kernel;
* no scratch (spill) access sits inside the kernel's inner loops, where the W
  fragments and the per-tile state live (a spill there would also stall every
  tile on the scratch round trip).

A VALU write to a matrix instruction's A or B registers right after it issues
does not change its result. This was checked on gfx950 with the matrix pipe
idle and busy, over 5e8 results each, so this test does not restrict it.

The assembly is generated here with the library's own flags (device code only,
about 15 s); no GPU is needed.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from ancestral_draft_token_amd import _build

KERNEL = "markov_bias_gumbel_argmax_resident_mfma"
VARIANTS = ["ILb0ELb0EE", "ILb1ELb0EE", "ILb0ELb1EE", "ILb1ELb1EE"]   # <bf16 base, ragged vocabulary>


@pytest.fixture(scope="module")
def asm(tmp_path_factory) -> str:
    if not os.path.exists(_build.hipcc()):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "dspark.s"
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", f"-I{_build.INCLUDE}", "-o", str(out), _build.SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _function(asm: str, variant: str) -> list:
    name = f"_ZN6dspark{len(KERNEL)}{KERNEL}{variant}EvNS_6MfArgsE"
    start = asm.index(f"\n{name}:")
    end = asm.index(".Lfunc_end", start)
    return asm[start:end].splitlines()


def _scratch_by_depth(lines: list) -> list:
    """(loop depth, instruction) of every scratch access, the depth taken from
    the compiler's basic-block comments."""
    depth, out = 0, []
    for line in lines:
        if line.startswith(".LBB") or line.startswith("; %bb"):
            m = re.search(r"Depth=(\d+)", line)
            depth = int(m.group(1)) if m else 0
        s = line.strip()
        if s.startswith("scratch_"):
            out.append((depth, s))
    return out


@pytest.mark.parametrize("variant", VARIANTS)
def test_matrix_kernel_is_a_full_mfma_kernel(asm, variant):
    lines = _function(asm, variant)
    assert sum(1 for l in lines if "v_mfma_f32_16x16x32_bf16" in l) >= 8 * 13


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_agpr_spill(asm, variant):
    bad = [s for _, s in _scratch_by_depth(_function(asm, variant)) if s.startswith("scratch_store") and " a[" in s]
    assert not bad, bad[:5]


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_spill_in_inner_loops(asm, variant):
    bad = [s for d, s in _scratch_by_depth(_function(asm, variant)) if d >= 2]
    assert not bad, bad[:5]


def test_depth_parser():
    lines = [
        ".LBB4_312:                              ; =>This Loop Header: Depth=1",
        "\tscratch_load_dwordx2 v[16:17], off, off offset:8",
        "; %bb.348:                              ;   in Loop: Header=BB4_315 Depth=2",
        "\tscratch_store_dwordx4 off, a[4:7], off",
        ".LBB4_400:",
        "\tscratch_store_dword off, v1, off",
    ]
    assert _scratch_by_depth(lines) == [
        (1, "scratch_load_dwordx2 v[16:17], off, off offset:8"),
        (2, "scratch_store_dwordx4 off, a[4:7], off"),
        (0, "scratch_store_dword off, v1, off"),
    ]


# ---- the windowed block attention ------------------------------------------------

@pytest.fixture(scope="module")
def attn_asm(tmp_path_factory) -> str:
    if not os.path.exists(_build.hipcc()):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "window_attn.s"
    src = [s for s in _build.SOURCES if s.endswith("window_attn.hip")][0]
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", f"-I{_build.INCLUDE}", "-o", str(out), src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _metadata(asm: str, name_part: str) -> dict:
    for blk in asm.split("  - .agpr_count")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        if name_part in name:
            return {"vgpr": int(re.search(r"\.vgpr_count:\s+(\d+)", blk).group(1)),
                    "scratch": int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk).group(1))}
    raise AssertionError(f"{name_part} not found")


def test_attention_kernel_has_no_scratch_and_four_waves_per_simd(attn_asm):
    """The tile loop's staging registers were once demoted to scratch (every
    tile then went through memory twice); and the kernel relies on four
    waves per SIMD (at most 128 registers) to hide the HBM latency."""
    md = _metadata(attn_asm, "wa_partials")
    assert md["scratch"] == 0, md
    assert md["vgpr"] <= 128, md
    lines = attn_asm[attn_asm.index("wa_partials"):].splitlines()
    assert sum(1 for l in lines[:6000] if "v_mfma_f32_16x16x32_bf16" in l) >= 32
