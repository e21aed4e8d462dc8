"""Checks on the gfx950 assembly of the large-batch (MFMA) kernel, and on the
compiler's hazard model that its register reuse relies on; also that the
small-batch resident kernel has no scratch.

The kernel keeps W resident in registers: 62 of its 64 A-operand fragments
per lane live in AGPRs for the whole launch, read there by the matrix
instructions. A build in which the register allocator spilled some of those
fragments to scratch memory gave bias values that changed from run to run,
and the fragments were then reloaded inside the N-tile loop. That build can
no longer be produced (the allocator does not spill them with the current
source and compiler), and the compiler's hazard model guards the one hazard
its spill code showed (an AGPR write two instructions after a 16-byte spill
store of the same registers: the model requires two wait states there, as it
does for VGPR store data), so its cause is not known. This test keeps that
configuration out:

* no AGPR is spilled (no scratch store with AGPR data) anywhere in the kernel;
* no scratch (spill) access sits inside the kernel's inner loops, where the W
  fragments and the per-tile state live (a spill there would also stall every
  tile on the scratch round trip).

The kernel also overwrites a matrix instruction's A operand with the next
LDS fragment read right after issuing it (the LDS chains of the epilogue).
The kernel is written with compiler builtins only, so the backend's hazard
recognizer, which inserts the wait states the ISA requires between dependent
instructions, sees every one of those instructions. The tests below run that
recognizer (llc's post-RA hazard pass for gfx950) on fixed-register
sequences and pin what it requires after v_mfma_f32_16x16x32_bf16: wait
states before a VALU write of SrcC or a read of the result, none before a
VALU or LDS write of SrcA or SrcB (those operands are consumed at issue),
and two wait states before a write of a 16-byte store's data registers,
AGPRs included.

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
# <bf16 base, ragged vocabulary, packed W>
VARIANTS = [f"ILb{b}ELb{g}ELb{p}EE" for p in (0, 1) for g in (0, 1) for b in (0, 1)]


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


# The small-batch (VALU) resident kernel, <rows, bf16 base, packed W>: no
# scratch at all. Its position loop polls exchange words while the next
# position's noise and statistics are computed; a spill reload there waits for
# every load in flight, the polls included (a two-row build spilled Philox
# round keys, reloaded in the next position's noise).
SMALL = [f"ILi{rb}ELb{b}ELb{p}EE" for rb in (1, 2) for b in (0, 1) for p in (0, 1)]


@pytest.mark.parametrize("variant", SMALL)
def test_small_batch_kernel_has_no_scratch(asm, variant):
    kernel = "markov_bias_gumbel_argmax_resident"
    name = f"_ZN6dspark{len(kernel)}{kernel}{variant}EvNS_7ResArgsE"
    desc = re.search(r"\.amdhsa_kernel " + re.escape(name) + r"\n(.*?)\.end_amdhsa_kernel", asm, re.S).group(1)
    assert int(re.search(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", desc).group(1)) == 0
    start = asm.index(f"\n{name}:")
    body = asm[start:asm.index(".Lfunc_end", start)]
    assert "scratch_" not in body


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


# ---- the compiler's hazard model after a matrix instruction ------------------------

LLC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llc")
MFMA = ("$vgpr12_vgpr13_vgpr14_vgpr15 = V_MFMA_F32_16X16X32_BF16_vgprcd_e64 $vgpr4_vgpr5_vgpr6_vgpr7, "
        "$vgpr8_vgpr9_vgpr10_vgpr11, $vgpr0_vgpr1_vgpr2_vgpr3, 0, 0, 0, implicit $mode, implicit $exec")
ST_AGPR = ("SCRATCH_STORE_DWORDX4_ST $agpr0_agpr1_agpr2_agpr3, 0, 0, implicit $exec, implicit $flat_scr "
           ":: (store (s128), addrspace 5)")
ST_VGPR = ("SCRATCH_STORE_DWORDX4_ST $vgpr4_vgpr5_vgpr6_vgpr7, 0, 0, implicit $exec, implicit $flat_scr "
           ":: (store (s128), addrspace 5)")
HAZARD_CASES = {
    # name: (instructions, wait states the recognizer must insert before the last one)
    "valu_writes_srcC": ([MFMA, "$vgpr0 = V_MOV_B32_e32 $vgpr20, implicit $exec"], "some"),
    "valu_reads_result": ([MFMA, "$vgpr30 = V_MOV_B32_e32 $vgpr12, implicit $exec"], "some"),
    "valu_writes_srcA": ([MFMA, "$vgpr4 = V_MOV_B32_e32 $vgpr20, implicit $exec"], 0),
    "valu_writes_srcB": ([MFMA, "$vgpr8 = V_MOV_B32_e32 $vgpr20, implicit $exec"], 0),
    "lds_read_writes_srcA": ([MFMA, "$vgpr4_vgpr5_vgpr6_vgpr7 = DS_READ_B128_gfx9 $vgpr20, 0, 0, implicit $exec"], 0),
    "store_vgpr_data_then_write": ([ST_VGPR, "$vgpr4 = V_MOV_B32_e32 $vgpr20, implicit $exec"], 2),
    "store_agpr_data_then_write": ([ST_AGPR, "$agpr0 = V_ACCVGPR_WRITE_B32_e64 $vgpr20, implicit $exec"], 2),
}


@pytest.fixture(scope="module")
def hazard_out(tmp_path_factory) -> str:
    if not os.path.exists(LLC):
        pytest.skip("llc not available")
    lines = ["--- |"] + [f"  define amdgpu_kernel void @{n}() {{ ret void }}" for n in HAZARD_CASES] + ["..."]
    for n, (ins, _) in HAZARD_CASES.items():
        lines += ["---", f"name: {n}", "tracksRegLiveness: true", "body: |", "  bb.0:",
                  "    liveins: $vgpr0_vgpr1_vgpr2_vgpr3, $vgpr4_vgpr5_vgpr6_vgpr7, $vgpr8_vgpr9_vgpr10_vgpr11, "
                  "$agpr0_agpr1_agpr2_agpr3, $vgpr20"] + ["    " + i for i in ins] + ["    S_ENDPGM 0", "..."]
    mir = tmp_path_factory.mktemp("hazard") / "cases.mir"
    mir.write_text("\n".join(lines) + "\n")
    r = subprocess.run([LLC, "-mtriple=amdgcn-amd-amdhsa", "-mcpu=gfx950", "-run-pass=post-RA-hazard-rec",
                        "-o", "-", str(mir)], check=True, capture_output=True, text=True)
    return r.stdout


def _wait_states(out: str, name: str) -> int:
    body = out[out.index(f"name:            {name}"):]
    body = body[:body.index("S_ENDPGM")]
    return sum(int(m.group(1)) + 1 for m in re.finditer(r"S_NOP (\d+)", body))


@pytest.mark.parametrize("name", list(HAZARD_CASES))
def test_hazard_model(hazard_out, name):
    got = _wait_states(hazard_out, name)
    want = HAZARD_CASES[name][1]
    if want == "some":
        assert got > 0, name
    else:
        assert got == want, (name, got)
