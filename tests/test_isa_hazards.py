"""Checks on the gfx950 assembly of the large-batch (MFMA) kernel.

The compiler's hazard model for matrix instructions covers a late read of the
accumulator input, not of the A and B operands. A build in which a reloaded A
operand was rewritten by the very next VALU instruction produced bias values
that changed from run to run, so the kernel is written to keep that pattern
out, and this test holds it out:

* no VALU instruction writes a register that a matrix instruction read as its
  A or B operand among the first 8 VALU instructions after it (each takes at
  least 4 cycles on a 16-lane SIMD, so that is 32 cycles or more: at least the
  whole duration of a 16x16x32 bf16 matrix instruction). A matrix instruction
  that accumulates onto an earlier one's result ends that one's window (it
  cannot start before the earlier one has read its operands). Loads from LDS
  or memory are exempt: their results arrive a memory latency after issue;
* no scratch (spill) access sits inside the kernel's inner loops, where the W
  fragments and the per-tile state live.

The assembly is generated here with the library's own flags (device code only,
about 15 s); no GPU is needed.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from ancestral_draft_token_amd import _build

WINDOW = 8   # VALU instructions
KERNEL = "markov_bias_gumbel_argmax_resident_mfma"
VARIANTS = ["ILb0ELb0EE", "ILb1ELb0EE", "ILb0ELb1EE", "ILb1ELb1EE"]   # <bf16 base, ragged vocabulary>
_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


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


def _operand_overwrites(lines: list) -> list:
    """(VALU distance, mfma line, writer line, opcode) for VALU writes of A/B
    operands; the distance counts the VALU instructions after the MFMA, the
    writer included (scalar instructions and s_nop count as none)."""
    pending, hits = [], []   # (A/B registers, destination, line, distance)
    for ln, line in enumerate(lines):
        s = line.strip()
        if not s or s.startswith(";") or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        parts = [p.strip() for p in s[len(op):].split(";")[0].split(",")]
        if op.startswith("v_mfma"):
            src_c = _regs(parts[3]) if len(parts) > 3 else set()
            pending = [e for e in pending if not (e[1] & src_c)]
            pending.append((_regs(parts[1]) | _regs(parts[2]), _regs(parts[0]), ln, 0))
        elif op.startswith("v_"):
            pending = [(ab, dst, i, d + 1) for ab, dst, i, d in pending]
            written = _regs(parts[0]) if parts[0] else set()
            hits += [(d, i, ln, op) for ab, dst, i, d in pending if ab & written]
            pending = [e for e in pending if e[3] < WINDOW]
    return hits


@pytest.mark.parametrize("variant", VARIANTS)
def test_mfma_operands_not_rewritten_soon_after(asm, variant):
    lines = _function(asm, variant)
    assert any("v_mfma" in l for l in lines)
    hits = _operand_overwrites(lines)
    assert not hits, [(d, lines[i].strip(), lines[j].strip()) for d, i, j, _ in hits[:5]]


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_spill_in_inner_loops(asm, variant):
    depth, bad = 0, []
    for line in _function(asm, variant):
        m = re.search(r"Depth=(\d+)", line)
        if line.startswith(".LBB") or line.startswith("; %bb"):
            depth = int(m.group(1)) if m else 0
        if "scratch_" in line and depth >= 2:
            bad.append(line.strip())
    assert not bad, bad[:5]


def test_scanner_flags_a_planted_overwrite():
    """The scanner itself: A and B operands rewritten within the window are found
    (nops and scalar instructions do not widen it); one rewritten after 8 VALU
    instructions, or by an LDS load, is not."""
    mfma = "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], 0"
    add = "\tv_add_f32_e32 v1, v2, v3"
    write_a = "\tv_bitop3_b32 v5, v1, v2, v3 bitop3:0x96"
    write_b = "\tv_mad_u64_u32 v[10:11], s[0:1], v1, s38, 0"
    assert [h[3] for h in _operand_overwrites([mfma, add, write_a])] == ["v_bitop3_b32"]
    assert [h[0] for h in _operand_overwrites([mfma, "\ts_nop 7", "\ts_mov_b32 s0, 0", write_b])] == [1]
    assert _operand_overwrites([mfma] + [add] * 7 + [write_a]) != []
    assert _operand_overwrites([mfma] + [add] * 8 + [write_a]) == []
    assert _operand_overwrites([mfma, "\tds_read_b128 v[4:7], v12 offset:1024"]) == []
    chained = "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[12:15], v[16:19], a[0:3]"
    assert _operand_overwrites([mfma, chained, write_a]) == []
    assert [h[3] for h in _operand_overwrites([mfma, chained, "\tv_mov_b32_e32 v13, 0"])] == ["v_mov_b32_e32"]

