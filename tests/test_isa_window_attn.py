"""Checks on the gfx950 assembly of the single-launch window attention kernel
(wa_block, one instance per number of position slots a wave holds).

Its key tiles stream through an LDS ring filled by LDS-direct loads written
as inline assembly (s_mov_b32 m0 / global_load_lds_dwordx4), which the tile
loop waits for itself with vmcnt. Two properties of the generated code make
that correct and keep the ring full, and neither is visible in the source:

* M0 holds the LDS address of those loads. The compiler reserves M0 and does
  not track the assembly's writes to it, so no compiler-generated
  instruction of these kernels may use M0: every M0 reference sits inside
  an inline-assembly block.
* Inside the tile loop the only vmcnt waits are its own, each right before
  a barrier (a compiler wait for the query fragments, or for an LDS read it
  ties to the loads, would drain every tile in flight on each iteration).

Also: no scratch (spill) memory, and at most 256 registers a lane, so that
two 4-wave workgroups fit on a CU (two waves per SIMD). The assembly is
generated here with the library's own flags (device code only); no GPU is
needed.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from ancestral_draft_token_amd import _build

SRC = os.path.join(_build.PKG, "csrc", "window_attn.hip")
SLOTS = [1, 2]


@pytest.fixture(scope="module")
def asm(tmp_path_factory) -> str:
    if not os.path.exists(_build.hipcc()):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "window_attn.s"
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", f"-I{_build.INCLUDE}", "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _body(asm: str, slots: int) -> list[str]:
    name = f"_ZN9dspark_wa8wa_blockILi{slots}EEEvNS_6WaArgsE"
    i = asm.index(f"\n{name}:")
    j = asm.index(".Lfunc_end", i)
    return asm[i:j].split("\n")


def _descriptor(asm: str, slots: int) -> dict:
    name = f"_ZN9dspark_wa8wa_blockILi{slots}EEEvNS_6WaArgsE"
    body = re.search(r"\.amdhsa_kernel " + re.escape(name) + r"\n(.*?)\.end_amdhsa_kernel", asm, re.S).group(1)
    return {k: int(v) for k, v in re.findall(r"\.amdhsa_(\w+)\s+(\d+)", body)}


@pytest.mark.parametrize("slots", SLOTS)
def test_m0_only_in_the_lds_direct_loads(asm, slots):
    inside, n_asm, outside = False, 0, []
    for line in _body(asm, slots):
        if "ASMSTART" in line:
            inside = True
            continue
        if "ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0]
        if re.search(r"\bm0\b", code):
            if inside:
                n_asm += 1
            else:
                outside.append(line.strip())
    assert not outside, outside
    assert n_asm >= 8           # 4 loads (K and V, 2 each) in the prologue and in the loop


@pytest.mark.parametrize("slots", SLOTS)
def test_vmcnt_waits_only_before_the_tile_barriers(asm, slots):
    """Once the first LDS-direct load is issued, every vmcnt wait is one of
    the ring's own (the prologue's for tile 0 with two tiles of 4 loads
    behind it, the tile loop's with one, vmcnt(0) at the end of the range),
    and the barrier follows it with no memory instruction in between."""
    body = [l.split(";")[0].strip() for l in _body(asm, slots)]
    first = next(n for n, l in enumerate(body) if l.startswith("global_load_lds"))
    waits = [n for n, l in enumerate(body) if n > first and "vmcnt" in l]
    assert waits
    counts = set()
    for n in waits:
        m = re.fullmatch(r"s_waitcnt vmcnt\((\d+)\)", body[n])
        assert m, body[n]
        counts.add(int(m.group(1)))
        for l in body[n + 1:]:
            # the barrier, or a branch to it (the end-of-range waits sit in a
            # switch), before any memory instruction
            if l.startswith("s_barrier") or l.startswith("s_branch") or l.startswith("s_cbranch"):
                break
            assert not re.match(r"(ds_|global_|buffer_|scratch_|flat_)", l), (body[n], l)
        else:
            raise AssertionError(f"no barrier after {body[n]}")
    assert counts <= {0, 4, 8, 12, 16} and 4 in counts, counts


@pytest.mark.parametrize("slots", SLOTS)
def test_both_lane_swap_results_are_used(asm, slots):
    """The per-head maximum reduces over lanes with v_permlane32_swap and
    v_permlane16_swap, each of which leaves its two results in its two
    registers: both must be read before either is overwritten (a compiler
    that took the pair for one value would drop one, and the maximum would
    then cover only part of a head's lanes)."""
    body = [l.split(";")[0].strip() for l in _body(asm, slots)]
    swaps = [n for n, l in enumerate(body) if re.match(r"v_permlane(16|32)_swap", l)]
    assert len(swaps) >= 2 * slots
    for n in swaps:
        regs = re.findall(r"v\d+", body[n].split(None, 1)[1])
        assert len(regs) == 2, body[n]
        for r in regs:
            read = False
            for l in body[n + 1:n + 40]:
                parts = l.split(None, 1)
                if len(parts) < 2:
                    continue
                ops = [o.strip() for o in parts[1].split(",")]
                if any(re.fullmatch(re.escape(r), o) for o in ops[1:]):
                    read = True
                    break
                if ops and re.fullmatch(re.escape(r), ops[0]):
                    break          # overwritten without having been read
            assert read, (body[n], r)


@pytest.mark.parametrize("slots", SLOTS)
def test_registers_and_no_scratch(asm, slots):
    d = _descriptor(asm, slots)
    assert d["private_segment_fixed_size"] == 0
    assert d["next_free_vgpr"] <= 256
    assert not any(re.match(r"\s+scratch_", l) for l in _body(asm, slots))
