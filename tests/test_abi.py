"""The C-ABI library loads and exports every symbol the header declares; host-side
argument checks return their documented status before anything is enqueued.

No kernel runs here: every call below fails a host check (or has B == 0), so
the library returns before its first HIP call.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import ancestral_draft_token_amd as adt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(adt.LIB_PATH):
        from ancestral_draft_token_amd import _build
        _build.build_library()
    return adt.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(adt.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in (adt.DSPARK_OK, adt.DSPARK_ERR_ARG, adt.DSPARK_ERR_UNSUPPORTED,
                 adt.DSPARK_ERR_WORKSPACE, adt.DSPARK_ERR_HIP, adt.DSPARK_ERR_SCRATCH):
        assert adt.status_string(code) and adt.status_string(code) != "unknown status"
    assert adt.status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    small = adt.dspark_workspace_bytes(1, 7, 4096, 32)
    big = adt.dspark_workspace_bytes(96, 7, 200064, 256)
    assert 0 < small < big
    # partials for 1563 chunks of 96 rows (16 B each), plus stats and the embedding rows
    assert big >= 96 * 1563 * 16 + 96 * 7 * 8 + 96 * 256 * 2
    # plus the persistent path's exchange words and per-workgroup statistics
    assert big < 16 << 20
    assert adt.dspark_workspace_bytes(1, 7, 4100, 32) == 0      # V % 8 != 0
    assert adt.dspark_workspace_bytes(1, 7, 4096, 48) == 0      # r % 32 != 0
    assert adt.dspark_workspace_bytes(1, 7, 4096, 2048) == 0    # r > 1024
    assert adt.dspark_workspace_bytes(1, 256, 4096, 32) == 0    # K > 255
    assert adt.dspark_workspace_bytes(-1, 7, 4096, 32) == 0


FAKE = 1 << 20          # a 16-byte aligned address that is never dereferenced


def call(**kw):
    args = dict(base_logits=FAKE, base_dtype=adt.DSPARK_F32, E=FAKE, W=FAKE, prev_token=FAKE,
                seed=FAKE, offset=FAKE, temperature=FAKE, n_real=None, B=2, K=7, V=4096, r=32,
                tokens=FAKE, logits_f32=FAKE, draft_probs=FAKE, workspace=FAKE,
                workspace_bytes=adt.dspark_workspace_bytes(2, 7, 4096, 32), stream=0, check=False)
    args.update(kw)
    return adt.dspark_draft_block(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(V=4100), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(r=48), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(K=300), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(B=-1), adt.DSPARK_ERR_ARG),
    (dict(V=0), adt.DSPARK_ERR_ARG),
    (dict(base_dtype=7), adt.DSPARK_ERR_ARG),
    (dict(base_logits=None), adt.DSPARK_ERR_ARG),
    (dict(E=None), adt.DSPARK_ERR_ARG),
    (dict(W=None), adt.DSPARK_ERR_ARG),
    (dict(prev_token=None), adt.DSPARK_ERR_ARG),
    (dict(seed=None), adt.DSPARK_ERR_ARG),
    (dict(offset=None), adt.DSPARK_ERR_ARG),
    (dict(temperature=None), adt.DSPARK_ERR_ARG),
    (dict(tokens=None), adt.DSPARK_ERR_ARG),
    (dict(logits_f32=None), adt.DSPARK_ERR_ARG),
    (dict(draft_probs=None), adt.DSPARK_ERR_ARG),
    (dict(base_logits=FAKE + 4), adt.DSPARK_ERR_ARG),
    (dict(W=FAKE + 2), adt.DSPARK_ERR_ARG),
    (dict(draft_probs=FAKE + 8), adt.DSPARK_ERR_ARG),
    (dict(workspace=None), adt.DSPARK_ERR_WORKSPACE),
    (dict(workspace_bytes=100), adt.DSPARK_ERR_WORKSPACE),
])
def test_host_checks(lib, kw, status):
    assert call(**kw) == status


def test_bad_chunking(lib):
    assert call(chunk_cols=100) == adt.DSPARK_ERR_UNSUPPORTED
    assert call(chunk_cols=-128) == adt.DSPARK_ERR_UNSUPPORTED


def test_empty_block_enqueues_nothing(lib):
    assert call(B=0, tokens=None, logits_f32=None, draft_probs=None, workspace=None) == adt.DSPARK_OK
    assert call(K=0, tokens=None, logits_f32=None, draft_probs=None, workspace=None) == adt.DSPARK_OK


def test_noalloc_host_checks(lib):
    assert adt.dspark_noalloc_scratch_bytes() == 8 << 20
    args = dict(base_logits=FAKE, base_dtype=adt.DSPARK_F32, E=FAKE, W=FAKE, prev_token=FAKE, seed=FAKE,
                offset=FAKE, temperature=FAKE, n_real=None, B=2, K=7, V=4096, r=32, tokens=FAKE,
                logits_f32=FAKE, draft_probs=FAKE, stream=0, check=False)
    assert adt.dspark_draft_block_noalloc(**dict(args, V=4100)) == adt.DSPARK_ERR_UNSUPPORTED
    assert adt.dspark_draft_block_noalloc(**dict(args, E=None)) == adt.DSPARK_ERR_ARG
    assert adt.dspark_draft_block_noalloc(**dict(args, draft_probs=FAKE + 4)) == adt.DSPARK_ERR_ARG
    assert adt.dspark_draft_block_noalloc(**dict(args, B=0, tokens=None)) == adt.DSPARK_OK


def test_packed_w_host_checks(lib):
    """The packed-W entries' checks that need no device: sizes no resident plan
    runs pack to nothing, bad arguments fail, and the packed block checks its
    own pointer before the rest (here every call returns before a HIP call)."""
    assert adt.dspark_packed_w_bytes(4100, 32) == 0          # V % 8 != 0
    assert adt.dspark_packed_w_bytes(4096, 48) == 0          # r % 32 != 0
    assert adt.dspark_packed_w_bytes(4096, 512) == 0         # r > 256
    assert adt.dspark_packed_w_bytes(1 << 19, 32) == 0       # V > 2^18
    assert adt.dspark_packed_w_bytes(0, 32) == 0
    assert adt.dspark_pack_w(FAKE, 0, 32, FAKE, 1 << 20, stream=0, check=False) == adt.DSPARK_ERR_ARG
    assert adt.dspark_pack_w(FAKE, 4096, -32, FAKE, 1 << 20, stream=0, check=False) == adt.DSPARK_ERR_ARG
    assert adt.dspark_pack_w(FAKE, 4096, 512, FAKE, 1 << 20, stream=0, check=False) == adt.DSPARK_ERR_UNSUPPORTED
    assert lib.dspark_draft_block_packed(FAKE, 0, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, None, 2, 7, 4096, 32,
                                         FAKE, FAKE, FAKE, FAKE, 1 << 20, None, None, 0) == adt.DSPARK_ERR_ARG
    assert call(W_packed=FAKE, packed_bytes=1, V=4100) == adt.DSPARK_ERR_UNSUPPORTED
    assert call(W_packed=FAKE + 8, packed_bytes=1) == adt.DSPARK_ERR_ARG
    assert call(W_packed=FAKE, packed_bytes=1, E=None) == adt.DSPARK_ERR_ARG
    assert call(W_packed=FAKE, packed_bytes=1, workspace=None) == adt.DSPARK_ERR_WORKSPACE
    assert call(W_packed=FAKE, packed_bytes=1, B=0, tokens=None) == adt.DSPARK_OK
    with pytest.raises(ValueError):
        call(W_packed=FAKE, packed_bytes=1, chunk_cols=128)


def call_slots(**kw):
    args = dict(base_logits=FAKE, base_dtype=adt.DSPARK_F32, E=FAKE, W=FAKE, prev_token=FAKE,
                seed=FAKE, offset=FAKE, temperature=FAKE, n_real=None, slot_index=FAKE, n_slots=4,
                B=2, K=7, V=4096, r=32, tokens=FAKE, logits_f32=FAKE, draft_probs=FAKE, workspace=FAKE,
                workspace_bytes=adt.dspark_workspace_bytes(2, 7, 4096, 32), stream=0, check=False)
    args.update(kw)
    return adt.dspark_draft_block_slots(**args)


def test_slot_entry_host_checks(lib):
    """The slot-indexed entry's checks that need no device (every call here
    returns before a HIP call)."""
    assert call_slots(slot_index=None) == adt.DSPARK_ERR_ARG
    assert call_slots(n_slots=0) == adt.DSPARK_ERR_ARG
    assert call_slots(n_slots=-3) == adt.DSPARK_ERR_ARG
    assert call_slots(V=4100) == adt.DSPARK_ERR_UNSUPPORTED
    assert call_slots(draft_probs=FAKE + 4) == adt.DSPARK_ERR_ARG
    assert call_slots(workspace=None) == adt.DSPARK_ERR_WORKSPACE
    assert call_slots(W_packed=FAKE + 8, packed_bytes=1) == adt.DSPARK_ERR_ARG
    assert call_slots(W_packed=FAKE, packed_bytes=1, V=4100) == adt.DSPARK_ERR_UNSUPPORTED
    assert call_slots(B=0, tokens=None) == adt.DSPARK_OK
    with pytest.raises(adt.DSparkError):
        call_slots(n_slots=0, check=True)


def test_block_status_checks_its_pointer(lib):
    assert lib.dspark_block_status(None, None) == adt.DSPARK_ERR_ARG


def test_wait_limit_round_trip(lib):
    prev = adt.dspark_set_wait_limit(5)
    try:
        assert prev == 1 << 20
        assert adt.dspark_set_wait_limit(7) == 5
    finally:
        adt.dspark_set_wait_limit(prev)
    assert adt.dspark_set_wait_limit(prev) == prev


def test_binding_raises_on_error(lib):
    with pytest.raises(adt.DSparkError):
        call(V=4100, check=True)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(adt, "_lib", None)
    with pytest.raises(RuntimeError):
        adt.load_library(str(tmp_path / "nope.so"))


# ---- standard verification: host checks (nothing is enqueued) ---------------

def _verify(lib, rule="standard", **kw):
    a = dict(draft=16, q=16, p=16, seed=16, offset=16, B=2, K=3, V=64, n=16, out=16, ws=16,
             ws_bytes=1 << 20)
    a.update(kw)
    fn = lib.dspark_verify_standard if rule == "standard" else lib.dspark_verify_block
    return fn(a["draft"], a["q"], a["p"], a["seed"], a["offset"], a["B"], a["K"], a["V"], a["n"], a["out"],
              a["ws"], a["ws_bytes"], None)


def test_verify_workspace_bytes(lib):
    assert adt.dspark_verify_workspace_bytes(88, 7, 200064) >= 88 * 25 * 8
    assert adt.dspark_verify_workspace_bytes(1, 7, 8) > 0
    assert adt.dspark_verify_workspace_bytes(1, 256, 64) == 0      # K > 255
    assert adt.dspark_verify_workspace_bytes(1, 7, 66) == 0        # V % 4 != 0


def test_verify_block_workspace_bytes(lib):
    # 98 chunks of 2048 columns per row: a partial mass per position, a key per position and the bonus
    assert adt.dspark_verify_block_workspace_bytes(88, 7, 200064) >= 88 * 98 * (7 + 8) * 8
    assert adt.dspark_verify_block_workspace_bytes(1, 0, 8) > 0
    assert adt.dspark_verify_block_workspace_bytes(1, 256, 64) == 0
    assert adt.dspark_verify_block_workspace_bytes(1, 7, 66) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(p=None), adt.DSPARK_ERR_ARG),
    (dict(q=None), adt.DSPARK_ERR_ARG),
    (dict(n=None), adt.DSPARK_ERR_ARG),
    (dict(p=24), adt.DSPARK_ERR_ARG),                  # p not 16-byte aligned
    (dict(V=66), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(K=256), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(B=-1), adt.DSPARK_ERR_ARG),
    (dict(ws=None), adt.DSPARK_ERR_WORKSPACE),
    (dict(ws_bytes=8), adt.DSPARK_ERR_WORKSPACE),
])
@pytest.mark.parametrize("rule", ["standard", "block"])
def test_verify_host_checks(lib, kw, status, rule):
    assert _verify(lib, rule, **kw) == status


@pytest.mark.parametrize("rule", ["standard", "block"])
def test_verify_empty_batch_enqueues_nothing(lib, rule):
    assert _verify(lib, rule, B=0, draft=None, q=None, p=None) == adt.DSPARK_OK


def _attn(lib, layout=None, **kw):
    a = dict(q=16, k=16, v=16, ctx=16, B=2, K=7, Hq=64, Hkv=4, D=128, L=9000, W=4096, scale=0.088, out=16,
             lse=16, ws=16, ws_bytes=1 << 30)
    a.update(kw)
    head = (a["q"], a["k"], a["v"], a["ctx"], a["B"], a["K"], a["Hq"], a["Hkv"], a["D"], a["L"], a["W"], a["scale"])
    tail = (a["out"], a["lse"], a["ws"], a["ws_bytes"], None)
    if layout is None:
        return lib.dspark_window_block_attention(*head, *tail)
    return lib.dspark_window_block_attention_layout(*head, layout, *tail)


def test_window_attention_workspace_bytes(lib):
    # B=8, 4 key/value heads (32 pairs): the key range split over workgroups,
    # partial outputs and (max, sum) per split
    n = adt.dspark_window_attention_workspace_bytes(8, 7, 64, 4, 128, 8199, 4096)
    assert n >= 8 * 4 * 2 * 7 * 16 * (128 + 2) * 4
    # from 256 (row, key/value head) pairs one launch keeps nothing: a token size
    assert adt.dspark_window_attention_workspace_bytes(88, 7, 64, 4, 128, 8199, 4096) == 256
    assert adt.dspark_window_attention_workspace_bytes(64, 7, 64, 4, 128, 8199, 4096) == 256
    assert adt.dspark_window_attention_workspace_bytes(63, 7, 64, 4, 128, 8199, 4096) > 256
    assert adt.dspark_window_attention_workspace_bytes(1, 7, 64, 4, 64, 8199, 4096) == 0    # D != 128
    assert adt.dspark_window_attention_workspace_bytes(1, 7, 48, 4, 128, 8199, 4096) == 0   # Hq != 16 Hkv
    assert adt.dspark_window_attention_workspace_bytes(1, 9, 64, 4, 128, 8199, 4096) == 0   # K > 8
    assert adt.dspark_window_attention_workspace_bytes(1, 7, 64, 4, 128, 8199, 4) == 0      # K > W


def test_window_attention_split_plan_at_one_row(lib):
    """The split plan shows in the workspace size: partial outputs and (max,
    sum) for B * Hkv * S * K * 16 rows, each region rounded up to 256 bytes.
    One row of the benchmark shape (window 4096: 65 tiles of 64 keys) takes
    33 splits of two tiles, the fastest measured (65 splits of one tile, the
    choice when the merge's read batches were left out of the cost, was 23.0
    against 18.7 us a call)."""
    def size(S, B=1, K=7, Hkv=4):
        rows = B * Hkv * S * K * 16
        up = lambda x: (x + 255) // 256 * 256
        return up(rows * 128 * 4) + up(rows * 2 * 4)
    assert adt.dspark_window_attention_workspace_bytes(1, 7, 64, 4, 128, 8199, 4096) == size(33)
    assert adt.dspark_window_attention_workspace_bytes(1, 8, 64, 4, 128, 8200, 4096) == size(33, K=8)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), adt.DSPARK_ERR_ARG),
    (dict(ctx=None), adt.DSPARK_ERR_ARG),
    (dict(lse=None), adt.DSPARK_ERR_ARG),
    (dict(k=24), adt.DSPARK_ERR_ARG),                  # cache not 16-byte aligned
    (dict(scale=0.0), adt.DSPARK_ERR_ARG),
    (dict(D=64), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(Hq=32), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(K=9), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(L=3), adt.DSPARK_ERR_UNSUPPORTED),
    (dict(K=0), adt.DSPARK_ERR_ARG),
    (dict(ws=None), adt.DSPARK_ERR_WORKSPACE),
    (dict(ws_bytes=8), adt.DSPARK_ERR_WORKSPACE),
])
@pytest.mark.parametrize("layout", [None, adt.DSPARK_KV_LAYOUT_BLHD, adt.DSPARK_KV_LAYOUT_BHLD])
def test_window_attention_host_checks(lib, kw, status, layout):
    assert _attn(lib, layout=layout, **kw) == status


@pytest.mark.parametrize("layout", [-1, 2, 7])
def test_window_attention_rejects_unknown_layout(lib, layout):
    assert _attn(lib, layout=layout) == adt.DSPARK_ERR_ARG


def test_window_attention_empty_batch_enqueues_nothing(lib):
    assert _attn(lib, B=0, q=None, k=None, v=None, ctx=None, out=None, lse=None) == adt.DSPARK_OK
