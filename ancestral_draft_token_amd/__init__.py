"""DSpark ancestral draft-block sampler for MI355X (gfx950).

A thin Python binding over the C ABI of ``libdspark.so`` (declared in
``include/dspark.h``). Every step of the sampler runs in the library's HIP
kernels; this module only loads the library and turns torch device tensors
into pointers and sizes. It has no fallback: if the library is missing or a
call fails, it raises.

PyTorch supplies device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdspark.so")

DSPARK_F32 = 0
DSPARK_BF16 = 1
DSPARK_OK = 0
DSPARK_ERR_ARG = -1
DSPARK_ERR_UNSUPPORTED = -2
DSPARK_ERR_WORKSPACE = -3
DSPARK_ERR_HIP = -4
DSPARK_ERR_SCRATCH = -5

# key/value cache layouts of the window attention
DSPARK_KV_LAYOUT_BLHD = 0   # [B, L, Hkv, D]
DSPARK_KV_LAYOUT_BHLD = 1   # [B, Hkv, L, D]

EXPORTED = ("dspark_init", "dspark_workspace_bytes", "dspark_draft_block",
            "dspark_draft_block_chunked", "dspark_draft_block_events", "dspark_launch_plan",
            "dspark_status_string", "dspark_verify_workspace_bytes", "dspark_verify_standard",
            "dspark_verify_block_workspace_bytes", "dspark_verify_block",
            "dspark_window_attention_workspace_bytes", "dspark_window_block_attention",
            "dspark_block_status", "dspark_set_wait_limit",
            "dspark_draft_block_noalloc", "dspark_noalloc_scratch_bytes",
            "dspark_window_block_attention_layout", "dspark_packed_w_bytes", "dspark_pack_w",
            "dspark_draft_block_packed", "dspark_draft_block_slots")

LAUNCH_KINDS = {0: "markov_bias_gumbel_argmax", 1: "pick_and_gather", 2: "proposal_softmax",
                4: "markov_bias_gumbel_argmax"}

_lib = None


class DSparkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status} ({status_string(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load ``libdspark.so`` (built by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime; import it first so the library binds to
    # that same runtime (one runtime per process: streams and pointers agree)
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.dspark_init.argtypes = []
    lib.dspark_init.restype = I
    lib.dspark_workspace_bytes.argtypes = [I, I, I, I]
    lib.dspark_workspace_bytes.restype = Z
    block_args = [P, I, P, P, P, P, P, P, P, I, I, I, I]
    out_args = [P, P, P, P, Z, P]
    lib.dspark_draft_block.argtypes = block_args + out_args
    lib.dspark_draft_block.restype = I
    lib.dspark_draft_block_chunked.argtypes = block_args + [I] + out_args
    lib.dspark_draft_block_chunked.restype = I
    lib.dspark_draft_block_events.argtypes = block_args + out_args + [P, I]
    lib.dspark_draft_block_events.restype = I
    lib.dspark_launch_plan.argtypes = [I, I, I, I, P, I]
    lib.dspark_launch_plan.restype = I
    lib.dspark_status_string.argtypes = [I]
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_verify_workspace_bytes.argtypes = [I, I, I]
    lib.dspark_verify_workspace_bytes.restype = Z
    lib.dspark_verify_standard.argtypes = [P, P, P, P, P, I, I, I, P, P, P, Z, P]
    lib.dspark_verify_standard.restype = I
    lib.dspark_verify_block_workspace_bytes.argtypes = [I, I, I]
    lib.dspark_verify_block_workspace_bytes.restype = Z
    lib.dspark_verify_block.argtypes = [P, P, P, P, P, I, I, I, P, P, P, Z, P]
    lib.dspark_verify_block.restype = I
    lib.dspark_window_attention_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.dspark_window_attention_workspace_bytes.restype = Z
    lib.dspark_window_block_attention.argtypes = [P, P, P, P, I, I, I, I, I, I, I, ctypes.c_float, P, P, P, Z, P]
    lib.dspark_window_block_attention.restype = I
    lib.dspark_window_block_attention_layout.argtypes = [P, P, P, P, I, I, I, I, I, I, I, ctypes.c_float, I,
                                                         P, P, P, Z, P]
    lib.dspark_window_block_attention_layout.restype = I
    lib.dspark_block_status.argtypes = [P, P]
    lib.dspark_block_status.restype = I
    lib.dspark_set_wait_limit.argtypes = [ctypes.c_uint]
    lib.dspark_set_wait_limit.restype = ctypes.c_uint
    lib.dspark_draft_block_noalloc.argtypes = block_args + [P, P, P, P]
    lib.dspark_draft_block_noalloc.restype = I
    lib.dspark_noalloc_scratch_bytes.argtypes = []
    lib.dspark_noalloc_scratch_bytes.restype = Z
    lib.dspark_packed_w_bytes.argtypes = [I, I]
    lib.dspark_packed_w_bytes.restype = Z
    lib.dspark_pack_w.argtypes = [P, I, I, P, Z, P]
    lib.dspark_pack_w.restype = I
    lib.dspark_draft_block_packed.argtypes = [P, I, P, P, P, Z, P, P, P, P, P, I, I, I, I] + out_args + [P, I]
    lib.dspark_draft_block_packed.restype = I
    lib.dspark_draft_block_slots.argtypes = [P, I, P, P, P, Z, P, P, P, P, P, P, I, I, I, I, I] + out_args
    lib.dspark_draft_block_slots.restype = I
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().dspark_status_string(int(status)).decode()


def dspark_init() -> None:
    rc = load_library().dspark_init()
    if rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_init")


def dspark_workspace_bytes(B: int, K: int, V: int, r: int) -> int:
    return int(load_library().dspark_workspace_bytes(B, K, V, r))


def dspark_launch_plan(B: int, K: int, V: int, r: int):
    """The launch kinds (ints) one block enqueues on the current device, in order."""
    lib = load_library()
    kinds = (ctypes.c_int * (2 * K + 4))()
    n = lib.dspark_launch_plan(B, K, V, r, kinds, len(kinds))
    if n < 0:
        raise DSparkError(n, "dspark_launch_plan")
    return [int(kinds[i]) for i in range(n)]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dspark_draft_block(base_logits, base_dtype: int, E, W, prev_token, seed, offset, temperature,
                       n_real, B: int, K: int, V: int, r: int, tokens, logits_f32, draft_probs,
                       workspace, workspace_bytes: int, stream=None, chunk_cols: Optional[int] = None,
                       events=None, check: bool = True, W_packed=None, packed_bytes: int = 0) -> int:
    """Enqueue one draft block; arguments as in ``include/dspark.h``.

    Tensor arguments may be torch device tensors or raw device addresses
    (ints); ``n_real`` may be None. ``stream`` is a torch stream, a raw
    hipStream_t, or None for torch's current stream. Returns the status; with
    ``check`` a nonzero status raises. ``events`` (a ctypes array of
    hipEvent_t handles, at least 2K + 2) selects ``dspark_draft_block_events``.
    ``W_packed`` (from ``dspark_pack_w``, with its ``packed_bytes``) selects
    ``dspark_draft_block_packed`` (events optional; no explicit chunking).
    """
    lib = load_library()
    args = [_ptr(base_logits), int(base_dtype), _ptr(E), _ptr(W), _ptr(prev_token), _ptr(seed),
            _ptr(offset), _ptr(temperature), _ptr(n_real), int(B), int(K), int(V), int(r)]
    outs = [_ptr(tokens), _ptr(logits_f32), _ptr(draft_probs), _ptr(workspace), int(workspace_bytes),
            _stream_ptr(stream)]
    if W_packed is not None:
        if chunk_cols is not None:
            raise ValueError("a packed W goes with the library's own chunking")
        ev = (ctypes.cast(events, ctypes.c_void_p), len(events)) if events is not None else (None, 0)
        rc = lib.dspark_draft_block_packed(*args[:4], _ptr(W_packed), int(packed_bytes), *args[4:], *outs, *ev)
        where = "dspark_draft_block_packed"
    elif events is not None:
        rc = lib.dspark_draft_block_events(*args, *outs, ctypes.cast(events, ctypes.c_void_p), len(events))
        where = "dspark_draft_block_events"
    elif chunk_cols is None:
        rc = lib.dspark_draft_block(*args, *outs)
        where = "dspark_draft_block"
    else:
        rc = lib.dspark_draft_block_chunked(*args, int(chunk_cols), *outs)
        where = "dspark_draft_block_chunked"
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, where)
    return rc


def dspark_draft_block_slots(base_logits, base_dtype: int, E, W, prev_token, seed, offset, temperature,
                             n_real, slot_index, n_slots: int, B: int, K: int, V: int, r: int, tokens,
                             logits_f32, draft_probs, workspace, workspace_bytes: int, stream=None,
                             W_packed=None, packed_bytes: int = 0, check: bool = True) -> int:
    """Enqueue one draft block whose proposals go to ``draft_probs`` rows
    ``slot_index[b]`` (``[n_slots, K, V]``); arguments as in ``include/dspark.h``
    (``W_packed`` optional). Returns the status; with ``check`` a nonzero
    status raises."""
    lib = load_library()
    rc = lib.dspark_draft_block_slots(
        _ptr(base_logits), int(base_dtype), _ptr(E), _ptr(W), _ptr(W_packed),
        int(packed_bytes) if W_packed is not None else 0, _ptr(prev_token), _ptr(seed), _ptr(offset),
        _ptr(temperature), _ptr(n_real), _ptr(slot_index), int(n_slots), int(B), int(K), int(V), int(r),
        _ptr(tokens), _ptr(logits_f32), _ptr(draft_probs), _ptr(workspace), int(workspace_bytes),
        _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_draft_block_slots")
    return rc


def dspark_packed_w_bytes(V: int, r: int) -> int:
    """Bytes of W packed for the resident kernels on the current device (0: nothing to pack)."""
    return int(load_library().dspark_packed_w_bytes(int(V), int(r)))


def dspark_pack_w(W, V: int, r: int, W_packed, packed_bytes: int, stream=None, check: bool = True) -> int:
    """Enqueue the packing of W [r, V] (bf16) into ``W_packed``; see ``include/dspark.h``."""
    rc = load_library().dspark_pack_w(_ptr(W), int(V), int(r), _ptr(W_packed), int(packed_bytes),
                                      _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_pack_w")
    return rc


def dspark_draft_block_noalloc(base_logits, base_dtype: int, E, W, prev_token, seed, offset, temperature,
                               n_real, B: int, K: int, V: int, r: int, tokens, logits_f32, draft_probs,
                               stream=None, check: bool = True) -> int:
    """Enqueue one draft block without a workspace (the library's static
    scratch); arguments as in ``include/dspark.h``."""
    rc = load_library().dspark_draft_block_noalloc(
        _ptr(base_logits), int(base_dtype), _ptr(E), _ptr(W), _ptr(prev_token), _ptr(seed), _ptr(offset),
        _ptr(temperature), _ptr(n_real), int(B), int(K), int(V), int(r), _ptr(tokens), _ptr(logits_f32),
        _ptr(draft_probs), _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_draft_block_noalloc")
    return rc


def dspark_noalloc_scratch_bytes() -> int:
    return int(load_library().dspark_noalloc_scratch_bytes())


def dspark_block_status(status, stream=None, check: bool = True) -> int:
    """Enqueue the status read of the last resident block on the current device
    into ``status`` (a device int32 tensor or address); see ``include/dspark.h``."""
    rc = load_library().dspark_block_status(_ptr(status), _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_block_status")
    return rc


def dspark_set_wait_limit(reads: int) -> int:
    """Set the resident kernels' wait limit (reads of an exchange word) for later
    calls; returns the previous limit."""
    return int(load_library().dspark_set_wait_limit(int(reads)))


def dspark_verify_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().dspark_verify_workspace_bytes(B, K, V))


def dspark_verify_standard(draft_tokens, draft_probs, target_probs, seed, offset, B: int, K: int, V: int,
                           n_accepted, out_tokens, workspace, workspace_bytes: int, stream=None,
                           check: bool = True) -> int:
    """Enqueue standard token-level verification; arguments as in ``include/dspark.h``
    (torch device tensors or raw device addresses; ``stream`` as for
    ``dspark_draft_block``)."""
    lib = load_library()
    rc = lib.dspark_verify_standard(_ptr(draft_tokens), _ptr(draft_probs), _ptr(target_probs), _ptr(seed),
                                    _ptr(offset), int(B), int(K), int(V), _ptr(n_accepted), _ptr(out_tokens),
                                    _ptr(workspace), int(workspace_bytes), _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_verify_standard")
    return rc


def dspark_verify_block_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().dspark_verify_block_workspace_bytes(B, K, V))


def dspark_verify_block(draft_tokens, draft_probs, target_probs, seed, offset, B: int, K: int, V: int,
                        n_accepted, out_tokens, workspace, workspace_bytes: int, stream=None,
                        check: bool = True) -> int:
    """Enqueue block verification; arguments as in ``include/dspark.h`` (the same
    as ``dspark_verify_standard``)."""
    lib = load_library()
    rc = lib.dspark_verify_block(_ptr(draft_tokens), _ptr(draft_probs), _ptr(target_probs), _ptr(seed),
                                 _ptr(offset), int(B), int(K), int(V), _ptr(n_accepted), _ptr(out_tokens),
                                 _ptr(workspace), int(workspace_bytes), _stream_ptr(stream))
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, "dspark_verify_block")
    return rc


def dspark_window_attention_workspace_bytes(B: int, K: int, Hq: int, Hkv: int, D: int, L: int, W: int) -> int:
    return int(load_library().dspark_window_attention_workspace_bytes(B, K, Hq, Hkv, D, L, W))


def dspark_window_block_attention(q, k_cache, v_cache, ctx_len, B: int, K: int, Hq: int, Hkv: int, D: int, L: int,
                                  W: int, scale: float, out, lse, workspace, workspace_bytes: int, stream=None,
                                  check: bool = True, layout: int | None = None) -> int:
    """Enqueue the drafter's non-causal windowed block attention; arguments as in
    ``include/dspark.h``. ``layout`` None calls dspark_window_block_attention
    (caches [B, L, Hkv, D]); a DSPARK_KV_LAYOUT_* value calls
    dspark_window_block_attention_layout with it."""
    lib = load_library()
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), int(B), int(K), int(Hq), int(Hkv), int(D), int(L),
            int(W), float(scale))
    tail = (_ptr(out), _ptr(lse), _ptr(workspace), int(workspace_bytes), _stream_ptr(stream))
    if layout is None:
        name = "dspark_window_block_attention"
        rc = lib.dspark_window_block_attention(*head, *tail)
    else:
        name = "dspark_window_block_attention_layout"
        rc = lib.dspark_window_block_attention_layout(*head, int(layout), *tail)
    if check and rc != DSPARK_OK:
        raise DSparkError(rc, name)
    return rc
