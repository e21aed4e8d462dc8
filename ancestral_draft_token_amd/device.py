"""Device buffers for one draft-block problem (PyTorch as memory and stream plumbing).

``DeviceProblem`` copies a host workload to the GPU, allocates the outputs
and the workspace once, and enqueues the library's draft block on a stream.
Nothing here computes any part of the sampler.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (DSPARK_BF16, DSPARK_F32, dspark_draft_block, dspark_init, dspark_pack_w, dspark_packed_w_bytes,
               dspark_workspace_bytes)
from .inputs import Workload


class DeviceProblem:
    def __init__(self, w: Workload, device: str = "cuda:0", chunk_cols: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None, packed: bool = False):
        self.w = w
        self.device = torch.device(device)
        self.chunk_cols = chunk_cols
        dev = self.device
        dspark_init()
        self.base_dtype = DSPARK_BF16 if w.base_dtype == "bf16" else DSPARK_F32
        base = torch.from_numpy(np.ascontiguousarray(w.base))
        if w.base_dtype == "bf16":
            base = base.view(torch.int16)
        self.base = base.to(dev)
        self.E = torch.from_numpy(w.E.view(np.int16)).to(dev)
        self.W = torch.from_numpy(w.W.view(np.int16)).to(dev)
        self.prev = torch.from_numpy(np.ascontiguousarray(w.prev_token, np.int32)).to(dev)
        self.seed = torch.from_numpy(np.ascontiguousarray(w.seed, np.int64)).to(dev)
        self.offset = torch.from_numpy(np.ascontiguousarray(w.offset, np.int64)).to(dev)
        self.temperature = torch.from_numpy(np.ascontiguousarray(w.temperature, np.float32)).to(dev)
        self.n_real = None
        if w.n_real is not None:
            self.n_real = torch.tensor([w.n_real], dtype=torch.int32, device=dev)
        B, K, V, r = w.B, w.K, w.V, w.r
        self.tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
        self.logits = torch.empty((B, K, V), dtype=torch.float32, device=dev)
        self.q = torch.empty((B, K, V), dtype=torch.float32, device=dev)
        self.ws_bytes = dspark_workspace_bytes(B, K, V, r)
        if workspace is not None:
            # a workspace shared by several problems (calls run one at a time)
            if workspace.numel() * workspace.element_size() < self.ws_bytes:
                raise ValueError("shared workspace is too small")
            self.workspace = workspace
        else:
            self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        # W packed once for the resident kernels (a weight: the same for every block)
        self.W_packed, self.packed_bytes = None, 0
        if packed and chunk_cols is None:
            self.packed_bytes = dspark_packed_w_bytes(V, r)
            if self.packed_bytes:
                self.W_packed = torch.empty(self.packed_bytes, dtype=torch.uint8, device=dev)
                dspark_pack_w(self.W, V, r, self.W_packed, self.packed_bytes)
                torch.cuda.synchronize(dev)

    def enqueue(self, stream=None, **overrides) -> int:
        """Enqueue one block on ``stream`` (torch stream / raw handle / None = current)."""
        w = self.w
        kw = dict(base_logits=self.base, base_dtype=self.base_dtype, E=self.E, W=self.W,
                  prev_token=self.prev, seed=self.seed, offset=self.offset,
                  temperature=self.temperature, n_real=self.n_real, B=w.B, K=w.K, V=w.V, r=w.r,
                  tokens=self.tokens, logits_f32=self.logits, draft_probs=self.q,
                  workspace=self.workspace, workspace_bytes=self.ws_bytes, stream=stream,
                  chunk_cols=self.chunk_cols)
        if self.W_packed is not None:
            kw.update(W_packed=self.W_packed, packed_bytes=self.packed_bytes)
        kw.update(overrides)
        return dspark_draft_block(**kw)

    def run(self):
        """Enqueue one block on the current stream, wait, and return host copies."""
        self.enqueue()
        torch.cuda.synchronize(self.device)
        return self.outputs()

    def outputs(self):
        return (self.tokens.cpu().numpy(), self.logits.cpu().numpy(), self.q.cpu().numpy())
