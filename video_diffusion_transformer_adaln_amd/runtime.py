"""Device-memory plumbing around the C ABI, on torch tensors.

torch provides HBM allocations and the current stream; every step of the
block runs in libh3k's kernels.  ``DitStack`` owns the weights of L blocks
and a workspace sized by ``h3k_dit_workspace_size``.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import binding as B


def torch_dtype(code: int):
    import torch
    return {B.H3K_F32: torch.float32, B.H3K_BF16: torch.bfloat16, B.H3K_INT8: torch.int8}[code]


def upload(storage: np.ndarray, kind: str, device="cuda"):
    """Host array -> device tensor.  kind: 'f32', 'bf16' (uint16 patterns) or 'int8'."""
    import torch
    if kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16)
    elif kind == "f32":
        t = torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32))
    elif kind == "int8":
        t = torch.from_numpy(np.ascontiguousarray(storage, dtype=np.int8))
    else:
        raise ValueError(kind)
    return t.to(device)


def alloc_workspace(cfg: B.DitConfig, n_blocks: int = 1, device="cuda"):
    """A 256-byte aligned uint8 workspace tensor of the size the plan needs."""
    import torch
    nbytes = B.h3k_dit_workspace_size(cfg, n_blocks)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def quantize_int8(w, stream=None):
    """Per-row symmetric int8 of a 2-D fp32/bf16 device tensor via the library's quantiser."""
    import torch
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    s = torch.empty((rows,), dtype=torch.float32, device=w.device)
    code = B.H3K_F32 if w.dtype == torch.float32 else B.H3K_BF16
    B.h3k_quantize_weights_int8(w, code, rows, cols, q, s, stream)
    return q, s


def quantize_int8_groups(w, group: int, stream=None):
    """Group-wise symmetric int8 (blocks of `group` columns) of a 2-D fp32/bf16 device tensor."""
    import torch
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=w.device)
    s = torch.empty((rows, cols // group), dtype=torch.float32, device=w.device)
    code = B.H3K_F32 if w.dtype == torch.float32 else B.H3K_BF16
    B.h3k_quantize_weights_int8_groups(w, code, rows, cols, group, q, s, stream)
    return q, s


class DitStack:
    """L blocks of weights on the device plus the shared workspace."""

    def __init__(self, cfg: B.DitConfig, blocks: Sequence[Dict[str, object]], device="cuda"):
        self.cfg = cfg
        self.tensors: List[Dict[str, object]] = list(blocks)
        self.structs = [B.make_weights(t) for t in self.tensors]
        self.workspace = alloc_workspace(cfg, len(self.structs), device)

    def forward(self, x, c, out, n_layers: Optional[int] = None, stream=None,
                stats: Optional[B.DitStats] = None):
        n = len(self.structs) if n_layers is None else n_layers
        if n == 1:
            B.h3k_dit_block_forward(self.cfg, self.structs[0], x, c, out, self.workspace, stream=stream,
                                    stats=stats)
        else:
            B.h3k_dit_stack_forward(self.cfg, self.structs[:n], x, c, out, self.workspace, stream=stream,
                                    stats=stats)
        return out
