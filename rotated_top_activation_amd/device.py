"""Device-side set-up of rotated sparse linears: upload, prepare, fold.

Marshalling around the C ABI only: tensors are allocated by torch and every
step (transposing the rotation, folding it into the weight, the forward
pass) runs in liblarosa's kernels.
"""
from __future__ import annotations

import numpy as np

from . import _lib
from .workloads import to_torch


class RotatedLinear:
    """One rotated sparse linear on the GPU.

    q_blocks: packed rotation [d_in // q_block, q_block, q_block]; w:
    [d_in, d_out]; either float64 arrays of stored values or device tensors
    of the storage dtype. Keeps Q, the prepared Qt, W (unless keep_w is
    False) and the folded W'.
    """

    def __init__(self, q_blocks, w, dtype: str, k: int, device: str = "cuda",
                 keep_w: bool = True):
        import torch
        nb, qb, _ = q_blocks.shape
        self.d_in = nb * qb
        self.q_block = qb
        self.d_out = w.shape[1]
        self.k = k
        self.dtype = dtype
        if isinstance(q_blocks, torch.Tensor):  # already on the device
            self.Q = q_blocks.reshape(self.d_in, qb).contiguous()
        else:
            self.Q = to_torch(q_blocks.reshape(self.d_in, qb), dtype, device)
        self.Qt = self.Q.new_empty(self.Q.shape)
        _lib.larosa_prepare_rotation(self.Q, self.Qt, self.d_in, qb)
        W = w.contiguous() if isinstance(w, torch.Tensor) else to_torch(w, dtype, device)
        self.Wf = W.new_empty(W.shape)
        _lib.larosa_fold_weights(self.Qt, qb, W, self.Wf, self.d_in, self.d_out)
        self.W = W if keep_w else None

    def workspace(self, B: int, mode: int = _lib.UNFUSED):
        import torch
        n = _lib.larosa_workspace_bytes(B, self.d_in, self.d_out, self.k, mode)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=self.Wf.device)
        _lib.larosa_workspace_init(ws)
        return ws

    def forward(self, x, y, ws, idx_out=None, xrot_out=None, mode: int = _lib.UNFUSED,
                stream=None):
        B = x.shape[0]
        _lib.larosa_layer_forward(x, self.Qt, self.q_block, self.Wf, B, self.d_in, self.d_out,
                                  self.k, y, idx_out=idx_out, xrot_out=xrot_out, mode=mode,
                                  ws=ws, stream=stream)
