"""A LLaMA-shaped decoder layer whose four linear inputs are rotated and
Top-K sparsified (every linear layer's input, per the LaRoSA summary page,
方法详解 · 技术框架), driven through the C ABI.

Marshalling only: buffers are torch tensors, and every step (RMSNorm, the
rotated sparse linears, rotary embedding, attention over the key/value cache,
SwiGLU, residual adds) is one of liblarosa's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from . import workloads as wl
from .device import RotatedLinear

ROLES = ("attn_in", "o_in", "mlp_in", "down_in")


class DecoderLayer:
    """Device state of one layer: four RotatedLinears and its KV cache.

    Row layout of the q|k|v projection output: n_heads query heads, then
    n_kv_heads key heads, then n_kv_heads value heads (d_head channels each).
    The cache is [B, n_kv_heads, ctx, d_head] (head-major). The gate|up
    linear also keeps its folded weight with gate and up columns interleaved
    (w_il), which the SwiGLU-folded layer call reads."""

    def __init__(self, shape: wl.DecoderShape, tensors: dict, ks: dict, k_cache, v_cache,
                 dtype: str = "bf16"):
        self.shape = shape
        self.lin = {}
        for role in ROLES:
            qname, wname = wl.ROLE_TENSORS[role]
            self.lin[role] = RotatedLinear(tensors[qname], tensors[wname], dtype, ks[role],
                                           keep_w=False)
        g = self.lin["mlp_in"]
        self.w_il = g.Wf.new_empty(g.Wf.shape)
        _lib.larosa_interleave_gate_up(g.Wf, self.w_il, g.d_in, shape.f)
        self.k_cache = k_cache
        self.v_cache = v_cache
        self.ws = {}

    def workspaces(self, B: int, mode: int):
        key = (B, mode)
        if key not in self.ws:
            ws = {r: self.lin[r].workspace(B, mode) for r in ROLES if r != "mlp_in"}
            g = self.lin["mlp_in"]
            n = _lib.larosa_swiglu_workspace_bytes(B, g.d_in, self.shape.f, g.k, mode)
            ws["mlp_in"] = torch.empty(max(n, 16), dtype=torch.uint8, device=g.Wf.device)
            _lib.larosa_workspace_init(ws["mlp_in"])
            self.ws[key] = ws
        return self.ws[key]


class DecoderBuffers:
    """Activations of one decode step for a batch of B tokens (reused by every
    layer)."""

    def __init__(self, shape: wl.DecoderShape, B: int, device="cuda"):
        s = shape
        bf = dict(dtype=torch.bfloat16, device=device)
        self.a = torch.empty((B, s.d), **bf)
        self.qkv = torch.empty((B, s.qkv_out), **bf)
        self.q = torch.empty((B, s.n_heads * s.d_head), **bf)
        self.k = torch.empty((B, s.n_kv_heads * s.d_head), **bf)
        self.att = torch.empty((B, s.n_heads * s.d_head), **bf)
        self.o = torch.empty((B, s.d), **bf)
        self.m = torch.empty((B, s.d), **bf)
        self.hh = torch.empty((B, s.f), **bf)
        self.dn = torch.empty((B, s.d), **bf)
        n = _lib.larosa_decode_attention_workspace_bytes(B, s.ctx, s.n_heads)
        self.att_ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def layer_forward(layer: DecoderLayer, h, buf: DecoderBuffers, mode: int = _lib.UNFUSED,
                  trace: dict | None = None):
    """One decode step through `layer`, updating h [B, d] in place. `trace`,
    if given, receives the rotated inputs and kept indices of the four
    linears (fp32 / int32 device tensors)."""
    s = layer.shape
    B = h.shape[0]
    ws = layer.workspaces(B, mode)

    def lin(role, x, y):
        L = layer.lin[role]
        xr = idx = None
        if trace is not None:
            xr = torch.empty((B, L.d_in), dtype=torch.float32, device=h.device)
            idx = torch.empty((B, L.k), dtype=torch.int32, device=h.device)
            trace[role] = (xr, idx)
        if role == "mlp_in":  # y is h = SiLU(gate)·up, folded into the gate|up call
            _lib.larosa_swiglu_layer_forward(x, L.Qt, L.q_block, layer.w_il, B, L.d_in, s.f, L.k,
                                             y, idx_out=idx, xrot_out=xr, mode=mode,
                                             ws=ws[role])
        else:
            L.forward(x, y, ws[role], idx_out=idx, xrot_out=xr, mode=mode)

    _lib.larosa_rmsnorm(h, buf.a, B, s.d)
    lin("attn_in", buf.a, buf.qkv)
    _lib.larosa_rope(buf.qkv, s.qkv_out, buf.q, buf.k, B, s.n_heads, s.n_kv_heads, s.d_head,
                     s.ctx)
    v_new = buf.qkv[:, (s.n_heads + s.n_kv_heads) * s.d_head:]
    _lib.larosa_decode_attention(buf.q, buf.k, s.n_kv_heads * s.d_head, v_new, s.qkv_out,
                                 layer.k_cache, layer.v_cache, buf.att, B, s.ctx, s.n_heads,
                                 s.n_kv_heads, s.d_head, ws=buf.att_ws)
    lin("o_in", buf.att, buf.o)
    _lib.larosa_residual_add(h, buf.o, B * s.d)
    _lib.larosa_rmsnorm(h, buf.m, B, s.d)
    lin("mlp_in", buf.m, buf.hh)
    lin("down_in", buf.hh, buf.dn)
    _lib.larosa_residual_add(h, buf.dn, B * s.d)


def upload_base(base: dict, dtype: str = "bf16") -> dict:
    """The per-role draws of workloads.base_decoder_tensors as device tensors."""
    return {name: wl.to_torch(arr, dtype) for name, arr in base.items()}


def build_layer(cfg: int, layer_idx: int, shape: wl.DecoderShape, base_dev: dict, kv_base,
                B: int, sparsity_pct: int, run_seed: int = 0):
    """One layer's seeded tensors (signed permutations of one draw per role,
    see workloads) built on the device from the uploaded draws. Returns
    (DecoderLayer, {role: index arrays}, kv offsets)."""
    dev = base_dev["q_attn"].device
    tens, idxs = {}, {}
    for role in ROLES:
        qname, wname = wl.ROLE_TENSORS[role]
        idx = wl.layer_tensor_indices(cfg, layer_idx, role, shape, run_seed)
        idxs[role] = idx
        rows, signs, w_rows, w_cols = (torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                                       for a in idx)
        q = base_dev[qname][:, rows, :] * signs.to(base_dev[qname].dtype)[None, None, :]
        tens[qname] = q.contiguous()
        tens[wname] = base_dev[wname].index_select(0, w_rows).index_select(1, w_cols).contiguous()
    ks = {r: wl.k_for(shape.f if r == "down_in" else shape.d, sparsity_pct) for r in ROLES}
    kb, vb = kv_base
    offs = wl.kv_offsets(cfg, layer_idx, B, shape.ctx, run_seed)
    kc = torch.stack([torch.roll(kb, int(o), dims=1) for o in offs]).contiguous()
    vc = torch.stack([torch.roll(vb, int(o), dims=1) for o in offs]).contiguous()
    layer = DecoderLayer(shape, tens, ks, kc, vc)
    del tens
    return layer, idxs, offs
