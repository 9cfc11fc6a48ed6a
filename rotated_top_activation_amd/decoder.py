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
        # one token, norms folded into the rotations: the second residual
        # buffer, a zero row (the residual sum of a first layer) and the two
        # rotated norm outputs
        self.h2 = torch.empty((B, s.d), **bf)
        self.zero = torch.zeros((B, s.d), **bf)
        self.xr_attn = torch.empty((B, s.d), dtype=torch.float32, device=device)
        self.xr_mlp = torch.empty((B, s.d), dtype=torch.float32, device=device)


def folds_norms(layer: DecoderLayer, B: int, mode: int) -> bool:
    """Whether layer_forward folds the two RMSNorms (with their residual adds)
    into the rotations of the q|k|v and gate|up inputs: one token, unfused
    steps, dense rotations of those inputs (larosa_residual_rmsnorm_rotate)."""
    s = layer.shape
    return (B == 1 and mode == _lib.UNFUSED and s.d % 8 == 0 and 256 < s.d <= 8192 and
            all(layer.lin[r].q_block == s.d for r in ("attn_in", "mlp_in")))


def layer_forward(layer: DecoderLayer, h, buf: DecoderBuffers, mode: int = _lib.UNFUSED,
                  trace: dict | None = None, normed: bool = False, norm_next: bool = False,
                  pending: bool = False, defer: bool = False):
    """One decode step through `layer`, updating h [B, d] in place. `trace`,
    if given, receives the rotated inputs and kept indices of the four
    linears (fp32 / int32 device tensors).

    normed: buf.a already holds RMSNorm(h) (the previous layer's norm_next),
    so the layer's first norm is skipped. norm_next: the closing residual add
    also writes RMSNorm of the new h into buf.a, the next layer's first norm,
    in the same launch. A stack of layers runs layer 0 with normed=False and
    every later one with normed=True, every layer but the last with
    norm_next=True.

    Where folds_norms holds (one token, unfused), the two norms run inside
    the rotations instead, and normed / norm_next are not used: pending says
    that buf.dn holds the previous layer's down output, still to be added to
    h (it is added inside the first folded norm); defer leaves this layer's
    down output in buf.dn for the next layer, so h ends the layer as the
    residual after attention. A stack runs layer 0 with pending=False and
    later ones with pending=True, every layer but the last with defer=True.
    buf.a and buf.m still receive the two norms' outputs."""
    s = layer.shape
    B = h.shape[0]
    ws = layer.workspaces(B, mode)
    if folds_norms(layer, B, mode):
        _layer_forward_folded(layer, h, buf, ws, trace, pending, defer)
        return

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

    if not normed:
        _lib.larosa_rmsnorm(h, buf.a, B, s.d)
    Hd, Kd = s.n_heads * s.d_head, s.n_kv_heads * s.d_head
    if B == 1:
        # one token: q and k are rotated in place inside qkv, in the q|k|v
        # product's epilogue (no RoPE launch); attention reads them there
        L = layer.lin["attn_in"]
        xr = idx = None
        if trace is not None:
            xr = torch.empty((B, L.d_in), dtype=torch.float32, device=h.device)
            idx = torch.empty((B, L.k), dtype=torch.int32, device=h.device)
            trace["attn_in"] = (xr, idx)
            trace["rope_in_qkv"] = True
        _lib.larosa_qkv_rope_layer_forward(buf.a, L.Qt, L.q_block, L.Wf, B, L.d_in, L.k,
                                           s.n_heads, s.n_kv_heads, s.d_head, s.ctx, buf.qkv,
                                           idx_out=idx, xrot_out=xr, mode=mode,
                                           ws=ws["attn_in"])
        q, k, k_stride = buf.qkv[:, :Hd], buf.qkv[:, Hd:Hd + Kd], s.qkv_out
    else:
        lin("attn_in", buf.a, buf.qkv)
        _lib.larosa_rope(buf.qkv, s.qkv_out, buf.q, buf.k, B, s.n_heads, s.n_kv_heads,
                         s.d_head, s.ctx)
        q, k, k_stride = buf.q, buf.k, Kd
    v_new = buf.qkv[:, Hd + Kd:]
    _lib.larosa_decode_attention(q, k, k_stride, v_new, s.qkv_out, layer.k_cache,
                                 layer.v_cache, buf.att, B, s.ctx, s.n_heads, s.n_kv_heads,
                                 s.d_head, ws=buf.att_ws)
    lin("o_in", buf.att, buf.o)
    _lib.larosa_residual_rmsnorm(h, buf.o, buf.m, B, s.d)  # h += o; m = RMSNorm(h)
    lin("mlp_in", buf.m, buf.hh)
    lin("down_in", buf.hh, buf.dn)
    if norm_next:
        _lib.larosa_residual_rmsnorm(h, buf.dn, buf.a, B, s.d)  # h += dn; the next layer's a
    else:
        _lib.larosa_residual_add(h, buf.dn, B * s.d)


def _layer_forward_folded(layer: DecoderLayer, h, buf: DecoderBuffers, ws: dict,
                          trace: dict | None, pending: bool, defer: bool):
    """layer_forward for one token with the norms folded into the rotations.
    The residual moves h -> buf.h2 (the first norm's sum) -> h (the second),
    since a folded norm cannot write its sum in place."""
    s = layer.shape
    B = 1
    Hd, Kd = s.n_heads * s.d_head, s.n_kv_heads * s.d_head
    pre = _lib.UNFUSED | _lib.PREROTATED

    def rotated(role, default):
        L = layer.lin[role]
        if trace is None:
            return default, None
        xr = torch.empty((B, L.d_in), dtype=torch.float32, device=h.device)
        idx = torch.empty((B, L.k), dtype=torch.int32, device=h.device)
        trace[role] = (xr, idx)
        return xr, idx

    # h + dn (or + 0 for a first layer) -> h2; x_rot of RMSNorm(h2)
    La = layer.lin["attn_in"]
    xr, idx = rotated("attn_in", buf.xr_attn)
    _lib.larosa_residual_rmsnorm_rotate(h, buf.dn if pending else buf.zero, buf.h2, La.Qt, xr,
                                        s.d, a_out=buf.a)
    if trace is not None:
        trace["rope_in_qkv"] = True
    _lib.larosa_qkv_rope_layer_forward(xr, None, La.q_block, La.Wf, B, La.d_in, La.k, s.n_heads,
                                       s.n_kv_heads, s.d_head, s.ctx, buf.qkv, idx_out=idx,
                                       mode=pre, ws=ws["attn_in"])
    q, k = buf.qkv[:, :Hd], buf.qkv[:, Hd:Hd + Kd]
    _lib.larosa_decode_attention(q, k, s.qkv_out, buf.qkv[:, Hd + Kd:], s.qkv_out,
                                 layer.k_cache, layer.v_cache, buf.att, B, s.ctx, s.n_heads,
                                 s.n_kv_heads, s.d_head, ws=buf.att_ws)
    Lo = layer.lin["o_in"]
    xr_o = idx_o = None
    if trace is not None:
        xr_o, idx_o = rotated("o_in", None)
    Lo.forward(buf.att, buf.o, ws["o_in"], idx_out=idx_o, xrot_out=xr_o, mode=_lib.UNFUSED)
    # h2 + o -> h; x_rot of RMSNorm(h)
    Lm = layer.lin["mlp_in"]
    xr, idx = rotated("mlp_in", buf.xr_mlp)
    _lib.larosa_residual_rmsnorm_rotate(buf.h2, buf.o, h, Lm.Qt, xr, s.d, a_out=buf.m)
    _lib.larosa_swiglu_layer_forward(xr, None, Lm.q_block, layer.w_il, B, Lm.d_in, s.f, Lm.k,
                                     buf.hh, idx_out=idx, mode=pre, ws=ws["mlp_in"])
    Ld = layer.lin["down_in"]
    xr_d = idx_d = None
    if trace is not None:
        xr_d, idx_d = rotated("down_in", None)
    Ld.forward(buf.hh, buf.dn, ws["down_in"], idx_out=idx_d, xrot_out=xr_d, mode=_lib.UNFUSED)
    if not defer:
        _lib.larosa_residual_add(h, buf.dn, B * s.d)


def decoder_step(layers: list, h, buf: DecoderBuffers, mode: int = _lib.UNFUSED,
                 traces: list | None = None):
    """One decode step through a stack of layers, h [B, d] updated in place
    (the chained norms of layer_forward). traces: one dict per layer, or
    None."""
    n = len(layers)
    if n == 0:
        return
    B = h.shape[0]
    folded = folds_norms(layers[0], B, mode)
    if not folded:
        _lib.larosa_rmsnorm(h, buf.a, B, layers[0].shape.d)
    for i, L in enumerate(layers):
        tr = traces[i] if traces is not None else None
        if folded:
            layer_forward(L, h, buf, mode, trace=tr, pending=i > 0, defer=i < n - 1)
        else:
            layer_forward(L, h, buf, mode, trace=tr, normed=True, norm_next=i < n - 1)


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
