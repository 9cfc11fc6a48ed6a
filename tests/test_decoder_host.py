"""The decoder glue's host logic on the CPU: which library calls a decode step
makes, in which order and on which buffers. The library's compute entry
points are replaced by recorders (nothing runs on a device); the size
functions are the library's own.

One token, unfused: the two RMSNorms run inside the rotations
(larosa_residual_rmsnorm_rotate) and the layer calls take the rotated input
(LAROSA_PREROTATED). The residual moves h -> h2 -> h within a layer, each
layer's down output is added by the next layer's first folded norm (a zero
row for the first layer), and only the last layer adds its own. Batches and
the one-launch mode keep the chained residual + RMSNorm launches."""
import types

import pytest
import torch

from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import decoder as D
from rotated_top_activation_amd import workloads as wl

SHAPE = wl.DecoderShape(d=512, f=1024, n_heads=4, n_kv_heads=2, d_head=128, ctx=64,
                        q2_block=512)


class FakeLinear:
    def __init__(self, role, d_in, q_block, calls):
        self.role, self.d_in, self.q_block, self.k = role, d_in, q_block, d_in // 2
        self.Qt, self.Wf = f"Qt_{role}", f"Wf_{role}"
        self.calls = calls

    def forward(self, x, y, ws, idx_out=None, xrot_out=None, mode=_lib.UNFUSED, stream=None):
        self.calls.append(("forward", self.role, x, y, mode))


class FakeLayer:
    def __init__(self, calls, dense_q=True):
        s = SHAPE
        qb = s.d if dense_q else s.d // 2
        self.shape = s
        self.lin = {"attn_in": FakeLinear("attn_in", s.d, qb, calls),
                    "o_in": FakeLinear("o_in", s.d, s.d, calls),
                    "mlp_in": FakeLinear("mlp_in", s.d, qb, calls),
                    "down_in": FakeLinear("down_in", s.f, s.q2_block, calls)}
        self.w_il = "w_il"
        self.k_cache, self.v_cache = "kc", "vc"

    def workspaces(self, B, mode):
        return {r: f"ws_{r}" for r in D.ROLES}


@pytest.fixture
def calls(monkeypatch):
    rec = []

    def recorder(name):
        def f(*args, **kw):
            rec.append((name, args, kw))
        return f

    for name in ("larosa_residual_rmsnorm_rotate", "larosa_qkv_rope_layer_forward",
                 "larosa_decode_attention", "larosa_swiglu_layer_forward", "larosa_residual_add",
                 "larosa_rmsnorm", "larosa_residual_rmsnorm", "larosa_rope"):
        monkeypatch.setattr(_lib, name, recorder(name))
    return rec


def names(rec):
    return [c[0] if c[0] != "forward" else f"forward:{c[1]}" for c in rec]


def test_one_token_folds_the_norms_and_chains_the_residual(calls):
    layers = [FakeLayer(calls) for _ in range(3)]
    assert D.folds_norms(layers[0], 1, _lib.UNFUSED)
    buf = D.DecoderBuffers(SHAPE, 1, device="cpu")
    h = torch.zeros((1, SHAPE.d), dtype=torch.bfloat16)
    D.decoder_step(layers, h, buf, _lib.UNFUSED)
    per_layer = ["larosa_residual_rmsnorm_rotate", "larosa_qkv_rope_layer_forward",
                 "larosa_decode_attention", "forward:o_in", "larosa_residual_rmsnorm_rotate",
                 "larosa_swiglu_layer_forward", "forward:down_in"]
    assert names(calls) == per_layer * 3 + ["larosa_residual_add"]
    norms = [c for c in calls if c[0] == "larosa_residual_rmsnorm_rotate"]
    for li in range(3):
        first, second = norms[2 * li], norms[2 * li + 1]
        # (h, o, h_out, Qt, x_rot, d): h + (previous down output, or zero) -> h2
        assert first[1][0] is h and first[1][2] is buf.h2
        assert first[1][1] is (buf.zero if li == 0 else buf.dn)
        assert first[1][3] == "Qt_attn_in" and first[1][4] is buf.xr_attn
        assert first[2]["a_out"] is buf.a
        # h2 + o -> h
        assert second[1][0] is buf.h2 and second[1][1] is buf.o and second[1][2] is h
        assert second[1][3] == "Qt_mlp_in" and second[1][4] is buf.xr_mlp
        assert second[2]["a_out"] is buf.m
    pre = _lib.UNFUSED | _lib.PREROTATED
    for c in calls:
        if c[0] in ("larosa_qkv_rope_layer_forward", "larosa_swiglu_layer_forward"):
            assert c[1][1] is None and c[2]["mode"] == pre  # x_rot given, Qt not passed
    qkv = [c for c in calls if c[0] == "larosa_qkv_rope_layer_forward"]
    assert all(c[1][0] is buf.xr_attn for c in qkv)
    last = calls[-1]
    assert last[1][0] is h and last[1][1] is buf.dn


def test_one_token_trace_gets_every_rotated_input(calls):
    layer = FakeLayer(calls)
    buf = D.DecoderBuffers(SHAPE, 1, device="cpu")
    h = torch.zeros((1, SHAPE.d), dtype=torch.bfloat16)
    trace = {}
    D.layer_forward(layer, h, buf, _lib.UNFUSED, trace=trace, pending=True, defer=False)
    assert set(D.ROLES) <= set(trace) and trace["rope_in_qkv"]
    norms = [c for c in calls if c[0] == "larosa_residual_rmsnorm_rotate"]
    assert norms[0][1][4] is trace["attn_in"][0] and norms[1][1][4] is trace["mlp_in"][0]
    assert norms[0][1][1] is buf.dn  # pending: the previous down output is added first
    assert names(calls)[-1] == "larosa_residual_add"


@pytest.mark.parametrize("B,mode,dense_q", [(2, _lib.UNFUSED, True), (1, _lib.FUSED, True),
                                            (1, _lib.UNFUSED, False)])
def test_batches_and_other_modes_keep_the_chained_norm_launches(calls, B, mode, dense_q):
    layers = [FakeLayer(calls, dense_q) for _ in range(2)]
    assert not D.folds_norms(layers[0], B, mode)
    buf = D.DecoderBuffers(SHAPE, B, device="cpu")
    h = torch.zeros((B, SHAPE.d), dtype=torch.bfloat16)
    D.decoder_step(layers, h, buf, mode)
    got = names(calls)
    assert "larosa_residual_rmsnorm_rotate" not in got
    assert got[0] == "larosa_rmsnorm"
    norms = [c for c in calls if c[0] == "larosa_residual_rmsnorm"]
    # per layer h += o (-> m); between layers h += dn (-> the next layer's a)
    assert [(c[1][1] is buf.o, c[1][2] is buf.m) for c in norms[::2]] == [(True, True)] * 2
    assert norms[1][1][1] is buf.dn and norms[1][1][2] is buf.a
    assert got[-1] == "larosa_residual_add"
