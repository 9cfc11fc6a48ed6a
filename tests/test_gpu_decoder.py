"""GPU parity of the decoder-layer glue and of the full LLaMA2-7B-shaped
32-layer decode step with every linear input rotated and Top-K sparsified.

Each layer is checked teacher-forced on the GPU's own layer input and
intermediates: RMSNorm, the four rotations (rigorous fp32 bound), the four
kept index sets (bit-exact against the oracle's selection on the GPU's
rotated activations), sampled output columns of the four products, rotary
embedding, attention over the key/value cache, the gate|up call's folded
SwiGLU and both residual adds.
"""
import functools

import numpy as np
import pytest
import torch

from oracle import decoder_ref as dec
from oracle import larosa_ref as ref
from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import decoder as D
from rotated_top_activation_amd import workloads as wl

from gpu_helpers import dev, host, host_f32, ulp_bf16
from test_gpu_parity import rotation_bound

pytestmark = pytest.mark.gpu

TOL = 2e-2


def close_bf16(got, want, extra=0.0):
    """Within one bf16 spacing (plus `extra` absolute) elementwise."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    spacing = np.maximum(ulp_bf16(want), ulp_bf16(got))
    return np.all(np.abs(got - want) <= spacing * 1.0001 + extra)


# ------------------------------------------------------------- glue ops ----

@pytest.mark.parametrize("B,d", [(1, 4096), (16, 4096), (3, 520)])
def test_rmsnorm(B, d):
    h = wl.decoder_hidden(3, B, d)
    out = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_rmsnorm(dev(h, "bf16"), out, B, d)
    torch.cuda.synchronize()
    want = dec.rmsnorm(h)
    # fp32 sum of squares: relative error far below a bf16 spacing
    assert close_bf16(host(out), want, extra=1e-6)


@pytest.mark.parametrize("B,H,Hkv", [(1, 32, 32), (4, 64, 8)])
def test_rope(B, H, Hkv):
    dh = 128
    rng = np.random.default_rng(B * H)
    n = (H + 2 * Hkv) * dh
    qkv = wl.quantize(rng.standard_normal((B, n)), "bf16")
    q = torch.empty((B, H * dh), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, Hkv * dh), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_rope(dev(qkv, "bf16"), n, q, k, B, H, Hkv, dh, 2048)
    torch.cuda.synchronize()
    # fp64 angles, fp32 products: within one bf16 spacing of the exact result
    want_q = dec.rope(qkv[:, :H * dh], H, dh, 2048)
    want_k = dec.rope(qkv[:, H * dh:(H + Hkv) * dh], Hkv, dh, 2048)
    assert close_bf16(host(q), want_q, extra=1e-6)
    assert close_bf16(host(k), want_k, extra=1e-6)


@pytest.mark.parametrize("B,H,Hkv,T", [(1, 32, 32, 2048), (4, 32, 32, 2048), (2, 64, 8, 300),
                                       (2, 4, 4, 0), (1, 8, 8, 255), (3, 8, 2, 256),
                                       (1, 4, 4, 4100)])
def test_decode_attention(B, H, Hkv, T):
    dh = 128
    rng = np.random.default_rng(T + B)
    q = wl.quantize(rng.standard_normal((B, H * dh)), "bf16")
    kn = wl.quantize(rng.standard_normal((B, Hkv * dh)), "bf16")
    vn = wl.quantize(rng.standard_normal((B, Hkv * dh)), "bf16")
    kc = wl.quantize(rng.standard_normal((B, Hkv, T, dh)), "bf16")
    vc = wl.quantize(rng.standard_normal((B, Hkv, T, dh)), "bf16")
    out = torch.empty((B, H * dh), dtype=torch.bfloat16, device="cuda")
    kc_d = dev(kc.reshape(-1), "bf16") if T else torch.empty(8, dtype=torch.bfloat16, device="cuda")
    vc_d = dev(vc.reshape(-1), "bf16") if T else torch.empty(8, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(_lib.larosa_decode_attention_workspace_bytes(B, T, H), dtype=torch.uint8,
                     device="cuda")
    _lib.larosa_decode_attention(dev(q, "bf16"), dev(kn, "bf16"), Hkv * dh, dev(vn, "bf16"),
                                 Hkv * dh, kc_d, vc_d, out, B, T, H, Hkv, dh, ws=ws)
    torch.cuda.synchronize()
    want = dec.decode_attention(q, kn, vn, kc, vc, H, Hkv, dh)
    assert ref.rel_error(host(out), want) <= TOL


def test_residual_add_matches_rounded_sum():
    rng = np.random.default_rng(9)
    a = wl.quantize(rng.standard_normal((3, 4096)), "bf16")
    b = wl.quantize(rng.standard_normal((3, 4096)), "bf16")
    h = dev(a, "bf16")
    _lib.larosa_residual_add(h, dev(b, "bf16"), a.size)
    torch.cuda.synchronize()
    # the fp32 sum of two bf16 values is exact, so one rounding: bit-exact
    np.testing.assert_array_equal(host(h), dec.residual_add(a, b))


# ------------------------------------------------------- decoder layers ----

def _check_linear(x_in, q_blocks, xr_gpu, idx_gpu, y_gpu, wf_dev, k, cols):
    bound, exact = rotation_bound(x_in, q_blocks)
    assert np.all(np.abs(xr_gpu.astype(np.float64) - exact) <= bound), "rotation bound"
    want_idx = ref.select(xr_gpu, k)
    np.testing.assert_array_equal(idx_gpu, want_idx)
    wf_cols = host(wf_dev[:, torch.from_numpy(cols).cuda()])
    want = ref.round_to(ref.gather_product(xr_gpu, want_idx, wf_cols), "bf16")
    assert ref.rel_error(y_gpu[:, cols], want) <= TOL


def _check_swiglu_linear(x_in, q_blocks, xr_gpu, idx_gpu, h_gpu, wf_dev, k, f, cols):
    """The gate|up linear with SiLU(gate)·up folded in: h on gate columns
    `cols` (each paired with up column f + c) against the oracle's SwiGLU of
    the product over the GPU's kept rows, teacher-forced."""
    bound, exact = rotation_bound(x_in, q_blocks)
    assert np.all(np.abs(xr_gpu.astype(np.float64) - exact) <= bound), "rotation bound"
    want_idx = ref.select(xr_gpu, k)
    np.testing.assert_array_equal(idx_gpu, want_idx)
    both = np.concatenate([cols, cols + f])
    wf_cols = host(wf_dev[:, torch.from_numpy(both).cuda()])
    gu = ref.round_to(ref.gather_product(xr_gpu, want_idx, wf_cols), "bf16")
    want = ref.swiglu(gu, len(cols), "bf16")
    assert ref.rel_error(h_gpu[:, cols], want) <= TOL


@functools.lru_cache(maxsize=1)
def _base(cfg):
    shape = wl.LLAMA7B
    base = wl.base_decoder_tensors(cfg, shape)
    return base, D.upload_base(base), wl.kv_cache_base(cfg, shape)


def run_decoder(B, sparsity, n_layers, mode, n_checked=None, seed_cols=0):
    """Run n_layers of the 7B-shaped decoder on one batch and check every
    layer (or the first n_checked) against the oracle, teacher-forced."""
    cfg = 3
    shape = wl.LLAMA7B
    base, base_dev, (kb, vb) = _base(cfg)
    kv_dev = (dev(kb.reshape(-1), "bf16").view(kb.shape), dev(vb.reshape(-1), "bf16").view(vb.shape))
    h0 = wl.decoder_hidden(cfg, B, shape.d)
    h = dev(h0, "bf16")
    buf = D.DecoderBuffers(shape, B)
    rng = np.random.default_rng(seed_cols)
    checked = 0
    for l in range(n_layers):
        layer, idxs, offs = D.build_layer(cfg, l, shape, base_dev, kv_dev, B, sparsity)
        h_in = host(h)
        trace = {}
        D.layer_forward(layer, h, buf, mode=mode, trace=trace)
        torch.cuda.synchronize()
        if n_checked is not None and checked >= n_checked:
            del layer
            continue
        checked += 1
        a, qkv, att, o, m, hh, dn = (host(t) for t in (buf.a, buf.qkv, buf.att, buf.o, buf.m,
                                                        buf.hh, buf.dn))
        q, k = host(buf.q), host(buf.k)
        h_out = host(h)
        assert close_bf16(a, dec.rmsnorm(h_in), extra=1e-6), f"layer {l} rmsnorm"
        lin_in = {"attn_in": a, "o_in": att, "mlp_in": m, "down_in": hh}
        lin_out = {"attn_in": qkv, "o_in": o, "mlp_in": hh, "down_in": dn}
        for role in D.ROLES:
            qn, _ = wl.ROLE_TENSORS[role]
            xr, idx = trace[role]
            L = layer.lin[role]
            q_host = wl.layer_rotation(base[qn], idxs[role])
            if role == "mlp_in":  # h = SiLU(gate)·up straight from the gate|up call
                cols = np.sort(rng.choice(shape.f, size=256, replace=False))
                _check_swiglu_linear(m, q_host, host_f32(xr), host(idx), hh, L.Wf, L.k,
                                     shape.f, cols)
                continue
            cols = np.sort(rng.choice(L.d_out, size=min(256, L.d_out), replace=False))
            _check_linear(lin_in[role], q_host, host_f32(xr), host(idx), lin_out[role], L.Wf,
                          L.k, cols)
        Hd = shape.n_heads * shape.d_head
        Kd = shape.n_kv_heads * shape.d_head
        assert close_bf16(q, dec.rope(qkv[:, :Hd], shape.n_heads, shape.d_head, shape.ctx),
                          extra=1e-6), f"layer {l} rope q"
        assert close_bf16(k, dec.rope(qkv[:, Hd:Hd + Kd], shape.n_kv_heads, shape.d_head,
                                      shape.ctx), extra=1e-6), f"layer {l} rope k"
        kc = np.stack([np.roll(kb, int(o_), axis=1) for o_ in offs])
        vc = np.stack([np.roll(vb, int(o_), axis=1) for o_ in offs])
        want_att = dec.decode_attention(q, k, qkv[:, Hd + Kd:], kc, vc, shape.n_heads,
                                        shape.n_kv_heads, shape.d_head)
        assert ref.rel_error(att, want_att) <= TOL, f"layer {l} attention"
        h_mid = dec.residual_add(h_in, o)
        assert close_bf16(m, dec.rmsnorm(h_mid), extra=1e-6), f"layer {l} residual/rmsnorm"
        np.testing.assert_array_equal(h_out, dec.residual_add(h_mid, dn))
        del layer
    assert np.all(np.isfinite(host(h)))


@pytest.mark.parametrize("B", [1, 4, 16])
def test_decoder_layer_7b_shape(B):
    run_decoder(B, 40, n_layers=2, mode=_lib.UNFUSED)


def test_decoder_layer_fused_single_token():
    run_decoder(1, 40, n_layers=2, mode=_lib.FUSED)


@pytest.mark.parametrize("B,sp", [(1, 25), (1, 40), (1, 50), (4, 40), (16, 40)])
def test_decoder_32_layers(B, sp):
    """The full 32-layer decode step; every layer checked."""
    run_decoder(B, sp, n_layers=32, mode=_lib.FUSED if B == 1 else _lib.UNFUSED)
