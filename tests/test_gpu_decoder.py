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
from rotated_top_activation_amd.device import RotatedLinear

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


@pytest.mark.parametrize("B,H,Hkv,mode,pos", [
    (1, 8, 8, _lib.UNFUSED, 2048), (1, 16, 4, _lib.UNFUSED, 777), (1, 8, 8, _lib.UNFUSED, 0),
    (4, 8, 8, _lib.UNFUSED, 2048), (1, 8, 8, _lib.FUSED, 2048),
    (1, 8, 2, _lib.UNFUSED | _lib.ROTATE_FP64, 5)])
def test_qkv_rope_layer_equals_layer_then_rope(B, H, Hkv, mode, pos):
    """larosa_qkv_rope_layer_forward: RoPE folded into the one-token
    product's epilogue (or applied in place after the other paths) gives the
    bits of larosa_layer_forward followed by larosa_rope."""
    d, dh = 1024, 128
    d_out = (H + 2 * Hkv) * dh
    k = wl.k_for(d, 40)
    rng = np.random.default_rng(H * 31 + Hkv + pos)
    q = wl.quantize(wl.rotation_fp64(4, 1, "attn_in", d, 512), "bf16")
    w = wl.quantize(rng.standard_normal((d, d_out)) * 0.02, "bf16")
    x = wl.quantize(rng.standard_normal((B, d)), "bf16")
    lin = RotatedLinear(q, w, "bf16", k, keep_w=False)
    x_d = dev(x, "bf16")
    y1 = torch.empty((B, d_out), dtype=torch.bfloat16, device="cuda")
    idx1 = torch.empty((B, k), dtype=torch.int32, device="cuda")
    _lib.larosa_qkv_rope_layer_forward(x_d, lin.Qt, lin.q_block, lin.Wf, B, d, k, H, Hkv, dh,
                                       pos, y1, idx_out=idx1, mode=mode,
                                       ws=lin.workspace(B, mode))
    y2 = torch.empty_like(y1)
    idx2 = torch.empty_like(idx1)
    lin.forward(x_d, y2, lin.workspace(B, mode), idx_out=idx2, mode=mode)
    qo = torch.empty((B, H * dh), dtype=torch.bfloat16, device="cuda")
    ko = torch.empty((B, Hkv * dh), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_rope(y2, d_out, qo, ko, B, H, Hkv, dh, pos)
    torch.cuda.synchronize()
    Hd, Kd = H * dh, Hkv * dh
    assert torch.equal(idx1, idx2)
    assert torch.equal(y1[:, :Hd], qo)
    assert torch.equal(y1[:, Hd:Hd + Kd], ko)
    assert torch.equal(y1[:, Hd + Kd:], y2[:, Hd + Kd:])
    if pos == 0:  # angle 0: the plain product
        assert torch.equal(y1, y2)


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
    ws = torch.zeros(_lib.larosa_decode_attention_workspace_bytes(B, T, H), dtype=torch.uint8,
                     device="cuda")
    args = (dev(q, "bf16"), dev(kn, "bf16"), Hkv * dh, dev(vn, "bf16"), Hkv * dh, kc_d, vc_d)
    _lib.larosa_decode_attention(*args, out, B, T, H, Hkv, dh, ws=ws)
    torch.cuda.synchronize()
    want = dec.decode_attention(q, kn, vn, kc, vc, H, Hkv, dh)
    assert ref.rel_error(host(out), want) <= TOL
    # the chunks are combined in chunk order: a second call gives the same bits
    out2 = torch.empty_like(out)
    _lib.larosa_decode_attention(*args, out2, B, T, H, Hkv, dh, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_decode_attention_workspace_reused_across_shapes():
    """One workspace serves calls of changing context length, batch and head
    count in a row."""
    dh = 128
    ws = torch.empty(_lib.larosa_decode_attention_workspace_bytes(4, 2048, 32), dtype=torch.uint8,
                     device="cuda")
    for B, H, Hkv, T in [(2, 32, 8, 2048), (2, 32, 8, 100), (2, 32, 8, 0), (2, 32, 8, 1500),
                         (4, 32, 32, 2000), (1, 8, 8, 300)]:
        rng = np.random.default_rng(7 * T + H + B)
        q = wl.quantize(rng.standard_normal((B, H * dh)), "bf16")
        kn = wl.quantize(rng.standard_normal((B, Hkv * dh)), "bf16")
        vn = wl.quantize(rng.standard_normal((B, Hkv * dh)), "bf16")
        kc = wl.quantize(rng.standard_normal((B, Hkv, T, dh)), "bf16")
        vc = wl.quantize(rng.standard_normal((B, Hkv, T, dh)), "bf16")
        out = torch.empty((B, H * dh), dtype=torch.bfloat16, device="cuda")
        kc_d = dev(kc.reshape(-1), "bf16") if T else torch.empty(8, dtype=torch.bfloat16,
                                                                  device="cuda")
        vc_d = dev(vc.reshape(-1), "bf16") if T else torch.empty(8, dtype=torch.bfloat16,
                                                                  device="cuda")
        _lib.larosa_decode_attention(dev(q, "bf16"), dev(kn, "bf16"), Hkv * dh, dev(vn, "bf16"),
                                     Hkv * dh, kc_d, vc_d, out, B, T, H, Hkv, dh, ws=ws)
        torch.cuda.synchronize()
        want = dec.decode_attention(q, kn, vn, kc, vc, H, Hkv, dh)
        assert ref.rel_error(host(out), want) <= TOL, (B, H, Hkv, T)


def _rand_qt(d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn((d, d), generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)


@pytest.mark.parametrize("d,resid", [(4096, True), (4096, False), (5120, True), (520, True),
                                     (8192, True), (264, False)])
def test_residual_rmsnorm_rotate_equals_the_two_steps(d, resid):
    """The norm folded into the one-token rotation gives the bits of the
    residual add + RMSNorm launch followed by the rotation launch: the new
    residual, the normalised row and x_rot."""
    rng = np.random.default_rng(d + resid)
    h = dev(wl.quantize(rng.standard_normal((1, d)) * 3, "bf16"), "bf16")
    o = dev(wl.quantize(rng.standard_normal((1, d)), "bf16"), "bf16")
    qt = _rand_qt(d, d)
    h1, a1 = h.clone(), torch.empty_like(h)
    xr1 = torch.empty((1, d), dtype=torch.float32, device="cuda")
    if resid:
        _lib.larosa_residual_rmsnorm(h1, o, a1, 1, d)
    else:
        _lib.larosa_rmsnorm(h1, a1, 1, d)
    _lib.larosa_rotate(a1, qt, d, xr1, 1, d)
    h2, a2 = torch.full_like(h, 7.0), torch.empty_like(h)
    xr2 = torch.empty_like(xr1)
    _lib.larosa_residual_rmsnorm_rotate(h, o if resid else None, h2 if resid else None, qt, xr2,
                                        d, a_out=a2)
    torch.cuda.synchronize()
    assert torch.equal(a2, a1)
    assert torch.equal(xr2, xr1)
    if resid:
        assert torch.equal(h2, h1)
    else:
        assert bool((h2 == 7.0).all())  # no residual sum without o
    # and against the oracle: the norm within one bf16 spacing, x_rot in its bound
    want_a = dec.rmsnorm(host(h1))
    assert close_bf16(host(a2), want_a, extra=1e-6)


def test_residual_rmsnorm_rotate_rejects_in_place_and_bad_sizes():
    d = 4096
    h = torch.zeros((1, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(h)
    qt = torch.zeros((d, d), dtype=torch.bfloat16, device="cuda")
    xr = torch.empty((1, d), dtype=torch.float32, device="cuda")
    for args, code in [((h, o, h, qt, xr, d), 1), ((h, o, o, qt, xr, d), 1),
                       ((h, o, None, qt, xr, d), 1), ((h, o, torch.empty_like(h), qt, xr, 256), 2),
                       ((h, o, torch.empty_like(h), qt, xr, 8200), 2)]:
        with pytest.raises(_lib.LarosaError) as err:
            _lib.larosa_residual_rmsnorm_rotate(*args)
        assert err.value.status == code


@pytest.mark.parametrize("B", [1, 4, 16])
def test_prerotated_layer_calls_equal_the_rotating_calls(B):
    """LAROSA_PREROTATED: the layer calls given x_rot give the bits of the
    calls that rotate x themselves (plain, SwiGLU-folded and RoPE-folded)."""
    shape = wl.LLAMA7B
    d, f = shape.d, 1024
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=2 * f, q_block=d, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    x_d = wl.to_torch(x, "bf16")
    xr = torch.empty((B, d), dtype=torch.float32, device="cuda")
    ws = lin.workspace(B)
    pre = _lib.UNFUSED | _lib.PREROTATED
    y1 = torch.empty((B, 2 * f), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    i1 = torch.empty((B, case.k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    lin.forward(x_d, y1, ws, idx_out=i1, xrot_out=xr)
    lin.forward(xr, y2, ws, idx_out=i2, mode=pre)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(y1, y2)
    # SwiGLU folded (interleaved gate|up)
    w_il = torch.empty_like(lin.Wf)
    _lib.larosa_interleave_gate_up(lin.Wf, w_il, d, f)
    n = _lib.larosa_swiglu_workspace_bytes(B, d, f, case.k, _lib.UNFUSED)
    sws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _lib.larosa_workspace_init(sws)
    h1 = torch.empty((B, f), dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h1)
    _lib.larosa_swiglu_layer_forward(x_d, lin.Qt, d, w_il, B, d, f, case.k, h1, ws=sws)
    _lib.larosa_swiglu_layer_forward(xr, None, d, w_il, B, d, f, case.k, h2, mode=pre, ws=sws)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    # RoPE folded: 2 f columns as 16 heads of 128
    H, Hkv = 8, 4
    _lib.larosa_qkv_rope_layer_forward(x_d, lin.Qt, d, lin.Wf, B, d, case.k, H, Hkv, 128, 2048,
                                       y1, ws=ws)
    _lib.larosa_qkv_rope_layer_forward(xr, None, d, lin.Wf, B, d, case.k, H, Hkv, 128, 2048, y2,
                                       mode=pre, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # the flag's argument rules
    with pytest.raises(RuntimeError):
        lin.forward(xr, y2, ws, xrot_out=xr, mode=pre)
    with pytest.raises(RuntimeError):
        lin.forward(xr, y2, ws, mode=pre | _lib.ROTATE_FP64)


@pytest.mark.parametrize("B,d", [(1, 4096), (16, 4096), (3, 520), (2, 5120), (1, 8192)])
def test_residual_rmsnorm_matches_the_two_steps(B, d):
    """The fused residual add + RMSNorm gives the same bits as the add and
    the norm run one after the other, and matches the oracle."""
    rng = np.random.default_rng(B + d)
    a = wl.quantize(rng.standard_normal((B, d)), "bf16")
    b = wl.quantize(rng.standard_normal((B, d)) * 0.5, "bf16")
    h1, h2 = dev(a, "bf16"), dev(a, "bf16")
    o = dev(b, "bf16")
    out1 = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out1)
    _lib.larosa_residual_rmsnorm(h1, o, out1, B, d)
    _lib.larosa_residual_add(h2, o, B * d)
    _lib.larosa_rmsnorm(h2, out2, B, d)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(out1, out2)
    h_sum = dec.residual_add(a, b)
    np.testing.assert_array_equal(host(h1), h_sum)
    assert close_bf16(host(out1), dec.rmsnorm(h_sum), extra=1e-6)


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


def _check_qkv_rope_linear(x_in, q_blocks, xr_gpu, idx_gpu, qkv_gpu, wf_dev, k, shape, rng):
    """The q|k|v linear with RoPE folded in (one token): 6 sampled q and k
    heads against the oracle's RoPE of the product over the GPU's kept rows,
    and 256 sampled v columns against the product, teacher-forced."""
    bound, exact = rotation_bound(x_in, q_blocks)
    assert np.all(np.abs(xr_gpu.astype(np.float64) - exact) <= bound), "rotation bound"
    want_idx = ref.select(xr_gpu, k)
    np.testing.assert_array_equal(idx_gpu, want_idx)
    dh = shape.d_head
    n_rot = shape.n_heads + shape.n_kv_heads
    heads = np.sort(rng.choice(n_rot, size=6, replace=False))
    cols = np.concatenate([np.arange(hd * dh, (hd + 1) * dh) for hd in heads])
    wf_cols = host(wf_dev[:, torch.from_numpy(cols).cuda()])
    prod = ref.round_to(ref.gather_product(xr_gpu, want_idx, wf_cols), "bf16")
    want = dec.rope(prod, len(heads), dh, shape.ctx)
    assert ref.rel_error(qkv_gpu[:, cols], want) <= TOL, "q|k heads with RoPE"
    v0 = n_rot * dh
    vcols = np.sort(rng.choice(np.arange(v0, shape.qkv_out), size=256, replace=False))
    wf_v = host(wf_dev[:, torch.from_numpy(vcols).cuda()])
    want_v = ref.round_to(ref.gather_product(xr_gpu, want_idx, wf_v), "bf16")
    assert ref.rel_error(qkv_gpu[:, vcols], want_v) <= TOL, "v columns"


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


def run_decoder(B, sparsity, n_layers, mode, n_checked=None, seed_cols=0, check_every=1):
    """Run n_layers of the 7B-shaped decoder on one batch and check every
    layer (or the first n_checked, or every check_every-th and the last)
    against the oracle, teacher-forced."""
    cfg = 3
    shape = wl.LLAMA7B
    base, base_dev, (kb, vb) = _base(cfg)
    kv_dev = (dev(kb.reshape(-1), "bf16").view(kb.shape), dev(vb.reshape(-1), "bf16").view(vb.shape))
    h0 = wl.decoder_hidden(cfg, B, shape.d)
    h = dev(h0, "bf16")
    buf = D.DecoderBuffers(shape, B)
    rng = np.random.default_rng(seed_cols)
    checked = 0
    folded = None
    for l in range(n_layers):
        layer, idxs, offs = D.build_layer(cfg, l, shape, base_dev, kv_dev, B, sparsity)
        if folded is None:
            # one token, unfused: the norms run inside the rotations, and each
            # layer's down output is added to h by the next layer's first
            # folded norm. Otherwise the chained form: layer l's closing
            # residual add also writes the next layer's first RMSNorm (one
            # launch); the first layer's norm runs here.
            folded = D.folds_norms(layer, B, mode)
            if not folded:
                _lib.larosa_rmsnorm(h, buf.a, B, shape.d)
        torch.cuda.synchronize()
        h_in = host(h)
        if folded and l > 0:  # the previous layer's down output, still pending
            h_in = dec.residual_add(h_in, host(buf.dn))
        a = None if folded else host(buf.a)
        trace = {}
        last = l == n_layers - 1
        D.layer_forward(layer, h, buf, mode=mode, trace=trace, normed=True, norm_next=not last,
                        pending=l > 0, defer=not last)
        torch.cuda.synchronize()
        if folded:
            a = host(buf.a)  # written by the layer's first folded norm
        skip = (n_checked is not None and checked >= n_checked) or \
            (l % check_every != 0 and l != n_layers - 1)
        if skip:
            del layer
            continue
        checked += 1
        qkv, att, o, m, hh, dn = (host(t) for t in (buf.qkv, buf.att, buf.o, buf.m, buf.hh,
                                                     buf.dn))
        Hd = shape.n_heads * shape.d_head
        Kd = shape.n_kv_heads * shape.d_head
        rope_in_qkv = trace.get("rope_in_qkv", False)
        if rope_in_qkv:  # q and k rotated in place inside qkv
            q, k = qkv[:, :Hd], qkv[:, Hd:Hd + Kd]
        else:
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
            if role == "attn_in" and rope_in_qkv:
                _check_qkv_rope_linear(a, q_host, host_f32(xr), host(idx), qkv, L.Wf, L.k,
                                       shape, rng)
                continue
            cols = np.sort(rng.choice(L.d_out, size=min(256, L.d_out), replace=False))
            _check_linear(lin_in[role], q_host, host_f32(xr), host(idx), lin_out[role], L.Wf,
                          L.k, cols)
        if not rope_in_qkv:
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
        if folded and not last:  # dn is added by the next layer
            np.testing.assert_array_equal(h_out, h_mid)
        else:
            np.testing.assert_array_equal(h_out, dec.residual_add(h_mid, dn))
        if l < n_layers - 1 and not folded:  # the next layer's norm, written by the closing add
            assert close_bf16(host(buf.a), dec.rmsnorm(h_out), extra=1e-6), f"layer {l} next norm"
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


@pytest.mark.parametrize("sp", [25, 40, 50])
def test_decoder_32_layers_single_token_unfused(sp):
    """One token through 32 layers in the mode the benchmark reports (one
    launch for the selection and product after each rotation); every layer
    checked."""
    run_decoder(1, sp, n_layers=32, mode=_lib.UNFUSED)


@pytest.mark.parametrize("B,sp", [(4, 25), (4, 50), (16, 25), (16, 50)])
def test_decoder_32_layers_batch_sparsity_grid(B, sp):
    """The rest of the batch x sparsity grid of the 32-layer step (4 and 16
    tokens at 25% and 50%): all 32 layers run, every fourth and the last are
    checked."""
    run_decoder(B, sp, n_layers=32, mode=_lib.UNFUSED, check_every=4)
