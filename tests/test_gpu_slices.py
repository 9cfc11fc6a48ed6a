"""GPU parity of the 13B- and 70B-shaped layer slices: the four rotated
sparse linear inputs of one layer (q|k|v, o, gate|up, down) at their full
shapes and batch sizes, teacher-forced against the oracle. The q|k|v, o and
gate|up inputs are seeded synthetic activations (the slices give no
key/value context, so no attention core runs); the down input is the SwiGLU
of the gate|up output. Outputs are compared on sampled columns, since the
folded weights reach 0.9 GB."""
import numpy as np
import pytest
import torch

from oracle import larosa_ref as ref
from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import workloads as wl
from rotated_top_activation_amd.device import RotatedLinear

from gpu_helpers import dev, guarded, host, host_f32
from test_gpu_parity import rotation_bound

pytestmark = pytest.mark.gpu

SLICES = {
    # d, ffn, n_heads, n_kv_heads, q2_block, w_std, activations, sparsity %
    "13b": dict(cfg=4, d=5120, f=13824, H=40, Hkv=40, q2=3456, w_std=0.02, act="outlier",
                sp=40),
    "70b": dict(cfg=5, d=8192, f=28672, H=64, Hkv=8, q2=4096, w_std=0.01, act="heavy", sp=50),
}


def check_linear_sampled(lin, x, q, n_cols=512, seed=0, mode=_lib.UNFUSED):
    B = x.shape[0]
    y, ok_y = guarded((B, lin.d_out), torch.bfloat16)
    idx, ok_i = guarded((B, lin.k), torch.int32, fill=-3)
    xr, ok_x = guarded((B, lin.d_in), torch.float32)
    ws = lin.workspace(B, mode)
    x_d = dev(x, "bf16")
    lin.forward(x_d, y, ws, idx_out=idx, xrot_out=xr, mode=mode)
    torch.cuda.synchronize()
    assert ok_y() and ok_i() and ok_x()
    xr_g = host_f32(xr)
    bound, exact = rotation_bound(x, q)
    assert np.all(np.abs(xr_g.astype(np.float64) - exact) <= bound)
    want_idx = ref.select(xr_g, lin.k)
    np.testing.assert_array_equal(host(idx), want_idx)
    cols = np.sort(np.random.default_rng(seed).choice(lin.d_out, size=min(n_cols, lin.d_out),
                                                      replace=False))
    wf = host(lin.Wf[:, torch.from_numpy(cols).cuda()])
    want = ref.round_to(ref.gather_product(xr_g, want_idx, wf), "bf16")
    y_h = host(y)
    assert ref.rel_error(y_h[:, cols], want) <= 2e-2
    assert np.all(np.isfinite(y_h))
    return y_h


def slice_activations(s, role, B, d):
    if s["act"] == "outlier":
        return wl.outlier_activations(s["cfg"], 0, role, B, d, d // 100, 30.0, "bf16")
    return wl.heavy_tailed_activations(s["cfg"], 0, role, B, d, "bf16")


@pytest.mark.parametrize("name,B", [("13b", 8), ("70b", 32), ("70b", 64)])
def test_layer_slice(name, B):
    s = SLICES[name]
    cfg, d, f = s["cfg"], s["d"], s["f"]
    k_d = wl.k_for(d, s["sp"])
    k_f = wl.k_for(f, s["sp"])
    qkv_out = (s["H"] + 2 * s["Hkv"]) * 128
    roles = [("attn_in", d, d, qkv_out), ("o_in", d, d, d), ("mlp_in", d, d, 2 * f)]
    gu = None
    for role, d_in, qb, n in roles:
        q = wl.rotation(cfg, 0, role, d_in, qb, "bf16")
        if role == "mlp_in":
            w = np.concatenate([wl.gaussian_weight(cfg, 0, role, d_in, f, s["w_std"], "bf16", 0, 0),
                                wl.gaussian_weight(cfg, 0, role, d_in, f, s["w_std"], "bf16", 0, 1)],
                               axis=1)
        else:
            w = wl.gaussian_weight(cfg, 0, role, d_in, n, s["w_std"], "bf16")
        lin = RotatedLinear(q, w, "bf16", k_d, keep_w=False)
        del w
        x = slice_activations(s, role, B, d_in)
        y = check_linear_sampled(lin, x, q)
        if role == "mlp_in":
            gu = y
        del lin
        torch.cuda.empty_cache()
    # down input: SwiGLU of the gate|up output, on the GPU
    h = torch.empty((B, f), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_swiglu(dev(gu, "bf16"), h, B, f)
    torch.cuda.synchronize()
    h_g = host(h)
    assert ref.rel_error(h_g, ref.swiglu(gu, f, "bf16")) <= 2e-2
    q2 = wl.rotation(cfg, 0, "down_in", f, s["q2"], "bf16")
    w2 = wl.gaussian_weight(cfg, 0, "down_in", f, d, s["w_std"], "bf16")
    lin = RotatedLinear(q2, w2, "bf16", k_f, keep_w=False)
    check_linear_sampled(lin, h_g, q2)
