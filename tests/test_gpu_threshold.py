"""GPU parity of the magnitude-threshold selection (the R-Sparse-style
contrast to the fixed Top-K) and its calibration, against the oracle.

Index sets, counts and calibrated thresholds are integer results: compared
bit for bit. Products are compared teacher-forced on the GPU's own x_rot and
folded weight, within the method's tolerances (see test_gpu_parity)."""
import numpy as np
import pytest
import torch

from oracle import larosa_ref as ref
from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import workloads as wl
from rotated_top_activation_amd.device import RotatedLinear

from gpu_helpers import dev, guarded, host, host_f32
from test_gpu_parity import make_x_rot

pytestmark = pytest.mark.gpu


def _keep(n, p):
    return n * (100 - p) // 100


def _check_sets(idx, count, want, d, fill):
    """idx rows of capacity d hold the wanted sets; slots past count untouched."""
    idx = host(idx).reshape(len(want), d)
    count = host(count)
    for b, w in enumerate(want):
        assert count[b] == len(w), (b, count[b], len(w))
        np.testing.assert_array_equal(idx[b, :len(w)], w)
        assert np.all(idx[b, len(w):] == fill)


SELECT_CASES = [
    # (d, B, kind, threshold: a sparsity % to calibrate on the same data, or a value)
    (4, 1, "ties", 50), (100, 3, "ties", 40), (512, 1, "gauss", 40), (1000, 2, "heavy", 25),
    (4096, 4, "heavy", 40), (4096, 1, "ties", 40), (11008, 3, "gauss", 50),
    (13824, 2, "heavy", 40), (32768, 1, "ties", 50), (5120, 8, "heavy", 40),
    (1024, 2, "gauss", "zero"), (1024, 2, "gauss", "above"), (1028, 3, "ties", "tied"),
]


def _threshold_for(xr, spec):
    if spec == "zero":
        return 0.0
    if spec == "above":
        return float(np.abs(xr).max()) * 2
    if spec == "tied":
        return 2.0  # the "ties" inputs take the magnitudes 0 .. 4
    return float(ref.calibrate_threshold(xr, spec))


@pytest.mark.parametrize("d,B,kind,spec", SELECT_CASES)
def test_threshold_select_bit_exact(d, B, kind, spec):
    xr = make_x_rot(kind, B, d, seed=d * 7 + B)
    t = _threshold_for(xr, spec)
    want = ref.threshold_select(xr, t)
    xr_d = torch.from_numpy(xr).cuda()
    idx, ok_i = guarded((B * d,), torch.int32, fill=-7)
    count, ok_c = guarded((B,), torch.int32, fill=-5)
    val, ok_v = guarded((B * d,), torch.float32, fill=77.0)
    xs = torch.full((B, d), 99.0, device="cuda")
    _lib.larosa_threshold_select(xr_d, B, d, t, idx, count, val, xs)
    torch.cuda.synchronize()
    assert ok_i() and ok_c() and ok_v()
    _check_sets(idx, count, want, d, -7)
    v = host_f32(val).reshape(B, d)
    for b, w in enumerate(want):
        np.testing.assert_array_equal(v[b, :len(w)], xr[b, w])
    np.testing.assert_array_equal(host_f32(xs), ref.sparsify(xr, want).astype(np.float32))
    if B > 1:
        u_idx = torch.full((d,), -1, dtype=torch.int32, device="cuda")
        u_cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
        u_coef = torch.empty((d * B,), dtype=torch.float32, device="cuda")
        ws = torch.empty(_lib.larosa_workspace_bytes(B, d, 8, d), dtype=torch.uint8,
                         device="cuda")
        _lib.larosa_threshold_select(xr_d, B, d, t, idx, count, val, xs, u_idx, u_cnt, u_coef,
                                     ws)
        torch.cuda.synchronize()
        u = np.unique(np.concatenate(want)) if any(len(w) for w in want) else np.array([])
        n = int(host(u_cnt)[0])
        assert n == len(u)
        np.testing.assert_array_equal(host(u_idx)[:n], u)


@pytest.mark.parametrize("n,p", [(1, 0), (7, 80), (7, 0), (1000, 40), (4093, 50),
                                 (4096 * 64, 40), (11008 * 17, 25), (28672 * 9 + 4, 60)])
def test_calibrated_threshold_bit_exact(n, p):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.abs(rng.standard_t(3, size=n))).astype(np.float32)
    if n > 100:  # some exact ties
        x[::97] = 0.5
    t_d, ok = guarded((1,), torch.float32, fill=-1.0)
    ws = torch.empty(_lib.larosa_calibrate_workspace_bytes(), dtype=torch.uint8, device="cuda")
    keep = _keep(n, p)
    _lib.larosa_calibrate_threshold(torch.from_numpy(x).cuda(), n, keep, t_d, ws)
    torch.cuda.synchronize()
    assert ok()
    assert host_f32(t_d)[0] == ref.calibrate_threshold(x[None], p)


def _calib_t(case, q, p, n_tok=32):
    """t for a sparsity of p% from the oracle's rotation of calibration
    tokens drawn like the layer input (a different run seed)."""
    xc = wl.heavy_tailed_activations(case.cfg, case.layer, case.role, n_tok, case.d_in,
                                     case.dtype, run_seed=9)
    return float(ref.calibrate_threshold(ref.rotate(xc, q), p))


def _check_threshold_linear(lin, x, q, t, mode, tol, exact_rotation=False):
    B = x.shape[0]
    tdt = torch.float32 if lin.dtype == "f32" else torch.bfloat16
    y, ok_y = guarded((B, lin.d_out), tdt)
    idx, ok_i = guarded((B * lin.d_in,), torch.int32, fill=-3)
    count, ok_c = guarded((B,), torch.int32, fill=-4)
    xr = torch.empty((B, lin.d_in), dtype=torch.float32, device="cuda")
    ws = lin.workspace_for(B, lin.d_in, mode)
    x_d = dev(x, lin.dtype)
    _lib.larosa_threshold_layer_forward(x_d, lin.Qt, lin.q_block, lin.Wf, B, lin.d_in,
                                        lin.d_out, t, y, idx_out=idx, count_out=count,
                                        xrot_out=xr, mode=mode, ws=ws)
    y2 = torch.empty_like(y)
    _lib.larosa_threshold_layer_forward(x_d, lin.Qt, lin.q_block, lin.Wf, B, lin.d_in,
                                        lin.d_out, t, y2, mode=mode, ws=ws)
    torch.cuda.synchronize()
    assert ok_y() and ok_i() and ok_c()
    assert torch.equal(y, y2), "two runs differ"
    xr_g = host_f32(xr)
    if exact_rotation:
        np.testing.assert_array_equal(xr_g, ref.rotate(x, q))
    want = ref.threshold_select(xr_g, t)
    _check_sets(idx, count, want, lin.d_in, -3)
    want_y = ref.round_to(ref.gather_product(xr_g, want, host(lin.Wf)), lin.dtype)
    err = ref.rel_error(host(y), want_y)
    assert err <= tol, err
    return host(count)


class _Lin(RotatedLinear):
    def workspace_for(self, B, k, mode):
        n = _lib.larosa_workspace_bytes(B, self.d_in, self.d_out, k, mode)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=self.Wf.device)
        _lib.larosa_workspace_init(ws)
        return ws


LAYER_CASES = [
    # (d_in, q_block, d_out, B, sparsity %): B = 1 takes the one-launch
    # selection + product below 16384 channels and the separate steps above
    (4096, 4096, 22016, 1, 40), (11008, 2752, 4096, 1, 40), (1024, 256, 1032, 1, 50),
    (20480, 2048, 1024, 1, 50), (4096, 4096, 1032, 3, 40), (4096, 4096, 1032, 16, 40),
    (2048, 512, 4104, 40, 25), (1024, 256, 2056, 64, 40),
]


@pytest.mark.parametrize("d,qb,n,B,sp", LAYER_CASES)
def test_threshold_layer_forward(d, qb, n, B, sp):
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=sp,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = _Lin(q, w, "bf16", case.k)
    t = _calib_t(case, q, sp)
    counts = _check_threshold_linear(lin, x, q, t, _lib.UNFUSED, 2e-2)
    print(f"d={d} B={B}: kept per token {counts.tolist()} (Top-K would keep {case.k})")


def test_threshold_layer_forward_fp64_rotation_and_f32():
    case = wl.LinearCase(cfg=3, batch=2, d_in=4096, d_out=1032, q_block=4096, sparsity_pct=40,
                         dtype="bf16", role="down_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = _Lin(q, w, "bf16", case.k)
    t = _calib_t(case, q, 40)
    _check_threshold_linear(lin, x, q, t, _lib.UNFUSED | _lib.ROTATE_FP64, 2e-2,
                            exact_rotation=True)
    # one token with the fused mode flag runs the unfused steps
    _check_threshold_linear(lin, x[:1], q, t, _lib.FUSED | _lib.ROTATE_FP64, 2e-2,
                            exact_rotation=True)
    for nb in (1, 3):  # fp32: the one-launch form, then the vector product over a union
        c1, x1, q1, w1 = wl.single_linear_f32(batch=nb)
        lin1 = _Lin(q1, w1, "f32", c1.k)
        t1 = float(ref.calibrate_threshold(ref.rotate(x1, q1), 40))
        _check_threshold_linear(lin1, x1, q1, t1, _lib.UNFUSED, 1e-5)


def test_threshold_layer_extremes():
    """t = 0 keeps every channel (the dense product); t above every magnitude
    keeps none (y = 0)."""
    case = wl.LinearCase(cfg=3, batch=1, d_in=4096, d_out=1032, q_block=4096, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = _Lin(q, w, "bf16", case.k)
    c = _check_threshold_linear(lin, x, q, 0.0, _lib.UNFUSED, 2e-2)
    assert c[0] == 4096
    c = _check_threshold_linear(lin, x, q, 1e30, _lib.UNFUSED, 2e-2)
    assert c[0] == 0


@pytest.mark.parametrize("B", [1, 3])
def test_threshold_swiglu_layer(B):
    d, f, sp = 4096, 2816, 40
    case = wl.LinearCase(cfg=2, batch=B, d_in=d, d_out=2 * f, q_block=d, sparsity_pct=sp,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = _Lin(q, w, "bf16", case.k)
    t = _calib_t(case, q, sp)
    w_il = torch.empty_like(lin.Wf)
    _lib.larosa_interleave_gate_up(lin.Wf, w_il, d, f)
    x_d = dev(x, "bf16")
    # the layer over [W'_gate | W'_up], then SwiGLU, on the device
    gu = torch.empty((B, 2 * f), dtype=torch.bfloat16, device="cuda")
    h_ref = torch.empty((B, f), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_threshold_layer_forward(x_d, lin.Qt, d, lin.Wf, B, d, 2 * f, t, gu,
                                        ws=lin.workspace_for(B, d, _lib.UNFUSED))
    _lib.larosa_swiglu(gu, h_ref, B, f)
    ws = torch.zeros(_lib.larosa_swiglu_workspace_bytes(B, d, f, d, _lib.UNFUSED),
                     dtype=torch.uint8, device="cuda")
    h, ok_h = guarded((B, f), torch.bfloat16)
    idx, ok_i = guarded((B * d,), torch.int32, fill=-3)
    count = torch.empty((B,), dtype=torch.int32, device="cuda")
    xr = torch.empty((B, d), dtype=torch.float32, device="cuda")
    for _ in range(2):
        _lib.larosa_threshold_swiglu_layer_forward(x_d, lin.Qt, d, w_il, B, d, f, t, h,
                                                   idx_out=idx, count_out=count, xrot_out=xr,
                                                   ws=ws)
    torch.cuda.synchronize()
    assert ok_h() and ok_i()
    assert torch.equal(h, h_ref)
    xr_g = host_f32(xr)
    want = ref.threshold_select(xr_g, t)
    _check_sets(idx, count, want, d, -3)
    g_u = ref.round_to(ref.gather_product(xr_g, want, host(lin.Wf)), "bf16")
    assert ref.rel_error(host(h), ref.swiglu(g_u, f, "bf16")) <= 2e-2
