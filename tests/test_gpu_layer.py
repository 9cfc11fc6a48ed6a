"""GPU parity of the whole rotated sparse linear (larosa_layer_forward) and of
the SwiGLU MLP built from two of them, on the workload shapes, teacher-forced
against the oracle (see test_gpu_parity for the tolerance rules)."""
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


def check_linear(lin: RotatedLinear, x: np.ndarray, q: np.ndarray, mode=_lib.UNFUSED,
                 tol=None, report=None):
    """Run one layer_forward on x and check every stage against the oracle.

    Returns the GPU output (float64 values of its dtype)."""
    B = x.shape[0]
    act = lin.dtype
    tdt = torch.float32 if act == "f32" else torch.bfloat16
    y, ok_y = guarded((B, lin.d_out), tdt)
    idx, ok_i = guarded((B, lin.k), torch.int32, fill=-3)
    xr, ok_x = guarded((B, lin.d_in), torch.float32)
    ws = lin.workspace(B, mode)
    x_d = dev(x, act)
    lin.forward(x_d, y, ws, idx_out=idx, xrot_out=xr, mode=mode)
    y2 = torch.empty_like(y)
    lin.forward(x_d, y2, ws, mode=mode)
    torch.cuda.synchronize()
    assert ok_y() and ok_i() and ok_x()
    assert torch.equal(y, y2), "two runs differ"

    xr_g = host_f32(xr)
    # stage 1: rotation within the rigorous fp32 bound of the exact product
    bound, exact = rotation_bound(x, q)
    assert np.all(np.abs(xr_g.astype(np.float64) - exact) <= bound)
    # stage 2: the GPU's selection on its own x_rot is the oracle's, bit for bit
    want_idx = ref.select(xr_g, lin.k)
    np.testing.assert_array_equal(host(idx), want_idx)
    # stage 3: the product over the kept rows of the GPU's folded weight
    wf = host(lin.Wf)
    want_y = ref.round_to(ref.gather_product(xr_g, want_idx, wf), lin.dtype)
    tol = tol if tol is not None else (1e-5 if lin.dtype == "f32" else 2e-2)
    err = ref.rel_error(host(y), want_y)
    assert err <= tol, err
    if report is not None:
        # end to end (not teacher-forced): sets from the oracle's own x_rot;
        # any difference must be a near-tie within the rotation error bound
        own = ref.select(ref.rotate(x, q), lin.k)
        mism = 0
        for b in range(B):
            a, c = set(own[b].tolist()), set(want_idx[b].tolist())
            if a != c:
                mism += 1
                key = np.abs(exact[b])
                kth = np.sort(key)[::-1][lin.k - 1]
                for i in a ^ c:
                    assert abs(key[i] - kth) <= 2 * bound[b, i] + 2 * bound[b].max()
        report.append((B, mism, err))
    return host(y), xr_g, want_idx


MODES = [pytest.param(_lib.UNFUSED, id="unfused"), pytest.param(_lib.FUSED, id="fused")]


@pytest.mark.parametrize("mode", MODES)
def test_single_linear_f32_512x1536(mode):
    case, x, q, w = wl.single_linear_f32()
    lin = RotatedLinear(q, w, "f32", case.k)
    rep = []
    check_linear(lin, x, q, mode=mode, report=rep)
    assert case.k == 307


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("d,qb,n,sp", [(4096, 4096, 12288, 25), (11008, 2752, 4096, 40),
                                       (1024, 256, 1032, 50), (16384, 4096, 520, 40),
                                       (2048, 2048, 22016, 40)])
def test_single_token_linear_shapes(mode, d, qb, n, sp):
    case = wl.LinearCase(cfg=3, batch=1, d_in=d, d_out=n, q_block=qb, sparsity_pct=sp,
                         dtype="bf16", role="o_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    check_linear(lin, x, q, mode=mode)


@pytest.mark.parametrize("B,sp", [(2, 25), (4, 40), (8, 50), (3, 40), (16, 40), (16, 25)])
def test_batched_linear_union_4096_to_qkv(B, sp):
    d, n = 4096, 12288
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=d, sparsity_pct=sp,
                         dtype="bf16", role="attn_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    check_linear(lin, x, q)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("k", [1, 4096])
def test_linear_extreme_k(k, B, mode):
    case = wl.LinearCase(cfg=3, batch=B, d_in=4096, d_out=1032, q_block=4096, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", k)
    y, xr, idx = check_linear(lin, x, q, mode=mode)
    if k == 4096:
        # K = d keeps every channel: the dense x·W within bf16 tolerance
        dense = ref.round_to(x @ w, "bf16")
        assert ref.rel_error(y, dense) <= 2e-2


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("d,qb,n,levels,k", [
    (4096, 512, 22016, 5, 2457),    # five magnitudes: the K-th key is tied many times
    (4096, 512, 4104, 1, 1000),     # one magnitude: every channel ties with the K-th
    (8192, 1024, 4096, 5, 7000),    # K past the nonzero channels: the K-th key is 0
    (16384, 1024, 22016, 1, 9000),  # ranges of 1024 channels, all tied
])
def test_single_token_ties(mode, d, qb, n, levels, k):
    """Exact ties at the K-th key: a signed-permutation rotation keeps x's
    few integer magnitudes exactly, so the lowest-index rule decides which of
    the tied channels are kept."""
    rng = np.random.default_rng(d + 10 * levels + k)
    q = np.zeros((d // qb, qb, qb))
    for b in range(d // qb):
        perm, sign = wl.signed_permutation(rng, qb)
        q[b, np.arange(qb), perm] = sign
    mag = rng.integers(0, levels, (1, d)) if levels > 1 else np.ones((1, d))
    x = mag * np.where(rng.random((1, d)) < 0.5, -1.0, 1.0)
    w = wl.quantize(rng.standard_normal((d, n)) * 0.02, "bf16")
    lin = RotatedLinear(q, w, "bf16", k)
    _, xr, _ = check_linear(lin, x, q, mode=mode)
    key = np.abs(xr[0])
    assert np.sum(key == np.sort(key)[::-1][k - 1]) > 1  # the case really ties


@pytest.mark.parametrize("mode", MODES)
def test_llama7b_mlp_decode_b1(mode):
    """The 7B-shaped SwiGLU MLP at batch 1, 40%: gate|up (4096→22016),
    SiLU(gate)·up, down (11008→4096) with the 4×2752 block rotation."""
    case = wl.llama7b_mlp()
    x, q1, wgu, q2, wd = wl.mlp_case_inputs(case)
    l1 = RotatedLinear(q1, wgu, "bf16", case.k1)
    l2 = RotatedLinear(q2, wd, "bf16", case.k2)
    gu, _, _ = check_linear(l1, x, q1, mode=mode)
    h = torch.empty((1, case.f), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_swiglu(dev(gu, "bf16"), h, 1, case.f)
    torch.cuda.synchronize()
    h_g = host(h)
    h_ref = ref.swiglu(gu, case.f, "bf16")
    assert ref.rel_error(h_g, h_ref) <= 2e-2
    check_linear(l2, h_g, q2, mode=mode)
    assert (case.k1, case.k2) == (2457, 6604)


@pytest.mark.parametrize("mode", MODES)
def test_llama7b_mlp_bench_sequence_all_columns(mode):
    """The exact call sequence the benchmark times for one decode token of
    the 7B-shaped MLP: the SwiGLU-folded gate|up call over the interleaved
    folded weight (d = 4096, f = 11008, K = 2457), then the down call
    (4 x 2752 block rotation, K = 6604). Checked on every output column,
    stage by stage and teacher-forced on the GPU's own rotated inputs, then
    end to end against the oracle's own MLP (any difference in a kept set must
    be a certified near-tie)."""
    case = wl.llama7b_mlp()
    d, f, k1, k2 = case.d, case.f, case.k1, case.k2
    x, q1, wgu, q2, wd = wl.mlp_case_inputs(case)
    l1 = RotatedLinear(q1, wgu, "bf16", k1, keep_w=False)
    l2 = RotatedLinear(q2, wd, "bf16", k2, keep_w=False)
    w_il = torch.empty_like(l1.Wf)
    _lib.larosa_interleave_gate_up(l1.Wf, w_il, d, f)
    ws1 = torch.zeros(_lib.larosa_swiglu_workspace_bytes(1, d, f, k1, _lib.FUSED),
                      dtype=torch.uint8, device="cuda")
    ws2 = l2.workspace(1, _lib.FUSED)
    x_d = dev(x, "bf16")
    h = torch.empty((1, f), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((1, d), dtype=torch.bfloat16, device="cuda")
    # as the benchmark calls it (no optional outputs) ...
    _lib.larosa_swiglu_layer_forward(x_d, l1.Qt, l1.q_block, w_il, 1, d, f, k1, h, mode=mode,
                                     ws=ws1)
    _lib.larosa_layer_forward(h, l2.Qt, l2.q_block, l2.Wf, 1, f, d, k2, y, mode=mode, ws=ws2)
    # ... and again with the selections and rotated inputs copied out
    h2, ok_h = guarded((1, f), torch.bfloat16)
    y2, ok_y = guarded((1, d), torch.bfloat16)
    idx1, ok_i1 = guarded((1, k1), torch.int32, fill=-3)
    idx2, ok_i2 = guarded((1, k2), torch.int32, fill=-3)
    xr1 = torch.empty((1, d), dtype=torch.float32, device="cuda")
    xr2 = torch.empty((1, f), dtype=torch.float32, device="cuda")
    _lib.larosa_swiglu_layer_forward(x_d, l1.Qt, l1.q_block, w_il, 1, d, f, k1, h2, idx_out=idx1,
                                     xrot_out=xr1, mode=mode, ws=ws1)
    _lib.larosa_layer_forward(h2, l2.Qt, l2.q_block, l2.Wf, 1, f, d, k2, y2, idx_out=idx2,
                              xrot_out=xr2, mode=mode, ws=ws2)
    torch.cuda.synchronize()
    assert ok_h() and ok_y() and ok_i1() and ok_i2()
    assert torch.equal(h, h2) and torch.equal(y, y2)

    # stage 1, teacher-forced: rotation bound, kept set, h on all 11008 columns
    xr1_g = host_f32(xr1)
    bound1, exact1 = rotation_bound(x, q1)
    assert np.all(np.abs(xr1_g.astype(np.float64) - exact1) <= bound1)
    want_idx1 = ref.select(xr1_g, k1)
    np.testing.assert_array_equal(host(idx1), want_idx1)
    wf1 = host(l1.Wf)
    gu = ref.round_to(ref.gather_product(xr1_g, want_idx1, wf1), "bf16")
    h_ref = ref.swiglu(gu, f, "bf16")
    h_g = host(h)
    assert ref.rel_error(h_g, h_ref) <= 2e-2
    # stage 2, teacher-forced on the GPU's h: all 4096 columns of y
    xr2_g = host_f32(xr2)
    bound2, exact2 = rotation_bound(h_g, q2)
    assert np.all(np.abs(xr2_g.astype(np.float64) - exact2) <= bound2)
    want_idx2 = ref.select(xr2_g, k2)
    np.testing.assert_array_equal(host(idx2), want_idx2)
    wf2 = host(l2.Wf)
    y_ref = ref.round_to(ref.gather_product(xr2_g, want_idx2, wf2), "bf16")
    assert ref.rel_error(host(y), y_ref) <= 2e-2

    # end to end: the oracle's own MLP from x on the same folded weights. A
    # kept channel may differ only at a near-tie: within the rotation's error
    # bound for the first linear; for the down linear (whose input h may
    # differ from the oracle's by a bf16 rounding) within 1% of the K-th
    # magnitude. With equal sets on both linears y is within the tolerance.
    y_o, st = ref.mlp(x, q1, wf1, q2, wf2, k1, k2, f, act_dtype="bf16")
    same = True
    for own, got, k, near in ((st["idx1"], want_idx1, k1, lambda i, kth, key:
                               abs(key[i] - kth) <= 2 * bound1[0, i] + 2 * bound1[0].max()),
                              (st["idx2"], want_idx2, k2, lambda i, kth, key:
                               abs(key[i] - kth) <= 1e-2 * kth)):
        a, c = set(own[0].tolist()), set(got[0].tolist())
        if a != c:
            same = False
            key = np.abs(np.asarray(st["x_rot1"] if k == k1 else st["x_rot2"],
                                    dtype=np.float64)[0])
            kth = np.sort(key)[::-1][k - 1]
            for i in a ^ c:
                assert near(i, kth, key), (k, i)
    if same:
        assert ref.rel_error(host(y), y_o) <= 2e-2
    assert (k1, k2) == (2457, 6604)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B", [1, 4])
def test_graph_replay_matches_eager(B, mode):
    """A captured layer_forward replays to the eager result every time, with
    eager work and synchronisations between replays."""
    case = wl.LinearCase(cfg=3, batch=B, d_in=2048, d_out=4104, q_block=512, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    ws = lin.workspace(B, mode)
    x_d = dev(x, "bf16")
    y_eager = torch.empty((B, case.d_out), dtype=torch.bfloat16, device="cuda")
    lin.forward(x_d, y_eager, ws, mode=mode)
    torch.cuda.synchronize()
    y_g = torch.zeros_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lin.forward(x_d, y_g, ws, mode=mode)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lin.forward(x_d, y_g, ws, mode=mode)
    for rep in range(4):
        y_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_eager), f"replay {rep} differs"
        other = torch.empty_like(y_eager)
        lin.forward(x_d, other, ws, mode=mode)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, y_eager)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B", [1, 4])
def test_graph_replay_with_changing_inputs(B, mode):
    """A captured layer_forward replayed on new inputs written into its input
    buffer: every replay equals the eager call on the same input. Any state a
    launch keeps between calls (the one-launch kernel's epoch) has to live on
    the device for this to hold."""
    case = wl.LinearCase(cfg=3, batch=B, d_in=2048, d_out=4104, q_block=512, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    ws = lin.workspace(B, mode)
    x_static = dev(x, "bf16")
    y_g = torch.zeros((B, case.d_out), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lin.forward(x_static, y_g, ws, mode=mode)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lin.forward(x_static, y_g, ws, mode=mode)
    rng = np.random.default_rng(100 + B + mode)
    ws_eager = lin.workspace(B, mode)
    for rep in range(5):
        xn = dev(wl.quantize(x * rng.uniform(0.25, 4.0, x.shape), "bf16"), "bf16")
        x_static.copy_(xn)
        y_g.zero_()
        g.replay()
        y_e = torch.empty_like(y_g)
        lin.forward(xn, y_e, ws_eager, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep} differs"


@pytest.mark.parametrize("mode", MODES)
def test_changing_inputs_through_one_workspace(mode):
    """Different inputs through one workspace, call after call: every output
    matches the oracle (a stale partial sum from an earlier call would not)."""
    case = wl.LinearCase(cfg=3, batch=1, d_in=4096, d_out=22016, q_block=4096,
                         sparsity_pct=40, dtype="bf16")
    _, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    ws = lin.workspace(1, mode)
    wf = host(lin.Wf)
    rng = np.random.default_rng(77)
    for it in range(6):
        x = wl.quantize(rng.standard_normal((1, 4096)) * (it + 1), "bf16")
        y = torch.empty((1, case.d_out), dtype=torch.bfloat16, device="cuda")
        xr = torch.empty((1, 4096), device="cuda")
        lin.forward(dev(x, "bf16"), y, ws, xrot_out=xr, mode=mode)
        torch.cuda.synchronize()
        xr_g = host_f32(xr)
        idx = ref.select(xr_g, case.k)
        want = ref.round_to(ref.gather_product(xr_g, idx, wf), "bf16")
        assert ref.rel_error(host(y), want) <= 2e-2, it


def test_fused_and_unfused_share_one_workspace():
    """Alternating modes on one workspace: both stay correct and agree on the
    kept index sets."""
    case = wl.LinearCase(cfg=3, batch=1, d_in=4096, d_out=4104, q_block=1024, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    ws = lin.workspace(1, _lib.FUSED)
    x_d = dev(x, "bf16")
    outs = []
    for it in range(6):
        mode = _lib.FUSED if it % 2 else _lib.UNFUSED
        y = torch.empty((1, case.d_out), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((1, case.k), dtype=torch.int32, device="cuda")
        lin.forward(x_d, y, ws, idx_out=idx, mode=mode)
        torch.cuda.synchronize()
        outs.append((mode, host(y), host(idx)))
    for mode, y, idx in outs:
        np.testing.assert_array_equal(idx, outs[0][2])
        assert ref.rel_error(y, outs[0][1]) <= 2e-2


@pytest.mark.parametrize("B,d,qb,n", [(32, 2048, 512, 2056), (64, 1024, 1024, 1032),
                                      (11, 4096, 4096, 520), (6, 1000, 200, 264)])
def test_large_batches(B, d, qb, n):
    """Matrix-core batches, including d = 1000, whose last mask word of the
    row union is partly past the channels."""
    case = wl.LinearCase(cfg=5, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=50,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.01)
    lin = RotatedLinear(q, w, "bf16", case.k)
    check_linear(lin, x, q)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,d,qb,n", [(1, 8192, 1024, 4096), (1, 4096, 4096, 22016),
                                      (3, 4096, 1024, 4104), (16, 2048, 512, 2056)])
def test_workspace_stays_in_bounds(mode, B, d, qb, n):
    """K from 1 to d, each on a fresh workspace of exactly the advertised size
    with canaries on both sides: no call writes outside it. (Fewer kept rows
    can make the gather plan choose more splits than the all-rows plan.)"""
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k, keep_w=False)
    x_d = dev(x, "bf16")
    ks = {1, 2, 63, 64, 65, d // 7, d // 3, d - 1, d} | set(range(d // 16, d, d // 16))
    pad = 4096
    for k in sorted(ks):
        nbytes = _lib.larosa_workspace_bytes(B, d, n, k, mode)
        buf = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
        ws = buf[pad:pad + nbytes]
        _lib.larosa_workspace_init(ws)
        y = torch.empty((B, n), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            _lib.larosa_layer_forward(x_d, lin.Qt, qb, lin.Wf, B, d, n, k, y, mode=mode, ws=ws)
        torch.cuda.synchronize()
        b = buf.cpu()
        assert bool((b[:pad] == 0xA5).all() and (b[pad + nbytes:] == 0xA5).all()), k
        assert bool(torch.isfinite(y).all()), k


# ------------------------------------------- SwiGLU folded into gate|up --

def _interleave_ref(w, f, block):
    """The column permutation larosa_interleave_gate_up documents."""
    out = np.empty_like(w)
    for i in range(f):
        c = (i // block) * 2 * block + i % block
        out[:, c] = w[:, i]
        out[:, c + block] = w[:, f + i]
    return out


@pytest.mark.parametrize("dt,d,f", [("bf16", 64, 512), ("f32", 40, 384)])
def test_interleave_gate_up_is_the_documented_permutation(dt, d, f):
    rng = np.random.default_rng(f)
    w = wl.quantize(rng.standard_normal((d, 2 * f)), dt)
    w_d = dev(w, dt)
    out = torch.empty_like(w_d)
    _lib.larosa_interleave_gate_up(w_d, out, d, f)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), _interleave_ref(w, f, 256 if dt == "bf16" else 128))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,f", [(1, 2816), (3, 2816), (16, 2816), (1, 11008), (4, 11008),
                                 (16, 11008)])
def test_swiglu_layer_matches_layer_then_swiglu(B, f, mode):
    """h from the gate|up linear with SiLU(gate)·up folded in equals, bit for
    bit, the plain layer over [W'_gate | W'_up] followed by the SwiGLU step,
    and both match the oracle (teacher-forced on the GPU's x_rot). f = 11008
    is the 7B MLP's gate|up."""
    d, sp = 4096, 40
    case = wl.LinearCase(cfg=2, batch=B, d_in=d, d_out=2 * f, q_block=d, sparsity_pct=sp,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    w_il = torch.empty_like(lin.Wf)
    _lib.larosa_interleave_gate_up(lin.Wf, w_il, d, f)
    x_d = dev(x, "bf16")
    # the two-step reference on the device
    gu = torch.empty((B, 2 * f), dtype=torch.bfloat16, device="cuda")
    h_ref = torch.empty((B, f), dtype=torch.bfloat16, device="cuda")
    lin.forward(x_d, gu, lin.workspace(B, mode), mode=mode)
    _lib.larosa_swiglu(gu, h_ref, B, f)
    # folded
    nbytes = _lib.larosa_swiglu_workspace_bytes(B, d, f, case.k, mode)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    h, ok_h = guarded((B, f), torch.bfloat16)
    idx, ok_i = guarded((B, case.k), torch.int32, fill=-3)
    xr = torch.empty((B, d), dtype=torch.float32, device="cuda")
    for _ in range(2):  # the second call checks the workspace was left ready
        _lib.larosa_swiglu_layer_forward(x_d, lin.Qt, d, w_il, B, d, f, case.k, h, idx_out=idx,
                                         xrot_out=xr, mode=mode, ws=ws)
    torch.cuda.synchronize()
    assert ok_h() and ok_i()
    assert torch.equal(h, h_ref)
    xr_g = host_f32(xr)
    want_idx = ref.select(xr_g, case.k)
    np.testing.assert_array_equal(host(idx), want_idx)
    g_u = ref.round_to(ref.gather_product(xr_g, want_idx, host(lin.Wf)), "bf16")
    want_h = ref.swiglu(g_u, f, "bf16")
    assert ref.rel_error(host(h), want_h) <= 2e-2


@pytest.mark.parametrize("B,d,qb,n", [(16, 4096, 4096, 1032), (64, 11008, 2752, 520),
                                      (40, 2048, 512, 1032), (2, 5120, 5120, 1032)])
def test_batched_selection_adds_the_rotation_parts_in_order(B, d, qb, n):
    """From 2 tokens the matrix-core rotation's k-range partial sums are added
    by the Top-K selection itself, with no separate summing launch. That
    x_rot must equal, bit for bit, the threshold layer's, whose rotation runs
    the same split and adds the partials in the separate step, and the kept
    sets must be the oracle's selection of it."""
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=40,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    x_d = dev(x, "bf16")
    y, ok_y = guarded((B, n), torch.bfloat16)
    idx, ok_i = guarded((B, case.k), torch.int32, fill=-3)
    xr, ok_x = guarded((B, d), torch.float32)
    lin.forward(x_d, y, lin.workspace(B), idx_out=idx, xrot_out=xr)
    y_t = torch.empty_like(y)
    xr_t = torch.empty((B, d), dtype=torch.float32, device="cuda")
    ws_t = torch.zeros(_lib.larosa_workspace_bytes(B, d, n, d, _lib.UNFUSED), dtype=torch.uint8,
                       device="cuda")
    _lib.larosa_threshold_layer_forward(x_d, lin.Qt, qb, lin.Wf, B, d, n, 1.0, y_t, xrot_out=xr_t,
                                        ws=ws_t)
    torch.cuda.synchronize()
    assert ok_y() and ok_i() and ok_x()
    assert torch.equal(xr, xr_t)
    np.testing.assert_array_equal(host(idx), ref.select(host_f32(xr), case.k))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B", [1, 2, 3, 8, 16, 33, 64])
def test_exact_arithmetic_end_to_end(B, dt, mode):
    """Signed-permutation rotations with small-integer x and W make every step
    exact: x_rot = x·Q is a signed permutation of x, the fold only permutes and
    negates W's rows, and every partial sum of the product is an integer below
    2^24, so no summation order can change it. The kept index sets are then
    the oracle's on its own x_rot (end to end, not teacher-forced; the
    integer magnitudes tie heavily at the K-th key, so the lowest-index rule
    decides), and y is the oracle's exact product rounded to the output type,
    bit for bit, through the one-token, vector and matrix-core paths and the
    one-launch form."""
    d, qb, n, k = 1024, 256, 1544, 410
    rng = np.random.default_rng(1000 * B + (dt == "f32"))
    q = np.zeros((d // qb, qb, qb))
    for c in range(d // qb):
        perm, sign = wl.signed_permutation(rng, qb)
        q[c, np.arange(qb), perm] = sign
    x = rng.integers(-8, 9, (B, d)).astype(np.float64)
    w = rng.integers(-4, 5, (d, n)).astype(np.float64)
    lin = RotatedLinear(q, w, dt, k)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    y, ok_y = guarded((B, n), tdt)
    idx, ok_i = guarded((B, k), torch.int32, fill=-3)
    xr, ok_x = guarded((B, d), torch.float32)
    lin.forward(dev(x, dt), y, lin.workspace(B, mode), idx_out=idx, xrot_out=xr, mode=mode)
    torch.cuda.synchronize()
    assert ok_y() and ok_i() and ok_x()
    want_y, want_xr, want_idx = ref.linear(x, q, ref.fold(q, w, dt), k, dt)
    np.testing.assert_array_equal(host_f32(xr), want_xr.astype(np.float32))
    np.testing.assert_array_equal(host(idx), want_idx)
    np.testing.assert_array_equal(host(y), want_y)
    key = np.abs(want_xr[0])
    assert np.sum(key == np.sort(key)[::-1][k - 1]) > 1  # the K-th key is tied
