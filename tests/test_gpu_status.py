"""GPU tests of the boundary's failure reporting: the LAROSA_VALIDATE mode
(non-finite rotated input turned into LAROSA_ERR_NONFINITE before the
selection runs) and the one-launch kernel's bounded waits (a host-set spin
limit of zero makes every wait give up; each kernel still runs to its end,
the workspace's status word reports LAROSA_ERR_TIMEOUT, and the next call
on the same workspace is correct again)."""
import numpy as np
import pytest
import torch

from oracle import larosa_ref as ref
from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import workloads as wl
from rotated_top_activation_amd.device import RotatedLinear

from gpu_helpers import dev, host, host_f32

pytestmark = pytest.mark.gpu


def _linear(B, d=1024, qb=256, n=1032, sp=40):
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=sp,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    return case, x, RotatedLinear(q, w, "bf16", case.k)


@pytest.mark.parametrize("mode", [_lib.UNFUSED, _lib.FUSED, _lib.UNFUSED | _lib.ROTATE_FP64])
@pytest.mark.parametrize("B", [1, 4, 16])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_validate_rejects_nonfinite_rotated_input(B, mode, bad):
    case, x, lin = _linear(B)
    x_bad = x.copy()
    x_bad[B - 1, 17] = bad          # one channel of the last token
    ws = lin.workspace(B, mode)
    y = torch.full((B, case.d_out), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.LarosaError) as ei:
        lin.forward(dev(x_bad, "bf16"), y, ws, mode=mode | _lib.VALIDATE)
    assert ei.value.status == _lib.ERR_NONFINITE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "y was written although the call failed"
    # the same workspace then serves a finite input, with and without the check
    y1 = torch.empty_like(y)
    y2 = torch.empty_like(y)
    lin.forward(dev(x, "bf16"), y1, ws, mode=mode | _lib.VALIDATE)
    lin.forward(dev(x, "bf16"), y2, ws, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_validate_on_the_swiglu_and_low_rank_calls():
    d, f = 1024, 512
    case = wl.LinearCase(cfg=2, batch=1, d_in=d, d_out=2 * f, q_block=256, sparsity_pct=40,
                         dtype="bf16", role="mlp_in")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    w_il = torch.empty_like(lin.Wf)
    _lib.larosa_interleave_gate_up(lin.Wf, w_il, d, f)
    ws = torch.zeros(_lib.larosa_swiglu_workspace_bytes(1, d, f, case.k, _lib.UNFUSED),
                     dtype=torch.uint8, device="cuda")
    h = torch.empty((1, f), dtype=torch.bfloat16, device="cuda")
    x_bad = x.copy()
    x_bad[0, 3] = float("nan")
    with pytest.raises(_lib.LarosaError) as ei:
        _lib.larosa_swiglu_layer_forward(dev(x_bad, "bf16"), lin.Qt, 256, w_il, 1, d, f, case.k,
                                         h, mode=_lib.VALIDATE, ws=ws)
    assert ei.value.status == _lib.ERR_NONFINITE
    r = 16
    a_r = torch.zeros((d, r), dtype=torch.bfloat16, device="cuda")
    w_ext = torch.cat([lin.Wf, torch.zeros((r, 2 * f), dtype=torch.bfloat16, device="cuda")])
    ws_lr = torch.zeros(_lib.larosa_lowrank_workspace_bytes(1, d, 2 * f, case.k, r),
                        dtype=torch.uint8, device="cuda")
    y = torch.empty((1, 2 * f), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.LarosaError) as ei:
        _lib.larosa_lowrank_layer_forward(dev(x_bad, "bf16"), lin.Qt, 256, w_ext, a_r, r, 1, d,
                                          2 * f, case.k, y, mode=_lib.VALIDATE, ws=ws_lr)
    assert ei.value.status == _lib.ERR_NONFINITE


def _status(ws):
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    _lib.larosa_workspace_status(ws, out)
    torch.cuda.synchronize()
    return int(out.item())


@pytest.mark.parametrize("d,qb,n", [(1024, 256, 1032), (4096, 4096, 22016)])
def test_fused_waits_give_up_with_a_status_and_recover(d, qb, n):
    """Spin limit 0: every bounded wait of the one-launch kernel gives up at
    once. The launch still completes, the status word says so, and with the
    limit restored the next call on the same workspace matches the oracle
    and reports no error."""
    case = wl.LinearCase(cfg=3, batch=1, d_in=d, d_out=n, q_block=qb, sparsity_pct=40,
                         dtype="bf16")
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    lin = RotatedLinear(q, w, "bf16", case.k)
    ws = lin.workspace(1, _lib.FUSED)
    x_d = dev(x, "bf16")
    y = torch.empty((1, n), dtype=torch.bfloat16, device="cuda")
    assert _status(ws) == _lib.OK
    prev = _lib.larosa_set_spin_limit(0)
    try:
        for _ in range(3):
            lin.forward(x_d, y, ws, mode=_lib.FUSED)
        torch.cuda.synchronize()
    finally:
        _lib.larosa_set_spin_limit(prev)
    assert _status(ws) == _lib.ERR_TIMEOUT
    assert _status(ws) == _lib.OK          # taking the status cleared it
    # recovered: the next calls are right, and report nothing
    for _ in range(2):
        xr = torch.empty((1, d), dtype=torch.float32, device="cuda")
        idx = torch.empty((1, case.k), dtype=torch.int32, device="cuda")
        lin.forward(x_d, y, ws, idx_out=idx, xrot_out=xr, mode=_lib.FUSED)
        torch.cuda.synchronize()
        assert _status(ws) == _lib.OK
        xr_g = host_f32(xr)
        want_idx = ref.select(xr_g, case.k)
        np.testing.assert_array_equal(host(idx), want_idx)
        want = ref.round_to(ref.gather_product(xr_g, want_idx, host(lin.Wf)), "bf16")
        assert ref.rel_error(host(y), want) <= 2e-2


def test_unfused_calls_leave_the_status_clear():
    case, x, lin = _linear(1)
    ws = lin.workspace(1, _lib.UNFUSED)
    y = torch.empty((1, case.d_out), dtype=torch.bfloat16, device="cuda")
    prev = _lib.larosa_set_spin_limit(0)
    try:
        lin.forward(dev(x, "bf16"), y, ws, mode=_lib.UNFUSED)   # has no waits
    finally:
        _lib.larosa_set_spin_limit(prev)
    assert _status(ws) == _lib.OK
