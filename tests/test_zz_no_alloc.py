"""larosa_layer_forward_noalloc (the entry point for callers that cannot
allocate) against larosa_layer_forward with a caller workspace: the same
outputs bit for bit, on two calls in a row, the second one smaller (another
shape, so the library's device-resident array is cleared again for it)."""
import pytest
import torch

from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import workloads as wl
from rotated_top_activation_amd.device import RotatedLinear

from gpu_helpers import dev

pytestmark = pytest.mark.gpu

# (B, d_in, q_block, d_out, sparsity %, mode): the 7B gate|up at one token,
# then smaller calls
SEQUENCES = [
    [(1, 4096, 4096, 22016, 40, _lib.UNFUSED), (1, 1024, 256, 1032, 40, _lib.UNFUSED)],
    [(4, 2048, 512, 4104, 40, _lib.UNFUSED), (2, 1024, 1024, 520, 25, _lib.UNFUSED)],
    [(1, 11008, 2752, 4096, 40, _lib.UNFUSED | _lib.ROTATE_FP64),
     (1, 4096, 4096, 4096, 50, _lib.UNFUSED)],
]


def _case(B, d, qb, n, sp, seed):
    case = wl.LinearCase(cfg=3, batch=B, d_in=d, d_out=n, q_block=qb, sparsity_pct=sp,
                         dtype="bf16", run_seed=seed)
    x, q, w = wl.linear_case_inputs(case, w_std=0.02)
    return case, x, RotatedLinear(q, w, "bf16", case.k, keep_w=False)


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_workspace_call(seq):
    for i, (B, d, qb, n, sp, mode) in enumerate(SEQUENCES[seq]):
        case, x, lin = _case(B, d, qb, n, sp, seed=10 * seq + i)
        x_d = dev(x, "bf16")
        y_ref = torch.empty((B, n), dtype=torch.bfloat16, device="cuda")
        idx_ref = torch.empty((B, case.k), dtype=torch.int32, device="cuda")
        xr_ref = torch.empty((B, d), dtype=torch.float32, device="cuda")
        lin.forward(x_d, y_ref, lin.workspace(B, mode), idx_out=idx_ref, xrot_out=xr_ref,
                    mode=mode)
        y = torch.full((B, n), 3.0, dtype=torch.bfloat16, device="cuda")
        idx = torch.full((B, case.k), -1, dtype=torch.int32, device="cuda")
        xr = torch.empty((B, d), dtype=torch.float32, device="cuda")
        for _ in range(2):  # and again on the array the first call left behind
            _lib.larosa_layer_forward_noalloc(x_d, lin.Qt, qb, lin.Wf, B, d, n, case.k, y,
                                              idx_out=idx, xrot_out=xr, mode=mode)
            torch.cuda.synchronize()
            assert torch.equal(xr, xr_ref), (seq, i)
            assert torch.equal(idx, idx_ref), (seq, i)
            assert torch.equal(y, y_ref), (seq, i)


def test_noalloc_rejects_what_it_cannot_serve():
    case, x, lin = _case(1, 1024, 256, 1032, 40, seed=3)
    y = torch.empty((1, 1032), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.LarosaError) as ei:   # the one-launch form needs a workspace
        _lib.larosa_layer_forward_noalloc(dev(x, "bf16"), lin.Qt, 256, lin.Wf, 1, 1024, 1032,
                                          case.k, y, mode=_lib.FUSED)
    assert ei.value.status == _lib.ERR_INVALID_ARG
    assert _lib.larosa_workspace_bytes(16, 4096, 22016, 2457) > 16 << 20
    xb = torch.zeros((16, 4096), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((16, 22016), dtype=torch.bfloat16, device="cuda")
    big = torch.zeros((4096, 22016), dtype=torch.bfloat16, device="cuda")
    qt = torch.zeros((4096, 4096), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.LarosaError) as ei:   # beyond the 16 MiB array
        _lib.larosa_layer_forward_noalloc(xb, qt, 4096, big, 16, 4096, 22016, 2457, yb)
    assert ei.value.status == _lib.ERR_WORKSPACE
