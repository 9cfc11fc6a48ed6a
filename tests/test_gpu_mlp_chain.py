"""GPU parity of larosa_mlp_forward, the whole SwiGLU MLP in one call, by
default the two layer calls; with LAROSA_CHAIN, for one token the down
linear's rotation runs inside the gate|up product's launch (the chained
form). Its outputs must equal the two layer calls'
(larosa_swiglu_layer_forward, then larosa_layer_forward) bit for bit where
the rotation's summation order is the same (Q2 blocks of 2056..4096
channels), match the oracle teacher-forced otherwise, stay right call after
call on one workspace and under graph replay (the chain keeps its epoch and
queues on the device), and report a wait that gives up."""
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


class Mlp:
    def __init__(self, d, f, q2_block, sp=40, seed=0):
        case = wl.llama7b_mlp(q2_block=q2_block) if (d, f) == (4096, 11008) else None
        if case is not None:
            x, q1, wgu, q2, wd = wl.mlp_case_inputs(case)
            self.k1, self.k2 = case.k1, case.k2
        else:
            rng = np.random.default_rng(seed)
            q1 = wl.quantize(wl.rotation_fp64(2, 0, "mlp_in", d, d), "bf16")
            q2 = wl.quantize(wl.rotation_fp64(2, 0, "down_in", f, q2_block), "bf16")
            wgu = wl.quantize(rng.standard_normal((d, 2 * f)) * 0.02, "bf16")
            wd = wl.quantize(rng.standard_normal((f, d)) * 0.02, "bf16")
            x = wl.heavy_tailed_activations(2, 0, "mlp_in", 1, d, "bf16", run_seed=seed)
            self.k1, self.k2 = wl.k_for(d, sp), wl.k_for(f, sp)
        self.d, self.f, self.qb2 = d, f, q2_block
        self.x, self.q1, self.q2 = x, q1, q2
        self.l1 = RotatedLinear(q1, wgu, "bf16", self.k1, keep_w=False)
        self.l2 = RotatedLinear(q2, wd, "bf16", self.k2, keep_w=False)
        self.w_il = torch.empty_like(self.l1.Wf)
        _lib.larosa_interleave_gate_up(self.l1.Wf, self.w_il, d, f)

    def ws(self, B=1, mode=_lib.CHAIN):
        return torch.zeros(_lib.larosa_mlp_workspace_bytes(B, self.d, self.f, self.k1, self.k2,
                                                           mode), dtype=torch.uint8,
                           device="cuda")

    def chain(self, x_d, ws, mode=_lib.CHAIN, outs=True):
        B = x_d.shape[0]
        h = torch.empty((B, self.f), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((B, self.d), dtype=torch.bfloat16, device="cuda")
        o = {}
        if outs:
            o = dict(idx1_out=torch.empty((B, self.k1), dtype=torch.int32, device="cuda"),
                     xrot1_out=torch.empty((B, self.d), device="cuda"),
                     idx2_out=torch.empty((B, self.k2), dtype=torch.int32, device="cuda"),
                     xrot2_out=torch.empty((B, self.f), device="cuda"))
        _lib.larosa_mlp_forward(x_d, self.l1.Qt, self.l1.q_block, self.w_il, self.l2.Qt,
                                self.qb2, self.l2.Wf, B, self.d, self.f, self.k1, self.k2, h, y,
                                mode=mode, ws=ws, **o)
        return h, y, o

    def two_calls(self, x_d, mode=_lib.UNFUSED):
        B = x_d.shape[0]
        h = torch.empty((B, self.f), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((B, self.d), dtype=torch.bfloat16, device="cuda")
        idx1 = torch.empty((B, self.k1), dtype=torch.int32, device="cuda")
        idx2 = torch.empty((B, self.k2), dtype=torch.int32, device="cuda")
        xr1 = torch.empty((B, self.d), device="cuda")
        xr2 = torch.empty((B, self.f), device="cuda")
        ws1 = torch.zeros(_lib.larosa_swiglu_workspace_bytes(B, self.d, self.f, self.k1, mode),
                          dtype=torch.uint8, device="cuda")
        _lib.larosa_swiglu_layer_forward(x_d, self.l1.Qt, self.l1.q_block, self.w_il, B, self.d,
                                         self.f, self.k1, h, idx_out=idx1, xrot_out=xr1,
                                         mode=mode, ws=ws1)
        _lib.larosa_layer_forward(h, self.l2.Qt, self.qb2, self.l2.Wf, B, self.f, self.d,
                                  self.k2, y, idx_out=idx2, xrot_out=xr2, mode=mode,
                                  ws=self.l2.workspace(B, mode))
        return h, y, dict(idx1_out=idx1, xrot1_out=xr1, idx2_out=idx2, xrot2_out=xr2)


def _status(ws):
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    _lib.larosa_workspace_status(ws, out)
    torch.cuda.synchronize()
    return int(out.item())


@pytest.mark.parametrize("d,f,qb2", [(4096, 11008, 2752), (1024, 2816, 2816), (2048, 5632, 2816)])
def test_chain_equals_the_two_layer_calls(d, f, qb2):
    m = Mlp(d, f, qb2)
    ws = m.ws()
    rng = np.random.default_rng(d + f)
    for it in range(4):  # one workspace, call after call, changing inputs
        x = m.x if it == 0 else wl.quantize(m.x * rng.uniform(0.5, 2.0, m.x.shape), "bf16")
        x_d = dev(x, "bf16")
        h, y, o = m.chain(x_d, ws)
        h2, y2, o2 = m.two_calls(x_d)
        torch.cuda.synchronize()
        for key in o:
            assert torch.equal(o[key], o2[key]), (it, key)
        assert torch.equal(h, h2), it
        assert torch.equal(y, y2), it
        assert _status(ws) == _lib.OK
    # the call without optional outputs gives the same h and y
    h3, y3, _ = m.chain(x_d, ws, outs=False)
    torch.cuda.synchronize()
    assert torch.equal(h3, h) and torch.equal(y3, y)


@pytest.mark.parametrize("d,f,qb2", [(1024, 2816, 256), (1024, 2816, 704), (1024, 2816, 1408)])
def test_chain_matches_the_oracle_for_other_block_widths(d, f, qb2):
    """Block widths whose one-token rotation sums in another order: checked
    stage by stage against the oracle on the GPU's own intermediates."""
    m = Mlp(d, f, qb2, seed=5)
    ws = m.ws()
    x_d = dev(m.x, "bf16")
    h, y, o = m.chain(x_d, ws)
    torch.cuda.synchronize()
    xr1 = host_f32(o["xrot1_out"])
    b1, e1 = rotation_bound(m.x, m.q1)
    assert np.all(np.abs(xr1.astype(np.float64) - e1) <= b1)
    idx1 = ref.select(xr1, m.k1)
    np.testing.assert_array_equal(host(o["idx1_out"]), idx1)
    gu = ref.round_to(ref.gather_product(xr1, idx1, host(m.l1.Wf)), "bf16")
    h_g = host(h)
    assert ref.rel_error(h_g, ref.swiglu(gu, f, "bf16")) <= 2e-2
    xr2 = host_f32(o["xrot2_out"])
    b2, e2 = rotation_bound(h_g, m.q2)
    assert np.all(np.abs(xr2.astype(np.float64) - e2) <= b2)
    idx2 = ref.select(xr2, m.k2)
    np.testing.assert_array_equal(host(o["idx2_out"]), idx2)
    y_ref = ref.round_to(ref.gather_product(xr2, idx2, host(m.l2.Wf)), "bf16")
    assert ref.rel_error(host(y), y_ref) <= 2e-2


@pytest.mark.parametrize("B,mode", [(4, _lib.UNFUSED), (1, _lib.FUSED),
                                    (1, _lib.UNFUSED | _lib.ROTATE_FP64)])
def test_other_batches_and_modes_run_the_two_calls(B, mode):
    m = Mlp(1024, 2816, 704, seed=7)
    rng = np.random.default_rng(3)
    x = wl.quantize(rng.standard_normal((B, 1024)), "bf16")
    x_d = dev(x, "bf16")
    h, y, o = m.chain(x_d, m.ws(B, mode), mode=mode | _lib.CHAIN)
    h2, y2, o2 = m.two_calls(x_d, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(y, y2)
    for key in o:
        assert torch.equal(o[key], o2[key]), key


def test_chain_wait_gives_up_with_a_status_and_recovers():
    m = Mlp(1024, 2816, 2816, seed=9)
    ws = m.ws()
    x_d = dev(m.x, "bf16")
    h_ok, y_ok, _ = m.two_calls(x_d)
    prev = _lib.larosa_set_spin_limit(0)
    try:
        for _ in range(3):
            m.chain(x_d, ws, outs=False)
        torch.cuda.synchronize()
    finally:
        _lib.larosa_set_spin_limit(prev)
    st = _status(ws)
    # with no wait allowed a workgroup that found its block not yet complete
    # says so; one that found it complete (its block finished first) has
    # nothing to report, so either status is possible, but a give-up must not
    # leave anything behind: the next calls are right again
    assert st in (_lib.OK, _lib.ERR_TIMEOUT)
    for _ in range(2):
        h, y, _ = m.chain(x_d, ws, outs=False)
        torch.cuda.synchronize()
        assert torch.equal(h, h_ok) and torch.equal(y, y_ok)
        assert _status(ws) == _lib.OK


def test_standalone_chained_kernel_equals_its_two_steps():
    """larosa_topk_swiglu_rotate (the chained launch alone) gives the bits of
    larosa_topk_swiglu_gemv followed by the one-token rotation, call after
    call on one workspace."""
    m = Mlp(4096, 11008, 2752)
    d, f = m.d, m.f
    ws = m.l1.workspace(1)
    x_d = dev(m.x, "bf16")
    xr1 = torch.empty((1, d), device="cuda")
    _lib.larosa_rotate(x_d, m.l1.Qt, m.l1.q_block, xr1, 1, d)
    ws_ref = m.l1.workspace(1)
    for it in range(3):
        xr = xr1 * (1.0 + 0.25 * it)
        h, ok_h = guarded((1, f), torch.bfloat16)
        xr2, ok_x = guarded((1, f), torch.float32)
        idx = torch.empty((1, m.k1), dtype=torch.int32, device="cuda")
        _lib.larosa_topk_swiglu_rotate(xr, d, m.k1, m.w_il, h, f, m.l2.Qt, m.qb2, xr2,
                                       idx_out=idx, ws=ws)
        h_ref = torch.empty((1, f), dtype=torch.bfloat16, device="cuda")
        idx_ref = torch.empty((1, m.k1), dtype=torch.int32, device="cuda")
        _lib.larosa_topk_swiglu_gemv(xr, d, m.k1, m.w_il, h_ref, f, idx_out=idx_ref, ws=ws_ref)
        xr2_ref = torch.empty((1, f), device="cuda")
        _lib.larosa_rotate(h_ref, m.l2.Qt, m.qb2, xr2_ref, 1, f)
        torch.cuda.synchronize()
        assert ok_h() and ok_x()
        assert torch.equal(h, h_ref) and torch.equal(idx, idx_ref), it
        assert torch.equal(xr2, xr2_ref), it
    assert _status(ws) == _lib.OK


def test_graph_replay_of_the_mlp_with_changing_inputs():
    """larosa_mlp_forward captured once and replayed on new inputs written
    into its input buffer: h and y equal the eager call's every time."""
    m = Mlp(4096, 11008, 2752)
    ws = m.ws()
    x_static = dev(m.x, "bf16")
    h_g = torch.zeros((1, m.f), dtype=torch.bfloat16, device="cuda")
    y_g = torch.zeros((1, m.d), dtype=torch.bfloat16, device="cuda")

    def call():
        _lib.larosa_mlp_forward(x_static, m.l1.Qt, m.l1.q_block, m.w_il, m.l2.Qt, m.qb2,
                                m.l2.Wf, 1, m.d, m.f, m.k1, m.k2, h_g, y_g, mode=_lib.CHAIN,
                                ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    rng = np.random.default_rng(11)
    ws_eager = m.ws()
    for rep in range(6):
        xn = dev(wl.quantize(m.x * rng.uniform(0.25, 4.0, m.x.shape), "bf16"), "bf16")
        x_static.copy_(xn)
        h_g.zero_()
        y_g.zero_()
        g.replay()
        h_e, y_e, _ = m.chain(xn, ws_eager, outs=False)
        torch.cuda.synchronize()
        assert torch.equal(h_g, h_e), f"replay {rep}: h differs"
        assert torch.equal(y_g, y_e), f"replay {rep}: y differs"
        if rep % 2:
            m.chain(xn, ws, outs=False)  # eager calls on the captured workspace in between
            torch.cuda.synchronize()
    assert _status(ws) == _lib.OK


def test_default_mode_is_the_two_layer_calls():
    """Without LAROSA_CHAIN the call runs the two layer calls: same bits, and
    the unfused workspace size."""
    m = Mlp(1024, 2816, 2816, seed=13)
    assert (_lib.larosa_mlp_workspace_bytes(1, m.d, m.f, m.k1, m.k2, _lib.UNFUSED) ==
            _lib.larosa_mlp_workspace_bytes(1, m.d, m.f, m.k1, m.k2, _lib.CHAIN))
    x_d = dev(m.x, "bf16")
    h, y, o = m.chain(x_d, m.ws(1, _lib.UNFUSED), mode=_lib.UNFUSED)
    h2, y2, o2 = m.two_calls(x_d)
    torch.cuda.synchronize()
    assert torch.equal(h, h2) and torch.equal(y, y2)
    for key in o:
        assert torch.equal(o[key], o2[key]), key
