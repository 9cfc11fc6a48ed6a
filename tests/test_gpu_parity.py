"""GPU parity of every entry point against the CPU oracle.

Index sets are compared bit for bit. Floating-point outputs are compared
teacher-forced: the oracle takes the GPU's own rotated activation and folded
weight, so a correct kernel cannot be failed by a legitimate fp32 summation
order (two correct orders can swap a near-tie at the K boundary). The
tolerances are the ones stated for the method's outputs: max relative error
(rel_error) <= 1e-5 for fp32 weights and <= 2e-2 for bf16 weights with fp32
accumulation; intermediate fp32 sums are held to the rigorous bound
|fl(Σ) − Σ| <= γ_n·Σ|terms| + half an ulp of the final rounding.
"""
import numpy as np
import pytest
import torch

from oracle import larosa_ref as ref
from rotated_top_activation_amd import _lib
from rotated_top_activation_amd import workloads as wl
from rotated_top_activation_amd.device import RotatedLinear

from gpu_helpers import dev, guarded, host, host_f32, ulp_bf16

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def gamma(n):
    return n * U32 / (1 - n * U32)


def rotation_bound(x, q_blocks):
    """Per-element bound on |fp32 x·Q − exact x·Q| for any summation order."""
    nb, b, _ = q_blocks.shape
    absum = ref.rotate_exact(np.abs(x), np.abs(q_blocks))
    exact = ref.rotate_exact(x, q_blocks)
    return gamma(b) * absum + ulp_f32(exact) / 2, exact


def ulp_f32(a):
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(np.where(a == 0, 1e-45, a))
    return np.ldexp(1.0, np.maximum(e - 24, -149))


def make_x_rot(kind, B, d, seed):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        return rng.standard_normal((B, d)).astype(np.float32)
    if kind == "ties":
        m = rng.integers(0, 5, (B, d)).astype(np.float32)
        s = np.where(rng.random((B, d)) < 0.5, -1.0, 1.0).astype(np.float32)
        return m * s
    if kind == "heavy":
        sc = np.abs(rng.standard_t(3, size=d))
        return (rng.standard_normal((B, d)) * sc).astype(np.float32)
    raise ValueError(kind)


# ----------------------------------------------------------------- select ---

SELECT_CASES = [
    (4, 1, 1, "ties"), (4, 4, 1, "ties"), (8, 3, 2, "ties"), (100, 37, 3, "ties"),
    (512, 307, 1, "gauss"), (1000, 600, 2, "heavy"), (1024, 1, 1, "gauss"),
    (1028, 1028, 1, "ties"), (4096, 2457, 1, "heavy"), (4096, 2457, 4, "ties"),
    (11008, 6604, 1, "heavy"), (13824, 8294, 2, "gauss"), (28672, 14336, 1, "heavy"),
    (32768, 16384, 1, "ties"), (5120, 3072, 8, "heavy"),
]


@pytest.mark.parametrize("d,k,B,kind", SELECT_CASES)
def test_select_bit_exact(d, k, B, kind):
    xr = make_x_rot(kind, B, d, seed=d * 31 + k)
    xr_d = torch.from_numpy(xr).cuda()
    idx, ok_idx = guarded((B, k), torch.int32, fill=-7)
    val, ok_val = guarded((B, k), torch.float32)
    xs = torch.full((B, d), 99.0, device="cuda")
    _lib.larosa_topk_select(xr_d, B, d, k, idx, val, xs)
    torch.cuda.synchronize()
    want = ref.select(xr, k)
    np.testing.assert_array_equal(host(idx), want)
    np.testing.assert_array_equal(host_f32(val), np.take_along_axis(xr, want, axis=1))
    np.testing.assert_array_equal(host_f32(xs), ref.sparsify(xr, want).astype(np.float32))
    assert ok_idx() and ok_val()


@pytest.mark.parametrize("d,k,B", [(512, 100, 2), (4100, 1700, 5), (11008, 6604, 8),
                                   (64, 64, 3), (2048, 1, 6),
                                   # 64 tokens, and a ragged last group of union rows
                                   (1000, 300, 64), (132, 100, 40)])
def test_union_matches_set_union(d, k, B):
    xr = make_x_rot("heavy", B, d, seed=B * 1000 + d)
    xr_d = torch.from_numpy(xr).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, k), device="cuda")
    xs = torch.empty((B, d), device="cuda")
    u_idx = torch.full((d,), -1, dtype=torch.int32, device="cuda")
    u_cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    u_coef = torch.full((d, B), 5.0, device="cuda")
    ws = torch.zeros(_lib.larosa_workspace_bytes(B, d, 64, k), dtype=torch.uint8, device="cuda")
    _lib.larosa_topk_select(xr_d, B, d, k, idx, val, xs, u_idx, u_cnt, u_coef, ws)
    torch.cuda.synchronize()
    sel = ref.select(xr, k)
    u = ref.row_union(sel)
    n = int(host(u_cnt)[0])
    assert n == len(u)
    np.testing.assert_array_equal(host(u_idx)[:n], u)
    xs_ref = ref.sparsify(xr, sel)
    np.testing.assert_array_equal(host_f32(u_coef)[:n], xs_ref[:, u].T.astype(np.float32))
    assert np.all(host_f32(u_coef)[n:] == 0)


# ---------------------------------------------------------------- rotation --

ROTATE_CASES = [
    # (x dtype, Q dtype, d, q_block, B)
    ("f32", "f32", 512, 512, 1), ("bf16", "bf16", 4096, 4096, 1),
    ("bf16", "bf16", 11008, 2752, 1), ("bf16", "bf16", 1024, 256, 5),
    ("f32", "bf16", 768, 768, 2), ("bf16", "f32", 256, 64, 3), ("bf16", "bf16", 13824, 3456, 8),
    # 2 to 8 tokens over blocks of 4096 or more, and fp32 batches: the
    # one-wave-per-channel form with the tokens' x staged in LDS
    ("bf16", "bf16", 4096, 4096, 2), ("bf16", "bf16", 4096, 4096, 3),
    ("bf16", "bf16", 5120, 5120, 4), ("f32", "f32", 512, 512, 4), ("f32", "f32", 2048, 1024, 7),
    ("bf16", "bf16", 4096, 4096, 8), ("bf16", "bf16", 8192, 8192, 6),
    # batches of 16 and more in bf16 take the matrix-core form
    ("bf16", "bf16", 4096, 4096, 16), ("bf16", "bf16", 11008, 2752, 33),
    ("bf16", "bf16", 8192, 8192, 64), ("bf16", "bf16", 1152, 96, 17),
    # one token, short blocks: several output channels per wave (8, 16 or 32
    # lanes each, the last with idle lanes)
    ("bf16", "bf16", 11008, 256, 1), ("bf16", "bf16", 1024, 64, 1), ("f32", "f32", 512, 64, 1),
    ("bf16", "bf16", 1152, 96, 1), ("f32", "f32", 384, 128, 1), ("bf16", "bf16", 11008, 344, 1),
]


@pytest.mark.parametrize("xdt,qdt,d,qb,B", ROTATE_CASES)
def test_rotate_within_rigorous_bound(xdt, qdt, d, qb, B):
    q = wl.rotation(4, 0, "single", d, qb, qdt)
    x = wl.heavy_tailed_activations(4, 0, "single", B, d, xdt)
    q_d = dev(q.reshape(d, qb), qdt)
    qt = torch.empty_like(q_d)
    _lib.larosa_prepare_rotation(q_d, qt, d, qb)
    xr, ok = guarded((B, d), torch.float32)
    _lib.larosa_rotate(dev(x, xdt), qt, qb, xr, B, d)
    torch.cuda.synchronize()
    bound, exact = rotation_bound(x, q)
    got = host(xr)
    assert np.all(np.abs(got - exact) <= bound)
    assert ref.rel_error(got, ref.rotate(x, q)) < 1e-5
    assert ok()


@pytest.mark.parametrize("dt,d,qb,B", [("bf16", 4096, 4096, 3), ("f32", 1024, 1024, 4),
                                        ("f32", 2048, 512, 7), ("bf16", 4096, 4096, 8)])
def test_batched_rotation_is_batch_invariant(dt, d, qb, B):
    """The few-token form sums each token in the one-token kernel's order:
    every token's x_rot equals its own one-token call bit for bit."""
    q = wl.rotation(4, 2, "single", d, qb, dt)
    x = wl.heavy_tailed_activations(4, 2, "single", B, d, dt)
    q_d = dev(q.reshape(d, qb), dt)
    qt = torch.empty_like(q_d)
    _lib.larosa_prepare_rotation(q_d, qt, d, qb)
    x_d = dev(x, dt)
    xr = torch.empty((B, d), device="cuda")
    _lib.larosa_rotate(x_d, qt, qb, xr, B, d)
    one = torch.empty((B, d), device="cuda")
    for b in range(B):
        _lib.larosa_rotate(x_d[b:b + 1], qt, qb, one[b:b + 1], 1, d)
    torch.cuda.synchronize()
    assert torch.equal(xr, one)


def test_rotate_exact_for_signed_permutation_and_identity():
    rng = np.random.default_rng(3)
    d = 2048
    x = wl.quantize(rng.standard_normal((3, d)), "bf16")
    perm, sign = wl.signed_permutation(rng, d)
    p = np.zeros((d, d))
    p[np.arange(d), perm] = sign
    for q in (p, np.eye(d)):
        q_d = dev(q, "bf16")
        qt = torch.empty_like(q_d)
        _lib.larosa_prepare_rotation(q_d, qt, d, d)
        xr = torch.empty((3, d), device="cuda")
        _lib.larosa_rotate(dev(x, "bf16"), qt, d, xr, 3, d)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_f32(xr), ref.rotate(x, q[None]))


def test_prepare_rotation_is_a_blockwise_transpose():
    q = wl.rotation(4, 1, "single", 640, 128, "bf16")
    q_d = dev(q.reshape(640, 128), "bf16")
    qt = torch.empty_like(q_d)
    _lib.larosa_prepare_rotation(q_d, qt, 640, 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(qt).reshape(5, 128, 128), np.transpose(q, (0, 2, 1)))


# -------------------------------------------------------------------- fold --

@pytest.mark.parametrize("dt,d,qb,n", [("bf16", 512, 128, 264), ("f32", 512, 512, 1536),
                                        ("bf16", 2752 * 2, 2752, 136)])
def test_fold_within_one_ulp(dt, d, qb, n):
    q = wl.rotation(5, 0, "single", d, qb, dt)
    w = wl.gaussian_weight(5, 0, "single", d, n, 0.02, dt)
    lin = RotatedLinear(q, w, dt, k=1)
    torch.cuda.synchronize()
    got = host(lin.Wf)
    exact = ref.fold_exact(q, w)
    absum = ref.fold_exact(np.abs(q), np.abs(w))
    if dt == "bf16":
        # fp32 accumulation then one bf16 rounding, against the once-rounded
        # exact value: at most one bf16 spacing apart, plus the fp32 sum's own
        # error (which dominates only where the folded value cancels to
        # near zero).
        want = ref.fold(q, w, "bf16")
        diff = np.abs(got - want)
        spacing = np.maximum(ulp_bf16(want), ulp_bf16(got))
        assert np.all(diff <= spacing + gamma(qb) * absum)
        assert np.mean(diff == 0) > 0.99
    else:
        assert np.all(np.abs(got - exact) <= gamma(qb) * absum + ulp_f32(exact) / 2)


def test_fold_exact_for_identity_and_signed_permutation():
    rng = np.random.default_rng(8)
    d, n = 256, 72
    w = wl.quantize(rng.standard_normal((d, n)), "bf16")
    perm, sign = wl.signed_permutation(rng, d)
    p = np.zeros((d, d))
    p[np.arange(d), perm] = sign
    for q in (np.eye(d), p):
        lin = RotatedLinear(q[None], w, "bf16", k=1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(lin.Wf), ref.fold(q[None], w, "bf16"))


# ------------------------------------------------------------------ gather --

def _gather_ws(B, d_in, d_out, k):
    n = _lib.larosa_workspace_bytes(B, d_in, d_out, k)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("dt,d_in,d_out,k", [("bf16", 4096, 22016, 2457), ("bf16", 11008, 4096, 6604),
                                              ("f32", 512, 1536, 307), ("bf16", 1000, 1544, 1),
                                              ("bf16", 300, 8, 300)])
def test_sparse_gemv_parity(dt, d_in, d_out, k):
    rng = np.random.default_rng(d_in + d_out)
    w = wl.quantize(rng.standard_normal((d_in, d_out)) * 0.02, dt)
    xr = make_x_rot("heavy", 1, d_in, seed=k)
    idx = ref.select(xr, k)
    val = np.take_along_axis(xr, idx, axis=1)
    y, ok = guarded((1, d_out), torch.float32 if dt == "f32" else torch.bfloat16)
    ws = _gather_ws(1, d_in, d_out, k)
    args = (torch.from_numpy(idx[0].astype(np.int32)).cuda(), None, k,
            torch.from_numpy(val[0]).cuda(), dev(w, dt))
    _lib.larosa_sparse_gemv(*args, y, 1, d_in, d_out, ws)
    y2 = torch.empty_like(y)
    _lib.larosa_sparse_gemv(*args, y2, 1, d_in, d_out, ws)   # counters were left at zero
    torch.cuda.synchronize()
    want = ref.round_to(ref.gather_product(xr, idx, w), dt)
    tol = 1e-5 if dt == "f32" else 2e-2
    assert ref.rel_error(host(y), want) <= tol
    assert torch.equal(y, y2)
    assert ok()


TOPK_GEMV_CASES = [
    # (weight dtype, d_in, d_out, k, activation kind)
    ("bf16", 4096, 22016, 2457, "heavy"), ("bf16", 11008, 4096, 6604, "gauss"),
    ("f32", 512, 1536, 307, "heavy"), ("bf16", 16384, 520, 9000, "heavy"),
    ("bf16", 1000, 1544, 1, "gauss"), ("bf16", 300, 8, 300, "heavy"),
    ("bf16", 4100, 2056, 1700, "ties"), ("bf16", 12288, 1032, 6000, "ties"),
    ("bf16", 2048, 11008, 2047, "gauss"),
]


@pytest.mark.parametrize("dt,d_in,d_out,k,kind", TOPK_GEMV_CASES)
def test_topk_gemv_selection_exact_and_product_within_tolerance(dt, d_in, d_out, k, kind):
    """The one-token selection folded into the product: the kept index list
    equals the oracle's selection bit for bit (ties included), the output is
    within tolerance of the oracle's product over those rows, and a second
    call on the same workspace gives identical bits."""
    rng = np.random.default_rng(d_in * 7 + k)
    w = wl.quantize(rng.standard_normal((d_in, d_out)) * 0.02, dt)
    xr = make_x_rot(kind, 1, d_in, seed=d_in + k)
    ydt = torch.float32 if dt == "f32" else torch.bfloat16
    y, ok_y = guarded((d_out,), ydt)
    idx, ok_i = guarded((k,), torch.int32, fill=-5)
    ws = _gather_ws(1, d_in, d_out, k)
    xr_d = torch.from_numpy(xr[0]).cuda()
    w_d = dev(w, dt)
    _lib.larosa_topk_gemv(xr_d, d_in, k, w_d, y, d_out, idx_out=idx, ws=ws)
    y2 = torch.empty_like(y)
    _lib.larosa_topk_gemv(xr_d, d_in, k, w_d, y2, d_out, ws=ws)
    torch.cuda.synchronize()
    assert ok_y() and ok_i()
    want_idx = ref.select(xr, k)
    np.testing.assert_array_equal(host(idx)[None, :], want_idx)
    want = ref.round_to(ref.gather_product(xr, want_idx, w), dt)
    assert ref.rel_error(host(y)[None, :], want) <= (1e-5 if dt == "f32" else 2e-2)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("B,d_in,d_out,k", [(16, 4096, 22016, 2457), (40, 4096, 1032, 1000),
                                             (64, 2048, 4104, 1024), (17, 11008, 4096, 6604)])
def test_sparse_gemv_batched_union_parity(B, d_in, d_out, k):
    """The product over the row union of a batch (packed coefficients, the
    count on the device), against each token's product over its own kept
    rows."""
    rng = np.random.default_rng(B * d_out + k)
    w = wl.quantize(rng.standard_normal((d_in, d_out)) * 0.02, "bf16")
    xr = make_x_rot("heavy", B, d_in, seed=k + B)
    idx = ref.select(xr, k)
    u = ref.row_union(idx)
    xs = ref.sparsify(xr, idx)
    coef = np.ascontiguousarray(xs[:, u].T.astype(np.float32))
    max_rows = min(d_in, B * k)
    rows = np.full(max_rows, -7, dtype=np.int32)
    rows[:len(u)] = u
    coef_full = np.zeros((max_rows, B), dtype=np.float32)
    coef_full[:len(u)] = coef
    n_dev = torch.tensor([len(u)], dtype=torch.int32, device="cuda")
    y, ok = guarded((B, d_out), torch.bfloat16)
    ws = _gather_ws(B, d_in, d_out, k)
    args = (torch.from_numpy(rows).cuda(), n_dev, max_rows, torch.from_numpy(coef_full).cuda(),
            dev(w, "bf16"))
    _lib.larosa_sparse_gemv(*args, y, B, d_in, d_out, ws)
    y2 = torch.empty_like(y)
    _lib.larosa_sparse_gemv(*args, y2, B, d_in, d_out, ws)
    torch.cuda.synchronize()
    want = ref.round_to(ref.gather_product(xr, idx, w), "bf16")
    assert ref.rel_error(host(y), want) <= 2e-2
    assert torch.equal(y, y2)
    assert ok()


@pytest.mark.parametrize("B", [3, 16, 64])
def test_sparse_gemv_small_integers_are_bit_exact_and_bounds_checked(B):
    """Integer weights and coefficients make every summation order exact, so
    the fp32 output must equal the oracle exactly. Row entries outside
    [0, d_in) and entries past the device-side count contribute nothing."""
    rng = np.random.default_rng(21 + B)
    d_in, d_out = 700, 2056
    w = rng.integers(-64, 65, (d_in, d_out)).astype(np.float64)
    rows = np.array(sorted(rng.choice(d_in, 200, replace=False)), dtype=np.int32)
    rows_bad = np.concatenate([rows[:150], [-1, d_in, 10 ** 6], rows[150:]]).astype(np.int32)
    coef = rng.integers(-9, 10, (len(rows_bad), B)).astype(np.float32)
    n_dev = torch.tensor([len(rows_bad) - 10], dtype=torch.int32, device="cuda")
    # The vector form (B < 16) is checked on an fp32 output. The matrix-core
    # form writes bf16 only: its fp32 sums are exact too (integers below 2^24),
    # so the output must be the bf16 rounding of the exact sum.
    ydt = torch.float32 if B < 16 else torch.bfloat16
    y = torch.empty((B, d_out), device="cuda", dtype=ydt)
    ws = _gather_ws(B, d_in, d_out, d_in)
    _lib.larosa_sparse_gemv(torch.from_numpy(rows_bad).cuda(), n_dev, len(rows_bad),
                            torch.from_numpy(coef).cuda(), dev(w, "bf16"), y, B, d_in, d_out, ws)
    torch.cuda.synchronize()
    used = len(rows_bad) - 10
    want = np.zeros((B, d_out))
    for j in range(used):
        r = rows_bad[j]
        if 0 <= r < d_in:
            want += coef[j][:, None].astype(np.float64) * w[r][None, :]
    np.testing.assert_array_equal(host(y), want if B < 16 else ref.round_to(want, "bf16"))


@pytest.mark.parametrize("dt,B,d_in,d_out", [("bf16", 1, 4096, 11008), ("f32", 2, 512, 1536),
                                              ("bf16", 8, 1024, 520), ("bf16", 16, 1024, 520),
                                              ("bf16", 64, 4096, 1032), ("bf16", 33, 300, 8)])
def test_dense_gemv_parity(dt, B, d_in, d_out):
    rng = np.random.default_rng(B * d_in)
    w = wl.quantize(rng.standard_normal((d_in, d_out)) * 0.02, dt)
    x = wl.quantize(rng.standard_normal((B, d_in)), dt)
    y = torch.empty((B, d_out), device="cuda", dtype=torch.float32 if dt == "f32" else torch.bfloat16)
    _lib.larosa_dense_gemv(dev(x, dt), dev(w, dt), y, B, d_in, d_out, _gather_ws(B, d_in, d_out, 1))
    torch.cuda.synchronize()
    want = ref.round_to(x @ w, dt)
    assert ref.rel_error(host(y), want) <= (1e-5 if dt == "f32" else 2e-2)


def test_swiglu_within_one_ulp():
    rng = np.random.default_rng(4)
    B, f = 3, 11008
    gu = wl.quantize(rng.standard_normal((B, 2 * f)) * 3, "bf16")
    h = torch.empty((B, f), dtype=torch.bfloat16, device="cuda")
    _lib.larosa_swiglu(dev(gu, "bf16"), h, B, f)
    torch.cuda.synchronize()
    want = ref.swiglu(gu, f, "bf16")
    assert np.all(np.abs(host(h) - want) <= ulp_bf16(want) * 1.0001)
