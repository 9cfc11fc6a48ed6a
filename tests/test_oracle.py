"""Pins for the CPU oracle: checked against hand-worked examples, closed forms,
invariants and brute force, never against the oracle itself.

Each check is chosen so that a plausible slip in the oracle (a transposed
operand, a sign, a dropped term, the wrong tie order) fails at least one of
them; ``test_pins_catch_planted_mistakes`` plants such slips in copies of the
oracle's steps and confirms the pins reject them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import larosa_ref as ref
from rotated_top_activation_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(vals):
    return np.array([float(v) for v in vals], dtype=np.float32)


# ---------------------------------------------------------------- golden ----

def test_worked_example_rotation_fold_select_product():
    g = _load("worked_example_4x3.json")
    q = np.array(g["Q"])[None]          # one dense 4×4 block
    x = np.array([g["x"]])
    w = np.array(g["W"])
    x_rot = ref.rotate(x, q)
    np.testing.assert_array_equal(x_rot[0], _f32(g["x_rot"]))
    np.testing.assert_array_equal(ref.fold(q, w, "f32"), np.array(g["W_folded"]))
    for k_str, kept in g["kept"].items():
        k = int(k_str)
        idx = ref.select(x_rot, k)
        np.testing.assert_array_equal(idx[0], kept)
        y = ref.gather_product(x_rot, idx, ref.fold(q, w, "f32"))
        np.testing.assert_array_equal(y[0], g["y"][k_str])
        y2, _, _ = ref.linear(x, q, ref.fold(q, w, "f32"), k, "f32")
        np.testing.assert_array_equal(y2[0], g["y"][k_str])
    np.testing.assert_array_equal(g["y"]["4"], g["dense_xW"])
    for p, k in g["sparsity_pct_to_k"].items():
        assert wl.k_for(4, int(p)) == k


def test_select_tie_fixtures():
    g = _load("select_ties.json")
    for case in g["cases"]:
        x = _f32(case["x_rot"])
        for k_str, kept in case["kept"].items():
            assert list(ref.select_row(x, int(k_str))) == kept, (case["why"], k_str)
            assert list(ref.select_row_by_rank(x, int(k_str))) == kept


def test_k_counts_of_the_workloads():
    # 512 channels at 40% keep 307 (the single-linear workload's stated K).
    assert wl.k_for(512, 40) == 307
    assert wl.k_for(4096, 40) == 2457
    assert wl.k_for(11008, 40) == 6604
    assert wl.k_for(28672, 50) == 14336
    assert wl.k_for(4096, 0) == 4096


# ------------------------------------------------------- number formats ----

def test_round_bf16_against_library_cast_and_halfway_cases():
    import torch
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -1e-42, 3.0e38, -3.3e38]]).astype(np.float32)
    # from fp32 inputs the library cast rounds once, so it must agree exactly
    lib = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ref.round_bf16(v.astype(np.float64)), lib)
    # halfway cases go to the even neighbour
    assert ref.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert ref.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert ref.round_bf16(np.array([-(1 + 2 ** -8)]))[0] == -1.0
    # one rounding from fp64: just above halfway rounds up (a detour through
    # fp32 would land exactly on halfway and round down)
    assert ref.round_bf16(np.array([1 + 2 ** -8 + 2 ** -30]))[0] == 1 + 2 ** -7
    assert np.isinf(ref.round_bf16(np.array([3.4e38]))[0])


def test_magnitude_key_rejects_nan_and_orders_like_abs():
    with pytest.raises(ValueError):
        ref.magnitude_key(np.array([1.0, np.nan], dtype=np.float32))
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(5000) * 1e3).astype(np.float32)
    k = ref.magnitude_key(v)
    a = np.abs(v.astype(np.float64))
    order_k = np.argsort(k, kind="stable")
    order_a = np.argsort(a, kind="stable")
    np.testing.assert_array_equal(order_k, order_a)


# -------------------------------------------------------------- rotation ----

@pytest.mark.parametrize("d,qb", [(512, 512), (256, 64), (96, 32)])
def test_generated_rotation_is_orthogonal_and_reproducible(d, qb):
    q = wl.rotation_fp64(9, 0, "single", d, qb)
    for blk in q:
        assert np.max(np.abs(blk @ blk.T - np.eye(qb))) <= 1e-12
        assert np.max(np.abs(blk.T @ blk - np.eye(qb))) <= 1e-12
    q2 = wl.rotation_fp64(9, 0, "single", d, qb)
    assert q.tobytes() == q2.tobytes()
    q3 = wl.rotation_fp64(9, 1, "single", d, qb)
    assert q.tobytes() != q3.tobytes()


def test_rotation_preserves_norm_and_block_structure():
    q = wl.rotation_fp64(9, 0, "single", 96, 32)
    x = np.random.default_rng(1).standard_normal((3, 96))
    xr = ref.rotate_exact(x, q)
    np.testing.assert_allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-13)
    # a block only mixes its own channels: changing block 1's input leaves
    # blocks 0 and 2 of the output untouched
    x2 = x.copy()
    x2[:, 32:64] += 1.0
    xr2 = ref.rotate_exact(x2, q)
    np.testing.assert_array_equal(xr[:, :32], xr2[:, :32])
    np.testing.assert_array_equal(xr[:, 64:], xr2[:, 64:])
    assert not np.array_equal(xr[:, 32:64], xr2[:, 32:64])
    dense = ref.dense_rotation(q)
    np.testing.assert_allclose(xr, x @ dense, rtol=0, atol=1e-12)


def test_identity_and_signed_permutation_rotations_are_exact():
    rng = np.random.default_rng(5)
    d = 64
    x = wl.quantize(rng.standard_normal((2, d)), "f32")
    np.testing.assert_array_equal(ref.rotate(x, np.eye(d)[None]), x.astype(np.float32))
    perm, sign = wl.signed_permutation(rng, d)
    p = np.zeros((d, d))
    p[np.arange(d), perm] = sign                # row i has sign[i] at column perm[i]
    # (x·P)[perm[i]] = sign[i]·x[i]
    want = np.empty_like(x)
    want[:, perm] = x * sign[None, :]
    np.testing.assert_array_equal(ref.rotate(x, p[None]), want.astype(np.float32))


# ------------------------------------------------------------------ fold ----

def test_fold_identity_recovers_dense_product():
    q = wl.rotation_fp64(9, 0, "single", 256, 64)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256))
    w = rng.standard_normal((256, 48))
    lhs = ref.rotate_exact(x, q) @ ref.fold_exact(q, w)
    rhs = x @ w
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


def test_fold_with_identity_and_signed_permutation_is_exact():
    rng = np.random.default_rng(6)
    d, n = 32, 24
    w = wl.quantize(rng.standard_normal((d, n)), "bf16")
    np.testing.assert_array_equal(ref.fold(np.eye(d)[None], w, "bf16"), w)
    perm, sign = wl.signed_permutation(rng, d)
    p = np.zeros((d, d))
    p[np.arange(d), perm] = sign
    # Pᵀ·W: row perm[i] of the result is sign[i]·W[i]
    want = np.empty_like(w)
    want[perm] = w * sign[:, None]
    np.testing.assert_array_equal(ref.fold(p[None], w, "bf16"), want)


# ---------------------------------------------------------------- select ----

def _exhaustive_topk(key, k):
    """The unique k-subset S with every kept entry beating every dropped one."""
    d = len(key)
    found = []
    for s in itertools.combinations(range(d), k):
        ss = set(s)
        ok = all(key[i] > key[j] or (key[i] == key[j] and i < j)
                 for i in ss for j in range(d) if j not in ss)
        if ok:
            found.append(list(s))
    assert len(found) == 1
    return found[0]


def test_select_matches_exhaustive_subsets_on_tiny_tie_heavy_inputs():
    rng = np.random.default_rng(11)
    for trial in range(250):
        d = int(rng.integers(1, 9))
        mags = rng.integers(0, 4, d).astype(np.float32)     # many ties
        signs = np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
        x = mags * signs                                    # includes ±0
        if trial % 7 == 0:
            x[rng.integers(0, d)] = np.float32(np.inf) * signs[0]
        key = ref.magnitude_key(x)
        for k in range(1, d + 1):
            want = _exhaustive_topk(list(key), k)
            assert list(ref.select_row(x, k)) == want
            assert list(ref.select_row_by_rank(x, k)) == want


def test_select_special_cases_and_invariants():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(1000) * np.exp(rng.standard_normal(1000))).astype(np.float32)
    key = ref.magnitude_key(x)
    assert list(ref.select_row(x, 1000)) == list(range(1000))
    assert list(ref.select_row(x, 1)) == [int(np.argmax(key))]   # first maximum
    same = np.full(50, -2.5, dtype=np.float32)
    assert list(ref.select_row(same, 17)) == list(range(17))
    for k in (1, 7, 300, 600, 999):
        idx = ref.select_row(x, k)
        assert len(idx) == k and np.all(np.diff(idx) > 0)
        mask = np.zeros(1000, bool)
        mask[idx] = True
        assert key[mask].min() >= key[~mask].max()
        np.testing.assert_array_equal(idx, ref.select_row_by_rank(x, k))
    with pytest.raises(ValueError):
        ref.select_row(x, 0)
    with pytest.raises(ValueError):
        ref.select_row(x, 1001)


def test_sparsify_keeps_values_unscaled_and_zeroes_the_rest():
    x = _f32([0.5, -1.5, 3.5, -0.5])[None]
    xs = ref.sparsify(x, np.array([[1, 2]]))
    np.testing.assert_array_equal(xs[0], [0.0, -1.5, 3.5, 0.0])


def test_union_is_set_union_and_batch_invariant():
    rng = np.random.default_rng(13)
    x_rot = rng.standard_normal((5, 40)).astype(np.float32)
    idx = ref.select(x_rot, 13)
    u = ref.row_union(idx)
    assert set(u.tolist()) == set().union(*[set(r.tolist()) for r in idx])
    assert np.all(np.diff(u) > 0)
    w = np.round(rng.standard_normal((40, 6)) * 8)       # small integers: exact sums
    xi = np.round(x_rot * 16).astype(np.float32)
    y = ref.gather_product(xi, ref.select(xi, 13), w)
    for b in range(5):
        yb = ref.gather_product(xi[b:b + 1], ref.select(xi[b:b + 1], 13), w)
        np.testing.assert_array_equal(y[b], yb[0])


# --------------------------------------------------------------- product ----

def test_product_one_hot_and_small_integers_are_exact():
    rng = np.random.default_rng(14)
    w = wl.quantize(rng.standard_normal((30, 9)), "bf16")
    x = np.zeros((1, 30), np.float32)
    x[0, 17] = -3.25
    y = ref.gather_product(x, np.array([[17]]), w)
    np.testing.assert_array_equal(y[0], -3.25 * w[17])
    xi = rng.integers(-20, 21, (2, 30)).astype(np.float32)
    wi = rng.integers(-50, 51, (30, 9)).astype(np.float64)
    idx = np.array([[0, 3, 4, 29], [1, 2, 3, 4]])
    y = ref.gather_product(xi, idx, wi)
    for b in range(2):
        want = sum(float(xi[b, i]) * wi[i] for i in idx[b])
        np.testing.assert_array_equal(y[b], want)


def test_full_k_reproduces_the_dense_product():
    """K = d keeps every rotated channel, so the sparse linear equals x·W up to
    the fp32 rounding of x_rot and the rounding of W' and y."""
    q = wl.rotation_fp64(9, 0, "single", 128, 128)
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 128))
    w = rng.standard_normal((128, 40)) / np.sqrt(128)
    y, _, _ = ref.linear(x, q, ref.fold_exact(q, w), 128, "f32")
    dense = x @ w
    assert ref.rel_error(y, dense) < 2e-6
    yb, _, _ = ref.linear(x, wl.quantize(q, "bf16"),
                          ref.fold(wl.quantize(q, "bf16"), w, "bf16"), 128, "bf16")
    assert ref.rel_error(yb, dense) < 2e-2


# ------------------------------------------------------------ activation ----

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    s = ref.silu(np.array([0.0, ln3, -ln3, 40.0, -40.0]))
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * ln3) < 1e-15
    assert abs(s[2] + 0.25 * ln3) < 1e-15
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15
    z = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(ref.silu(z) - ref.silu(-z), z, atol=1e-14)
    gu = np.array([[ln3, 0.0, 2.0, 5.0]])
    h = ref.swiglu(gu, 2, "f32")
    np.testing.assert_allclose(h[0], [0.75 * ln3 * 2.0, 0.0], rtol=1e-7)


def _mlp_fixture():
    g = _load("mlp_worked_example.json")
    x = np.array([g["x"]])
    q1 = np.array(g["Q1"])[None]
    q2 = np.array(g["Q2"])[None]
    wgu = np.array(g["W_gate_up_folded"])
    wd = np.array(g["W_down_folded"])
    return g, x, q1, wgu, q2, wd


def test_mlp_worked_example_f32():
    """The MLP composition against the hand-worked closed forms (fp32
    activations): every intermediate is a multiple of ln 3."""
    g, x, q1, wgu, q2, wd = _mlp_fixture()
    ln3 = math.log(3.0)
    y, st = ref.mlp(x, q1, wgu, q2, wd, g["k1"], g["k2"], g["f"], act_dtype="f32")
    c = g["f32"]
    np.testing.assert_array_equal(st["x_rot1"][0], _f32(g["x_rot1"]))
    assert list(st["idx1"][0]) == g["idx1"]
    np.testing.assert_allclose(st["gu"][0, :2], np.array(c["gate_up_over_ln3"]) * ln3, rtol=1e-7)
    np.testing.assert_array_equal(st["gu"][0, 2:], c["up"])
    np.testing.assert_allclose(st["h"][0], np.array(c["h_over_ln3"]) * ln3, rtol=1e-6)
    np.testing.assert_allclose(st["x_rot2"][0], np.array(c["x_rot2_over_ln3"]) * ln3, rtol=1e-6)
    assert list(st["idx2"][0]) == g["idx2"]
    np.testing.assert_allclose(y[0], np.array(c["y_over_ln3"]) * ln3, rtol=1e-6)


def test_mlp_worked_example_bf16():
    """bf16 activations: every value in the fixture is a bf16 number, so the
    oracle must reproduce each exactly, including y[0], which depends on h
    being rounded to bf16 before the down linear."""
    g, x, q1, wgu, q2, wd = _mlp_fixture()
    y, st = ref.mlp(x, q1, wgu, q2, wd, g["k1"], g["k2"], g["f"], act_dtype="bf16")
    c = g["bf16"]
    np.testing.assert_array_equal(st["gu"][0], c["gate_up"])
    np.testing.assert_array_equal(st["h"][0], c["h"])
    np.testing.assert_array_equal(st["x_rot2"][0], _f32(c["x_rot2"]))
    assert list(st["idx1"][0]) == g["idx1"] and list(st["idx2"][0]) == g["idx2"]
    np.testing.assert_array_equal(y[0], c["y"])


def test_mlp_pins_catch_planted_mistakes():
    """Plausible slips in the MLP composition each fail the bf16 fixture."""
    g, x, q1, wgu, q2, wd = _mlp_fixture()
    f, k1, k2 = g["f"], g["k1"], g["k2"]
    want = np.array(g["bf16"]["y"])
    gu, _, _ = ref.linear(x, q1, wgu, k1, "bf16")
    h = ref.swiglu(gu, f, "bf16")
    # gate|up rows fed to the down linear instead of h (the slice takes gate)
    y_bad, _, _ = ref.linear(gu[:, :f], q2, wd, k2, "bf16")
    assert not np.array_equal(y_bad[0], want)
    # the gate|up linear's K reused for the down linear
    y_bad, _, _ = ref.linear(h, q2, wd, k1, "bf16")
    assert not np.array_equal(y_bad[0], want)
    # h left unrounded between the linears
    h_raw = ref.silu(gu[:, :f]) * gu[:, f:]
    y_bad, _, _ = ref.linear(h_raw, q2, wd, k2, "bf16")
    assert not np.array_equal(y_bad[0], want)
    np.testing.assert_array_equal(y_bad[0], g["bf16"]["y_if_h_unrounded"])
    # SiLU applied to up instead of gate
    h_swap = ref.round_to(ref.silu(gu[:, f:]) * gu[:, :f], "bf16")
    y_bad, _, _ = ref.linear(h_swap, q2, wd, k2, "bf16")
    assert not np.array_equal(y_bad[0], want)
    # the down linear run with the gate|up rotation's transpose convention (x·Qᵀ)
    xr_bad = ref.round_f32(h @ q2[0].T)
    idx_bad = ref.select(xr_bad, k2)
    y_bad = ref.round_to(ref.gather_product(xr_bad, idx_bad, wd), "bf16")
    assert not np.array_equal(y_bad[0], want)
    # the correct composition, for contrast
    y_ok, _, _ = ref.linear(h, q2, wd, k2, "bf16")
    np.testing.assert_array_equal(y_ok[0], want)


def test_rel_error_metric():
    y = np.array([1.0, -2.0, 0.0, 1e-9])
    assert ref.rel_error(y, y) == 0.0
    rms = math.sqrt((1 + 4) / 4)
    assert abs(ref.rel_error(y + np.array([0, 0, 0.01, 0]), y) - 0.01 / rms) < 1e-15


# ------------------------------------------------------ planted mistakes ----

def test_pins_catch_planted_mistakes():
    """Copies of oracle steps with one plausible slip each must fail a pin."""
    g = _load("worked_example_4x3.json")
    q = np.array(g["Q"])
    x = np.array(g["x"])
    w = np.array(g["W"])
    # rotation by Qᵀ instead of Q
    assert not np.array_equal(x @ q.T, g["x_rot"])
    # fold by Q·W instead of Qᵀ·W
    assert not np.array_equal(q @ w, g["W_folded"])
    # selection on signed value instead of magnitude
    xr = _f32(g["x_rot"])
    assert sorted(np.argsort(-xr, kind="stable")[:2]) != g["kept"]["2"]
    # highest index wins among ties
    key = ref.magnitude_key(xr)
    bad = np.sort(np.lexsort((-np.arange(4), -key))[:3])
    assert list(bad) != g["kept"]["3"]
    # the product dropping the last kept row
    rows = g["kept"]["3"][:-1]
    assert not np.array_equal(xr[rows] @ np.array(g["W_folded"])[rows], g["y"]["3"])
    # a sign slip in SiLU
    ln3 = math.log(3.0)
    assert abs(ln3 / (1 + math.exp(ln3)) - 0.75 * ln3) > 0.1


# ------------------------------------------------- threshold and low rank ----

def test_threshold_worked_example():
    g = _load("threshold_lowrank_example.json")
    x = _f32(g["threshold"]["x_rot"])
    for t, kept in g["threshold"]["kept"].items():
        assert list(ref.threshold_select_row(x, float(t))) == kept, t
    c = g["calibration"]
    xc = np.array(c["x_rot"], dtype=np.float32)
    for p, t in c["t"].items():
        assert ref.calibrate_threshold(xc, int(p)) == np.float32(t), p
    sel = ref.threshold_select(xc, ref.calibrate_threshold(xc, 50))
    assert [list(s) for s in sel] == c["kept_at_p50"]


def test_calibrated_threshold_brute_force_and_top_k_agreement():
    rng = np.random.default_rng(11)
    for trial in range(40):
        n_tok, d = int(rng.integers(1, 4)), int(rng.integers(1, 40))
        # small integers: many ties
        xc = rng.integers(-4, 5, (n_tok, d)).astype(np.float32)
        for p in (0, 10, 40, 50, 90):
            n = n_tok * d
            k_total = n * (100 - p) // 100
            if k_total < 1:
                with pytest.raises(ValueError):
                    ref.calibrate_threshold(xc, p)
                continue
            t = ref.calibrate_threshold(xc, p)
            mags = np.abs(xc.astype(np.float64)).reshape(-1)
            # characterisation: fewer than K_total entries are above t, and
            # at least K_total are at or above it; t is one of the magnitudes
            assert (mags > t).sum() < k_total <= (mags >= t).sum()
            assert t in mags
            kept = sum(len(s) for s in ref.threshold_select(xc, t))
            assert kept == (mags >= t).sum()
            if n_tok == 1:
                # one calibration token: the threshold keeps the Top-K set,
                # plus every channel tied with the K-th magnitude
                topk = set(ref.select_row(xc[0], k_total).tolist())
                thr = set(ref.threshold_select_row(xc[0], t).tolist())
                assert topk <= thr
                assert all(abs(xc[0, i]) == t for i in thr - topk)
    # without ties the two selections coincide
    x = rng.standard_normal(4096).astype(np.float32)
    t = ref.calibrate_threshold(x[None], 40)
    np.testing.assert_array_equal(ref.threshold_select_row(x, t), ref.select_row(x, 2457))


def test_threshold_special_cases():
    x = np.array([0.0, -0.0, 1.0, -np.inf, np.inf, 3.0], dtype=np.float32)
    assert list(ref.threshold_select_row(x, 0.0)) == [0, 1, 2, 3, 4, 5]
    assert list(ref.threshold_select_row(x, -0.0)) == [0, 1, 2, 3, 4, 5]
    assert list(ref.threshold_select_row(x, np.inf)) == [3, 4]
    assert list(ref.threshold_select_row(x, 3.0)) == [3, 4, 5]
    assert list(ref.threshold_select_row(x[:3], 2.0)) == []
    for bad in (-1.0, np.nan):
        with pytest.raises(ValueError):
            ref.threshold_select_row(x, bad)
    # a larger threshold keeps a subset
    rng = np.random.default_rng(2)
    y = rng.standard_normal(500).astype(np.float32)
    a = set(ref.threshold_select_row(y, 0.5).tolist())
    b = set(ref.threshold_select_row(y, 0.8).tolist())
    assert b <= a and len(a) > len(b)


def test_lowrank_worked_example():
    g = _load("threshold_lowrank_example.json")["lowrank"]
    w = np.array(g["W_folded"])
    a1, b1 = ref.lowrank_factors(w, 1)
    np.testing.assert_allclose(a1 @ b1, g["rank1_product"], atol=1e-15)
    xr = _f32(g["x_rot"])[None]
    for r, y in g["y"].items():
        a, b = ref.lowrank_factors(w, int(r))
        got = ref.lowrank_compensated_product(xr, [np.array(g["kept"])], w, a, b)
        np.testing.assert_allclose(got[0], y, atol=1e-14)


def test_lowrank_factors_closed_forms():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((48, 30))
    sv = np.linalg.svd(w, compute_uv=False)
    for r in (0, 1, 7, 30):
        a, b = ref.lowrank_factors(w, r)
        assert a.shape == (48, r) and b.shape == (r, 30)
        # Eckart–Young: the residual's energy is the dropped singular values'
        res = np.sum((w - a @ b) ** 2)
        assert abs(res - np.sum(sv[r:] ** 2)) <= 1e-10 * np.sum(sv ** 2)
        # balanced factors: AᵀA = B·Bᵀ = Σ_r
        np.testing.assert_allclose(a.T @ a, np.diag(sv[:r]), atol=1e-10)
        np.testing.assert_allclose(b @ b.T, np.diag(sv[:r]), atol=1e-10)
    with pytest.raises(ValueError):
        ref.lowrank_factors(w, 31)


def test_lowrank_compensation_limits():
    rng = np.random.default_rng(8)
    d, n, k = 64, 40, 25
    w = rng.standard_normal((d, n))
    xr = rng.standard_normal((3, d)).astype(np.float32)
    idx = ref.select(xr, k)
    plain = ref.gather_product(xr, idx, w)
    dense = xr.astype(np.float64) @ w
    a0, b0 = ref.lowrank_factors(w, 0)
    np.testing.assert_array_equal(ref.lowrank_compensated_product(xr, idx, w, a0, b0), plain)
    af, bf = ref.lowrank_factors(w, n)  # full rank: the dense product
    np.testing.assert_allclose(ref.lowrank_compensated_product(xr, idx, w, af, bf), dense,
                               rtol=1e-12, atol=1e-12)
    # nothing dropped (K = d): the compensation adds exactly zero
    all_idx = ref.select(xr, d)
    a5, b5 = ref.lowrank_factors(w, 5)
    np.testing.assert_array_equal(ref.lowrank_compensated_product(xr, all_idx, w, a5, b5),
                                  ref.gather_product(xr, all_idx, w))
    # an exactly rank-5 weight is recovered by rank 5 for any selection
    w5 = rng.standard_normal((d, 5)) @ rng.standard_normal((5, n))
    a, b = ref.lowrank_factors(w5, 5)
    np.testing.assert_allclose(ref.lowrank_compensated_product(xr, idx, w5, a, b),
                               xr.astype(np.float64) @ w5, rtol=1e-10, atol=1e-10)
    # the error shrinks as the rank grows
    errs = [np.abs(ref.lowrank_compensated_product(xr, idx, w, *ref.lowrank_factors(w, r))
                   - dense).max() for r in (0, 10, 20, 40)]
    assert errs[0] > errs[1] > errs[2] > errs[3]


def test_threshold_and_lowrank_pins_catch_planted_mistakes():
    g = _load("threshold_lowrank_example.json")
    x = _f32(g["threshold"]["x_rot"])
    # strict > instead of >= drops the channels equal to t
    key = ref.magnitude_key(x)
    tk = ref.threshold_key(1.0)
    assert list(np.nonzero(key > tk)[0]) != g["threshold"]["kept"]["1.0"]
    # calibration taking the K_total-th smallest instead of largest
    xc = np.array(g["calibration"]["x_rot"], dtype=np.float32)
    mk = np.sort(ref.magnitude_key(xc.reshape(-1)))
    wrong = np.array(mk[2 - 1], dtype=np.uint32).view(np.float32)  # p = 75: K_total = 2
    assert wrong != np.float32(g["calibration"]["t"]["75"])
    # compensating the kept part instead of the dropped one
    lr = g["lowrank"]
    w = np.array(lr["W_folded"])
    a, b = ref.lowrank_factors(w, 1)
    xr = _f32(lr["x_rot"])[None]
    xs = ref.sparsify(xr, [np.array(lr["kept"])])
    bad = ref.gather_product(xr, [np.array(lr["kept"])], w) + (xs @ a) @ b
    assert not np.allclose(bad[0], lr["y"]["1"])
    # B_r taken without the Σ^½ weight (U_r·V_rᵀ)
    u, sv, vt = np.linalg.svd(w)
    assert not np.allclose(u[:, :1] @ vt[:1], lr["rank1_product"])
