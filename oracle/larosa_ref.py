"""CPU oracle for the rotated Top-K sparse linear (LaRoSA decode path).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module. The product path
never calls it, and it imports nothing from the HIP path: it is written from
the method's definition, in float64 NumPy, one step at a time, so that a
reader can check each line against the pages.

Sources:
  [abstract]  "La RoSA: Enhancing LLM Efficiency via Layerwise Rotated Sparse
              Activation", abstract (PMLR 267 proceedings page; the same text
              is on the arXiv summary pages): a layerwise orthogonal rotation
              of each linear layer's input, then Top-K selection on the
              rotated activations; fixed K gives consistent model-level
              sparsity.
  [framework] the LaRoSA summary page (shd-paper.top), 方法详解 · 技术框架
              (method details, technical framework): stage 1 applies the
              orthogonal matrix to the layer's activation; stage 2 keeps the
              K entries of largest magnitude and sets the rest to zero.
  [design]    same page, 方法详解 · 关键设计 (key design): the rotation may be
              random or learned; the Top-K ratio sets the sparsity.
  [rsparse]   the R-Sparse summary page (R-Sparse: Rank-Aware Activation
              Sparsity, 研究流程与方法 · R-Sparse框架设计 (framework design)):
              input channels whose magnitude is below a threshold t(s) set by
              a sparsity budget s are masked; the masked remainder goes
              through a rank-r factorisation A_r·B_r of the weight taken from
              its SVD (A_r = U_r·Σ_r^½, B_r = Σ_r^½·V_rᵀ); the output is the
              sparse part plus that low-rank part.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * Folding: since Q·Qᵀ = I for an orthogonal Q, (x·Q)·(Qᵀ·W) = x·W, so the
    rotated input multiplies the folded weight W' = Qᵀ·W.
  * Selection runs on the fp32 rotated activation; the key of an entry is its
    fp32 bit pattern with the sign bit cleared (so |-0| = |+0| and ±inf rank
    highest); equal keys are broken by the lower index; NaN is rejected.
  * Selected values are kept unscaled; the indices are reported ascending.
  * With several tokens, each token selects its own K; the rows read are the
    union of the tokens' sets, which changes no token's result.

Shapes: x [B, d_in]; Q packed block-diagonal [d_in // b, b, b] (b = d_in is
one dense block); W, W' [d_in, d_out]; y [B, d_out].
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Number formats (written out here so the oracle owns its own rounding).


def round_f32(a) -> np.ndarray:
    """Round float64 values to float32 (IEEE round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even, in one step
    (no detour through float32). Returned as float64.

    bfloat16 has float32's exponent range and 8 significant bits; below the
    smallest normal (2^-126) the spacing is fixed at 2^-133.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, e = np.frexp(v)                      # v = m·2^e, 0.5 <= |m| < 1
    q = np.ldexp(1.0, np.maximum(e - 8, -133))   # spacing of bf16 values near v
    r = np.rint(v / q) * q                  # np.rint: halfway cases to even
    big = np.abs(r) > 3.3895313892515355e38  # beyond the largest finite bf16
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def round_to(a, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype ("f32" or "bf16"), as float64."""
    if dtype == "f32":
        return round_f32(a).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(a)
    raise ValueError(dtype)


def magnitude_key(x_rot_f32: np.ndarray) -> np.ndarray:
    """Selection key: the fp32 bit pattern with the sign bit cleared (int64).

    For finite and infinite fp32 values this orders exactly like |x|.
    """
    x = np.asarray(x_rot_f32, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN in the rotated activation: selection undefined")
    return (x.view(np.uint32) & np.uint32(0x7FFFFFFF)).astype(np.int64)


# ----------------------------------------------------------------------------
# The method's steps.


def dense_rotation(q_blocks: np.ndarray) -> np.ndarray:
    """Expand packed blocks [nb, b, b] into the dense block-diagonal [d, d]."""
    nb, b, _ = q_blocks.shape
    q = np.zeros((nb * b, nb * b))
    for c in range(nb):
        q[c * b:(c + 1) * b, c * b:(c + 1) * b] = q_blocks[c]
    return q


def rotate_exact(x: np.ndarray, q_blocks: np.ndarray) -> np.ndarray:
    """x·Q in float64 with no final rounding [framework, stage 1]."""
    x = np.asarray(x, dtype=np.float64)
    nb, b, _ = q_blocks.shape
    out = np.empty_like(x)
    for c in range(nb):
        out[:, c * b:(c + 1) * b] = x[:, c * b:(c + 1) * b] @ q_blocks[c]
    return out


def rotate(x: np.ndarray, q_blocks: np.ndarray) -> np.ndarray:
    """x_rot = fp32(x·Q): the product formed in float64, rounded once to fp32."""
    return round_f32(rotate_exact(x, q_blocks))


def fold_exact(q_blocks: np.ndarray, w: np.ndarray) -> np.ndarray:
    """W' = Qᵀ·W in float64 with no final rounding (the folding reading)."""
    w = np.asarray(w, dtype=np.float64)
    nb, b, _ = q_blocks.shape
    out = np.empty_like(w)
    for c in range(nb):
        out[c * b:(c + 1) * b] = q_blocks[c].T @ w[c * b:(c + 1) * b]
    return out


def fold(q_blocks: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """W' = Qᵀ·W, rounded once to the weight dtype."""
    return round_to(fold_exact(q_blocks, w), dtype)


def select_row(x_rot_row: np.ndarray, k: int) -> np.ndarray:
    """Top-K of one token [framework, stage 2]: the k indices of largest
    magnitude, lower index first among equal magnitudes, returned ascending.

    A stable sort on the descending key keeps equal keys in index order.
    """
    key = magnitude_key(x_rot_row)
    d = key.shape[0]
    if not 1 <= k <= d:
        raise ValueError(f"k={k} outside [1, {d}]")
    order = np.argsort(-key, kind="stable")
    return np.sort(order[:k]).astype(np.int32)


def select_row_by_rank(x_rot_row: np.ndarray, k: int) -> np.ndarray:
    """The same set by rank counting, O(d²): index i is kept iff fewer than k
    indices j beat it, where j beats i if key_j > key_i, or key_j == key_i
    and j < i."""
    key = magnitude_key(x_rot_row)
    d = key.shape[0]
    j = np.arange(d)
    beats = (key[None, :] > key[:, None]) | (
        (key[None, :] == key[:, None]) & (j[None, :] < j[:, None]))
    rank = beats.sum(axis=1)
    return np.nonzero(rank < k)[0].astype(np.int32)


def select(x_rot: np.ndarray, k: int) -> np.ndarray:
    """Per-token Top-K indices [B, k], each row ascending."""
    x_rot = np.asarray(x_rot, dtype=np.float32)
    return np.stack([select_row(x_rot[b], k) for b in range(x_rot.shape[0])])


def sparsify(x_rot: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """xs: the rotated values at the selected indices, unscaled; zero
    elsewhere [framework, stage 2]. Returned as float64 of the fp32 values."""
    x_rot = np.asarray(x_rot, dtype=np.float32)
    xs = np.zeros(x_rot.shape, dtype=np.float64)
    for b in range(x_rot.shape[0]):
        xs[b, idx[b]] = x_rot[b, idx[b]]
    return xs


def row_union(idx: np.ndarray) -> np.ndarray:
    """The ascending union of the tokens' selected indices: the weight rows a
    batched product has to read."""
    return np.unique(np.asarray(idx).reshape(-1)).astype(np.int32)


def gather_product(x_rot: np.ndarray, idx: np.ndarray,
                   w_folded: np.ndarray) -> np.ndarray:
    """y_b = Σ_{i ∈ S_b} x_rot[b, i] · W'[i, :] in float64 (unrounded).

    Only the selected rows of W' enter: the saving the abstract names
    (computation and memory transfers of the zeroed channels).
    """
    x_rot = np.asarray(x_rot, dtype=np.float32)
    w = np.asarray(w_folded, dtype=np.float64)
    y = np.zeros((x_rot.shape[0], w.shape[1]))
    for b in range(x_rot.shape[0]):
        rows = idx[b]
        y[b] = x_rot[b, rows].astype(np.float64) @ w[rows]
    return y


def linear(x: np.ndarray, q_blocks: np.ndarray, w_folded: np.ndarray, k: int,
           out_dtype: str):
    """One rotated sparse linear: rotate, select, product over the selected
    rows, round to the activation dtype. Returns (y, x_rot, idx)."""
    x_rot = rotate(x, q_blocks)
    idx = select(x_rot, k)
    y = round_to(gather_product(x_rot, idx, w_folded), out_dtype)
    return y, x_rot, idx


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z) in float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(gu: np.ndarray, f: int, out_dtype: str) -> np.ndarray:
    """h = SiLU(gate)·up for gu = [gate | up] ([B, 2F]), rounded to out_dtype."""
    gu = np.asarray(gu, dtype=np.float64)
    return round_to(silu(gu[:, :f]) * gu[:, f:2 * f], out_dtype)


def mlp(x, q1, w_gu_folded, q2, w_down_folded, k1: int, k2: int, f: int,
        act_dtype: str = "bf16"):
    """Rotated sparse SwiGLU MLP: gate|up = linear(x; Q1), h = SiLU(g)·u,
    y = linear(h; Q2). Returns y and the intermediates of both linears."""
    gu, xr1, idx1 = linear(x, q1, w_gu_folded, k1, act_dtype)
    h = swiglu(gu, f, act_dtype)
    y, xr2, idx2 = linear(h, q2, w_down_folded, k2, act_dtype)
    return y, dict(gu=gu, h=h, x_rot1=xr1, idx1=idx1, x_rot2=xr2, idx2=idx2)


# ----------------------------------------------------------------------------
# Variants next to the method's fixed Top-K (the contrast the pages draw).


def threshold_key(t) -> np.uint32:
    """The key a magnitude threshold t is compared with: fp32(t)'s bit
    pattern. t must be a non-negative number (−0 counts as 0)."""
    t32 = np.float32(t)
    if np.isnan(t32) or t32 < 0:
        raise ValueError(f"threshold {t!r} must be a non-negative number")
    return np.uint32(np.array(t32).view(np.uint32) & np.uint32(0x7FFFFFFF))


def calibrate_threshold(x_rot_calib: np.ndarray, sparsity_pct: int) -> np.float32:
    """t(s) [rsparse] from calibration activations: the K_total-th largest
    magnitude over all n entries, K_total = ⌊n·(100 − p)/100⌋ (the same floor
    rule as K). Keeping |x| ≥ t keeps K_total of the calibration entries, or
    more when the K_total-th magnitude is tied. Returned as the fp32 value."""
    key = magnitude_key(np.asarray(x_rot_calib, dtype=np.float32).reshape(-1))
    n = key.size
    k_total = n * (100 - int(sparsity_pct)) // 100
    if not 1 <= k_total <= n:
        raise ValueError(f"sparsity {sparsity_pct}% keeps {k_total} of {n} entries")
    kth = np.sort(key)[::-1][k_total - 1]
    return np.array(kth, dtype=np.uint32).view(np.float32)[()]


def threshold_select_row(x_rot_row: np.ndarray, t) -> np.ndarray:
    """Magnitude-threshold selection [rsparse]: the indices i with
    |x_rot[i]| ≥ t, ascending. How many are kept varies from token to token
    (the fluctuating sparsity [abstract] attributes to magnitude pruning)."""
    key = magnitude_key(x_rot_row)
    return np.nonzero(key >= threshold_key(t))[0].astype(np.int32)


def threshold_select(x_rot: np.ndarray, t) -> list:
    """Per-token threshold selections (a list of ascending index arrays)."""
    x_rot = np.asarray(x_rot, dtype=np.float32)
    return [threshold_select_row(x_rot[b], t) for b in range(x_rot.shape[0])]


def lowrank_factors(w_folded: np.ndarray, r: int):
    """A_r = U_r·Σ_r^½ [d_in, r] and B_r = Σ_r^½·V_rᵀ [r, d_out] from the SVD
    W' = U·Σ·Vᵀ [rsparse], so that A_r·B_r is the best rank-r approximation
    of W' (in the x·W orientation used here)."""
    w = np.asarray(w_folded, dtype=np.float64)
    if not 0 <= r <= min(w.shape):
        raise ValueError(f"rank {r} outside [0, {min(w.shape)}]")
    u, sv, vt = np.linalg.svd(w, full_matrices=False)
    root = np.sqrt(sv[:r])
    return u[:, :r] * root[None, :], root[:, None] * vt[:r]


def lowrank_compensated_product(x_rot: np.ndarray, idx, w_folded: np.ndarray,
                                a_r: np.ndarray, b_r: np.ndarray) -> np.ndarray:
    """y = xs·W' + (x_rot − xs)·(A_r·B_r) in float64 [rsparse]: the sparse
    product over the kept rows, plus the dropped remainder of the rotated
    input through the low-rank factors (first (x_rot − xs)·A_r, then ·B_r)."""
    xs = sparsify(x_rot, idx)
    dropped = np.asarray(x_rot, dtype=np.float32).astype(np.float64) - xs
    y_s = gather_product(x_rot, idx, w_folded)
    y_r = (dropped @ np.asarray(a_r, dtype=np.float64)) @ np.asarray(b_r, dtype=np.float64)
    return y_s + y_r


def rel_error(y_hat, y) -> float:
    """max_i |ŷ_i − y_i| / max(|y_i|, rms(y)): a relative error that stays
    meaningful where an output cancels to near zero."""
    y_hat = np.asarray(y_hat, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    rms = np.sqrt(np.mean(y * y)) if y.size else 0.0
    den = np.maximum(np.abs(y), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y_hat - y) / den)) if y.size else 0.0
