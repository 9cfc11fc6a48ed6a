"""Seeded synthetic inputs for the rotated Top-K sparse linear path.

This module only draws inputs: activations, weights, rotation matrices and
KV caches. It holds none of the method's arithmetic (no rotation, selection,
folding or product), so both the HIP path and the CPU oracle can be fed from
it without sharing any computation.

Every tensor comes from ``numpy.random.default_rng(SeedSequence([cfg, layer,
role, tensor, run_seed]))``. Values are returned as float64 arrays that are
exactly representable in the storage dtype ("f32" or "bf16"); ``to_torch``
turns them into device tensors of that dtype without any further rounding.

Shapes follow the x·W convention: x is [B, d_in], W is [d_in, d_out], so one
input channel of x owns one contiguous row of W.

Rotation matrices are random orthogonal blocks: the Q factor of the QR
decomposition of a Gaussian matrix, with column signs fixed so the diagonal
of R is positive. The LaRoSA summary page (方法详解 · 关键设计, "key design")
allows the rotation to be randomly initialised or learned; the random choice
is the one that needs no data. A block-diagonal rotation of width q_block is
stored packed as [d // q_block, q_block, q_block].
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

ROLE = {"single": 0, "attn_in": 0, "o_in": 1, "mlp_in": 2, "down_in": 3}
TENSOR = {"Q": 0, "W": 1, "x": 2, "scales": 3, "outliers": 4, "kv": 5, "perm": 6}


def rng_for(cfg: int, layer: int, role: str, tensor: str, run_seed: int = 0):
    """The generator for one (config, layer, role, tensor, run) key."""
    return np.random.default_rng(
        np.random.SeedSequence([cfg, layer, ROLE[role], TENSOR[tensor], run_seed]))


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round an input draw to the storage dtype; the result is float64.

    This is input quantisation (what the stored tensor holds), done with the
    library casts of numpy (fp32) and torch (bf16).
    """
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(
            torch.float64).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def haar_block(rng, n: int) -> np.ndarray:
    """One n×n random orthogonal matrix (float64): QR of N(0,1), sign-fixed."""
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


@functools.lru_cache(maxsize=16)
def _haar_blocks_cached(cfg, layer, role, d, q_block, run_seed):
    rng = rng_for(cfg, layer, role, "Q", run_seed)
    return np.stack([haar_block(rng, q_block) for _ in range(d // q_block)])


def rotation(cfg: int, layer: int, role: str, d: int, q_block: int,
             dtype: str, run_seed: int = 0) -> np.ndarray:
    """Packed block-diagonal rotation [d // q_block, q_block, q_block].

    Returns the stored (dtype-rounded) values as float64. q_block == d gives
    one dense block.
    """
    if d % q_block:
        raise ValueError("q_block must divide d")
    q64 = _haar_blocks_cached(cfg, layer, role, d, q_block, run_seed)
    return quantize(q64, dtype)


def rotation_fp64(cfg: int, layer: int, role: str, d: int, q_block: int,
                  run_seed: int = 0) -> np.ndarray:
    """The unrounded float64 rotation blocks behind ``rotation``."""
    return _haar_blocks_cached(cfg, layer, role, d, q_block, run_seed).copy()


def signed_permutation(rng, n: int) -> tuple[np.ndarray, np.ndarray]:
    """A random permutation and random signs (±1) of length n."""
    return rng.permutation(n), np.where(rng.random(n) < 0.5, -1.0, 1.0)


def gaussian_weight(cfg: int, layer: int, role: str, d_in: int, d_out: int,
                    std: float, dtype: str, run_seed: int = 0,
                    part: int = 0) -> np.ndarray:
    """W [d_in, d_out] ~ N(0, std²), rounded to dtype. ``part`` separates the
    projections that share one input (q/k/v, gate/up)."""
    rng = rng_for(cfg, layer, role, "W", run_seed * 16 + part)
    w = rng.standard_normal((d_in, d_out), dtype=np.float32).astype(np.float64)
    return quantize(w * std, dtype)


def heavy_tailed_activations(cfg: int, layer: int, role: str, batch: int,
                             d: int, dtype: str, run_seed: int = 0,
                             nu: float = 3.0) -> np.ndarray:
    """x[b, j] = s_j · z[b, j]: s_j = |t_j| with t_j ~ Student-t(nu) fixed per
    channel, z ~ N(0,1) per token."""
    s = np.abs(rng_for(cfg, layer, role, "scales", run_seed).standard_t(nu, size=d))
    z = rng_for(cfg, layer, role, "x", run_seed).standard_normal((batch, d))
    return quantize(z * s[None, :], dtype)


def outlier_activations(cfg: int, layer: int, role: str, batch: int, d: int,
                        n_outliers: int, factor: float, dtype: str,
                        run_seed: int = 0) -> np.ndarray:
    """x ~ N(0,1) with n_outliers seeded channels (no repeats) scaled by factor."""
    z = rng_for(cfg, layer, role, "x", run_seed).standard_normal((batch, d))
    ch = rng_for(cfg, layer, role, "outliers", run_seed).choice(
        d, size=n_outliers, replace=False)
    z[:, ch] *= factor
    return quantize(z, dtype)


def kv_cache(cfg: int, layer: int, batch: int, ctx: int, n_kv_heads: int,
             head_dim: int, dtype: str, run_seed: int = 0):
    """Seeded N(0,1) key and value caches [batch, ctx, n_kv_heads, head_dim]."""
    rng = rng_for(cfg, layer, "attn_in", "kv", run_seed)
    k = rng.standard_normal((batch, ctx, n_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, ctx, n_kv_heads, head_dim), dtype=np.float32)
    return quantize(k, dtype), quantize(v, dtype)


def k_for(d: int, sparsity_pct: int) -> int:
    """Number of kept channels for an integer sparsity percentage.

    The pages fix only the sparsity ratio (40% in the LaRoSA abstract). The
    count is floor(d·(100 − p)/100) in integer arithmetic, so the achieved
    sparsity is never below the nominal one (512 channels at 40% keep 307).
    """
    return (d * (100 - sparsity_pct)) // 100


# ----------------------------------------------------------------------------
# The five workload shapes.

@dataclasses.dataclass(frozen=True)
class LinearCase:
    """One rotated sparse linear: x [B, d_in] · W [d_in, d_out]."""
    cfg: int
    batch: int
    d_in: int
    d_out: int
    q_block: int
    sparsity_pct: int
    dtype: str
    role: str = "single"
    layer: int = 0
    run_seed: int = 0

    @property
    def k(self) -> int:
        return k_for(self.d_in, self.sparsity_pct)


def linear_case_inputs(case: LinearCase, w_std: float, act: str = "heavy",
                       n_outliers: int = 8, factor: float = 20.0):
    """(x, Q, W) for one linear as float64 arrays of stored values."""
    q = rotation(case.cfg, case.layer, case.role, case.d_in, case.q_block,
                 case.dtype, case.run_seed)
    w = gaussian_weight(case.cfg, case.layer, case.role, case.d_in, case.d_out,
                        w_std, case.dtype, case.run_seed)
    if act == "heavy":
        x = heavy_tailed_activations(case.cfg, case.layer, case.role,
                                     case.batch, case.d_in, case.dtype,
                                     case.run_seed)
    elif act == "outlier":
        x = outlier_activations(case.cfg, case.layer, case.role, case.batch,
                                case.d_in, n_outliers, factor, case.dtype,
                                case.run_seed)
    else:
        raise ValueError(act)
    return x, q, w


def single_linear_f32(run_seed: int = 0, batch: int = 1):
    """512→1536 fp32 linear at 40%: Q 512² random orthogonal, W ~ N(0, 1/512)
    (variance 1/d_in), x ~ N(0,1) with 8 outlier channels ×20."""
    case = LinearCase(cfg=1, batch=batch, d_in=512, d_out=1536, q_block=512,
                      sparsity_pct=40, dtype="f32", run_seed=run_seed)
    x, q, w = linear_case_inputs(case, w_std=1.0 / np.sqrt(512.0),
                                 act="outlier", n_outliers=8, factor=20.0)
    return case, x, q, w


def ffn_q_block(f: int) -> int:
    """Block width of the rotation on an FFN-wide input: the fewest equal
    blocks of width <= 4096 that are multiples of 64 (11008 → 4×2752,
    13824 → 4×3456, 28672 → 7×4096)."""
    for nb in range(1, f + 1):
        if f % nb == 0 and f // nb <= 4096 and (f // nb) % 64 == 0:
            return f // nb
    raise ValueError(f"no block width for {f}")


@dataclasses.dataclass(frozen=True)
class MlpCase:
    """SwiGLU MLP: gate|up d→F, SiLU(gate)·up, down F→d, both inputs rotated."""
    cfg: int
    batch: int
    d: int
    f: int
    q1_block: int
    q2_block: int
    sparsity_pct: int
    dtype: str = "bf16"
    w_std: float = 0.02
    layer: int = 0
    run_seed: int = 0

    @property
    def k1(self) -> int:
        return k_for(self.d, self.sparsity_pct)

    @property
    def k2(self) -> int:
        return k_for(self.f, self.sparsity_pct)


def mlp_case_inputs(case: MlpCase, act: str = "heavy", n_outliers: int = 0,
                    factor: float = 1.0):
    """(x, Q1, W_gu, Q2, W_down) as float64 arrays of stored values.

    W_gu is [d, 2F]: the gate columns first, then the up columns.
    """
    c, l, r, dt = case.cfg, case.layer, case.run_seed, case.dtype
    q1 = rotation(c, l, "mlp_in", case.d, case.q1_block, dt, r)
    q2 = rotation(c, l, "down_in", case.f, case.q2_block, dt, r)
    wg = gaussian_weight(c, l, "mlp_in", case.d, case.f, case.w_std, dt, r, 0)
    wu = gaussian_weight(c, l, "mlp_in", case.d, case.f, case.w_std, dt, r, 1)
    wd = gaussian_weight(c, l, "down_in", case.f, case.d, case.w_std, dt, r, 0)
    if act == "heavy":
        x = heavy_tailed_activations(c, l, "mlp_in", case.batch, case.d, dt, r)
    else:
        x = outlier_activations(c, l, "mlp_in", case.batch, case.d, n_outliers,
                                factor, dt, r)
    return x, q1, np.concatenate([wg, wu], axis=1), q2, wd


def llama7b_mlp(batch: int = 1, sparsity_pct: int = 40, q2_block: int | None = None,
                run_seed: int = 0) -> MlpCase:
    """LLaMA2-7B-shaped SwiGLU MLP decode: d 4096, F 11008, bf16."""
    return MlpCase(cfg=2, batch=batch, d=4096, f=11008, q1_block=4096,
                   q2_block=q2_block or ffn_q_block(11008),
                   sparsity_pct=sparsity_pct, run_seed=run_seed)


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    """A device tensor holding exactly the values of ``a`` in ``dtype``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t.to(device)


# ----------------------------------------------------------------------------
# Decoder-scale workloads. Drawing tens of fresh 4096² random orthogonal
# matrices and gigabytes of Gaussian weights per run would dominate the test
# time, so a layer's tensors are seeded signed permutations of one draw per
# role: for a random orthogonal Q and permutation/sign matrices P, D, the
# matrix P·Q·D is again random orthogonal with the same (Haar) law, and a
# row/column permutation of an i.i.d. Gaussian matrix is again i.i.d.
# Gaussian. The permutations are inputs like everything else here.

@dataclasses.dataclass(frozen=True)
class DecoderShape:
    """A LLaMA-shaped decoder layer."""
    d: int = 4096
    f: int = 11008
    n_heads: int = 32
    n_kv_heads: int = 32
    d_head: int = 128
    ctx: int = 2048
    q2_block: int = 2752
    w_std: float = 0.02

    @property
    def qkv_out(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.d_head


LLAMA7B = DecoderShape()


def base_decoder_tensors(cfg: int, shape: DecoderShape, dtype: str = "bf16",
                         run_seed: int = 0) -> dict:
    """One draw per role: rotations (packed blocks) and Gaussian weights."""
    d, f = shape.d, shape.f
    out = {
        "q_attn": rotation(cfg, 0, "attn_in", d, d, dtype, run_seed),
        "q_o": rotation(cfg, 0, "o_in", d, d, dtype, run_seed),
        "q_mlp": rotation(cfg, 0, "mlp_in", d, d, dtype, run_seed),
        "q_down": rotation(cfg, 0, "down_in", f, shape.q2_block, dtype, run_seed),
        "w_qkv": gaussian_weight(cfg, 0, "attn_in", d, shape.qkv_out, shape.w_std, dtype, run_seed),
        "w_o": gaussian_weight(cfg, 0, "o_in", d, d, shape.w_std, dtype, run_seed),
        "w_gu": np.concatenate(
            [gaussian_weight(cfg, 0, "mlp_in", d, f, shape.w_std, dtype, run_seed, 0),
             gaussian_weight(cfg, 0, "mlp_in", d, f, shape.w_std, dtype, run_seed, 1)], axis=1),
        "w_down": gaussian_weight(cfg, 0, "down_in", f, d, shape.w_std, dtype, run_seed),
    }
    return out


ROLE_TENSORS = {"attn_in": ("q_attn", "w_qkv"), "o_in": ("q_o", "w_o"),
                "mlp_in": ("q_mlp", "w_gu"), "down_in": ("q_down", "w_down")}


def layer_tensor_indices(cfg: int, layer: int, role: str, shape: DecoderShape,
                         run_seed: int = 0):
    """For layer `layer` and `role`: (rot_rows, rot_signs, w_rows, w_cols), the
    index arrays that turn the role's base draw into this layer's tensors:
    Q_l = base[:, rot_rows, :] · diag(rot_signs) per block, W_l = base[w_rows][:, w_cols].
    Layer 0 uses the base draw itself."""
    d_in = shape.f if role == "down_in" else shape.d
    qb = shape.q2_block if role == "down_in" else shape.d
    n_out = {"attn_in": shape.qkv_out, "o_in": shape.d, "mlp_in": 2 * shape.f,
             "down_in": shape.d}[role]
    if layer == 0:
        return (np.arange(qb), np.ones(qb), np.arange(d_in), np.arange(n_out))
    rng = rng_for(cfg, layer, role, "perm", run_seed)
    rot_rows, rot_signs = signed_permutation(rng, qb)
    return rot_rows, rot_signs, rng.permutation(d_in), rng.permutation(n_out)


def layer_rotation(base_q: np.ndarray, idx) -> np.ndarray:
    rot_rows, rot_signs = idx[0], idx[1]
    return base_q[:, rot_rows, :] * rot_signs[None, None, :]


def layer_weight(base_w: np.ndarray, idx) -> np.ndarray:
    return base_w[idx[2]][:, idx[3]]


def kv_cache_base(cfg: int, shape: DecoderShape, dtype: str = "bf16", run_seed: int = 0):
    """One seeded N(0,1) key and value cache [n_kv_heads, ctx, d_head]; token b
    of layer l reads it rolled by a seeded offset along the positions."""
    rng = rng_for(cfg, 0, "attn_in", "kv", run_seed)
    k = rng.standard_normal((shape.n_kv_heads, shape.ctx, shape.d_head), dtype=np.float32)
    v = rng.standard_normal((shape.n_kv_heads, shape.ctx, shape.d_head), dtype=np.float32)
    return quantize(k, dtype), quantize(v, dtype)


def kv_offsets(cfg: int, layer: int, batch: int, ctx: int, run_seed: int = 0) -> np.ndarray:
    return rng_for(cfg, layer, "o_in", "kv", run_seed).integers(0, ctx, size=batch)


def decoder_hidden(cfg: int, batch: int, d: int, dtype: str = "bf16", run_seed: int = 0):
    """The decode step's input hidden state: heavy-tailed channel scales."""
    return heavy_tailed_activations(cfg, 0, "attn_in", batch, d, dtype, run_seed)
