"""Pins for the decoder-layer oracle (RMSNorm, rotary embedding, single-query
attention, residual add): closed forms, invariants and a hand-worked fixture,
not the oracle's own formulas retyped."""
import json
import math
import os

import numpy as np

from oracle import decoder_ref as dec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rmsnorm_closed_forms_and_invariance():
    for c in (3.0, -0.5, 1e-3):
        x = np.full((1, 64), c)
        y = dec.rmsnorm(x, out_dtype="f32")
        want = np.sign(c) / math.sqrt(1.0 + 1e-5 / (c * c))
        np.testing.assert_allclose(y, want, rtol=1e-7)
    assert np.all(dec.rmsnorm(np.zeros((2, 16)), out_dtype="f32") == 0)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 256)) * 40
    np.testing.assert_allclose(dec.rmsnorm(x * 7, out_dtype="f32"),
                               dec.rmsnorm(x, out_dtype="f32"), rtol=1e-6)
    y = dec.rmsnorm(x, out_dtype="f32")
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-5)


def test_rope_hand_worked_head4():
    g = json.load(open(os.path.join(GOLDEN, "rope_dhead4.json")))
    x = np.array(g["inputs"], dtype=np.float64)
    got = dec.rope_exact(x, 1, 4, g["pos"])
    np.testing.assert_allclose(got, g["outputs"], atol=1e-15)
    # the interleaved pairing (2i, 2i+1) is a different reading and fails
    wrong = x.copy()
    ang = 100.0
    wrong[0] = [math.cos(ang), math.sin(ang), 0, 0]
    assert not np.allclose(wrong[0], g["outputs"][0])


def test_rope_invariants():
    rng = np.random.default_rng(2)
    H, dh = 4, 128
    x = rng.standard_normal((3, H * dh))
    np.testing.assert_array_equal(dec.rope_exact(x, H, dh, 0), x)
    a = dec.rope_exact(dec.rope_exact(x, H, dh, 700), H, dh, 1348)
    np.testing.assert_allclose(a, dec.rope_exact(x, H, dh, 2048), atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(dec.rope_exact(x, H, dh, 2048).reshape(3, H, dh), axis=2),
                               np.linalg.norm(x.reshape(3, H, dh), axis=2), rtol=1e-12)
    q, k = x[:1], rng.standard_normal((1, H * dh))
    lhs = (dec.rope_exact(q, H, dh, 2048).reshape(H, dh) * dec.rope_exact(k, H, dh, 2000).reshape(H, dh)).sum(1)
    rhs = (dec.rope_exact(q, H, dh, 48).reshape(H, dh) * k.reshape(H, dh)).sum(1)
    np.testing.assert_allclose(lhs, rhs, atol=1e-9)   # depends only on the offset


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    B, H, Hkv, dh, T = 2, 4, 2, 8, 5
    q = rng.standard_normal((B, H * dh))
    kn = rng.standard_normal((B, Hkv * dh))
    vn = rng.standard_normal((B, Hkv * dh))
    # empty cache: the new token's value, whatever the scores
    kc = np.zeros((B, Hkv, 0, dh))
    out = dec.decode_attention(q, kn, vn, kc, kc, H, Hkv, dh, "f32")
    want = np.repeat(vn.reshape(B, Hkv, 1, dh), H // Hkv, axis=1).reshape(B, H * dh)
    np.testing.assert_allclose(out, want, rtol=1e-7)
    # all keys equal: the plain mean of the values
    k_same = np.broadcast_to(kn.reshape(B, Hkv, 1, dh), (B, Hkv, T, dh)).copy()
    vc = rng.standard_normal((B, Hkv, T, dh))
    out = dec.decode_attention(q, kn, vn, k_same, vc, H, Hkv, dh, "f32")
    allv = np.concatenate([vc, vn.reshape(B, Hkv, 1, dh)], axis=2).mean(axis=2)
    np.testing.assert_allclose(out, np.repeat(allv, 2, axis=1).reshape(B, H * dh), rtol=1e-6)
    # two positions: a two-way softmax is a logistic function of the score gap
    qq = np.zeros((1, dh)); qq[0, 0] = 3.0
    k1 = np.zeros((1, 1, 1, dh)); k1[..., 0] = 1.0
    v1 = np.zeros((1, 1, 1, dh)); v1[..., 1] = 1.0
    v2 = np.zeros((1, dh)); v2[0, 2] = 1.0
    o = dec.decode_attention(qq, np.zeros((1, dh)), v2, k1, v1, 1, 1, dh, "f32")
    w = 1.0 / (1.0 + math.exp(-3.0 / math.sqrt(dh)))
    np.testing.assert_allclose(o[0, [1, 2]], [w, 1 - w], rtol=1e-6)


def test_residual_add_exact():
    a = np.array([[1.0, -2.5, 3.0]])
    b = np.array([[0.5, 2.5, -1.0]])
    np.testing.assert_array_equal(dec.residual_add(a, b), [[1.5, 0.0, 2.0]])
