"""Pins of the oracle's decoder against things other than itself: a library
rounding routine, exact rationals, closed forms, textbook constants,
invariants of the definition, and pure-Python brute force on tiny inputs."""

import json
import math
import os

import numpy as np
import pytest
import torch

import vdm_workloads as W
from oracle import brute, decoder as dec
from oracle.bf16 import round_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-39),  # subnormal range
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got.astype(np.float32), ref)


def test_bf16_ties_to_even_and_float64_inputs():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert round_bf16(1 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert round_bf16(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    # a float64 just above the tie must round up (no double rounding via float32)
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(x) == 1 + 2.0 ** -7
    rng = np.random.default_rng(2)
    for v in rng.standard_normal(300) * 10.0 ** rng.integers(-5, 5, 300):
        assert round_bf16(v) == brute.bf16(v)


# ---------------------------------------------------------------- grid

def test_grid_coords_exact_and_nested():
    for R in (16, 128):  # dyadic grids: 2i/R - 1 is exact
        i = np.arange(R + 1)
        np.testing.assert_array_equal(dec.grid_coord(i, R), (2.0 * i / R - 1).astype(np.float32))
    for R in (75, 150):
        i = np.arange(R + 1)
        a = dec.grid_coord(i, R)
        b = dec.grid_coord(2 * i, 2 * R)
        assert a.tobytes() == b.tobytes()
        assert a[0] == -1 and a[-1] == 1
    for i in range(76):  # correctly rounded quotient, checked with exact rationals
        assert float(dec.grid_coord(i, 75)) == brute.coord(i, 75)


def test_grid_points_order():
    p = dec.grid_points(4)
    assert p.shape == (125, 3)
    # x slowest, z fastest
    np.testing.assert_array_equal(p[1], [-1, -1, -0.5])
    np.testing.assert_array_equal(p[5], [-1, -0.5, -1])
    np.testing.assert_array_equal(p[25], [-0.5, -1, -1])


# ---------------------------------------------------------------- embedding

def test_embed_closed_forms():
    e = dec.embed(np.zeros((1, 3), np.float32))[0]
    assert e.shape == (51,)
    np.testing.assert_array_equal(e[:27], 0.0)  # xyz and every sine vanish at 0
    np.testing.assert_array_equal(e[27:], 1.0)  # every cosine is 1 at 0
    e = dec.embed(np.array([[0.5, 0.0, 0.0]], np.float32))[0]
    assert e[0] == 0.5
    # axis x, k=0: sin(pi/2) = 1 up to the float32 rounding of pi (|error| < 1e-14)
    assert abs(e[3] - 1.0) < 1e-14 and abs(e[27]) < 1e-6
    # axis x, k=1: sin(pi) = 0 up to float32 pi (|sin(fl(pi))| < 1e-7)
    assert abs(e[4]) < 1e-7 and abs(e[28] + 1.0) < 1e-13
    # layout: y's sines start at 3 + 8
    e = dec.embed(np.array([[0.0, 0.5, 0.0]], np.float32))[0]
    assert abs(e[11] - 1.0) < 1e-14 and e[3] == 0.0


def test_embed_vs_brute():
    pts = W.gen.random_points(3, 20)
    got = dec.embed(pts)
    for n in range(20):
        ref = brute.embed([float(v) for v in pts[n]])
        np.testing.assert_allclose(got[n], ref, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- attention

def _rand_qkv(seed, N=7, M=19, D=128):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, D)), rng.standard_normal((M, D)), rng.standard_normal((M, D))


def test_softmax_rows_sum_to_one():
    Q, K, _ = _rand_qkv(4)
    P = dec.attention_probs(Q * 5, K, 2)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-12
    assert np.all(P >= 0)


def test_attention_single_token_and_identical_keys():
    Q, K, V = _rand_qkv(5)
    o = dec.attention(Q, K[:1], V[:1], 2)
    np.testing.assert_array_equal(o, np.repeat(V[:1], Q.shape[0], 0))
    Ksame = np.repeat(K[:1], K.shape[0], 0)
    o = dec.attention(Q, Ksame, V, 2)
    np.testing.assert_allclose(o, np.repeat(V.mean(0, keepdims=True), Q.shape[0], 0), atol=1e-13)


def test_attention_token_permutation_invariance():
    Q, K, V = _rand_qkv(6)
    perm = np.random.default_rng(7).permutation(K.shape[0])
    np.testing.assert_allclose(dec.attention(Q, K, V, 2), dec.attention(Q, K[perm], V[perm], 2),
                               atol=1e-13)


def test_attention_heads_use_their_own_columns():
    Q, K, V = _rand_qkv(8)
    o = dec.attention(Q, K, V, 2)
    o0 = dec.attention(Q[:, :64], K[:, :64], V[:, :64], 1)
    np.testing.assert_array_equal(o[:, :64], o0)


# ---------------------------------------------------------------- MLP pieces

def test_gelu_textbook_values():
    g = json.load(open(os.path.join(GOLD, "textbook_constants.json")))
    tol = g["tolerance"]
    for x, phi in g["Phi"].items():
        x = float(x)
        assert abs(dec.gelu(np.array([x]))[0] - x * phi) < tol * max(1, abs(x))
    for x, v in g["erf"].items():
        x = float(x)  # gelu(x*sqrt2) = x*sqrt2 * (1 + erf(x)) / 2
        got = dec.gelu(np.array([x * math.sqrt(2)]))[0]
        assert abs(got - x * math.sqrt(2) * (1 + v) / 2) < 2 * tol
    assert dec.gelu(np.array([0.0]))[0] == 0.0
    assert abs(dec.gelu(np.array([9.0]))[0] - 9.0) < 1e-15
    assert abs(dec.gelu(np.array([-9.0]))[0]) < 1e-15


def test_analytic_closed_forms():
    P = W.Prim
    sph = P(0, np.array([0.1, -0.2, 0.3], np.float32), np.array([0.25, 0, 0], np.float32))
    box = P(1, np.array([0.0, 0.0, 0.0], np.float32), np.array([0.2, 0.3, 0.4], np.float32))
    c = sph.centre.astype(np.float64)
    pts = np.array([c, c + [0.5, 0, 0], c + [0, 0, 0.1]], np.float32)
    d = dec.analytic_sdf(pts, [sph])
    np.testing.assert_allclose(d, [-0.25, 0.25, -0.15], atol=2e-7)
    pts = np.array([[0, 0, 0], [0.5, 0, 0], [0.5, 0.7, 0], [0.19, 0, 0], [0.5, 0.7, 0.8]], np.float32)
    d = dec.analytic_sdf(pts, [box])
    ref = [-0.2, 0.3, math.hypot(0.3, 0.4), -0.01, math.sqrt(0.3 ** 2 + 0.4 ** 2 + 0.4 ** 2)]
    np.testing.assert_allclose(d, ref, atol=2e-7)
    both = dec.analytic_sdf(pts, [box, sph])
    np.testing.assert_array_equal(both, np.minimum(dec.analytic_sdf(pts, [box]), dec.analytic_sdf(pts, [sph])))


# ---------------------------------------------------------------- full decoder vs brute force

def _brute_decoder_inputs(w):
    Wl = {k: v.tolist() for k, v in w.weights.items()}
    K, V = brute.project_kv(w.Z.tolist(), Wl["Wk"], Wl["Wv"], w.dtype)
    return Wl, K, V


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decoder_vs_brute(dtype):
    w = W.gen.small_decoder(11, 64, 128, 16, dtype)
    od = dec.Decoder.from_workload(w)
    Wl, K, V = _brute_decoder_inputs(w)
    np.testing.assert_allclose(od.K, K, atol=1e-12, rtol=0)
    np.testing.assert_allclose(od.V, V, atol=1e-12, rtol=0)
    pts = np.concatenate([dec.grid_points(4)[::7], W.gen.random_points(12, 6)])
    got = od.sdf(pts)
    for n, p in enumerate(pts):
        ref = brute.decode_point([float(v) for v in p], Wl, K, V, w.H, w.prims, w.net_scale, dtype)
        assert abs(got[n] - ref) <= 1e-12, (n, got[n], ref)


def test_decoder_two_heads_vs_brute():
    w = W.gen.small_decoder(13, 128, 128, 8, "bf16")
    od = dec.Decoder.from_workload(w)
    Wl, K, V = _brute_decoder_inputs(w)
    pts = W.gen.random_points(14, 5)
    got = od.sdf(pts)
    for n, p in enumerate(pts):
        ref = brute.decode_point([float(v) for v in p], Wl, K, V, 2, w.prims, w.net_scale, "bf16")
        assert abs(got[n] - ref) <= 1e-12


def test_zero_query_weights_give_constant_network_term():
    w = W.gen.small_decoder(15, 64, 128, 16, "f32")
    w.weights["Wq"] = np.zeros_like(w.weights["Wq"])
    od = dec.Decoder.from_workload(w)
    pts = W.gen.random_points(16, 50)
    net = od.net(pts)
    assert np.ptp(net) <= 1e-12
    # q = 0: every logit is 0, attention is the token mean of V
    o = od.V.mean(0)
    c = dec.mlp_head(o[None, :], od.W)[0]
    assert abs(net[0] - c) <= 1e-12
    np.testing.assert_allclose(od.sdf(pts), dec.analytic_sdf(pts, w.prims) + 0.05 * c, atol=1e-12)


def test_zero_net_scale_gives_analytic_sdf():
    w = W.gen.small_decoder(17, 64, 128, 16, "f32")
    od = dec.Decoder(w.weights, w.Z, w.prims, "f32", net_scale=0.0)
    pts = W.gen.random_points(18, 40)
    np.testing.assert_array_equal(od.sdf(pts), dec.analytic_sdf(pts, w.prims))


def test_bf16_decoder_rounds_q_k_v():
    w = W.gen.small_decoder(19, 64, 128, 16, "bf16")
    od = dec.Decoder.from_workload(w)
    for A in (od.K, od.V, od.q(W.gen.random_points(1, 9))):
        np.testing.assert_array_equal(round_bf16(A), A)


def test_workload_shapes():
    w = W.make(0)
    assert (w.D, w.H, w.F, w.M) == (64, 1, 128, 64) and w.dtype == "f32"
    assert np.allclose(np.linalg.norm(w.source_points, axis=1), 0.5)
    w1 = W.make(1)
    assert (w1.D, w1.H, w1.F, w1.M) == (256, 4, 1024, 3072) and w1.query["R"] == 128
    np.testing.assert_array_equal(round_bf16(w1.Z), w1.Z)
    w4 = W.make(4)
    assert w4.M == 40960 and w4.query["xyz"].shape == (200000, 3)
    assert np.all(np.abs(w4.query["xyz"][:100000]) <= 1)
    # near-surface half: within 0.02 of a generated surface point, so |analytic| <= 0.02
    d = dec.analytic_sdf(w4.query["xyz"][100000:], w4.prims)
    assert np.max(np.abs(d)) <= 0.02 + 1e-6
