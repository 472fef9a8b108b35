"""Pins of the oracle's hierarchical volume decoding: brute force with per-cell
loops, the tau = inf special case (equals dense decoding), a Lipschitz
argument that makes the method exact for a pure distance field, closed-form
sphere geometry, the pages' hole claim for plain octree decoding, and the
structural invariants."""

import itertools
import math

import numpy as np
import pytest

import vdm_workloads as W
from oracle import brute, decoder as dec, hvd as hv


def _field(seed, Rf, thin=True, net_scale=0.05, zero_wq=False):
    """Dense oracle SDF on the finest grid plus a decode(R, lin) that reads it
    at the nested points (coordinates nest exactly, so this is the decode)."""
    w = W.gen.small_decoder(seed, 64, 128, 16, "f32", n_sph=2, n_box=1)
    prims = list(w.prims)
    if thin:  # a thin plate that coarse grids step over
        prims.append(W.Prim(1, np.array([0.13, -0.11, 0.07], np.float32),
                            np.array([0.5, 0.45, 0.012], np.float32)))
    if zero_wq:
        w.weights["Wq"] = np.zeros_like(w.weights["Wq"])
    od = dec.Decoder(w.weights, w.Z, prims, "f32", net_scale=net_scale)
    P = Rf + 1
    vol = od.sdf_grid(Rf).reshape(P, P, P)

    def decode(R, lin):
        s = Rf // R
        I, r = np.divmod(np.asarray(lin, np.int64), (R + 1) ** 2)
        J, K = np.divmod(r, R + 1)
        return vol[I * s, J * s, K * s]

    return vol, decode, od, prims


def _to_set3(mask):
    return set(map(tuple, np.argwhere(mask)))


@pytest.mark.parametrize("tau,dil", [(0.06, 1), (0.0, 0), (0.02, 2)])
def test_hvd_matches_brute(tau, dil):
    R0, levels = 4, 3
    vol, decode, _, _ = _field(21, R0 * 4)
    res = hv.hvd(decode, R0, levels, tau, dil)
    bvol, brec = brute.hvd(lambda R, t: float(decode(R, [(t[0] * (R + 1) + t[1]) * (R + 1) + t[2]])[0]),
                           R0, levels, tau, dil)
    for rec, b in zip(res["levels"], brec):
        assert rec["R"] == b["R"]
        assert list(rec["list"]) == b["list"]
        assert _to_set3(rec["active"]) == b["active"]
        assert _to_set3(rec["tested"]) == b["tested"]
        if "kept" in rec:
            assert _to_set3(rec["kept"]) == b["kept"]
    P = R0 * 2 ** (levels - 1) + 1
    ref = np.array([bvol[t] for t in itertools.product(range(P), repeat=3)]).reshape(P, P, P)
    np.testing.assert_array_equal(res["vol"], ref)


def test_tau_inf_equals_dense():
    R0, levels = 4, 3
    vol, decode, _, _ = _field(22, 16)
    res = hv.hvd(decode, R0, levels, np.inf, 1)
    np.testing.assert_array_equal(res["vol"], vol)
    for rec in res["levels"]:
        assert rec["active"].all()


def test_structural_invariants():
    R0, levels = 6, 3
    _, decode, _, _ = _field(23, 24)
    res = hv.hvd(decode, R0, levels, 0.03, 1)
    computed = None
    for L, rec in enumerate(res["levels"]):
        R, P = rec["R"], rec["R"] + 1
        keys = hv.blocked_key(rec["list"], P)
        assert np.all(np.diff(keys) > 0)  # strictly increasing, so no duplicates
        v32 = rec["vol"].astype(np.float32)
        sc = hv.cell_test(v32, rec["tested"], 0.0)  # sign-change cells among the tested
        assert not np.any(sc & ~rec["active"])
        if "kept" in rec:
            assert not np.any(rec["active"] & ~rec["kept"])
            nxt = res["levels"][L + 1]["tested"]
            assert np.all(hv.children(sc) <= nxt)  # refined set contains every sign-change cell
        if computed is not None:  # new queries were not computed before
            prevpts = np.zeros(P ** 3, bool)
            prevpts.reshape(P, P, P)[::2, ::2, ::2] = computed
            assert not np.any(prevpts[rec["list"]])
        c = np.zeros(P ** 3, bool)
        c[rec["list"]] = True
        if computed is not None:
            c.reshape(P, P, P)[::2, ::2, ::2] |= computed
        computed = c.reshape(P, P, P)
        # every tested cell has all 8 corners computed
        t = rec["tested"]
        for a, b, cc in itertools.product((0, 1), repeat=3):
            assert np.all(computed[a:a + R, b:b + R, cc:cc + R][t])


def test_lipschitz_band_makes_pure_distance_field_exact():
    # With net_scale = 0 the volume is a distance field (1-Lipschitz). If tau is
    # at least the coarse cell diagonal, a cell with all |s| >= tau cannot contain
    # surface, so every inherited point keeps the correct sign.
    R0, levels = 4, 3
    vol, decode, _, _ = _field(24, 16, net_scale=0.0)
    tau = 1.01 * math.sqrt(3) * 2.0 / R0
    res = hv.hvd(decode, R0, levels, tau, 0)
    np.testing.assert_array_equal(res["vol"] >= 0, vol >= 0)


def test_octree_without_band_and_dilation_leaves_holes():
    # FlashVDM summary, section 4.1 key details: plain octree decoding misses thin
    # parts. A plate z in [0.15, 0.35] lies between the R=4 grid planes z=0 and
    # z=0.5, so no coarse corner sees it; the R=16 grid (plane z=0.25) does.
    plate = W.Prim(1, np.array([0.0, 0.0, 0.25], np.float32), np.array([0.6, 0.6, 0.1], np.float32))
    w = W.gen.small_decoder(25, 64, 128, 16, "f32")
    od = dec.Decoder(w.weights, w.Z, [plate], "f32", net_scale=0.0)
    Rf, R0, levels = 16, 4, 3
    vol = od.sdf_grid(Rf).reshape((Rf + 1,) * 3)

    def decode(R, lin):
        s = Rf // R
        I, r = np.divmod(np.asarray(lin, np.int64), (R + 1) ** 2)
        J, K = np.divmod(r, R + 1)
        return vol[I * s, J * s, K * s]

    every = np.ones((Rf,) * 3, bool)
    dense_sc = hv.cell_test(vol.astype(np.float32), every, 0.0)
    assert np.count_nonzero(dense_sc) > 0
    plain = hv.hvd(decode, R0, levels, 0.0, 0)
    plain_sc = hv.cell_test(plain["vol"].astype(np.float32), every, 0.0)
    assert np.count_nonzero(dense_sc & ~plain_sc) > 0
    full = hv.hvd(decode, R0, levels, 1.01 * math.sqrt(3) * 2.0 / R0, 1)
    full_sc = hv.cell_test(full["vol"].astype(np.float32), every, 0.0)
    assert np.count_nonzero(dense_sc & ~full_sc) == 0


def test_zero_query_weights_sphere_geometry():
    # q = 0 makes the network term a constant c, so SDF = |p - centre| - r' with
    # r' = r - 0.05 c: sign-change cells follow from corner distances alone.
    w = W.gen.small_decoder(26, 64, 128, 16, "f32")
    w.weights["Wq"] = np.zeros_like(w.weights["Wq"])
    sph = W.Prim(0, np.array([0.05, -0.1, 0.02], np.float32), np.array([0.55, 0, 0], np.float32))
    od = dec.Decoder(w.weights, w.Z, [sph], "f32")
    c = od.net(np.zeros((1, 3), np.float32))[0]
    r_eff = 0.55 - od.net_scale * c
    R = 12
    vol = od.sdf_grid(R).reshape((R + 1,) * 3)
    act = hv.cell_test(vol.astype(np.float32), np.ones((R,) * 3, bool), 0.0)
    g = dec.grid_coord(np.arange(R + 1), R).astype(np.float64)
    X, Y, Z = np.meshgrid(g, g, g, indexing="ij")
    d = np.sqrt((X - 0.05) ** 2 + (Y + 0.1) ** 2 + (Z - 0.02) ** 2)
    cs = [d[a:a + R, b:b + R, cc:cc + R] for a, b, cc in itertools.product((0, 1), repeat=3)]
    dmin, dmax = np.min(cs, axis=0), np.max(cs, axis=0)
    geo = (dmin < r_eff) & (dmax >= r_eff)
    near = np.zeros_like(geo)
    for cv in cs:
        near |= np.abs(cv - r_eff) < 1e-6
    assert np.count_nonzero(geo) > 20
    np.testing.assert_array_equal(act[~near], geo[~near])


def test_blocked_key_order_and_ragged_blocks():
    P = 19  # 3 blocks per axis, the last one ragged (3 points)
    lin = np.arange(P ** 3)
    keys = hv.blocked_key(lin, P)
    assert len(np.unique(keys)) == P ** 3
    order = lin[np.argsort(keys)]
    # first 512 entries are exactly the first full block
    I, r = np.divmod(order[:512], P * P)
    J, K = np.divmod(r, P)
    assert I.max() == 7 and J.max() == 7 and K.max() == 7
    for t in [(0, 0, 0), (18, 18, 18), (7, 8, 9), (16, 2, 17)]:
        assert hv.blocked_key(np.array([(t[0] * P + t[1]) * P + t[2]]), P)[0] == brute.key(*t, P)


def test_query_reduction_on_the_hierarchical_workload_shape():
    # Aggregate sanity (not parity): with the analytic part of the 75->150->300
    # workload the number of decoded points is a small fraction of 301^3; the
    # FlashVDM summary reports 91.4% fewer queries on its own data.
    w = W.make(2)
    prims = w.prims
    Rf = 300

    def decode(R, lin):
        return dec.analytic_sdf(dec.grid_points(R, lin), prims)

    q = w.query
    res = hv.hvd(decode, q["R0"], q["levels"], q["tau"], q["dilation"])
    st = hv.stats(res)
    total = sum(s["queries"] for s in st)
    frac = total / (Rf + 1) ** 3
    assert 0.02 < frac < 0.15, st
