"""Pins of the oracle's local KNN decoder (AVS-Conv, MSVS-VAE page section
1.1): the neighbour sets against scipy's k-d tree and against brute force with
exact ties, the whole decoder against pure-Python loops on tiny inputs, and
closed forms (zero dynamic weights give the neighbour mean, a query on a
support, a zero hidden layer in the head), exact translation invariance on
dyadic coordinates, permutation invariance of the supports, and K = M."""

import numpy as np
import pytest
from scipy.spatial import cKDTree

import vdm_workloads as W
from oracle import brute, local as lo
from oracle.decoder import analytic_sdf, gelu


def _tiny(seed=3, M=30, C=8, F=16, n=10, K=5, hidden=4):
    return W.small_local(seed, M, C, F, n, K=K, hidden=hidden)


def test_knn_matches_kdtree():
    rng = np.random.default_rng(1)
    P = rng.uniform(-1, 1, (3000, 3)).astype(np.float32)
    X = rng.uniform(-1.1, 1.1, (200, 3)).astype(np.float32)
    got = lo.knn(P, X, 16)
    _, ref = cKDTree(P.astype(np.float64)).query(X.astype(np.float64), k=16)
    np.testing.assert_array_equal(np.sort(got, axis=1), np.sort(ref, axis=1))
    # nearest first
    d = np.stack([lo.sq_dist_f32(P, X[n])[got[n]] for n in range(X.shape[0])])
    assert np.all(np.diff(d, axis=1) >= 0)


def test_knn_ties_go_to_the_lower_index_and_match_brute_force():
    # supports on a coarse lattice, many repeated: exact distance ties
    rng = np.random.default_rng(2)
    base = rng.integers(-4, 5, (12, 3)).astype(np.float32) / 8
    P = np.concatenate([base, base[::-1], base[:5]])  # duplicates at other indices
    X = rng.integers(-8, 9, (25, 3)).astype(np.float32) / 16
    got = lo.knn(P, X, 7)
    for n in range(X.shape[0]):
        assert list(got[n]) == brute.local_neighbours(P.tolist(), X[n].tolist(), 7), n
    # duplicates: the lower index comes first among equal positions
    j = int(got[0][0])
    twins = [k for k in range(P.shape[0]) if np.array_equal(P[k], P[j])]
    assert j == min(twins)


def test_decoder_matches_pure_python_loops():
    w = _tiny()
    got = lo.sdf_of(w)
    for n in range(w.queries.shape[0]):
        ref = brute.local_point(w.xyz.tolist(), w.feats.tolist(), w.queries[n].tolist(),
                                {k: v.tolist() for k, v in w.weights.items()}, w.K, w.prims, w.net_scale)
        assert abs(got[n] - ref) < 1e-12, (n, got[n], ref)


def test_zero_offset_weights_give_the_neighbour_mean():
    w = _tiny(M=40, C=12)
    W0 = dict(w.weights, B=np.zeros_like(w.weights["B"]))
    nbr = lo.knn(w.xyz, w.queries, w.K)
    h = lo.fuse(w.xyz, w.feats, w.queries, nbr, W0)
    np.testing.assert_allclose(h, w.feats.astype(np.float64)[nbr].mean(axis=1), rtol=0, atol=1e-14)


def test_query_on_a_support_with_one_neighbour():
    # K = 1 and the query at a support's position: offset 0, so
    # h = B GELU(a) * f + f for that support
    w = _tiny(K=1)
    j = 7
    X = w.xyz[j:j + 1]
    nbr = lo.knn(w.xyz, X, 1)
    assert nbr[0, 0] == j
    h = lo.fuse(w.xyz, w.feats, X, nbr, w.weights)
    f = w.feats[j].astype(np.float64)
    want = (np.asarray(w.weights["B"], np.float64) @ gelu(np.asarray(w.weights["a"], np.float64))) * f + f
    np.testing.assert_allclose(h[0], want, rtol=0, atol=1e-13)


def test_zero_hidden_layer_leaves_the_linear_head():
    w = _tiny()
    W0 = dict(w.weights, W1=np.zeros_like(w.weights["W1"]))
    nbr = lo.knn(w.xyz, w.queries, w.K)
    h = lo.fuse(w.xyz, w.feats, w.queries, nbr, W0)
    net = lo.head(h, W0)
    np.testing.assert_allclose(net, h @ np.asarray(w.weights["w_head"], np.float64), rtol=0, atol=1e-13)
    s = lo.sdf_of(W.LocalWorkload(w.name, w.K, w.xyz, w.feats, W0, w.queries, w.prims, w.net_scale))
    np.testing.assert_allclose(s, analytic_sdf(w.queries, w.prims) + np.float32(0.05) * net, rtol=0, atol=1e-13)


def test_translation_invariance_on_dyadic_points():
    # coordinates and shift on a 2^-8 lattice: every float32 difference is exact,
    # so neighbours and offsets (hence h) are unchanged by a common shift
    rng = np.random.default_rng(4)
    w = _tiny(M=50, n=12)
    P = (rng.integers(-200, 200, (50, 3)) / 256).astype(np.float32)
    X = (rng.integers(-200, 200, (12, 3)) / 256).astype(np.float32)
    t = np.float32([0.25, -0.5, 0.125])
    n1 = lo.knn(P, X, w.K)
    n2 = lo.knn(P + t, X + t, w.K)
    np.testing.assert_array_equal(n1, n2)
    h1 = lo.fuse(P, w.feats, X, n1, w.weights)
    h2 = lo.fuse(P + t, w.feats, X + t, n2, w.weights)
    np.testing.assert_array_equal(h1, h2)


def test_support_permutation_invariance():
    w = _tiny(M=60, n=15)
    perm = np.random.default_rng(5).permutation(w.M)
    a = lo.sdf_of(w)
    b = lo.sdf_of(W.LocalWorkload(w.name, w.K, w.xyz[perm], w.feats[perm], w.weights, w.queries, w.prims,
                                  w.net_scale))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_all_supports_as_neighbours():
    w = _tiny(M=9, K=9)
    nbr = lo.knn(w.xyz, w.queries, 9)
    assert all(sorted(r) == list(range(9)) for r in nbr.tolist())
    h = lo.fuse(w.xyz, w.feats, w.queries, nbr, w.weights)
    # the sum over all supports in index order gives the same h
    order = np.tile(np.arange(9), (w.queries.shape[0], 1))
    np.testing.assert_allclose(h, lo.fuse(w.xyz, w.feats, w.queries, order, w.weights), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [64])
def test_full_size_workload_shape(n):
    # the 40,960-support workload: neighbour sets of a few queries against the k-d tree
    w = W.make_local(n_queries=n)
    assert w.M == 40960 and w.C == 256 and w.F == 1024 and w.K == 16
    got = lo.knn(w.xyz, w.queries, w.K)
    _, ref = cKDTree(w.xyz.astype(np.float64)).query(w.queries.astype(np.float64), k=w.K)
    same = np.all(np.sort(got, axis=1) == np.sort(ref, axis=1), axis=1)
    assert same.mean() > 0.95  # (float32 vs float64 distances may reorder a near tie)
