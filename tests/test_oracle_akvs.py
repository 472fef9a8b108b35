"""Pins of the oracle's adaptive KV selection: brute-force scores and a full
stable sort for top-k (with exact ties and a binding cap), the k = all special
case (equals full attention), the corner-probe geometry of ragged blocks, and
the HVD + selection loop against brute force on a tiny grid."""

import itertools

import numpy as np
import pytest

import vdm_workloads as W
from oracle import akvs, brute, decoder as dec, hvd as hv


def test_probe_scores_vs_brute():
    rng = np.random.default_rng(31)
    Qp = rng.standard_normal((8, 128)) * 2
    K = rng.standard_normal((24, 128))
    got = akvs.probe_scores(Qp, K, 2)
    ref = brute.scores(Qp.tolist(), K.tolist(), 2)
    np.testing.assert_allclose(got, ref, atol=1e-15, rtol=0)
    assert np.max(np.abs(got.sum(1) - 1)) < 1e-13


@pytest.mark.parametrize("k,cap", [(3, 24), (5, 24), (5, 9), (24, 24), (1, 1)])
def test_select_vs_brute_with_ties(k, cap):
    rng = np.random.default_rng(32 + k + cap)
    sc = rng.integers(0, 6, (8, 24)).astype(np.float64) / 7.0  # many exact ties
    got = akvs.select(sc, k, cap)
    assert list(got) == brute.select(sc.tolist(), k, cap)
    assert np.all(np.diff(got) > 0) and got.size <= min(cap, 8 * k)


def test_topk_ties_go_to_lower_index():
    s = np.array([0.5, 0.2, 0.5, 0.9, 0.5])
    assert list(akvs.topk_ids(s, 3)) == [3, 0, 2]


def test_cap_keeps_largest_max_scores():
    sc = np.zeros((2, 10))
    sc[0, [0, 1, 2]] = [0.9, 0.8, 0.1]
    sc[1, [5, 6, 7]] = [0.85, 0.05, 0.07]
    # union {0,1,2,5,6,7}; max scores 0.9, 0.8, 0.1, 0.85, 0.05, 0.07 -> keep 0, 5, 1, 2
    assert list(akvs.select(sc, 3, 4)) == [0, 1, 2, 5]


def test_k_all_is_full_attention():
    w = W.gen.small_decoder(33, 128, 128, 40, "bf16")
    od = dec.Decoder.from_workload(w)
    pts = W.gen.random_points(34, 16)
    sets = akvs.select_blocks(od, 16, np.array([0, 3, 7]), w.M, w.M)
    for s in sets.values():
        np.testing.assert_array_equal(s, np.arange(w.M))
    np.testing.assert_allclose(od.sdf(pts, od.K[np.arange(w.M)], od.V[np.arange(w.M)]), od.sdf(pts),
                               atol=1e-14)


def test_corner_probes_of_ragged_blocks():
    R = 75  # 76 points: blocks 0..9, the last spans 72..75
    idx = akvs.block_corner_indices(R, np.array([[9, 0, 3]]))[0]
    assert set(idx[:, 0]) == {72, 75} and set(idx[:, 1]) == {0, 7} and set(idx[:, 2]) == {24, 31}
    assert len({tuple(t) for t in idx}) == 8
    idx = akvs.block_corner_indices(8, np.array([[1, 1, 1]]))[0]  # single-point block
    assert np.all(idx == 8)


def test_splitmix64_reference_outputs():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")))
    assert akvs.splitmix64(0, 0) == int(g["seed_0_first"], 16)
    assert [akvs.splitmix64(1234567, c) for c in range(5)] == [int(x) for x in g["seed_1234567_first_5"]]


def test_random_probes_stay_in_their_blocks_and_cover_them():
    R, NB = 75, 10
    blocks = np.arange(NB ** 3)
    idx = akvs.block_random_indices(R, blocks, NB, seed=99)
    bijk = akvs.block_ijk(blocks, NB)
    lo = bijk[:, None, :] * 8
    hi = np.minimum(lo + 7, R)
    assert (idx >= lo).all() and (idx <= hi).all()
    # deterministic in the seed, different across seeds and blocks
    assert np.array_equal(idx, akvs.block_random_indices(R, blocks, NB, seed=99))
    assert not np.array_equal(idx, akvs.block_random_indices(R, blocks, NB, seed=100))
    # roughly uniform over the 8 offsets of a full block (8000 draws per axis)
    full = (bijk < 9).all(axis=1)
    off = (idx - lo)[full].reshape(-1)
    counts = np.bincount(off, minlength=8)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    # the single-point edge blocks of an R = 8 grid keep their one point
    idx = akvs.block_random_indices(8, np.array([7]), 2, seed=5)
    assert np.all(idx == 8)


def test_scores_mean_over_heads_of_softmax():
    rng = np.random.default_rng(35)
    Qp, K = rng.standard_normal((3, 256)), rng.standard_normal((50, 256))
    s = akvs.probe_scores(Qp, K, 4)
    ref = np.mean([dec.softmax_rows(Qp[:, 64 * h:64 * h + 64] @ K[:, 64 * h:64 * h + 64].T / 8)
                   for h in range(4)], axis=0)
    np.testing.assert_allclose(s, ref, atol=1e-15)


def test_hvd_with_selection_vs_brute():
    w = W.gen.small_decoder(36, 64, 64, 12, "bf16")
    od = dec.Decoder.from_workload(w)
    k, cap, R0, levels, tau = 3, 20, 4, 2, 0.1
    rec = {}
    res = hv.hvd(akvs.make_decode(od, k, cap, record=rec), R0, levels, tau, 1)
    Wl = {kk: v.tolist() for kk, v in w.weights.items()}
    K, V = od.K.tolist(), od.V.tolist()
    cache = {}

    def bdecode(R, t):
        P = R + 1
        NB = (P + 7) // 8
        b = ((t[0] // 8) * NB + t[1] // 8) * NB + t[2] // 8
        if (R, b) not in cache:
            bi, bj, bk = b // (NB * NB), (b // NB) % NB, b % NB
            lo = [8 * x for x in (bi, bj, bk)]
            hi = [min(8 * x + 7, R) for x in (bi, bj, bk)]
            probes = [[brute.coord(c, R) for c in corner]
                      for corner in itertools.product(*zip(lo, hi))]
            qs = [[brute.bf16(v) for v in brute.matvec(Wl["Wq"], brute.embed(p))] for p in probes]
            cache[(R, b)] = brute.select(brute.scores(qs, K, 1), k, cap)
        p = [brute.coord(c, R) for c in t]
        return brute.decode_point(p, Wl, K, V, 1, w.prims, w.net_scale, "bf16", tokens=cache[(R, b)])

    bvol, brec = brute.hvd(bdecode, R0, levels, tau, 1)
    for r, b in zip(res["levels"], brec):
        assert list(r["list"]) == b["list"]
    for (R, b), toks in cache.items():
        assert list(rec[R][b]) == toks
    P = R0 * 2 ** (levels - 1) + 1
    ref = np.array([bvol[t] for t in itertools.product(range(P), repeat=3)]).reshape(P, P, P)
    np.testing.assert_allclose(res["vol"], ref, atol=1e-12, rtol=0)


def test_per_head_scores_and_sets_vs_brute():
    rng = np.random.default_rng(35)
    Qp = rng.standard_normal((8, 128)) * 2
    K = rng.standard_normal((24, 128))
    got = akvs.probe_scores_per_head(Qp, K, 2)
    ref = brute.scores_per_head(Qp.tolist(), K.tolist(), 2)
    np.testing.assert_allclose(got, ref, atol=1e-15, rtol=0)
    # the head-mean score is the mean of the per-head scores
    np.testing.assert_allclose(got.mean(axis=0), akvs.probe_scores(Qp, K, 2), atol=1e-16, rtol=0)
    for h in range(2):
        assert list(akvs.select(got[h], 3, 10)) == brute.select(ref[h], 3, 10)
    # the heads rank differently: their sets differ
    assert not np.array_equal(akvs.select(got[0], 3, 24), akvs.select(got[1], 3, 24))


def test_per_head_sets_decode_vs_brute_and_special_cases():
    w = W.gen.small_decoder(36, 128, 128, 20, "f32")
    od = dec.Decoder.from_workload(w)
    pts = W.gen.random_points(37, 5)
    sets = [np.array([0, 3, 4, 9, 17]), np.array([1, 2, 3, 12, 13, 19])]
    got = akvs.sdf_per_head_sets(od, pts, sets)
    W64 = {k: v.astype(np.float64).tolist() for k, v in w.weights.items()}
    for n in range(pts.shape[0]):
        ref = brute.decode_point(pts[n].tolist(), W64, od.K.tolist(), od.V.tolist(), 2, w.prims, w.net_scale, "f32",
                                 head_tokens=[s.tolist() for s in sets])
        assert abs(got[n] - ref) < 1e-12
    # every head on the same set: attention restricted to that set
    same = [sets[0], sets[0]]
    np.testing.assert_allclose(akvs.sdf_per_head_sets(od, pts, same),
                               od.sdf(pts, od.K[sets[0]], od.V[sets[0]]), atol=1e-13, rtol=0)
    # every head on all tokens: full attention
    allt = [np.arange(w.M)] * 2
    np.testing.assert_allclose(akvs.sdf_per_head_sets(od, pts, allt), od.sdf(pts), atol=1e-13, rtol=0)


def test_per_head_selection_with_one_head_equals_head_mean():
    w = W.gen.small_decoder(38, 64, 128, 50, "bf16")
    od = dec.Decoder.from_workload(w)
    blocks = np.array([0, 2, 5])
    a = akvs.select_blocks(od, 12, blocks, 7, 30)
    b = akvs.select_blocks(od, 12, blocks, 7, 30, heads=True)
    for blk in blocks:
        np.testing.assert_array_equal(a[int(blk)], b[int(blk)][0])
