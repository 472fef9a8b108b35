"""Pins of the oracle's tie windows: the helpers that name which GPU/oracle
differences in integer outputs are excused (tokens near a top-k or cap cutoff,
cells with a corner value near a threshold). The benchmark spec's tolerance reads
"within 1e-4 of a threshold or tie"; the readings are a relative 1e-4 around a
token score cutoff and an absolute 1e-4 around the SDF thresholds 0 and +-tau.

Each input is built by hand so that a plausible slip fails one case: an
absolute window instead of a relative one (or the reverse), the wrong rank
index, a missing +-tau or -tau term, a window that ignores the cap stage, or a
window that lands on the wrong cells."""

import numpy as np

from oracle import akvs, hvd as hv

def _row(kth, k, M, spread=0.5):
    """A score row whose k-th largest value is ``kth`` and whose other values
    lie far (a factor 1 +- spread) from it: k - 1 above, M - k below."""
    above = kth * (1 + spread) * (1 + np.arange(k - 1) / M)
    below = kth * (1 - spread) * (1 - np.arange(M - k) / (2 * M))
    return np.concatenate([above, [kth], below])


def test_topk_window_is_relative_to_the_kth_score():
    k = 4
    for kth in (3e-4, 1e3):  # a probability scale and a large scale
        # ranks: one far above, two just above (1 + 2e-4, 1 + 0.5e-4), the k-th,
        # two just below (1 - 0.5e-4, 1 - 2e-4), then far below
        row = np.array([kth * 1.5, kth * (1 + 2e-4), kth * (1 + 0.5e-4), kth,
                        kth * (1 - 0.5e-4), kth * (1 - 2e-4), kth * 0.5, kth * 0.4])
        perm = np.array([5, 0, 7, 2, 4, 6, 1, 3])  # token ids of the ranks
        sc = np.empty_like(row)
        sc[perm] = row
        amb = set(akvs.near_tie_tokens(sc[None, :], k).tolist())
        assert amb == {int(perm[2]), int(perm[3]), int(perm[4])}, (kth, amb)


def test_topk_window_rejects_an_absolute_reading():
    # at probability scale an absolute 1e-4 window would cover +-30 %
    k, M = 3, 10
    kth = 3e-4
    row = _row(kth, k, M)
    row[9] = kth * 0.8
    assert set(akvs.near_tie_tokens(row[None, :], k).tolist()) == {k - 1}


def test_topk_window_uses_rank_k_not_a_neighbour_rank():
    # ranks k-1 and k+1 are 5 % away; a token 0.5e-4 from rank k is excused
    # only if the window sits on rank k itself
    k = 5
    row = np.array([10, 9, 8, 7.35, 7.0, 6.65, 3, 2, 1, 7.0 * (1 + 0.5e-4)], np.float64)
    # sorted: 10 9 8 7.35 7.00035 7.0 6.65 ... -> rank 5 is 7.00035 (index 9)
    amb = set(akvs.near_tie_tokens(row[None, :], k).tolist())
    assert amb == {4, 9}, amb


def test_topk_window_is_per_probe():
    k, M = 2, 12
    a = _row(1.0, k, M)
    b = _row(5.0, k, M)
    b[7] = 5.0 * (1 - 0.3e-4)  # near probe 1's cutoff; far from probe 0's
    amb = set(akvs.near_tie_tokens(np.stack([a, b]), k).tolist())
    assert 7 in amb
    # probe 0's own near-tie: none besides its k-th; probe 1's k-th too
    assert amb == {int(np.flatnonzero(a == 1.0)[0]), int(np.flatnonzero(b == 5.0)[0]), 7}


def test_cap_window_around_the_cap_cutoff():
    # two probes, k = 3 each, disjoint top sets: union of 6 tokens, cap 4.
    # max-over-probes scores of the union: 0.9, 0.8, 0.7, 0.6 (rank 4: the cutoff),
    # 0.6 (1 + 0.5e-4) (inside the cap window), 0.6 (1 - 2e-4) (outside)
    sc = np.full((2, 12), 1e-3)
    sc[0, [0, 1, 2]] = [0.9, 0.7, 0.6 * (1 + 0.5e-4)]
    sc[1, [5, 6, 7]] = [0.8, 0.6, 0.6 * (1 - 2e-4)]
    no_cap = set(akvs.near_tie_tokens(sc, 3).tolist())
    assert no_cap == {2, 7}  # each probe's k-th score only
    with_cap = set(akvs.near_tie_tokens(sc, 3, cap=4).tolist())
    # rank-4 max score over the union {0,1,2,5,6,7}: 0.9 0.8 0.7 0.60003 0.6 0.59988
    # -> cutoff 0.60003 (token 2); 6 lies 0.5e-4 below it, 7 lies 2.5e-4 below
    assert with_cap == no_cap | {6}, with_cap
    # and the oracle's own selection keeps exactly the first four by max score
    assert list(akvs.select(sc, 3, 4)) == [0, 1, 2, 5]


def test_cap_window_is_empty_when_the_cap_does_not_bind():
    sc = np.full((2, 12), 1e-3)
    sc[0, [0, 1, 2]] = [0.9, 0.7, 0.6]
    sc[1, [5, 6, 7]] = [0.8, 0.6 * (1 + 0.5e-4), 0.5]
    assert set(akvs.near_tie_tokens(sc, 3, cap=6).tolist()) == set(akvs.near_tie_tokens(sc, 3).tolist())


def _vol(R=2, fill=0.5):
    return np.full((R + 1,) * 3, fill)


def test_threshold_window_around_zero_and_both_taus():
    tau = 1 / 75
    # corner values: 0 +- 5e-5 and +-tau +- 5e-5 are near; 0 +- 2e-4 and
    # +-tau +- 2e-4 are not
    for v, near in [(5e-5, True), (-5e-5, True), (2e-4, False), (-2e-4, False),
                    (tau + 5e-5, True), (tau - 5e-5, True), (-tau + 5e-5, True), (-tau - 5e-5, True),
                    (tau + 2e-4, False), (tau - 2e-4, False), (-tau + 2e-4, False), (-tau - 2e-4, False)]:
        vol = _vol()
        vol[0, 0, 0] = v
        cells = hv.near_threshold_cells(vol, tau)
        assert bool(cells[0, 0, 0]) == near, (v, near)
        # only the one cell that owns the corner (0, 0, 0)
        assert int(cells.sum()) == (1 if near else 0), v


def test_threshold_window_marks_every_cell_around_a_corner():
    tau = 0.02
    vol = _vol(R=3)
    vol[1, 2, 1] = tau - 3e-5
    cells = hv.near_threshold_cells(vol, tau)
    want = np.zeros((3, 3, 3), bool)
    want[0:2, 1:3, 0:2] = True  # the 8 cells whose corner set holds (1, 2, 1)
    np.testing.assert_array_equal(cells, want)


def test_threshold_window_is_absolute_not_relative():
    # an absolute window around tau: 5e-5 from a tau of 0.5 is near (a relative
    # 1e-4 window would be 5e-5 wide and miss 8e-5), 2e-4 from it is not
    tau = 0.5
    vol = _vol(fill=0.9)
    vol[2, 2, 2] = tau + 8e-5
    assert hv.near_threshold_cells(vol, tau)[1, 1, 1]
    vol[2, 2, 2] = tau + 2e-4
    assert not hv.near_threshold_cells(vol, tau).any()
