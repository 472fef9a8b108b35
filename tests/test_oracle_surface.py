"""Pins of the surface-extraction oracle (marching cubes at SDF = 0): closed forms,
mesh invariants and convergence to the analytic sphere."""
import numpy as np
import pytest

from oracle import surface as S


def grid(R):
    x = -1.0 + 2.0 * np.arange(R + 1) / R
    return np.meshgrid(x, x, x, indexing="ij")


def directed_edges(T):
    return np.concatenate([T[:, [0, 1]], T[:, [1, 2]], T[:, [2, 0]]])


def closed_and_oriented(T):
    """Every directed mesh edge occurs once and its reverse once: a closed,
    consistently oriented 2-manifold (edge-wise)."""
    d = directed_edges(T)
    key = d[:, 0] * (1 << 32) + d[:, 1]
    rkey = d[:, 1] * (1 << 32) + d[:, 0]
    return len(np.unique(key)) == len(key) and np.array_equal(np.sort(key), np.sort(rkey))


def euler(V, T):
    e = np.unique(np.sort(directed_edges(T), axis=1), axis=0)
    return len(V) - len(e) + len(T)


def normals(V, T):
    a, b, c = V[T[:, 0]], V[T[:, 1]], V[T[:, 2]]
    return np.cross(b - a, c - a), (a + b + c) / 3


def enclosed_volume(V, T):
    a, b, c = V[T[:, 0]], V[T[:, 1]], V[T[:, 2]]
    return np.einsum("ij,ij->i", a, np.cross(b, c)).sum() / 6


def test_every_case_uses_each_crossing_edge_once_and_single_corners_give_one_triangle():
    counts = S.case_triangle_counts()
    assert counts[0] == 0 and counts[255] == 0
    for n, c in enumerate(S.CORNERS):
        # one inside corner: one triangle over its three edges, normal away from it
        loops = S.cell_loops(tuple(m == n for m in range(8)))
        assert len(loops) == 1 and len(loops[0]) == 3
        assert sorted(e[0] for e in loops[0]) != []
        p = [S._mid(e) for e in loops[0]]
        nrm = np.cross(p[1] - p[0], p[2] - p[0])
        assert np.dot(nrm, np.mean(p, axis=0) - np.array(c, float)) > 0
        # one outside corner: the same triangle, facing the corner
        loops = S.cell_loops(tuple(m != n for m in range(8)))
        p = [S._mid(e) for e in loops[0]]
        nrm = np.cross(p[1] - p[0], p[2] - p[0])
        assert len(loops) == 1 and np.dot(nrm, np.mean(p, axis=0) - np.array(c, float)) < 0
    # two inside corners on a cube edge: one quad
    assert counts[0b00000011] == 2
    # inside corners that touch only across face diagonals stay apart
    checker = sum(1 << n for n, c in enumerate(S.CORNERS) if sum(c) % 2 == 0)
    assert counts[checker] == 4 and counts[255 ^ checker] == 4
    assert counts.max() == 5


def test_single_inside_point_gives_the_octahedron():
    R = 4
    v = np.ones((R + 1,) * 3, dtype=np.float32)
    v[2, 2, 2] = -1.0
    V, T, E = S.extract(v, R)
    assert len(V) == 6 and len(T) == 8
    # each vertex halfway along its edge: half a grid step (0.25) from the centre
    assert np.allclose(np.sort(np.abs(V).sum(axis=1)), 0.25, atol=0)
    assert np.allclose(np.sort(np.linalg.norm(V, axis=1)), 0.25, atol=0)
    assert closed_and_oriented(T) and euler(V, T) == 2
    n, cen = normals(V, T)
    assert (np.einsum("ij,ij->i", n, cen) > 0).all()
    assert enclosed_volume(V, T) == pytest.approx(4.0 / 3.0 * 0.25 ** 3, rel=1e-12)  # octahedron |x|+|y|+|z| <= r


def test_plane_lies_on_the_zero_set_and_faces_the_positive_side():
    R = 20
    X, Y, Z = grid(R)
    v = (X - 0.13).astype(np.float32)
    V, T, E = S.extract(v, R)
    assert np.abs(V[:, 0] - 0.13).max() < 1e-6
    assert set(np.unique(E // (R + 1) ** 3)) == {0}  # only x edges cross
    assert len(V) == (R + 1) ** 2
    n, _ = normals(V, T)
    area = 0.5 * np.linalg.norm(n, axis=1)
    assert area.sum() == pytest.approx(4.0, rel=1e-6)
    assert (n[:, 0] > 0).all()


@pytest.mark.parametrize("R", [24, 48])
def test_sphere_is_closed_outward_and_converges(R):
    X, Y, Z = grid(R)
    r = 0.6
    v = (np.sqrt(X ** 2 + Y ** 2 + Z ** 2) - r).astype(np.float32)
    V, T, E = S.extract(v, R)
    assert closed_and_oriented(T) and euler(V, T) == 2
    n, cen = normals(V, T)
    assert (np.einsum("ij,ij->i", n, cen) > 0).all()
    assert np.abs(np.linalg.norm(V, axis=1) - r).max() < (2.0 / R) ** 2  # chord error of linear interpolation
    err = abs(enclosed_volume(V, T) - 4.0 / 3.0 * np.pi * r ** 3) / (4.0 / 3.0 * np.pi * r ** 3)
    assert err < {24: 0.015, 48: 0.004}[R]


def test_random_fields_cover_every_case_with_closed_oriented_meshes():
    rng = np.random.default_rng(7)
    seen = set()
    for s in range(40):
        P = 8
        if s % 2:
            v = rng.standard_normal((P, P, P)).astype(np.float32)
        else:  # many exact zeros (outside by definition)
            v = rng.integers(-1, 2, (P, P, P)).astype(np.float32)
        v[0], v[-1], v[:, 0], v[:, -1], v[:, :, 0], v[:, :, -1] = 1, 1, 1, 1, 1, 1
        V, T, E = S.extract(v, P - 1)
        assert closed_and_oriented(T)
        assert np.array_equal(E, S.crossing_edges(v))
        seen |= set(np.unique(S.cell_cases(v)).tolist())
    assert seen == set(range(256))


def test_cell_mask_keeps_exactly_the_masked_cells_triangles():
    rng = np.random.default_rng(3)
    R = 9
    v = rng.standard_normal((R + 1,) * 3).astype(np.float32)
    mask = (rng.random(R ** 3) < 0.4).astype(np.uint8)
    Vf, Tf, Ef = S.extract(v, R)
    Vm, Tm, Em = S.extract(v, R, mask)
    case = S.cell_cases(v)
    want = []
    for c in np.flatnonzero(mask):
        i, j, k = c // (R * R), (c // R) % R, c % R
        want += S.cell_triangles(i, j, k, int(case[i, j, k]), R + 1)
    assert np.array_equal(Em[Tm], np.array(want, dtype=np.int64).reshape(-1, 3))
    assert np.allclose(Vm, Vf[np.searchsorted(Ef, Em)])
