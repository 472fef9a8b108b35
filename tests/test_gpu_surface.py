"""GPU parity of surface extraction (marching cubes at SDF = 0) through the C ABI.

Small volumes: the GPU mesh equals the oracle's exactly (vertex edge ids, triangle
vertex ids, counts) and the vertex positions agree to float32 rounding. A volume
built to contain every one of the 256 cell cases, zeros, NaN, empty and full
volumes, cell masks and short output buffers are covered. Full size: the
hierarchical decode's 301^3 volume, checked through the definition where the
oracle can compute it at that size (every crossing edge, every cell's triangle
count) and cell by cell on a sample."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from oracle import surface as S
from tests.helpers import dev, gpu_decoder, gpu_kv

pytestmark = pytest.mark.gpu

POS_TOL = 2e-6  # |d position|: float32 interpolation and world-coordinate rounding


def V():
    import shape_vae_decoding_amd as mod

    return mod


def gpu_extract(vol, R, mask=None, max_verts=None, max_tris=None):
    vt = torch.from_numpy(np.ascontiguousarray(vol, np.float32).reshape(-1)).to(dev())
    mt = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8).reshape(-1)).to(dev())
    nv = max_verts if max_verts is not None else 3 * (R + 1) ** 3
    nt = max_tris if max_tris is not None else 5 * R ** 3
    verts = torch.full((max(nv, 1), 3), -7.0, dtype=torch.float32, device=dev())[:nv]
    tris = torch.full((max(nt, 1), 3), -7, dtype=torch.int32, device=dev())[:nt]
    edges = torch.full((max(nv, 1),), -7, dtype=torch.int64, device=dev())[:nv]
    counts = torch.full((2,), -1, dtype=torch.int64, device=dev())
    print(f"[surface] R={R} mask={'yes' if mask is not None else 'no'} max_verts={nv} max_tris={nt}", flush=True)
    V().vdm_extract_surface(vt, R, verts, tris, counts, cell_mask=mt, vert_edges=edges)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    return verts.cpu().numpy(), tris.cpu().numpy().astype(np.int64), edges.cpu().numpy(), int(c[0]), int(c[1])


def check_equal(vol, R, mask=None):
    Vo, To, Eo = S.extract(vol, R, mask)
    Vg, Tg, Eg, nv, nt = gpu_extract(vol, R, mask)
    assert (nv, nt) == (len(Vo), len(To))
    assert np.array_equal(Eg[:nv], Eo)
    assert np.array_equal(Tg[:nt], To)
    assert np.abs(Vg[:nv] - Vo).max(initial=0.0) <= POS_TOL
    return Vo, To


def grid(R):
    x = -1.0 + 2.0 * np.arange(R + 1) / R
    return np.meshgrid(x, x, x, indexing="ij")


def all_cases_volume():
    """Cells at even (i, j, k) have disjoint corners: 343 of them, the first 256
    take cases 0..255 (corner (di,dj,dk) inside when bit 4di+2dj+dk is set)."""
    R = 13
    rng = np.random.default_rng(11)
    v = rng.uniform(0.2, 1.0, (R + 1,) * 3).astype(np.float32)
    slots = [(a, b, c) for a in range(7) for b in range(7) for c in range(7)]
    for case, (a, b, c) in zip(range(256), slots):
        for di in range(2):
            for dj in range(2):
                for dk in range(2):
                    if case >> (4 * di + 2 * dj + dk) & 1:
                        v[2 * a + di, 2 * b + dj, 2 * c + dk] *= -1.0
    return v, R


def test_every_cell_case():
    v, R = all_cases_volume()
    assert set(np.unique(S.cell_cases(v)).tolist()) == set(range(256))
    check_equal(v, R)


@pytest.mark.parametrize("R", [40, 37])
def test_sphere(R):
    X, Y, Z = grid(R)
    v = (np.sqrt((X - 0.07) ** 2 + (Y + 0.11) ** 2 + Z ** 2) - 0.55).astype(np.float32)
    Vo, To = check_equal(v, R)
    assert len(To) > 1000


@pytest.mark.parametrize("R", [70, 126])
def test_rows_longer_than_a_word(R):
    # points k >= 32 and k >= 63 of a row (R = 126: rows of exactly two pieces of 63
    # points and one of 1); an off-centre sphere reaching close to the boundary
    X, Y, Z = grid(R)
    v = (np.sqrt((X - 0.05) ** 2 + (Y + 0.03) ** 2 + (Z - 0.04) ** 2) - 0.93).astype(np.float32)
    Vo, To = check_equal(v, R)
    assert np.abs(S.extract(v, R)[2] % (R + 1) - 63).min() == 0  # a vertex at k = 63


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_fields(seed):
    rng = np.random.default_rng(seed)
    R = [20, 17, 9][seed]
    if seed == 1:  # many exact zeros (outside)
        v = rng.integers(-1, 2, (R + 1,) * 3).astype(np.float32)
    else:
        v = rng.standard_normal((R + 1,) * 3).astype(np.float32)
    check_equal(v, R)


def test_single_point_empty_full_and_one_cell():
    v = np.ones((5, 5, 5), np.float32)
    v[2, 2, 2] = -0.5
    Vo, To = check_equal(v, 4)
    assert len(To) == 8
    for fill in (1.0, 0.0, -1.0):  # no crossing edge: empty mesh
        _, _, _, nv, nt = gpu_extract(np.full((9, 9, 9), fill, np.float32), 8)
        assert (nv, nt) == (0, 0)
    for case in (1, 0b01101001, 0b10010110, 127):
        v = np.ones((2, 2, 2), np.float32)
        for n in range(8):
            if case >> n & 1:
                v[n >> 2, (n >> 1) & 1, n & 1] = -1.0
        check_equal(v, 1)


def test_nan_counts_as_outside():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((12, 12, 12)).astype(np.float32)
    v[3, 4, 5] = np.nan
    v[7, 7, 7] = np.nan
    Vo, To, Eo = S.extract(v, 11)
    Vg, Tg, Eg, nv, nt = gpu_extract(v, 11)
    assert np.array_equal(Eg[:nv], Eo) and np.array_equal(Tg[:nt], To)
    fin = np.isfinite(Vo).all(axis=1)
    assert np.array_equal(fin, np.isfinite(Vg[:nv]).all(axis=1))
    assert np.abs(Vg[:nv][fin] - Vo[fin]).max() <= POS_TOL


def test_cell_mask():
    R = 24
    X, Y, Z = grid(R)
    v = (np.sqrt(X ** 2 + Y ** 2 + Z ** 2) - 0.6).astype(np.float32)
    rng = np.random.default_rng(9)
    mask = (rng.random(R ** 3) < 0.5).astype(np.uint8)
    check_equal(v, R, mask)
    check_equal(v, R, np.zeros(R ** 3, np.uint8))


def test_short_output_buffers_keep_the_counts_and_write_only_the_prefix():
    R = 30
    X, Y, Z = grid(R)
    v = (np.abs(X) + np.abs(Y) + np.abs(Z) - 1.1).astype(np.float32)
    Vo, To, Eo = S.extract(v, R)
    mv, mt = len(Vo) // 3, len(To) // 2
    Vg, Tg, Eg, nv, nt = gpu_extract(v, R, max_verts=mv, max_tris=mt)
    assert (nv, nt) == (len(Vo), len(To))
    assert np.array_equal(Eg, Eo[:mv]) and np.array_equal(Tg, To[:mt])
    assert np.abs(Vg - Vo[:mv]).max() <= POS_TOL
    _, _, _, nv0, nt0 = gpu_extract(v, R, max_verts=0, max_tris=0)
    assert (nv0, nt0) == (len(Vo), len(To))


def test_full_size_hierarchical_volume():
    """The 75 -> 150 -> 300 hierarchical decode's 301^3 volume."""
    w = W.make(2)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    q = w.query
    params = V().hier_params(R0=q["R0"], levels=q["levels"], tau=q["tau"], dilation=q["dilation"])
    R = 300
    vol = torch.empty((R + 1) ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_hier(dec, params, K, Vv, vol)
    torch.cuda.synchronize()
    v = vol.cpu().numpy().reshape((R + 1,) * 3)
    edges = S.crossing_edges(v)
    case = S.cell_cases(v).reshape(-1)
    ntri = S.case_triangle_counts()[case]
    Vg, Tg, Eg, nv, nt = gpu_extract(v, R, max_verts=len(edges) + 16, max_tris=int(ntri.sum()) + 16)
    print(f"[surface] 301^3: {nv} vertices, {nt} triangles", flush=True)
    assert nv == len(edges) and nt == int(ntri.sum())
    assert np.array_equal(Eg[:nv], edges)
    # positions on a sample of vertices
    rng = np.random.default_rng(4)
    pick = rng.choice(nv, size=min(nv, 20000), replace=False)
    assert np.abs(Vg[pick] - S.vertex_positions(v, edges[pick], R)).max() <= POS_TOL
    # triangles cell by cell on a sample of surface cells
    first = np.concatenate([[0], np.cumsum(ntri)])
    cells = np.flatnonzero(ntri)
    for c in rng.choice(cells, size=min(len(cells), 3000), replace=False):
        i, j, k = c // (R * R), (c // R) % R, c % R
        want = np.array(S.cell_triangles(int(i), int(j), int(k), int(case[c]), R + 1), np.int64)
        got = Eg[Tg[first[c]:first[c + 1]]]
        assert np.array_equal(got, want), (int(c), int(case[c]))
    # the whole mesh is closed and consistently oriented unless a crossing edge lies
    # in a boundary face of the volume
    P = R + 1
    a, p = Eg[:nv] // P ** 3, Eg[:nv] % P ** 3
    ijk = np.stack([p // (P * P), (p // P) % P, p % P], axis=1)
    in_face = np.zeros(nv, bool)
    for b in range(3):
        in_face |= (a != b) & ((ijk[:, b] == 0) | (ijk[:, b] == R))
    if not in_face.any():
        T = Tg[:nt]
        d = np.concatenate([T[:, [0, 1]], T[:, [1, 2]], T[:, [2, 0]]])
        key = np.sort(d[:, 0] * (1 << 32) + d[:, 1])
        rkey = np.sort(d[:, 1] * (1 << 32) + d[:, 0])
        assert len(np.unique(key)) == len(key) and np.array_equal(key, rkey)
