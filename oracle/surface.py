"""Surface extraction from a decoded SDF volume: TEST INFRASTRUCTURE ONLY.

The techwalker article on FlashVDM, part 1, lists the four stages of a vecset
diffusion pipeline: image encoding, diffusion sampling, VAE decoding and surface
extraction; the last turns the decoded volume into a mesh. The pages do not name
the extraction algorithm. Reading taken here (the plainest one for an SDF
sampled on a grid): marching cubes at SDF = 0 over the (R+1)^3 volume that the
hierarchical decode writes, every cell of the grid (or the cells of a given mask).

Definition (all of it is restated from the geometry, no case table is copied):

* A grid point is inside when its value is < 0 (0 and NaN are outside).
* Every grid edge whose two end points differ in that test carries one vertex,
  at the zero of the linear interpolant along the edge:
  t = v0 / (v0 - v1) from the lower end point, world coordinate -1 + 2 (i + t) / R
  on the edge's axis. Vertices are numbered by ascending edge id
  axis * P^3 + (i * P + j) * P + k (all x edges, then y, then z; P = R + 1),
  over the crossing edges of processed cells.
* Each cell's surface is found face by face. On a cube face with two crossing
  edges one segment joins them; on a face with four (two inside corners on a
  diagonal) each inside corner is cut off by its own segment, so inside corners
  never connect across a face (the choice is made on the face alone, so the two
  cells sharing it agree and the mesh is closed). Each segment is directed so
  that, seen from outside the cube, the surface normal points from the inside
  corners to the outside ones; the directed segments chain into loops.
* Each loop is split into a fan of triangles around one of its vertices, the
  apex: the vertex of smallest global edge id among those that share no cube
  face with any loop vertex other than their two neighbours in the loop. Such a
  vertex exists for every loop (checked over all 256 cases), and with it no
  triangle and no inner fan edge lies in a cube face, so the fans of two cells
  that share a face never overlap (a fan from the smallest id alone can put the
  same triangle, with opposite orientations, into both cells). The fan is
  (apex, v_m, v_m+1), m = 1..n-2, along the loop from the apex. The loops of a
  cell are ordered by their smallest global edge id, triangles by ascending
  cell id (i * R + j) * R + k. Triangle normals (right-hand rule) point to the
  outside (positive) side.

Parity: pinned by tests/test_oracle_surface.py (plane and single-point closed
forms, closed and consistently oriented meshes on spheres and random fields,
sphere area and volume convergence, Euler characteristic).
"""

from functools import lru_cache
from itertools import product
from typing import List, Optional, Tuple

import numpy as np

CORNERS = [c for c in product((0, 1), repeat=3)]  # (di, dj, dk)


def cube_edges() -> List[Tuple[Tuple[int, int, int], int]]:
    """The 12 edges of the unit cube as (lower corner, axis)."""
    return [(c, a) for c in CORNERS for a in range(3) if c[a] == 0]


def _mid(edge) -> np.ndarray:
    c, a = edge
    m = np.array(c, dtype=np.float64)
    m[a] += 0.5
    return m


def _ends(edge):
    c, a = edge
    d = list(c)
    d[a] = 1
    return c, tuple(d)


@lru_cache(maxsize=None)
def cell_loops(inside: Tuple[bool, ...]) -> Tuple[Tuple[Tuple[Tuple[int, int, int], int], ...], ...]:
    """Directed loops of crossing cube edges for one cell.

    inside[n] is the test of corner CORNERS[n]. Returns loops as tuples of cube
    edges (lower corner, axis) in traversal order (not yet canonicalised)."""
    ins = {c: bool(inside[n]) for n, c in enumerate(CORNERS)}
    crossing = lambda e: ins[_ends(e)[0]] != ins[_ends(e)[1]]
    nxt = {}
    for f in range(3):
        for s in (0, 1):
            n_out = np.zeros(3)
            n_out[f] = 2 * s - 1
            fc = [c for c in CORNERS if c[f] == s]
            fe = [e for e in cube_edges() if e[1] != f and e[0][f] == s]
            ce = [e for e in fe if crossing(e)]
            if not ce:
                continue
            segs = []  # (edge a, edge b, g): g points from the inside side to the outside side
            if len(ce) == 2:
                cin = [np.array(c, float) for c in fc if ins[c]]
                cout = [np.array(c, float) for c in fc if not ins[c]]
                segs.append((ce[0], ce[1], np.mean(cout, axis=0) - np.mean(cin, axis=0)))
            else:
                assert len(ce) == 4
                centre = np.mean([np.array(c, float) for c in fc], axis=0)
                for c in fc:
                    if ins[c]:
                        ea, eb = [e for e in fe if c in _ends(e)]
                        segs.append((ea, eb, centre - np.array(c, float)))
            for ea, eb, g in segs:
                t = np.cross(g, n_out)
                d = float(np.dot(_mid(eb) - _mid(ea), t))
                assert d != 0.0
                if d < 0:
                    ea, eb = eb, ea
                assert ea not in nxt
                nxt[ea] = eb
    loops = []
    todo = set(nxt)
    while todo:
        e0 = min(todo)
        loop = [e0]
        todo.discard(e0)
        e = nxt[e0]
        while e != e0:
            loop.append(e)
            todo.discard(e)
            e = nxt[e]
        loops.append(tuple(loop))
    assert sorted(e for lp in loops for e in lp) == sorted(e for e in cube_edges() if crossing(e))
    return tuple(loops)


def edge_faces(edge) -> set:
    """The two cube faces (axis, side) that contain a cube edge."""
    c, a = edge
    return {(f, c[f]) for f in range(3) if f != a}


def fan_apex(loop) -> List[int]:
    """Positions in the loop of the vertices whose chords avoid every cube face."""
    n = len(loop)
    ok = []
    for p in range(n):
        if all(not (edge_faces(loop[p]) & edge_faces(loop[(p + m) % n])) for m in range(2, n - 1)):
            ok.append(p)
    assert ok
    return ok


def edge_id(i: int, j: int, k: int, a: int, P: int) -> int:
    return a * P ** 3 + (i * P + j) * P + k


def crossing_edges(vol3: np.ndarray) -> np.ndarray:
    """Ascending ids of every grid edge whose end points differ in the inside test."""
    P = vol3.shape[0]
    ins = vol3 < 0
    ids = []
    for a in range(3):
        lo = [slice(None)] * 3
        hi = [slice(None)] * 3
        lo[a] = slice(0, P - 1)
        hi[a] = slice(1, P)
        x = np.argwhere(ins[tuple(lo)] != ins[tuple(hi)])
        ids.append(a * P ** 3 + (x[:, 0] * P + x[:, 1]) * P + x[:, 2])
    return np.sort(np.concatenate(ids)).astype(np.int64)


def cell_cases(vol3: np.ndarray) -> np.ndarray:
    """[R, R, R] int: bit n set when corner CORNERS[n] of the cell is inside."""
    ins = vol3 < 0
    R = vol3.shape[0] - 1
    case = np.zeros((R, R, R), dtype=np.int64)
    for n, (di, dj, dk) in enumerate(CORNERS):
        case |= ins[di:di + R, dj:dj + R, dk:dk + R].astype(np.int64) << n
    return case


def case_triangle_counts() -> np.ndarray:
    """Triangles per cell case (256 entries), from cell_loops."""
    out = np.zeros(256, dtype=np.int64)
    for case in range(256):
        loops = cell_loops(tuple(bool(case >> n & 1) for n in range(8)))
        out[case] = sum(len(lp) - 2 for lp in loops)
    return out


def cell_triangles(i: int, j: int, k: int, case: int, P: int) -> List[Tuple[int, int, int]]:
    """Triangles of one cell as triples of global edge ids, in the canonical order."""
    loops = cell_loops(tuple(bool(case >> n & 1) for n in range(8)))
    fans = []
    for lp in loops:
        ids = [edge_id(i + c[0], j + c[1], k + c[2], a, P) for c, a in lp]
        apex = min(fan_apex(lp), key=lambda p: ids[p])
        fans.append((min(ids), ids[apex:] + ids[:apex]))
    fans.sort()
    tris = []
    for _, ids in fans:
        for m in range(1, len(ids) - 1):
            tris.append((ids[0], ids[m], ids[m + 1]))
    return tris


def vertex_positions(vol3: np.ndarray, edges: np.ndarray, R: int) -> np.ndarray:
    """World coordinates (float64) of the vertices on the given edge ids."""
    P = R + 1
    v = vol3.astype(np.float64).reshape(-1)
    a = edges // P ** 3
    p = edges % P ** 3
    step = np.array([P * P, P, 1], dtype=np.int64)[a]
    v0, v1 = v[p], v[p + step]
    t = v0 / (v0 - v1)
    ijk = np.stack([p // (P * P), (p // P) % P, p % P], axis=1).astype(np.float64)
    ijk[np.arange(len(a)), a] += t
    return -1.0 + 2.0 * ijk / R


def extract(vol, R: int, cell_mask: Optional[np.ndarray] = None):
    """Marching cubes at SDF = 0 of the (R+1)^3 float32 volume.

    cell_mask: optional [R^3] (row-major cells) of 0/1; None = every cell.
    Returns (verts [nv, 3] float64 world coordinates, tris [nt, 3] int64 vertex
    indices, edges [nv] int64 edge id of each vertex)."""
    P = R + 1
    vol3 = np.asarray(vol, dtype=np.float32).reshape(P, P, P)
    case = cell_cases(vol3)
    todo = (case != 0) & (case != 255)
    if cell_mask is not None:
        todo &= np.asarray(cell_mask).reshape(R, R, R) != 0
    tri_edges = []
    for i, j, k in np.argwhere(todo):  # ascending cell id
        tri_edges.extend(cell_triangles(int(i), int(j), int(k), int(case[i, j, k]), P))
    te = np.array(tri_edges, dtype=np.int64).reshape(-1, 3)
    edges = np.unique(te)
    if cell_mask is None:
        assert np.array_equal(edges, crossing_edges(vol3))
    tris = np.searchsorted(edges, te)
    return vertex_positions(vol3, edges, R), tris.astype(np.int64), edges
