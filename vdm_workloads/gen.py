"""Seeded workload generator (data only; see the package docstring).

Recipe (the pages leave these details open; the plainest reading is taken):

* Decoder weights are N(0, 1/fan_in): Wq [D,51], Wk/Wv/Wo [D,D], W1 [F,D],
  W2 [D,F], w_head [D]. The 1024-wide decoder is drawn once and shared by the
  129^3 dense, hierarchical, KV-selection and 40,960-token workloads.
* A shape is a union of analytic primitives: spheres (centre, radius) and
  axis-aligned boxes (centre, per-axis half extent); centres U[-0.5,0.5]^3,
  sizes U[0.15,0.4].
* Latent tokens: M points on the union's surface (primitive chosen in
  proportion to its area, a uniform point on it, rejected when strictly
  inside another primitive), Fourier features of each point (xyz, then sin
  and cos of 2^k*pi*coordinate for k = 0..7, axis-major), a Gaussian
  projection G ~ N(0, 1/51) of those 51 features to D dims, plus noise of
  variance 0.01.
* bf16 workloads round every weight and latent to bf16 (round to nearest
  even) here, so both consumers see identical values.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

CONFIG_NAMES = {
    0: "tiny_dense_17cubed_fp32",
    1: "dense_129cubed_M3072_bf16",
    2: "hier_75_150_300_M3072_bf16",
    3: "hier_akvs_75_150_300_M3072_bf16",
    4: "dense_200k_M40960_bf16",
}

N_FREQ = 8
E_DIM = 3 + 2 * 3 * N_FREQ  # 51

# substream ids (seed sequence = [seed, stream])
_S_TINY = 10
_S_DEC256 = 20
_S_SHAPE1 = 30
_S_SHAPE4 = 40
_S_QUERY4 = 41


@dataclasses.dataclass
class Prim:
    """One analytic primitive: kind 0 = sphere (size[0] = radius),
    kind 1 = axis-aligned box (size = half extents)."""

    kind: int
    centre: np.ndarray  # float32 [3]
    size: np.ndarray  # float32 [3]


@dataclasses.dataclass
class Workload:
    cid: int
    name: str
    dtype: str  # "f32" or "bf16"
    D: int
    H: int
    F: int
    M: int
    weights: Dict[str, np.ndarray]  # float32 arrays
    Z: np.ndarray  # float32 [M, D]
    prims: List[Prim]
    net_scale: float
    query: Dict[str, object]
    source_points: np.ndarray  # float64 [M, 3]
    seed: int = 0

    @property
    def n_queries(self) -> Optional[int]:
        q = self.query
        if q["kind"] == "grid":
            return (int(q["R"]) + 1) ** 3
        if q["kind"] == "points":
            return int(q["xyz"].shape[0])
        return None


def round_bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of bf16-representable values (RNE),
    via torch's own conversion (input preparation, not decoder arithmetic)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy().copy()


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def _decoder_weights(rng: np.random.Generator, D: int, F: int) -> Dict[str, np.ndarray]:
    def w(shape, fan_in):
        return (rng.standard_normal(shape) / np.sqrt(fan_in)).astype(np.float32)

    return {
        "Wq": w((D, E_DIM), E_DIM),
        "Wk": w((D, D), D),
        "Wv": w((D, D), D),
        "Wo": w((D, D), D),
        "W1": w((F, D), D),
        "W2": w((D, F), F),
        "w_head": w((D,), D),
    }


def _random_prims(rng: np.random.Generator, n_sph: int, n_box: int) -> List[Prim]:
    prims = []
    for _ in range(n_sph):
        c = rng.uniform(-0.5, 0.5, 3).astype(np.float32)
        r = np.float32(rng.uniform(0.15, 0.4))
        prims.append(Prim(0, c, np.array([r, 0.0, 0.0], np.float32)))
    for _ in range(n_box):
        c = rng.uniform(-0.5, 0.5, 3).astype(np.float32)
        h = rng.uniform(0.15, 0.4, 3).astype(np.float32)
        prims.append(Prim(1, c, h))
    return prims


def _strictly_inside(p: np.ndarray, pr: Prim) -> np.ndarray:
    """Membership predicate used only for rejection sampling of surface points."""
    c = pr.centre.astype(np.float64)
    if pr.kind == 0:
        return np.sum((p - c) ** 2, axis=1) < float(pr.size[0]) ** 2
    h = pr.size.astype(np.float64)
    return np.all(np.abs(p - c) < h, axis=1)


def _area(pr: Prim) -> float:
    if pr.kind == 0:
        return 4.0 * np.pi * float(pr.size[0]) ** 2
    hx, hy, hz = (float(v) for v in pr.size)
    return 8.0 * (hx * hy + hy * hz + hx * hz)


def _sample_on(rng: np.random.Generator, pr: Prim, n: int) -> np.ndarray:
    c = pr.centre.astype(np.float64)
    if pr.kind == 0:
        d = rng.standard_normal((n, 3))
        d /= np.linalg.norm(d, axis=1, keepdims=True)
        return c + float(pr.size[0]) * d
    h = pr.size.astype(np.float64)
    # face pairs normal to x, y, z have areas 4*hy*hz, 4*hx*hz, 4*hx*hy (each side)
    fa = np.array([h[1] * h[2], h[0] * h[2], h[0] * h[1]])
    axis = rng.choice(3, size=n, p=fa / fa.sum())
    side = rng.choice(np.array([-1.0, 1.0]), size=n)
    u = rng.uniform(-1.0, 1.0, (n, 3)) * h
    u[np.arange(n), axis] = side * h[axis]
    return c + u


def sample_union_surface(rng: np.random.Generator, prims: List[Prim], n: int) -> np.ndarray:
    """n points uniformly on the surface of the union of ``prims``."""
    areas = np.array([_area(p) for p in prims])
    out = []
    have = 0
    while have < n:
        batch = max(1024, 2 * (n - have))
        which = rng.choice(len(prims), size=batch, p=areas / areas.sum())
        pts = np.empty((batch, 3))
        for i, pr in enumerate(prims):
            sel = np.nonzero(which == i)[0]
            if sel.size:
                pts[sel] = _sample_on(rng, pr, sel.size)
        keep = np.ones(batch, bool)
        for i, pr in enumerate(prims):
            inside = _strictly_inside(pts, pr) & (which != i)
            keep &= ~inside
        pts = pts[keep]
        out.append(pts)
        have += pts.shape[0]
    return np.concatenate(out, axis=0)[:n]


def _fourier_features_for_latents(s: np.ndarray) -> np.ndarray:
    """Input recipe: 51 Fourier features of the latent *source* points
    (xyz, sin then cos of 2^k*pi*coordinate, axis-major), float64."""
    f = (2.0 ** np.arange(N_FREQ)) * np.pi  # [8]
    arg = s[:, :, None] * f[None, None, :]  # [M, 3, 8]
    return np.concatenate(
        [s, np.sin(arg).reshape(len(s), -1), np.cos(arg).reshape(len(s), -1)], axis=1
    )


def _latents(rng: np.random.Generator, src: np.ndarray, D: int) -> np.ndarray:
    G = rng.standard_normal((D, E_DIM)) / np.sqrt(E_DIM)
    feats = _fourier_features_for_latents(src)
    noise = rng.standard_normal((src.shape[0], D)) * 0.1  # variance 0.01
    return (feats @ G.T + noise).astype(np.float32)


def _bf16_all(weights: Dict[str, np.ndarray], Z: np.ndarray):
    return {k: round_bf16_values(v) for k, v in weights.items()}, round_bf16_values(Z)


def _make_tiny(seed: int) -> Workload:
    D, H, F, M = 64, 1, 128, 64
    rng = _rng(seed, _S_TINY)
    weights = _decoder_weights(rng, D, F)
    d = rng.standard_normal((M, 3))
    src = 0.5 * d / np.linalg.norm(d, axis=1, keepdims=True)
    Z = _latents(rng, src, D)
    prims = [Prim(0, np.zeros(3, np.float32), np.array([0.5, 0, 0], np.float32))]
    return Workload(0, CONFIG_NAMES[0], "f32", D, H, F, M, weights, Z, prims,
                    0.05, {"kind": "grid", "R": 16}, src, seed)


def _dec256(seed: int):
    return _decoder_weights(_rng(seed, _S_DEC256), 256, 1024)


def _make_shape1(seed: int, M: int = 3072):
    rng = _rng(seed, _S_SHAPE1)
    prims = _random_prims(rng, 3, 2)
    src = sample_union_surface(rng, prims, M)
    Z = _latents(rng, src, 256)
    return prims, src, Z


def _make_shape4(seed: int, M: int = 40960):
    rng = _rng(seed, _S_SHAPE4)
    prims = _random_prims(rng, 5, 5)
    src = sample_union_surface(rng, prims, M)
    Z = _latents(rng, src, 256)
    return prims, src, Z


def _c4_queries(seed: int, prims: List[Prim], n: int = 200_000) -> np.ndarray:
    rng = _rng(seed, _S_QUERY4)
    half = n // 2
    uni = rng.uniform(-1.0, 1.0, (half, 3))
    surf = sample_union_surface(rng, prims, n - half)
    d = rng.standard_normal((n - half, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    r = 0.02 * rng.uniform(0.0, 1.0, n - half) ** (1.0 / 3.0)  # uniform in the ball
    near = surf + d * r[:, None]
    return np.concatenate([uni, near], axis=0).astype(np.float32)


HIER_DEFAULT = {
    "R0": 75,
    "levels": 3,
    # two voxel widths of the finest (300^3) level: 2 * (2/300), in float32
    "tau": float(np.float32(2.0 * 2.0 / 300.0)),
    "dilation": 1,
}
KVSEL_DEFAULT = {"block": 8, "k": 64, "cap": 512}


def make(cid: int, seed: int = 0, *, M: Optional[int] = None) -> Workload:
    """Build workload ``cid`` (0..4). ``M`` overrides the token count of the
    generated shape (used by tests to make smaller variants)."""
    if cid == 0:
        return _make_tiny(seed)
    weights = _dec256(seed)
    if cid in (1, 2, 3):
        prims, src, Z = _make_shape1(seed, M or 3072)
    elif cid == 4:
        prims, src, Z = _make_shape4(seed, M or 40960)
    else:
        raise ValueError(f"unknown workload {cid}")
    weights, Z = _bf16_all(weights, Z)
    if cid == 1:
        query = {"kind": "grid", "R": 128}
    elif cid == 2:
        query = dict(kind="hier", **HIER_DEFAULT)
    elif cid == 3:
        query = dict(kind="hier", kvsel=dict(KVSEL_DEFAULT), **HIER_DEFAULT)
    else:
        query = {"kind": "points", "xyz": _c4_queries(seed, prims)}
    return Workload(cid, CONFIG_NAMES[cid], "bf16", 256, 4, 1024, Z.shape[0], weights, Z,
                    prims, 0.05, query, src, seed)


def random_points(seed: int, n: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Uniform float32 query points in [lo, hi]^3 (test inputs)."""
    return _rng(seed, 99).uniform(lo, hi, (n, 3)).astype(np.float32)


def small_decoder(seed: int, D: int, F: int, M: int, dtype: str = "bf16", n_sph: int = 2,
                  n_box: int = 1) -> Workload:
    """A scaled-down decoder + shape with the same recipe (for parity tests that
    the oracle finishes in seconds)."""
    rng = _rng(seed, 77)
    weights = _decoder_weights(rng, D, F)
    prims = _random_prims(rng, n_sph, n_box)
    src = sample_union_surface(rng, prims, M)
    Z = _latents(rng, src, D)
    if dtype == "bf16":
        weights, Z = _bf16_all(weights, Z)
    return Workload(-1, f"small_D{D}_F{F}_M{M}_{dtype}", dtype, D, D // 64, F, M, weights, Z,
                    prims, 0.05, {"kind": "none"}, src, seed)


def unseen_key_directions(Wq: np.ndarray, H: int) -> np.ndarray:
    """[H, 64] unit vectors, one per head h, orthogonal to every column of the
    head's query weights Wq[64h:64h+64, :] (a head's queries span at most 51 of
    its 64 dimensions; the rest is the left null space of those rows). A key
    component along such a direction changes no logit of an exactly projected
    query, but raises the key's norm (test input construction)."""
    Wq = np.asarray(Wq, np.float64)
    out = np.empty((H, 64))
    for h in range(H):
        U, _, _ = np.linalg.svd(Wq[64 * h:64 * h + 64, :])
        u = U[:, Wq.shape[1]:].sum(axis=1)
        out[h] = u / np.linalg.norm(u)
    return out


def with_unseen_key(K: np.ndarray, Wq: np.ndarray, H: int, token: int, norm: float,
                    dtype: str = "bf16") -> np.ndarray:
    """K [M, 64 H] with ``norm`` times each head's unseen direction added to row
    ``token`` (rounded to bf16 for bf16 decoders)."""
    K = np.array(K, np.float64)
    K[token] += norm * unseen_key_directions(Wq, H).reshape(-1)
    K = K.astype(np.float32)
    return round_bf16_values(K) if dtype == "bf16" else K


# ---------------------------------------------------------------- local KNN decoder workload

_S_LOCAL = 50
LOCAL_K = 16       # neighbours per query
LOCAL_HIDDEN = 32  # width of the offset MLP
LOCAL_OFFSET_SCALE = 0.25  # offsets of this length reach the offset MLP's hidden units at unit scale


@dataclasses.dataclass
class LocalWorkload:
    """Inputs of the local KNN decoder (AVS-Conv) at the 200K-query x 40,960-token
    shape: supports (anchor positions and their latent features), offset-MLP and
    head weights, query points, analytic prior."""

    name: str
    K: int
    xyz: np.ndarray       # float32 [M, 3] support positions
    feats: np.ndarray     # float32 [M, C] support features (bf16 values)
    weights: Dict[str, np.ndarray]  # A [Hw,3], a [Hw] (float32); B [C,Hw], W1 [F,C], W2 [C,F] (bf16 values); w_head [C]
    queries: np.ndarray   # float32 [N, 3]
    prims: List[Prim]
    net_scale: float

    @property
    def M(self) -> int:
        return int(self.xyz.shape[0])

    @property
    def C(self) -> int:
        return int(self.feats.shape[1])

    @property
    def F(self) -> int:
        return int(self.weights["W1"].shape[0])


def _local_weights(rng: np.random.Generator, C: int, Hw: int) -> Dict[str, np.ndarray]:
    # A ~ N(0, 1/3) / LOCAL_OFFSET_SCALE, a ~ N(0, 1), B ~ N(0, 1/Hw)
    A = (rng.standard_normal((Hw, 3)) / np.sqrt(3.0) / LOCAL_OFFSET_SCALE).astype(np.float32)
    a = rng.standard_normal(Hw).astype(np.float32)
    B = round_bf16_values((rng.standard_normal((C, Hw)) / np.sqrt(Hw)).astype(np.float32))
    return {"A": A, "a": a, "B": B}


def make_local(seed: int = 0, *, M: Optional[int] = None, n_queries: Optional[int] = None) -> LocalWorkload:
    """The local decoder at the MSVS-VAE page's decode-speed shape: the
    40,960-token shape's latents as supports at the surface points they were
    drawn from, the 200,000 query points of that workload, the 1024-wide head
    of the vecset decoder (W1, W2, w_head) and a fresh offset MLP."""
    base = make(4, seed, M=M)
    lw = _local_weights(_rng(seed, _S_LOCAL), base.D, LOCAL_HIDDEN)
    weights = dict(lw, W1=base.weights["W1"], W2=base.weights["W2"], w_head=base.weights["w_head"])
    q = base.query["xyz"] if n_queries is None else base.query["xyz"][:n_queries]
    return LocalWorkload(f"local_knn_{q.shape[0]}q_M{base.M}", LOCAL_K, base.source_points.astype(np.float32),
                         base.Z, weights, np.ascontiguousarray(q), base.prims, 0.05)


def small_local(seed: int, M: int, C: int, F: int, n_queries: int, K: int = LOCAL_K,
                hidden: int = LOCAL_HIDDEN) -> LocalWorkload:
    """A scaled-down local decoder with the same recipe (supports on a union of
    primitives, features = latents of those points, uniform and near-surface
    queries)."""
    rng = _rng(seed, 78)
    prims = _random_prims(rng, 2, 1)
    src = sample_union_surface(rng, prims, M)
    Z = round_bf16_values(_latents(rng, src, C))
    head = _decoder_weights(rng, C, F)
    lw = _local_weights(rng, C, hidden)
    weights = dict(lw, W1=round_bf16_values(head["W1"]), W2=round_bf16_values(head["W2"]), w_head=head["w_head"])
    half = n_queries // 2
    uni = rng.uniform(-1.0, 1.0, (half, 3))
    near = sample_union_surface(rng, prims, n_queries - half) + rng.normal(0.0, 0.01, (n_queries - half, 3))
    q = np.concatenate([uni, near]).astype(np.float32)
    return LocalWorkload(f"small_local_M{M}_C{C}", K, src.astype(np.float32), Z, weights, q, prims, 0.05)
