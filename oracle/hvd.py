"""Hierarchical Volume Decoding, written plainly (oracle; test infrastructure only).

Follows the FlashVDM summary page, section 4.1 item 1: decode the whole
volume on a coarse grid; find the voxels the surface passes through (the SDF
sign differs between neighbouring samples); split those voxels into
higher-resolution children and query only the new positions; repeat up to the
target resolution. Its key-details paragraph adds two fixes against holes:
voxels whose truncated SDF is below a threshold are also kept (thin
structures), and the kept set is dilated once by its neighbours. The
techwalker article (part 2) adds that regions wholly inside or outside skip
the detailed computation and keep their inside/outside label.

Readings (the pages leave these open):
  * level L has R_L = R_0 * 2^L cells and R_L + 1 points per axis;
  * a cell is tested when its 8 corners were all computed at level L (every
    cell at level 0; the 8 children of each kept parent afterwards);
  * a tested cell is active when its corner values include both s < 0 and
    s >= 0, or when the smallest |s| over its corners is below tau
    (the band test on the decoded SDF stands in for the trained tSDF head);
  * active cells are dilated with the 3x3x3 (26-neighbour) stencil, clipped
    at the border, ``dilation`` times;
  * every corner of every child of a kept cell is a candidate; candidates not
    computed before are the next level's queries;
  * every other point inherits the value of its nearest ancestor, the point
    (floor(I/2), floor(J/2), floor(K/2)) of the previous level;
  * decisions are taken on float32 values (the precision of the volume).

Lists hold row-major linear indices (I*P + J)*P + K ordered by the blocked
key: 8x8x8-point blocks in row-major block order, row-major inside a block.
"""

from __future__ import annotations

import itertools
from typing import Callable, Dict, List

import numpy as np

BLOCK = 8


def nblocks(P: int, block: int = BLOCK) -> int:
    return -(-P // block)


def blocked_key(lin: np.ndarray, P: int, block: int = BLOCK) -> np.ndarray:
    lin = np.asarray(lin, np.int64)
    I, r = np.divmod(lin, P * P)
    J, K = np.divmod(r, P)
    NB = nblocks(P, block)
    b = ((I // block) * NB + J // block) * NB + K // block
    loc = ((I % block) * block + J % block) * block + K % block
    return b * block ** 3 + loc


def block_of(lin: np.ndarray, P: int, block: int = BLOCK) -> np.ndarray:
    return blocked_key(lin, P, block) // block ** 3


def blocked_order(mask3: np.ndarray) -> np.ndarray:
    """Linear indices of the set points of a (P,P,P) mask, in blocked order."""
    P = mask3.shape[0]
    lin = np.flatnonzero(mask3.reshape(-1))
    return lin[np.argsort(blocked_key(lin, P), kind="stable")]


def cell_test(vol3: np.ndarray, tested: np.ndarray, tau: float) -> np.ndarray:
    """Active cells of a (P,P,P) float32 volume among the ``tested`` (R,R,R) cells."""
    v = np.asarray(vol3, np.float32)
    R = v.shape[0] - 1
    cs = [v[a:a + R, b:b + R, c:c + R] for a, b, c in itertools.product((0, 1), repeat=3)]
    neg = np.zeros((R, R, R), bool)
    nonneg = np.zeros((R, R, R), bool)
    minabs = np.full((R, R, R), np.inf, np.float32)
    for c in cs:
        neg |= c < 0
        nonneg |= c >= 0
        minabs = np.minimum(minabs, np.abs(c))
    return tested & ((neg & nonneg) | (minabs < np.float32(tau)))


def dilate(mask: np.ndarray, times: int = 1) -> np.ndarray:
    """OR over the 3x3x3 neighbourhood (cells outside the grid count as unset)."""
    m = mask.copy()
    R = m.shape[0]
    for _ in range(times):
        pad = np.zeros((R + 2,) * 3, bool)
        pad[1:-1, 1:-1, 1:-1] = m
        out = np.zeros_like(m)
        for a, b, c in itertools.product((0, 1, 2), repeat=3):
            out |= pad[a:a + R, b:b + R, c:c + R]
        m = out
    return m


def children(mask: np.ndarray) -> np.ndarray:
    """Each cell of an (R,R,R) mask -> its 2x2x2 children at the next level."""
    return mask.repeat(2, 0).repeat(2, 1).repeat(2, 2)


def candidates(kept: np.ndarray) -> np.ndarray:
    """Points of the next level that are corners of a child of a kept cell."""
    ch = children(kept)
    n = ch.shape[0]
    cand = np.zeros((n + 1,) * 3, bool)
    for a, b, c in itertools.product((0, 1), repeat=3):
        cand[a:a + n, b:b + n, c:c + n] |= ch
    return cand


def upsample(vol3: np.ndarray) -> np.ndarray:
    """Next-level volume where every point holds its nearest ancestor's value."""
    P = vol3.shape[0]
    idx = np.arange(2 * P - 1) // 2
    return vol3[np.ix_(idx, idx, idx)]


def refine_step(vol3: np.ndarray, computed: np.ndarray, tested: np.ndarray, tau: float,
                dilation: int = 1) -> Dict[str, np.ndarray]:
    """One level transition from level-L data, without decoding.

    Returns the level-L active and kept (dilated) cells, the next level's
    query list (blocked order), its inherited volume (before the new queries
    are written), its 'computed before' mask and its tested cells."""
    active = cell_test(vol3, tested, tau)
    kept = dilate(active, dilation) if dilation > 0 else active.copy()
    cand = candidates(kept)
    P1 = cand.shape[0]
    prev = np.zeros((P1,) * 3, bool)
    prev[::2, ::2, ::2] = computed
    new = cand & ~prev
    return {
        "active": active,
        "kept": kept,
        "list": blocked_order(new),
        "vol_inherited": upsample(vol3),
        "computed_next": prev | new,
        "tested_next": children(kept),
    }


def hvd(decode: Callable[[int, np.ndarray], np.ndarray], R0: int, levels: int, tau: float,
        dilation: int = 1) -> Dict[str, object]:
    """The level loop. ``decode(R, lin)`` returns SDF values at grid points
    ``lin`` (blocked order) of the R-cell grid. Values are stored as decoded
    (float64 from the oracle decoder) and decisions use their float32
    rounding."""
    P = R0 + 1
    lin = blocked_order(np.ones((P,) * 3, bool))
    vol = np.empty(P ** 3, np.float64)
    vol[lin] = decode(R0, lin)
    vol3 = vol.reshape((P,) * 3)
    computed = np.ones((P,) * 3, bool)
    tested = np.ones((R0,) * 3, bool)
    R = R0
    levels_out: List[Dict[str, object]] = []
    for L in range(levels):
        rec: Dict[str, object] = {"R": R, "list": lin, "vol": vol3.copy(), "tested": tested}
        if L == levels - 1:
            rec["active"] = cell_test(vol3.astype(np.float32), tested, tau)
            levels_out.append(rec)
            break
        st = refine_step(vol3.astype(np.float32), computed, tested, tau, dilation)
        rec["active"], rec["kept"] = st["active"], st["kept"]
        levels_out.append(rec)
        R *= 2
        lin = st["list"]
        # inherited values come from the float64 volume, not its float32 copy
        nxt = upsample(vol3).reshape(-1).copy()
        if lin.size:
            nxt[lin] = decode(R, lin)
        vol3 = nxt.reshape((R + 1,) * 3)
        computed = st["computed_next"]
        tested = st["tested_next"]
    return {"vol": vol3, "levels": levels_out}


def stats(result: Dict[str, object]) -> List[Dict[str, float]]:
    """Per-level counts and fractions: tested/active/kept cells over R^3,
    queries over (R+1)^3."""
    out = []
    for rec in result["levels"]:
        R = rec["R"]
        d = {
            "R": R,
            "tested": int(np.count_nonzero(rec["tested"])),
            "active": int(np.count_nonzero(rec["active"])),
            "queries": int(np.asarray(rec["list"]).size),
        }
        if "kept" in rec:
            d["kept"] = int(np.count_nonzero(rec["kept"]))
        d["active_frac"] = d["active"] / R ** 3
        d["query_frac"] = d["queries"] / (R + 1) ** 3
        out.append(d)
    return out


def near_threshold_cells(vol3: np.ndarray, tau: float, window: float = 1e-4) -> np.ndarray:
    """Cells with a corner value within ``window`` of 0 or of +-tau: their
    decision can flip under a perturbation of that size."""
    v = np.asarray(vol3, np.float64)
    R = v.shape[0] - 1
    near = np.zeros((R, R, R), bool)
    for a, b, c in itertools.product((0, 1), repeat=3):
        cv = v[a:a + R, b:b + R, c:c + R]
        near |= (np.abs(cv) < window) | (np.abs(np.abs(cv) - tau) < window)
    return near
