"""Adaptive KV Selection, written plainly (oracle; test infrastructure only).

Follows the FlashVDM summary page, section 4.1 item 2: split the decoded
volume into sub-volumes; in each, a few probe queries attend to every latent
token; the attention scores pick the top-K tokens for that sub-volume; every
other query of the sub-volume attends only to those tokens. The techwalker
article (part 5) describes the same probe-then-reuse scheme.

Readings (the pages leave these open):
  * sub-volumes are blocks of 8x8x8 grid points of the current level (block
    b spans indices 8b .. min(8b+7, R) on each axis), at every level;
  * the probes are the block's 8 corner points (corners make the selection
    independent of any random stream), or, as the pages describe, 8 random
    points of the block: probe n of block b takes, along axis a, the grid
    index lo_a + (u mod e_a), where lo_a is the block's first index, e_a its
    number of points along a, and u the c-th output (c = (8 b + n) * 3 + a,
    counted from 0) of the SplitMix64 stream seeded with the call's seed
    (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    2014; the mixing constants of Vigna's reference splitmix64.c);
  * a token's score for a probe is the head-mean of its softmax probability;
  * each probe keeps its top-k tokens (ties go to the lower token index); the
    block keeps the union; if the union exceeds ``cap`` tokens, those with the
    largest max-over-probes score are kept (ties to the lower index);
  * the kept set is stored in ascending token order;
  * ranking uses float32 scores (the precision a GPU kernel ranks in);
  * per-head sets (the alternative reading of the multi-head score): head h
    ranks tokens by its own softmax probability and keeps its own union and cap,
    and its attention in the sub-volume runs over that set only.
"""

from __future__ import annotations

import itertools
from typing import Dict, Optional

import numpy as np

from . import decoder as dec
from . import hvd as hv


def block_corner_indices(R: int, bijk: np.ndarray, block: int = 8) -> np.ndarray:
    """[nblk, 8, 3] grid indices of the 8 corner probes of blocks (bi, bj, bk).
    Corner order: i in {lo, hi} outermost, then j, then k."""
    bijk = np.asarray(bijk, np.int64).reshape(-1, 3)
    lo = bijk * block
    hi = np.minimum(lo + block - 1, R)
    out = np.empty((bijk.shape[0], 8, 3), np.int64)
    for n, (a, b, c) in enumerate(itertools.product((0, 1), repeat=3)):
        out[:, n, 0] = np.where(a, hi[:, 0], lo[:, 0])
        out[:, n, 1] = np.where(b, hi[:, 1], lo[:, 1])
        out[:, n, 2] = np.where(c, hi[:, 2], lo[:, 2])
    return out


MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, c: int) -> int:
    """The c-th output (from 0) of the SplitMix64 stream seeded with ``seed``:
    the state advances by the golden-ratio increment, then is mixed."""
    z = (seed + (c + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def block_random_indices(R: int, blocks: np.ndarray, NB: int, seed: int, block: int = 8) -> np.ndarray:
    """[nblk, 8, 3] grid indices of the 8 random probes of the given block ids."""
    blocks = np.asarray(blocks, np.int64).reshape(-1)
    bijk = block_ijk(blocks, NB)
    out = np.empty((blocks.size, 8, 3), np.int64)
    for r, b in enumerate(blocks.tolist()):
        for n in range(8):
            for a in range(3):
                lo = int(bijk[r, a]) * block
                ext = min(block, R + 1 - lo)
                out[r, n, a] = lo + splitmix64(seed, (8 * b + n) * 3 + a) % ext
    return out


def block_ijk(b: np.ndarray, NB: int) -> np.ndarray:
    b = np.asarray(b, np.int64)
    bi, r = np.divmod(b, NB * NB)
    bj, bk = np.divmod(r, NB)
    return np.stack([bi, bj, bk], axis=-1)


def probe_scores(Qp: np.ndarray, K: np.ndarray, H: int) -> np.ndarray:
    """[n_probe, M]: mean over heads of each probe's softmax probability."""
    return dec.attention_probs(np.asarray(Qp, np.float64), np.asarray(K, np.float64), H).mean(axis=0)


def probe_scores_per_head(Qp: np.ndarray, K: np.ndarray, H: int) -> np.ndarray:
    """[H, n_probe, M]: each head's softmax probability for each probe."""
    return dec.attention_probs(np.asarray(Qp, np.float64), np.asarray(K, np.float64), H)


def attention_per_head_sets(Q: np.ndarray, K: np.ndarray, V: np.ndarray, H: int, sets) -> np.ndarray:
    """Attention of queries Q [N, D] where head h attends only to tokens sets[h]
    (columns 64h .. 64h+63 of K and V)."""
    Q = np.asarray(Q, np.float64)
    out = np.empty_like(Q)
    for h in range(H):
        c = slice(dec.HEAD_DIM * h, dec.HEAD_DIM * (h + 1))
        t = np.asarray(sets[h])
        s_ = (Q[:, c] @ np.asarray(K, np.float64)[t][:, c].T) / np.sqrt(dec.HEAD_DIM)
        out[:, c] = dec.softmax_rows(s_) @ np.asarray(V, np.float64)[t][:, c]
    return out


def sdf_per_head_sets(decoder: dec.Decoder, xyz: np.ndarray, sets, K=None, V=None) -> np.ndarray:
    """SDF at float32 points with head h attending only to sets[h]."""
    K = decoder.K if K is None else K
    V = decoder.V if V is None else V
    xyz = np.asarray(xyz, np.float32)
    O = attention_per_head_sets(decoder.q(xyz), K, V, decoder.H, sets)
    return dec.analytic_sdf(xyz, decoder.prims) + decoder.net_scale * dec.mlp_head(O, decoder.W)


def topk_ids(score: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores; equal scores go to the lower index."""
    M = score.shape[0]
    order = np.lexsort((np.arange(M), -score))  # primary: score descending
    return order[:k]


def select(scores: np.ndarray, k: int, cap: int) -> np.ndarray:
    """Ascending token set for one block from its probes' scores [n_probe, M]."""
    s32 = np.asarray(scores, np.float64).astype(np.float32)
    union = np.unique(np.concatenate([topk_ids(s, k) for s in s32]))
    if union.size > cap:
        key = s32[:, union].max(axis=0)
        order = np.lexsort((union, -key))
        union = np.sort(union[order[:cap]])
    return union


def near_tie_tokens(scores: np.ndarray, k: int, cap: Optional[int] = None, rel: float = 1e-4) -> np.ndarray:
    """Tokens whose membership in the block's set can flip under a relative
    perturbation ``rel`` of the scores [n_probe, M] (the tie window of the
    selection):

    * top-k stage: tokens whose score, for some probe, lies within ``rel`` of
      that probe's k-th largest score;
    * cap stage (``cap`` given and the union of the probes' top-k sets, as
      ``select`` forms it, larger than ``cap``): union tokens whose
      max-over-probes score lies within ``rel`` of the cap-th largest such
      score, the cutoff of the cap.
    """
    s = np.asarray(scores, np.float64)
    amb = np.zeros(s.shape[1], bool)
    for row in s:
        kth = np.sort(row)[::-1][k - 1]
        amb |= np.abs(row - kth) <= rel * abs(kth)
    if cap is not None:
        s32 = s.astype(np.float32)
        union = np.unique(np.concatenate([topk_ids(r, k) for r in s32]))
        if union.size > cap:
            key = s[:, union].max(axis=0)
            cut = np.sort(key)[::-1][cap - 1]
            amb[union[np.abs(key - cut) <= rel * abs(cut)]] = True
    return np.flatnonzero(amb)


def select_blocks(decoder: dec.Decoder, R: int, blocks: np.ndarray, k: int, cap: int,
                  block: int = 8, Qfn=None, probes: str = "corners", seed: int = 0,
                  heads: bool = False) -> Dict[int, np.ndarray]:
    """Token sets for the given block ids of the R-cell grid. ``Qfn`` maps
    float32 probe points to projections (default: the oracle's own). ``probes``:
    "corners" or "random" (SplitMix64 stream seeded with ``seed``). ``heads``:
    one set per head (a list of H arrays per block) instead of one per block."""
    NB = hv.nblocks(R + 1, block)
    if probes == "random":
        idx = block_random_indices(R, blocks, NB, seed, block)
    else:
        idx = block_corner_indices(R, block_ijk(blocks, NB), block)
    out = {}
    for n, b in enumerate(np.asarray(blocks, np.int64)):
        pts = dec.grid_coord(idx[n], R).astype(np.float32)
        Qp = decoder.q(pts) if Qfn is None else Qfn(pts)
        if heads:
            sc = probe_scores_per_head(Qp, decoder.K, decoder.H)
            out[int(b)] = [select(sc[h], k, cap) for h in range(decoder.H)]
        else:
            out[int(b)] = select(probe_scores(Qp, decoder.K, decoder.H), k, cap)
    return out


def make_decode(decoder: dec.Decoder, k: int, cap: int, block: int = 8, record: Optional[dict] = None,
                probes: str = "corners", seed: int = 0, heads: bool = False):
    """A ``decode(R, lin)`` for ``hvd.hvd`` that groups the queries by block,
    selects each block's tokens with its probes (random probes: the level with
    R cells uses the stream seeded with seed + R), and decodes the block's
    queries against those tokens only."""

    def decode(R: int, lin: np.ndarray) -> np.ndarray:
        P = R + 1
        blk = hv.block_of(lin, P, block)
        ub = np.unique(blk)
        sets = select_blocks(decoder, R, ub, k, cap, block, probes=probes, seed=(seed + R) & MASK64, heads=heads)
        if record is not None:
            record[R] = sets
        out = np.empty(lin.size, np.float64)
        pts = dec.grid_points(R, lin)
        for b in ub:
            m = blk == b
            sel = sets[int(b)]
            if heads:
                out[m] = sdf_per_head_sets(decoder, pts[m], sel)
            else:
                out[m] = decoder.sdf(pts[m], decoder.K[sel], decoder.V[sel])
        return out

    return decode
