"""The local KNN decoder (AVS-Conv) of the MSVS-VAE page, written plainly
(oracle; test infrastructure only).

What it computes follows the MSVS-VAE page (kwkr.cn), section 1.1: instead
of global attention, a query gathers features only from its K nearest
supports by Euclidean distance; an MLP turns each neighbour's offset relative
to the query into dynamic weights; the neighbours' features are fused by a
weighted sum, next to a mean-pooling residual branch. In the decoder the
supports are the latent tokens at their anchor positions and the queries are
grid points (section 1.1); a light network then maps the fused feature to the
SDF (section 1.3). Section 3.3 times 200K queries against 40K tokens.

Readings (the page leaves these open; the plainest reading is taken):

  * K = 16 neighbours, offset MLP of width 32 (the page gives neither);
  * neighbours: the K supports of smallest squared distance
        d_j = fl(fl(fl(dx*dx) + fl(dy*dy)) + fl(dz*dz)),  dx = fl(p_jx - x_x), ...
    evaluated in float32 (both this oracle and the GPU take this integer
    decision in float32), ascending, equal distances to the lower index;
  * offset delta_j = p_j - x (the float32 differences above);
  * dynamic weights w_j = B GELU(A delta_j + a): A [Hw, 3], a [Hw], B [C, Hw],
    exact-erf GELU, one weight per feature channel;
  * fusion h = (1/K) sum_j w_j * f_j + (1/K) sum_j f_j over the K neighbours
    (the weighted fusion as a weighted mean, beside the mean-pool residual:
    h does not grow with K);
  * head (the light network): y = h + W2 GELU(W1 h), net = w_head . y,
    SDF = analytic(x) + net_scale * net -- the slim head of the vecset
    decoder, so the two decoders differ only in how a query gathers its
    latent feature;
  * one latent scale (the multi-scale query of section 1.3 would repeat the
    gather per scale and concatenate; the synthetic supports have one scale).

Everything after the neighbour decision is float64 on the given float32 /
bf16-valued inputs.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .decoder import analytic_sdf, gelu


def sq_dist_f32(P: np.ndarray, x: np.ndarray) -> np.ndarray:
    """float32 squared distances of supports P [M,3] from one point x [3], in
    the stated order of operations (no fused multiply-add)."""
    P = np.asarray(P, np.float32)
    x = np.asarray(x, np.float32)
    d = P - x[None, :]                       # float32 differences
    sq = d * d                               # float32 products
    return (sq[:, 0] + sq[:, 1]) + sq[:, 2]  # float32 sums, x then y then z


def knn(P: np.ndarray, X: np.ndarray, K: int) -> np.ndarray:
    """[N, K] indices of each query's K nearest supports, nearest first
    (float32 squared distance ascending, then the lower index)."""
    X = np.asarray(X, np.float32)
    M = np.asarray(P).shape[0]
    out = np.empty((X.shape[0], K), np.int64)
    idx = np.arange(M)
    for n in range(X.shape[0]):
        d = sq_dist_f32(P, X[n])
        out[n] = np.lexsort((idx, d))[:K]  # primary key: d, then index
    return out


def offset_weights(delta: np.ndarray, W: dict) -> np.ndarray:
    """w = B GELU(A delta + a) for offsets delta [..., 3] -> [..., C]."""
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    u = np.asarray(delta, np.float64) @ f("A").T + f("a")
    return gelu(u) @ f("B").T


def fuse(P: np.ndarray, Fe: np.ndarray, X: np.ndarray, nbr: np.ndarray, W: dict) -> np.ndarray:
    """h [N, C] = mean_j w_j * f_j + mean_j f_j over each query's neighbours."""
    P32 = np.asarray(P, np.float32)
    X32 = np.asarray(X, np.float32)
    Fe = np.asarray(Fe, np.float64)
    K = nbr.shape[1]
    delta = (P32[nbr] - X32[:, None, :]).astype(np.float64)  # float32 differences, [N, K, 3]
    w = offset_weights(delta, W)                             # [N, K, C]
    f = Fe[nbr]                                              # [N, K, C]
    return (w * f).sum(axis=1) / K + f.sum(axis=1) / K


def head(h: np.ndarray, W: dict) -> np.ndarray:
    """net = w_head . (h + W2 GELU(W1 h))."""
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    y = h + gelu(h @ f("W1").T) @ f("W2").T
    return y @ f("w_head")


def sdf(P: np.ndarray, Fe: np.ndarray, X: np.ndarray, W: dict, K: int, prims: Sequence, net_scale: float,
        nbr: Optional[np.ndarray] = None) -> np.ndarray:
    """SDF at float32 query points X [N, 3]; ``nbr`` overrides the neighbour
    sets (identical-input comparisons)."""
    X = np.asarray(X, np.float32)
    if nbr is None:
        nbr = knn(P, X, K)
    net = head(fuse(P, Fe, X, nbr, W), W)
    return analytic_sdf(X, prims) + float(np.float32(net_scale)) * net


def sdf_of(w, X: Optional[np.ndarray] = None, nbr: Optional[np.ndarray] = None) -> np.ndarray:
    """SDF of a ``vdm_workloads.LocalWorkload`` at X (default: its queries)."""
    X = w.queries if X is None else X
    return sdf(w.xyz, w.feats, X, w.weights, w.K, w.prims, w.net_scale, nbr)
