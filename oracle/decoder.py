"""The vecset decoder, written plainly (oracle; test infrastructure only).

What it computes follows the FlashVDM summary page ("Unleashing Vecset
Diffusion Model for Fast Shape Generation"), section 3: the decoder maps
a set of latent tokens to the SDF at any query point by cross-attention
from the query point to the tokens; section 4.1 item 3 describes the slim
decoder (narrower width, lower MLP ratio, fewer LayerNorms). The pages do
not print the layer equations, so this module takes the plainest reading:

  e(p)   = [x, y, z, sin(f_k x).., sin(f_k y).., sin(f_k z).., cos(same)]
           with f_k = 2^k * pi, k = 0..7                       (51 dims)
  q      = Wq e                                    (no bias, no extra layer)
  k_j    = Wk z_j,  v_j = Wv z_j
  per head h (columns 64h..64h+63):
  o_h    = sum_j softmax_j(q_h . k_hj / sqrt(64)) v_hj
  a      = Wo [o_0 .. o_{H-1}]
  y      = a + W2 GELU(W1 a)                 (exact erf GELU, residual)
  net    = w_head . y
  SDF(p) = analytic(p) + net_scale * net

No LayerNorm and no biases (the slim design removes LayerNorms; the
synthetic decoder has none). Every quantity is float64 except the
two rounding points a bf16 decoder exposes at its interface (Q and K/V),
which ``dtype="bf16"`` reproduces with ``bf16.round_bf16``.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
from scipy.special import erf

from .bf16 import round_bf16

N_FREQ = 8
E_DIM = 51
HEAD_DIM = 64


# ---------------------------------------------------------------- geometry

def grid_coord(i, R: int) -> np.ndarray:
    """Coordinate of grid index i on a grid of R cells (R+1 points) over
    [-1, 1]: the float32 value nearest to 2i/R - 1, i.e. the float32
    quotient of the exact integers (2i - R) and R. Index 2i on the 2R grid
    therefore gives the same float32 value as index i on the R grid."""
    i = np.asarray(i, dtype=np.int64)
    num = (2 * i - R).astype(np.float32)
    return num / np.float32(R)  # IEEE float32 division, correctly rounded


def grid_points(R: int, lin: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 [N,3] coordinates of grid points (row-major linear index,
    x slowest, z fastest). All (R+1)^3 points when ``lin`` is None."""
    P = R + 1
    if lin is None:
        lin = np.arange(P ** 3, dtype=np.int64)
    lin = np.asarray(lin, dtype=np.int64)
    i, r = np.divmod(lin, P * P)
    j, k = np.divmod(r, P)
    return np.stack([grid_coord(i, R), grid_coord(j, R), grid_coord(k, R)], axis=1)


# ---------------------------------------------------------------- embedding

def freqs_f32() -> np.ndarray:
    """f_k = 2^k * pi as float32 (the float32 of pi scaled by 2^k, exact)."""
    return (np.float32(math.pi) * (2.0 ** np.arange(N_FREQ))).astype(np.float32)


def embed(xyz: np.ndarray) -> np.ndarray:
    """Fourier embedding e(p) of float32 points, [N,3] -> float64 [N,51].

    The argument of sin/cos is the float32 product f_k * c (one rounding),
    and sin/cos are evaluated in float64 from that float32 argument.
    Layout: xyz, then sin for axis x (k=0..7), y, z, then cos in the same
    order."""
    xyz = np.asarray(xyz, dtype=np.float32)
    f = freqs_f32()
    arg = (xyz[:, :, None] * f[None, None, :]).astype(np.float32)  # float32 product
    arg = arg.astype(np.float64).reshape(xyz.shape[0], 3 * N_FREQ)
    return np.concatenate([xyz.astype(np.float64), np.sin(arg), np.cos(arg)], axis=1)


def qproj(e: np.ndarray, Wq: np.ndarray, dtype: str) -> np.ndarray:
    """q = Wq e for each row of e; bf16 decoders round q to bf16."""
    q = e @ np.asarray(Wq, np.float64).T
    return round_bf16(q) if dtype == "bf16" else q


def kv_proj(Z: np.ndarray, Wk: np.ndarray, Wv: np.ndarray, dtype: str):
    """k_j = Wk z_j, v_j = Wv z_j for every token; bf16 decoders round both."""
    Z = np.asarray(Z, np.float64)
    K = Z @ np.asarray(Wk, np.float64).T
    V = Z @ np.asarray(Wv, np.float64).T
    if dtype == "bf16":
        K, V = round_bf16(K), round_bf16(V)
    return K, V


# ---------------------------------------------------------------- attention

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first."""
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=-1, keepdims=True)


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, H: int) -> np.ndarray:
    """Multi-head cross-attention of queries Q [N,D] over tokens K,V [M,D].
    Head h uses columns 64h..64h+63; logits are scaled by 1/sqrt(64)."""
    N, D = Q.shape
    out = np.empty((N, D), np.float64)
    for h in range(H):
        c = slice(HEAD_DIM * h, HEAD_DIM * (h + 1))
        s = (Q[:, c] @ K[:, c].T) / math.sqrt(HEAD_DIM)
        out[:, c] = softmax_rows(s) @ V[:, c]
    return out


def attention_probs(Q: np.ndarray, K: np.ndarray, H: int) -> np.ndarray:
    """Softmax probabilities per head, [H, N, M] (used by KV selection)."""
    P = []
    for h in range(H):
        c = slice(HEAD_DIM * h, HEAD_DIM * (h + 1))
        P.append(softmax_rows((Q[:, c] @ K[:, c].T) / math.sqrt(HEAD_DIM)))
    return np.stack(P)


# ---------------------------------------------------------------- MLP + head

def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def mlp_head(O: np.ndarray, W: dict) -> np.ndarray:
    """net = w_head . (a + W2 GELU(W1 a)), a = Wo o."""
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    a = O @ f("Wo").T
    y = a + gelu(a @ f("W1").T) @ f("W2").T
    return y @ f("w_head")


# ---------------------------------------------------------------- analytic prior

def analytic_sdf(xyz: np.ndarray, prims: Sequence) -> np.ndarray:
    """SDF of the union of primitives = min over primitives of
    sphere: |p - c| - r;  box: |max(q, 0)| + min(max_i q_i, 0), q = |p - c| - h."""
    p = np.asarray(xyz, np.float64)
    best = np.full(p.shape[0], np.inf)
    for pr in prims:
        c = np.asarray(pr.centre, np.float64)
        if pr.kind == 0:
            d = np.sqrt(np.sum((p - c) ** 2, axis=1)) - float(pr.size[0])
        else:
            q = np.abs(p - c) - np.asarray(pr.size, np.float64)
            d = np.sqrt(np.sum(np.maximum(q, 0.0) ** 2, axis=1)) + np.minimum(q.max(axis=1), 0.0)
        best = np.minimum(best, d)
    return best


# ---------------------------------------------------------------- full decode

class Decoder:
    """A decoder instance: weights, latents and analytic prior of one shape."""

    def __init__(self, weights: dict, Z: np.ndarray, prims, dtype: str, net_scale: float = 0.05,
                 H: Optional[int] = None):
        self.W = {k: np.asarray(v, np.float64) for k, v in weights.items()}
        self.dtype = dtype
        self.D = self.W["Wq"].shape[0]
        self.H = H if H is not None else self.D // HEAD_DIM
        self.prims = list(prims)
        self.net_scale = float(np.float32(net_scale))
        self.K, self.V = kv_proj(Z, self.W["Wk"], self.W["Wv"], dtype)

    @classmethod
    def from_workload(cls, w):
        return cls(w.weights, w.Z, w.prims, w.dtype, w.net_scale, w.H)

    def q(self, xyz: np.ndarray) -> np.ndarray:
        return qproj(embed(xyz), self.W["Wq"], self.dtype)

    def net(self, xyz: np.ndarray, K=None, V=None, chunk: int = 512) -> np.ndarray:
        """Network scalar at float32 points, chunked over queries."""
        K = self.K if K is None else K
        V = self.V if V is None else V
        xyz = np.asarray(xyz, np.float32)
        out = np.empty(xyz.shape[0], np.float64)
        for s in range(0, xyz.shape[0], chunk):
            Q = self.q(xyz[s:s + chunk])
            out[s:s + chunk] = mlp_head(attention(Q, K, V, self.H), self.W)
        return out

    def sdf(self, xyz: np.ndarray, K=None, V=None, chunk: int = 512) -> np.ndarray:
        xyz = np.asarray(xyz, np.float32)
        return analytic_sdf(xyz, self.prims) + self.net_scale * self.net(xyz, K, V, chunk)

    def sdf_from_q(self, xyz: np.ndarray, Q: np.ndarray, K=None, V=None) -> np.ndarray:
        """SDF from given query projections (identical-input comparisons)."""
        K = self.K if K is None else K
        V = self.V if V is None else V
        net = mlp_head(attention(np.asarray(Q, np.float64), K, V, self.H), self.W)
        return analytic_sdf(xyz, self.prims) + self.net_scale * net

    def sdf_grid(self, R: int, lin: Optional[np.ndarray] = None, chunk: int = 512) -> np.ndarray:
        return self.sdf(grid_points(R, lin), chunk=chunk)
