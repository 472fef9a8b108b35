"""Shared helpers for the GPU parity tests (the GPU side goes through the C ABI
binding; the reference side is the oracle)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import decoder as odec

TOL_BF16 = 2e-3  # max |dSDF| for bf16 decoders
TOL_F32 = 1e-5   # max |dSDF| for fp32 decoders
DECODE_TILE = 128  # queries per decode work item, for every supported decoder


def dev():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    return torch.device("cuda:0")


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def gpu_decoder(w, net_scale=None, weights=None, prims=None):
    import shape_vae_decoding_amd as V

    d = dev()
    W = weights if weights is not None else w.weights
    wt = {}
    for k, v in W.items():
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(d)
        wt[k] = t if k == "w_head" else t.to(tdtype(w))
    return V.Decoder(wt, prims if prims is not None else w.prims, w.net_scale if net_scale is None else net_scale)


def gpu_kv(dec, w, Z=None):
    import shape_vae_decoding_amd as V

    Zt = torch.from_numpy(np.ascontiguousarray(w.Z if Z is None else Z, np.float32)).to(dev()).to(tdtype(w))
    K = torch.empty_like(Zt)
    Vv = torch.empty_like(Zt)
    V.vdm_project_kv(dec, Zt, K, Vv)
    return K, Vv


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_decoder(w, net_scale=None, weights=None, prims=None):
    return odec.Decoder(weights if weights is not None else w.weights, w.Z,
                        prims if prims is not None else w.prims, w.dtype,
                        w.net_scale if net_scale is None else net_scale, w.H)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^-7 relative)."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(np.maximum(x, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def bf16_close(g: np.ndarray, r: np.ndarray, abs_terms: np.ndarray, n_terms: int) -> np.ndarray:
    """Both sides round a dot product to bf16: the GPU from an fp32 sum (error at
    most n_terms * 2^-24 * sum |terms|), the oracle from the exact value. They agree
    to one bf16 step plus that accumulation error (which matters only where the
    terms cancel to a small result)."""
    return np.abs(g - r) <= ulp_bf16(r) * 1.0001 + 2.0 * n_terms * 2.0 ** -24 * abs_terms


def report(name, err, tol):
    print(f"[parity] {name}: max|d| = {err:.3e} (tol {tol:.1e})", flush=True)


def tile_sample(n, bq):
    """One index in each bq-query tile of [0, n): tile t takes lane (37 t) mod bq,
    the last tile its last query if that lane lies past n."""
    t = np.arange(-(-n // bq), dtype=np.int64)
    return np.minimum(bq * t + (37 * t) % bq, n - 1)
