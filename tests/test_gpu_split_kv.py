"""The tail split of the dense decode over token ranges (split-KV), through the
C ABI. With many tokens (M >= 8192) and a last round of the persistent grid at
most half full, the last round's tiles are each cut into ranges of token tiles
that run as separate work units; the last range to finish a tile adds every
range's partial O and row sums in range order and runs the epilogue.

- Parity with the oracle at every point of launches whose tiles are all split
  (fewer tiles than the grid), over 9,000 tokens, so that the last range ends in
  a partial token tile; the 40,960-token workload (split tail) is checked at one
  query per tile in test_gpu_dense.py.
- Agreement with the unsplit decode: vdm_decode_dense_noalloc never splits, and
  the two differ only in the fp32 order in which the same products are summed.
- Run-to-run bit equality: whichever range arrives last, the partials are added
  in range order.
- A key outside every query's span forces the exact-maximum softmax shift; it is
  taken over all tokens, so every range of a tile shares it."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from tests.helpers import TOL_BF16, dev, f64, gpu_decoder, gpu_kv, oracle_decoder, report, tdtype

pytestmark = pytest.mark.gpu

M_SPLIT = 9000  # 282 token tiles, the last one partial


def V():
    import shape_vae_decoding_amd as mod

    return mod


def _inputs(n, seed=0, unseen=False):
    w = W.make(4)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w, Z=w.Z[:M_SPLIT])
    if unseen:
        K2 = W.with_unseen_key(f64(K), w.weights["Wq"], w.H, 11, 400.0, w.dtype)
        K = torch.from_numpy(K2).to(dev()).to(tdtype(w))
    xyz = W.gen.random_points(seed, n, -1.05, 1.05)
    od = oracle_decoder(w)
    od.K, od.V = f64(K), f64(Vv)
    return w, dec, K, Vv, xyz, od


def _decode(dec, K, Vv, xyz, noalloc=False):
    x = torch.from_numpy(xyz).to(dev())
    sdf = torch.empty(xyz.shape[0], dtype=torch.float32, device=dev())
    if noalloc:
        V().vdm_decode_dense_noalloc(dec, V().queries_points(x), K, Vv, sdf)
    else:
        V().vdm_decode_dense(dec, V().queries_points(x), K, Vv, sdf)
    torch.cuda.synchronize()
    return sdf.cpu().numpy().astype(np.float64)


def test_split_is_planned():
    # the split's scratch shows in the workspace: a whole number of rounds (no
    # tail) needs none, a tail of 16 tiles does (grid of 256 workgroups)
    w = W.make(4)
    dec = gpu_decoder(w)
    ws = V().vdm_dense_workspace_size
    whole_rounds = ws(dec, M_SPLIT, 256 * 128)
    assert ws(dec, M_SPLIT, 2000) > whole_rounds
    assert ws(dec, 3072, 2000) == ws(dec, 3072, 256 * 128)  # fewer than 8192 tokens: never split


@pytest.mark.parametrize("n", [2000, 130, 1])
def test_split_tiles_match_oracle_at_every_point(n):
    # 16, 2 and 1 tiles: every tile split (16 ranges each)
    w, dec, K, Vv, xyz, od = _inputs(n, seed=n)
    out = _decode(dec, K, Vv, xyz)
    assert np.all(np.isfinite(out))
    err = np.abs(out - od.sdf(xyz, chunk=64)).max()
    report(f"split-KV {n} points x {M_SPLIT} tokens, every point", err, TOL_BF16)
    assert err <= TOL_BF16


def test_split_equals_unsplit_up_to_summation_order():
    w, dec, K, Vv, xyz, od = _inputs(2000, seed=5)
    split = _decode(dec, K, Vv, xyz)
    whole = _decode(dec, K, Vv, xyz, noalloc=True)
    d = np.abs(split - whole).max()
    print(f"[split-KV] max |split - unsplit| = {d:.3e}", flush=True)
    assert d <= 2e-5


def test_split_deterministic():
    w, dec, K, Vv, xyz, od = _inputs(2000, seed=6)
    a = _decode(dec, K, Vv, xyz)
    b = _decode(dec, K, Vv, xyz)
    assert np.array_equal(a, b)


def test_split_with_shifted_softmax_waves():
    w, dec, K, Vv, xyz, od = _inputs(1500, seed=7, unseen=True)
    out = _decode(dec, K, Vv, xyz)
    assert np.all(np.isfinite(out))
    err = np.abs(out - od.sdf(xyz, chunk=64)).max()
    report(f"split-KV with an unseen key, {xyz.shape[0]} points", err, TOL_BF16)
    assert err <= TOL_BF16
