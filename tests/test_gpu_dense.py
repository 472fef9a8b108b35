"""GPU parity of the dense decoder path through the C ABI against the oracle:
K/V projection, fused embedding + Q projection, and the full decode (fp32 tiny
workload, bf16 1024-wide decoder on ragged point sets, grids and lists), plus
special cases with closed forms and run-to-run determinism."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from oracle import decoder as odec
from oracle.bf16 import round_bf16
from tests.helpers import (DECODE_TILE, TOL_BF16, TOL_F32, bf16_close, tile_sample, dev, f64, gpu_decoder, gpu_kv, oracle_decoder,
                           report, tdtype)

pytestmark = pytest.mark.gpu


def V():
    import shape_vae_decoding_amd as mod

    return mod


@pytest.mark.parametrize("cid", [0, 1, 4])
def test_kv_projection(cid):
    w = W.make(cid)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    torch.cuda.synchronize()
    od = oracle_decoder(w)
    Zabs = np.abs(w.Z.astype(np.float64))
    for name, g, r, Wm in (("K", f64(K), od.K, w.weights["Wk"]), ("V", f64(Vv), od.V, w.weights["Wv"])):
        d = np.abs(g - r)
        if w.dtype == "bf16":
            ok = bf16_close(g, r, Zabs @ np.abs(Wm.astype(np.float64)).T, w.D)
            assert np.all(ok), (name, np.argwhere(~ok)[:5], g[~ok][:5], r[~ok][:5])
            frac = np.mean(d > 0)
            print(f"[parity] {name} c{cid}: {frac:.2%} elements one bf16 step apart", flush=True)
            assert frac < 0.02
        else:
            report(f"{name} c{cid}", d.max(), 1e-5)
            assert d.max() <= 1e-5 * max(1.0, np.abs(r).max())


@pytest.mark.parametrize("cid", [0, 1])
def test_embed_queries(cid):
    w = W.make(cid)
    dec = gpu_decoder(w)
    xyz = np.concatenate([W.gen.random_points(5, 1000), odec.grid_points(6)])  # 1343: ragged last tile
    Q = torch.empty((xyz.shape[0], w.D), dtype=tdtype(w), device=dev())
    V().vdm_embed_queries(dec, torch.from_numpy(xyz).to(dev()), Q)
    torch.cuda.synchronize()
    e = odec.embed(xyz)
    ref = odec.qproj(e, w.weights["Wq"], w.dtype)
    g = f64(Q)
    d = np.abs(g - ref)
    if w.dtype == "bf16":
        ok = bf16_close(g, ref, np.abs(e) @ np.abs(w.weights["Wq"].astype(np.float64)).T, 64)
        assert np.all(ok), (np.argwhere(~ok)[:5], g[~ok][:5], ref[~ok][:5])
        print(f"[parity] Q c{cid}: {np.mean(d > 0):.3%} elements one bf16 step apart", flush=True)
        assert np.mean(d > 0) < 0.01
    else:
        report("Q c0", d.max(), 1e-5)
        assert d.max() <= 2e-6 * max(1.0, np.abs(ref).max())


def test_dense_tiny_fp32_grid():
    w = W.make(0)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = w.query["R"]
    sdf = torch.empty((R + 1) ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, sdf)
    torch.cuda.synchronize()
    ref = oracle_decoder(w).sdf_grid(R)
    err = np.abs(f64(sdf) - ref).max()
    report("tiny fp32 17^3", err, TOL_F32)
    assert err <= TOL_F32


def _bf16_identical_inputs(w, K, Vv):
    """Oracle decoder fed the GPU's K/V (identical inputs for the attention)."""
    od = oracle_decoder(w)
    od.K, od.V = f64(K), f64(Vv)
    return od


@pytest.mark.parametrize("n", [1, 37, 1000, 4097])
def test_dense_bf16_points_ragged(n):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    xyz = W.gen.random_points(100 + n, n, -1.05, 1.05)
    sdf = torch.empty(n, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(dev())), K, Vv, sdf)
    torch.cuda.synchronize()
    od = _bf16_identical_inputs(w, K, Vv)
    ref = od.sdf(xyz)
    err = np.abs(f64(sdf) - ref).max()
    report(f"bf16 points n={n}", err, TOL_BF16)
    assert err <= TOL_BF16
    # the oracle's own K/V (not the GPU's) agree as well
    err2 = np.abs(f64(sdf) - oracle_decoder(w).sdf(xyz)).max()
    report(f"bf16 points n={n} (oracle K/V)", err2, TOL_BF16)
    assert err2 <= TOL_BF16


def test_dense_small_decoder_bf16_d64():
    w = W.gen.small_decoder(41, 64, 128, 100, "bf16")
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 13
    sdf = torch.empty((R + 1) ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, sdf)
    torch.cuda.synchronize()
    od = _bf16_identical_inputs(w, K, Vv)
    err = np.abs(f64(sdf) - od.sdf_grid(R)).max()
    report("bf16 D=64 M=100 14^3", err, TOL_BF16)
    assert err <= TOL_BF16


@pytest.mark.parametrize("D,F,dtype", [(256, 256, "bf16"), (256, 768, "bf16"), (256, 4096, "bf16"),
                                       (64, 64, "bf16"), (64, 64, "f32"), (64, 192, "f32")])
def test_dense_mlp_widths(D, F, dtype):
    # the epilogue's weight ring runs through Wo, then W1 and W2 per hidden chunk
    # (256 wide for D = 256, 64 for D = 64): one chunk, an odd count and the
    # widest MLP the library accepts, over a ragged grid (13^3 = 2,197 points:
    # 17 tiles, the last one partial) and a ragged token count
    w = W.gen.small_decoder(90 + F + D, D, F, 100, dtype)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 12
    sdf = torch.empty((R + 1) ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, sdf)
    torch.cuda.synchronize()
    od = _bf16_identical_inputs(w, K, Vv) if dtype == "bf16" else oracle_decoder(w)
    err = np.abs(f64(sdf) - od.sdf_grid(R)).max()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    report(f"{dtype} D={D} F={F} 13^3", err, tol)
    assert err <= tol


def test_dense_modes_agree_bitwise():
    # every query's value depends only on its own position: grid, list and point
    # modes (different tile compositions) give identical bits
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 20
    P3 = (R + 1) ** 3
    d = dev()
    a = torch.empty(P3, dtype=torch.float32, device=d)
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, a)
    perm = np.random.default_rng(3).permutation(P3).astype(np.int32)
    b = torch.empty(P3, dtype=torch.float32, device=d)
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(perm).to(d)), K, Vv, b)
    xyz = odec.grid_points(R)[perm]
    c = torch.empty(P3, dtype=torch.float32, device=d)
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(d)), K, Vv, c)
    torch.cuda.synchronize()
    A = a.cpu().numpy()
    assert np.array_equal(A[perm], b.cpu().numpy())
    assert np.array_equal(A[perm], c.cpu().numpy())


def test_dense_deterministic():
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 40
    outs = []
    for _ in range(2):
        s = torch.empty((R + 1) ** 3, dtype=torch.float32, device=dev())
        V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, s)
        outs.append(s.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("cid", [0, 1])
def test_softmax_normalises_constant_values(cid):
    # V = 1 for every token: each head's output is sum_j p_j / sum_j p_j = 1 for any
    # logits, so the network term is the same constant at every query
    w = W.make(cid)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    ones = torch.ones_like(K)
    xyz = W.gen.random_points(7, 3000)
    sdf = torch.empty(3000, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(dev())), K, ones, sdf)
    torch.cuda.synchronize()
    od = oracle_decoder(w)
    net_ref = odec.mlp_head(np.ones((1, w.D)), od.W)[0]
    ref = odec.analytic_sdf(xyz, w.prims) + od.net_scale * net_ref
    err = np.abs(f64(sdf) - ref).max()
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    report(f"V=1 c{cid}", err, tol)
    assert err <= tol


def test_token_permutation_invariance():
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.M)).to(dev())
    xyz = torch.from_numpy(W.gen.random_points(8, 2000)).to(dev())
    a = torch.empty(2000, dtype=torch.float32, device=dev())
    b = torch.empty(2000, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(xyz), K, Vv, a)
    V().vdm_decode_dense(dec, V().queries_points(xyz), K[perm].contiguous(), Vv[perm].contiguous(), b)
    torch.cuda.synchronize()
    err = (a - b).abs().max().item()
    report("token permutation", err, TOL_BF16)
    assert err <= TOL_BF16


def test_dense_full_grid_129_one_query_per_tile():
    # the 129^3 dense workload, in the launch configuration the benchmark times:
    # one query of every 128-query tile (16,771 tiles; the lane offset rotates
    # from tile to tile), plus the first 200 points and the last one
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = w.query["R"]
    n = (R + 1) ** 3
    sdf = torch.empty(n, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, sdf)
    torch.cuda.synchronize()
    out = sdf.cpu().numpy()
    bq = DECODE_TILE
    lin = np.unique(np.concatenate([tile_sample(n, bq), np.arange(0, 200), [n - 1]]))
    assert np.unique(lin // bq).size == -(-n // bq)
    od = _bf16_identical_inputs(w, K, Vv)
    ref = od.sdf(odec.grid_points(R, lin))
    err = np.abs(out[lin].astype(np.float64) - ref).max()
    report(f"129^3, one query per tile ({lin.size} points)", err, TOL_BF16)
    assert err <= TOL_BF16
    assert np.all(np.isfinite(out))


def test_large_token_set_one_query_per_tile():
    # the 40,960-token x 200K-query workload: one query of every 128-query tile
    w = W.make(4)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    xyz = w.query["xyz"]
    n = xyz.shape[0]
    sdf = torch.empty(n, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(dev())), K, Vv, sdf)
    torch.cuda.synchronize()
    out = sdf.cpu().numpy()
    assert np.all(np.isfinite(out))
    idx = tile_sample(n, DECODE_TILE)
    od = _bf16_identical_inputs(w, K, Vv)
    ref = od.sdf(xyz[idx], chunk=64)
    err = np.abs(out[idx].astype(np.float64) - ref).max()
    report(f"200K x 40960, one query per tile ({idx.size} points)", err, TOL_BF16)
    assert err <= TOL_BF16


def _unseen_key_inputs(w, dec, K, norm=400.0, token=7):
    """The GPU's K with one token given a large component outside every head's
    query span (vdm_workloads.with_unseen_key), on the device, and the oracle
    decoder fed the same K and V."""
    K2 = W.with_unseen_key(f64(K), w.weights["Wq"], w.H, token, norm, w.dtype)
    return torch.from_numpy(K2).to(dev()).to(tdtype(w))


@pytest.mark.parametrize("cid", [1, 0])
def test_dense_key_outside_query_span(cid):
    # One key with a large component that no query sees makes the Cauchy-Schwarz
    # logit bound B exceed the true maximum logit by more than 213 (base 2) for
    # every query here (checked below with the oracle's numbers): a softmax
    # shifted by the bound alone would underflow to an all-zero row sum. The
    # decode must stay finite and within tolerance of the oracle on the same K.
    w = W.make(cid)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    K2 = _unseen_key_inputs(w, dec, K)
    n = 4097 if cid == 1 else 1000  # ragged last tile
    xyz = W.gen.random_points(300 + cid, n, -1.05, 1.05)
    od = oracle_decoder(w)
    od.K, od.V = f64(K2), f64(Vv)
    q = odec.qproj(odec.embed(xyz), od.W["Wq"], od.dtype) * (np.log2(np.e) / 8)
    gaps = []
    for h in range(w.H):
        c = slice(64 * h, 64 * h + 64)
        B = 1.00390625 * np.linalg.norm(q[:, c], axis=1) * np.linalg.norm(od.K[:, c], axis=1).max()
        gaps.append(B - (q[:, c] @ od.K[:, c].T).max(axis=1))
    gap = np.min(gaps, axis=0)
    print(f"[unseen key] c{cid}: bound minus max logit, min {gap.min():.1f}, median {np.median(gap):.1f}",
          flush=True)
    assert np.mean(gap > 213) > 0.9
    sdf = torch.empty(n, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(dev())), K2, Vv, sdf)
    torch.cuda.synchronize()
    out = f64(sdf)
    assert np.all(np.isfinite(out))
    tol = TOL_BF16 if w.dtype == "bf16" else TOL_F32
    err = np.abs(out - od.sdf(xyz)).max()
    report(f"key outside the query span, c{cid}", err, tol)
    assert err <= tol


def _head_gain_weights(w, gains):
    """Wq with the rows of head h multiplied by gains[h] (powers of two, so the
    bf16 weights stay exact): larger logit bounds for chosen heads."""
    weights = dict(w.weights)
    weights["Wq"] = (w.weights["Wq"] * np.repeat(np.asarray(gains, np.float32), 64)[:, None]).astype(np.float32)
    return weights


def _logit_bounds(od, xyz, H):
    """Per head and query: |q|_2 max_j |k_j|_2 log2(e)/sqrt(64), the bound of the
    base-2 logits (oracle Q and K)."""
    q = odec.qproj(odec.embed(xyz), od.W["Wq"], od.dtype)
    c = np.log2(np.e) / 8
    return np.stack([np.linalg.norm(q[:, 64 * h:64 * h + 64], axis=1)
                     * np.linalg.norm(od.K[:, 64 * h:64 * h + 64], axis=1).max() * c for h in range(H)])


@pytest.mark.parametrize("gains", [(8, 8, 8, 8), (16, 1, 1, 1)])
def test_large_logits_shifted_softmax(gains):
    # Logit bounds above 64 (base 2) make a wave shift its softmax. Gain 8 puts
    # about a third of the queries of every head above the bound; gain 16 on head 0
    # alone puts all of that head's waves on the shifted path beside unshifted
    # waves of the other heads in every workgroup. The tolerance covers rounding q
    # after the logit scale rather than before it (the oracle rounds q itself):
    # that placement alone moves the SDF by up to 8.4e-4 at gain 16.
    w = W.make(1)
    weights = _head_gain_weights(w, gains)
    dec = gpu_decoder(w, weights=weights)
    K, Vv = gpu_kv(dec, w)
    xyz = W.gen.random_points(11, 3000)
    od = oracle_decoder(w, weights=weights)
    B = _logit_bounds(od, xyz, w.H)
    frac = (B > 64).mean(axis=1)
    assert frac[0] > 0.2 and (gains[1] > 1 or frac[1:].max() == 0.0), frac
    sdf = torch.empty(3000, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_points(torch.from_numpy(xyz).to(dev())), K, Vv, sdf)
    torch.cuda.synchronize()
    ref = od.sdf(xyz, f64(K), f64(Vv))
    err = np.abs(f64(sdf) - ref).max()
    report(f"logit gains {gains} (queries above the bound per head {np.round(frac, 2)})", err, TOL_BF16)
    assert np.all(np.isfinite(f64(sdf)))
    assert err <= TOL_BF16


@pytest.mark.parametrize("mode", ["grid", "points"])
def test_batched_decode_equals_single_shape_calls_bitwise(mode):
    # B vecsets in one decode launch: every shape's SDF equals its own vdm_decode_dense
    # call bit for bit; shape 0 against the oracle on a sample
    w = W.make(1)
    dec = gpu_decoder(w)
    rng = np.random.default_rng(21)
    Zs = [w.Z] + [w.Z * np.float32(0.8) + np.float32(0.2) * rng.standard_normal(w.Z.shape).astype(np.float32)
                  for _ in range(2)]
    KV = [gpu_kv(dec, w, Z) for Z in Zs]
    K = torch.stack([k for k, _ in KV]).contiguous()
    Vv = torch.stack([v for _, v in KV]).contiguous()
    if mode == "grid":
        R = 24
        q = V().queries_grid(R)
    else:
        xyz = torch.from_numpy(rng.uniform(-1, 1, (1001, 3)).astype(np.float32)).to(dev())
        q = V().queries_points(xyz)
    print(f"[batch] {mode}: B={len(Zs)} N={q.N}", flush=True)
    out = torch.empty((len(Zs), q.N), dtype=torch.float32, device=dev())
    V().vdm_decode_dense_batch(dec, q, K, Vv, out)
    for b in range(len(Zs)):
        one = torch.empty(q.N, dtype=torch.float32, device=dev())
        V().vdm_decode_dense(dec, q, K[b], Vv[b], one)
        torch.cuda.synchronize()
        assert torch.equal(out[b], one), b
    # a batch of one is the single call
    one = torch.empty((1, q.N), dtype=torch.float32, device=dev())
    V().vdm_decode_dense_batch(dec, q, K[1:2].contiguous(), Vv[1:2].contiguous(), one)
    torch.cuda.synchronize()
    assert torch.equal(one[0], out[1])
    od = oracle_decoder(w)
    od.K, od.V = f64(K[0]), f64(Vv[0])
    pick = np.sort(rng.choice(q.N, 200, replace=False))
    ref = od.sdf_grid(R, pick) if mode == "grid" else od.sdf(f64(xyz)[pick])
    err = np.abs(out[0].cpu().numpy()[pick].astype(np.float64) - ref).max()
    report(f"batched decode ({mode}), shape 0 vs oracle", err, TOL_BF16)
    assert err <= TOL_BF16


def test_device_info_matches_the_runtime():
    # compute units as torch reports them; a peak shader clock in a plausible range
    di = V().vdm_device_info()
    props = torch.cuda.get_device_properties(0)
    assert di["compute_units"] == props.multi_processor_count
    assert 500_000 <= di["peak_clock_khz"] <= 5_000_000, di
