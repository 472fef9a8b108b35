"""GPU parity of adaptive KV selection and the gathered decode through the C ABI.

Selection is compared on identical inputs: the oracle scores the GPU's own
probe projections (vdm_embed_queries at the same corner points) against the
GPU's K, and the selected sets must match exactly except for tokens within a
relative 1e-4 of a probe's k-th score (counted). The gathered decode is
compared with the oracle's attention restricted to the GPU's token sets."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from oracle import akvs as oak
from oracle import decoder as odec
from oracle import hvd as hv
from tests.helpers import (DECODE_TILE, TOL_BF16, dev, f64, gpu_decoder, gpu_kv, oracle_decoder, report, tdtype,
                           tile_sample)

pytestmark = pytest.mark.gpu


def V():
    import shape_vae_decoding_amd as mod

    return mod


def gpu_probe_q(dec, w, R, blocks, block=8, probes="corners", seed=0):
    NB = hv.nblocks(R + 1, block)
    if probes == "random":
        idx = oak.block_random_indices(R, blocks, NB, seed, block)
    else:
        idx = oak.block_corner_indices(R, oak.block_ijk(blocks, NB), block)
    pts = odec.grid_coord(idx.reshape(-1, 3), R).astype(np.float32)
    Q = torch.empty((pts.shape[0], w.D), dtype=tdtype(w), device=dev())
    V().vdm_embed_queries(dec, torch.from_numpy(pts).to(dev()), Q)
    return f64(Q).reshape(len(blocks), 8, w.D)


def compare_sets(dec, w, K, R, blocks, k, cap, sel_idx, sel_cnt, block=8, probes="corners", seed=0):
    Qp = gpu_probe_q(dec, w, R, blocks, block, probes, seed)
    Kh = f64(K)
    n_amb = 0
    for r, b in enumerate(blocks):
        sc = oak.probe_scores(Qp[r], Kh, w.H)
        ref = oak.select(sc, k, cap)
        got = sel_idx[r, : sel_cnt[r]]
        assert np.all(np.diff(got) > 0) and np.all(sel_idx[r, sel_cnt[r]:] == -1)
        sym = np.setxor1d(ref, got)
        if sym.size:
            amb = oak.near_tie_tokens(sc, k, cap)
            n_amb += sym.size
            assert np.all(np.isin(sym, amb)), (b, sym, got.size, ref.size)
    print(f"[parity] selection R={R} k={k} cap={cap}: {len(blocks)} blocks, {n_amb} near-tie tokens differ",
          flush=True)


def run_select(dec, w, K, R, blocks, k, cap, block=8, probes="corners", seed=0):
    nb = len(blocks)
    sel_idx = torch.empty((nb, cap), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb, dtype=torch.int32, device=dev())
    bt = torch.from_numpy(np.asarray(blocks, np.int32)).to(dev())
    V().vdm_select_kv(dec, R, block, k, cap, K, bt, sel_idx, sel_cnt, probes=probes, seed=seed)
    torch.cuda.synchronize()
    return sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()


@pytest.mark.parametrize("R,k,cap,block", [(75, 64, 512, 8), (75, 64, 100, 8), (150, 32, 512, 8), (75, 64, 512, 16),
                                           (150, 64, 512, 4)])
def test_select_matches_oracle(R, k, cap, block):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    nb = hv.nblocks(R + 1, block)
    blocks = np.sort(np.random.default_rng(R + k + cap).choice(nb ** 3, 60, replace=False))
    blocks = np.unique(np.concatenate([blocks, [0, nb ** 3 - 1]]))  # include the ragged corner block
    sel_idx, sel_cnt = run_select(dec, w, K, R, blocks, k, cap, block)
    assert np.all(sel_cnt <= cap) and np.all(sel_cnt >= k)
    if cap == 100:
        assert np.all(sel_cnt == 100)  # the cap binds: 8 probes x 64 exceed it
    compare_sets(dec, w, K, R, blocks, k, cap, sel_idx, sel_cnt, block)


@pytest.mark.parametrize("R,seed", [(75, 0), (150, 0x0123456789ABCDEF)])
def test_select_with_random_probes_matches_oracle(R, seed):
    # the pages' own probes: 8 random points per block from the SplitMix64 stream
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    nb = hv.nblocks(R + 1)
    blocks = np.sort(np.random.default_rng(R).choice(nb ** 3, 60, replace=False))
    blocks = np.unique(np.concatenate([blocks, [0, nb ** 3 - 1]]))
    sel_idx, sel_cnt = run_select(dec, w, K, R, blocks, 64, 512, probes="random", seed=seed)
    compare_sets(dec, w, K, R, blocks, 64, 512, sel_idx, sel_cnt, probes="random", seed=seed)
    # and the sets differ from the corner probes' (other probe points)
    ci, cc = run_select(dec, w, K, R, blocks, 64, 512)
    assert any(not np.array_equal(ci[r, : cc[r]], sel_idx[r, : sel_cnt[r]]) for r in range(len(blocks)))


def test_select_all_blocks_ragged_token_count():
    w = W.gen.small_decoder(61, 64, 128, 100, "bf16")  # 100 tokens: a ragged 32-token tile
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    R = 20
    nb = hv.nblocks(R + 1)
    sel_idx = torch.empty((nb ** 3, 40), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, 8, 5, 40, K, None, sel_idx, sel_cnt)
    torch.cuda.synchronize()
    compare_sets(dec, w, K, R, np.arange(nb ** 3), 5, 40, sel_idx.cpu().numpy(), sel_cnt.cpu().numpy())


def test_k_equal_all_tokens_is_full_attention():
    w = W.gen.small_decoder(62, 256, 1024, 200, "bf16")
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 15
    nb = hv.nblocks(R + 1)
    sel_idx = torch.empty((nb ** 3, w.M), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, 8, w.M, w.M, K, None, sel_idx, sel_cnt)
    lst = hv.blocked_order(np.ones((R + 1,) * 3, bool)).astype(np.int32)
    lt = torch.from_numpy(lst).to(dev())
    a = torch.empty(lst.size, dtype=torch.float32, device=dev())
    b = torch.empty(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, lt), K, Vv, a, sel=V().kvsel(8, w.M, sel_idx, sel_cnt))
    V().vdm_decode_dense(dec, V().queries_list(R, lt), K, Vv, b)
    torch.cuda.synchronize()
    assert np.all(sel_cnt.cpu().numpy() == w.M)
    assert np.array_equal(sel_idx.cpu().numpy(), np.tile(np.arange(w.M, dtype=np.int32), (nb ** 3, 1)))
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("block", [8, 4, 16])
def test_gathered_decode_matches_restricted_attention(block):
    # sub-volumes of block^3 points (the pages' size trade-off); the list in the
    # blocked order of that block size
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 30
    nb = hv.nblocks(R + 1, block)
    sel_idx = torch.empty((nb ** 3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, block, 64, 512, K, None, sel_idx, sel_cnt)
    lin = np.arange((R + 1) ** 3)
    lst = lin[np.argsort(hv.blocked_key(lin, R + 1, block), kind="stable")].astype(np.int32)
    out = torch.empty(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(lst).to(dev())), K, Vv, out,
                         sel=V().kvsel(block, 512, sel_idx, sel_cnt))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    si, sc = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    od = oracle_decoder(w)
    Kh, Vh = f64(K), f64(Vv)
    blk = hv.block_of(lst, R + 1, block)
    rng = np.random.default_rng(4)
    worst = 0.0
    ub = np.unique(blk)
    for b in rng.choice(ub, min(12, ub.size), replace=False):
        m = np.nonzero(blk == b)[0][:40]
        toks = si[b, : sc[b]]
        ref = od.sdf(odec.grid_points(R, lst[m]), Kh[toks], Vh[toks])
        worst = max(worst, np.abs(out[m].astype(np.float64) - ref).max())
    report(f"gathered decode vs restricted attention (blocks of {block}^3)", worst, TOL_BF16)
    assert worst <= TOL_BF16


@pytest.mark.parametrize("probes", ["corners", "random"])
def test_hier_with_selection_full_workload(probes):
    # the 75 -> 150 -> 300 workload with adaptive KV selection at every level
    # (random probes: level L draws from the stream seeded with seed + R_L)
    w = W.make(3)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    q = w.query
    seed = 20251203
    kv = dict(q["kvsel"], probes=probes, seed=seed)
    params = V().hier_params(R0=q["R0"], levels=q["levels"], tau=q["tau"], dilation=q["dilation"], kvsel=kv)
    levels = params.levels
    vol = torch.empty(301 ** 3, dtype=torch.float32, device=dev())
    stats = torch.zeros(levels * V().STAT_FIELDS, dtype=torch.int64, device=dev())
    dbg = V().HierDebug(params, with_sel=True)
    V().vdm_decode_hier(dec, params, K, Vv, vol, stats, dbg)
    dense = torch.empty(301 ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(300), K, Vv, dense)
    torch.cuda.synchronize()
    st = V().stats_dict(stats, levels)
    od = oracle_decoder(w)
    Kh, Vh = f64(K), f64(Vv)
    rng = np.random.default_rng(8)
    vol_np, dense_np = vol.cpu().numpy(), dense.cpu().numpy()
    for L in range(levels):
        R = 75 << L
        s = st[L]
        d = dbg.levels[L]
        nocc = s["blocks"]
        blocks = d["sel_blocks"][:nocc].cpu().numpy()
        cnt = d["sel_cnt"][:nocc].cpu().numpy()
        idx = d["sel_idx"][: nocc * kv["cap"]].cpu().numpy().reshape(nocc, kv["cap"])
        print(f"[akvs] R={R}: {nocc} blocks, mean selected {cnt.mean():.1f} tokens, queries {s['queries']}",
              flush=True)
        assert s["selected"] == int(cnt.sum())
        lst = d["list"][: s["queries"]].cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(blocks, np.unique(hv.block_of(lst, R + 1)))
        pick = np.sort(rng.choice(nocc, min(nocc, 40), replace=False))
        compare_sets(dec, w, K, R, blocks[pick], kv["k"], kv["cap"], idx[pick], cnt[pick], probes=probes,
                     seed=seed + R)
        # decoded values with each block's selected tokens (identical inputs): one
        # point of every work item (an occupied block's queries, in list order, cut
        # into DECODE_TILE-query items), the lane offset rotating with the item
        volL = d["vol"].cpu().numpy()
        blk = hv.block_of(lst, R + 1)
        starts = np.searchsorted(blk, blocks)
        ends = np.searchsorted(blk, blocks, side="right")
        worst, n_items = 0.0, 0
        for r in range(nocc):
            m = lst[starts[r]:ends[r]][tile_sample(ends[r] - starts[r], DECODE_TILE)]
            n_items += m.size
            toks = idx[r, : cnt[r]]
            ref = od.sdf(odec.grid_points(R, m), Kh[toks], Vh[toks])
            worst = max(worst, np.abs(volL[m].astype(np.float64) - ref).max())
        assert n_items == s["items"]
        report(f"selection level {L}: one point per work item ({n_items}) vs restricted attention", worst, TOL_BF16)
        assert worst <= TOL_BF16
    # quality against dense decoding (reported, as on the pages: not a parity bound)
    comp = np.zeros(301 ** 3, bool)
    last = dbg.levels[levels - 1]["list"][: st[-1]["queries"]].cpu().numpy().astype(np.int64)
    comp[last] = True
    dd = np.abs(vol_np[comp].astype(np.float64) - dense_np[comp])
    flips = int(np.sum((vol_np < 0) != (dense_np < 0)))
    inter = np.sum((vol_np < 0) & (dense_np < 0))
    union = np.sum((vol_np < 0) | (dense_np < 0))
    print(f"[akvs] {probes} probes vs dense at finest decoded points: max|dSDF| {dd.max():.3e} mean {dd.mean():.3e}; "
          f"sign flips over the volume {flips}; occupancy IoU {inter / union:.5f}", flush=True)


def test_gathered_decode_mixed_softmax_paths():
    # head 0 with 16x larger logits: its waves take the shifted softmax, the other
    # heads' waves in the same workgroups do not, while all pass the per-tile
    # barriers of the gathered loop together
    w = W.make(1)
    weights = dict(w.weights)
    weights["Wq"] = (w.weights["Wq"] * np.repeat(np.float32([16, 1, 1, 1]), 64)[:, None]).astype(np.float32)
    dec = gpu_decoder(w, weights=weights)
    K, Vv = gpu_kv(dec, w)
    R = 30
    nb = hv.nblocks(R + 1)
    sel_idx = torch.empty((nb ** 3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt)
    lst = hv.blocked_order(np.ones((R + 1,) * 3, bool)).astype(np.int32)
    out = torch.empty(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(lst).to(dev())), K, Vv, out,
                         sel=V().kvsel(8, 512, sel_idx, sel_cnt))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    si, sc = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    od = oracle_decoder(w, weights=weights)
    Kh, Vh = f64(K), f64(Vv)
    blk = hv.block_of(lst, R + 1)
    rng = np.random.default_rng(5)
    worst = 0.0
    ub = np.unique(blk)
    for b in rng.choice(ub, min(12, ub.size), replace=False):
        m = np.nonzero(blk == b)[0][:40]
        toks = si[b, : sc[b]]
        ref = od.sdf(odec.grid_points(R, lst[m]), Kh[toks], Vh[toks])
        worst = max(worst, np.abs(out[m].astype(np.float64) - ref).max())
    assert np.all(np.isfinite(out))
    report("gathered decode, mixed softmax paths", worst, TOL_BF16)
    assert worst <= TOL_BF16


@pytest.mark.parametrize("repeat", [1, 3])
def test_select_ties_go_to_the_lower_index(repeat):
    # Keys made of `repeat` distinct rows, each repeated: whole groups of tokens
    # share one score, so the k-th score has many copies and the set must take the
    # lowest-indexed of them (exactly, no tie window). repeat = 1: every score is
    # equal, so every value is a candidate of the threshold search (more than its
    # candidate list holds); repeat = 3: three score levels.
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    M = w.M
    rows = K[torch.arange(M, device=dev()) % repeat * 97].contiguous()
    R, k, cap = 75, 64, 512
    nb = hv.nblocks(R + 1)
    blocks = np.array([0, 5, nb ** 3 // 2, nb ** 3 - 1])
    sel_idx, sel_cnt = run_select(dec, w, rows, R, blocks, k, cap)
    Qp = gpu_probe_q(dec, w, R, blocks)
    Kh = f64(rows)
    for r in range(len(blocks)):
        sc = oak.probe_scores(Qp[r], Kh, w.H)
        ref = oak.select(sc, k, cap)
        got = sel_idx[r, : sel_cnt[r]]
        assert np.array_equal(np.sort(ref), got), (blocks[r], ref[:8], got[:8])
    if repeat == 1:
        assert np.all(sel_cnt == k) and np.array_equal(sel_idx[:, :k], np.tile(np.arange(k), (len(blocks), 1)))
    print(f"[parity] selection ties (repeat={repeat}): {len(blocks)} blocks exact", flush=True)


@pytest.mark.parametrize("M", [1000, 33])
def test_select_ragged_token_count_full_width(M):
    # the 4-head, 256-wide decoder with a token count that leaves a partial last key
    # tile (1000 = 31 tiles + 8 keys; 33 = 1 tile + 1 key): only that tile is masked
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    K = K[:M].contiguous()
    R = 75
    nb = hv.nblocks(R + 1)
    blocks = np.sort(np.random.default_rng(M).choice(nb ** 3, 40, replace=False))
    blocks = np.unique(np.concatenate([blocks, [0, nb ** 3 - 1]]))
    k = min(64, M)
    print(f"[select] ragged M={M} k={k}", flush=True)
    sel_idx, sel_cnt = run_select(dec, w, K, R, blocks, k, 512)
    assert np.all(sel_cnt >= k) and np.all(sel_cnt <= min(512, M))
    compare_sets(dec, w, K, R, blocks, k, 512, sel_idx, sel_cnt)


def test_gathered_decode_key_outside_query_span():
    # One key with a large component outside every head's query span: its norm
    # sets the softmax bound of every block whose set holds it, far above any
    # logit (see test_gpu_dense.py::test_dense_key_outside_query_span). The
    # gathered decode must stay finite and match attention restricted to each
    # block's set on the same K.
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 30
    nb = hv.nblocks(R + 1)
    sel_idx = torch.empty((nb ** 3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    # the token: the first of block 0's set (its logits barely move, so it stays selected)
    V().vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt)
    tok = int(sel_idx[0, 0].item())
    K2 = torch.from_numpy(W.with_unseen_key(f64(K), w.weights["Wq"], w.H, tok, 400.0)).to(dev()).to(tdtype(w))
    V().vdm_select_kv(dec, R, 8, 64, 512, K2, None, sel_idx, sel_cnt)
    lst = hv.blocked_order(np.ones((R + 1,) * 3, bool)).astype(np.int32)
    out = torch.empty(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(lst).to(dev())), K2, Vv, out,
                         sel=V().kvsel(8, 512, sel_idx, sel_cnt))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    si, sc = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    od = oracle_decoder(w)
    Kh, Vh = f64(K2), f64(Vv)
    blk = hv.block_of(lst, R + 1)
    # blocks whose set holds the token and blocks whose set does not
    has7 = np.array([tok in si[b, : sc[b]] for b in range(nb ** 3)])
    assert has7.any()
    worst = 0.0
    rng = np.random.default_rng(6)
    for b in np.concatenate([rng.choice(np.flatnonzero(has7), min(10, has7.sum()), replace=False),
                             rng.choice(np.flatnonzero(~has7), min(4, (~has7).sum()), replace=False)]):
        m = np.nonzero(blk == b)[0][:40]
        toks = si[b, : sc[b]]
        ref = od.sdf(odec.grid_points(R, lst[m]), Kh[toks], Vh[toks])
        worst = max(worst, np.abs(out[m].astype(np.float64) - ref).max())
    report(f"gathered decode, key outside the query span ({int(has7.sum())} sets hold it)", worst, TOL_BF16)
    assert worst <= TOL_BF16


def test_gathered_decode_list_outside_preconditions():
    # Lists outside the documented preconditions stay defined: an entry outside
    # the grid gets NaN and no work item, a run of one block longer than block^3
    # (repeated entries) is decoded in full, each copy equal to the point's value
    # in a valid list, and an empty token set gives a finite value.
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 30
    P = R + 1
    nb = hv.nblocks(P)
    sel_idx = torch.empty((nb ** 3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt)
    valid = hv.blocked_order(np.ones((P,) * 3, bool)).astype(np.int32)
    ref = torch.empty(valid.size, dtype=torch.float32, device=dev())
    sel = V().kvsel(8, 512, sel_idx, sel_cnt)
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(valid).to(dev())), K, Vv, ref, sel=sel)
    p0 = int(valid[3])  # a point of block 0
    lst = np.concatenate([valid[:100], [-5, P ** 3 + 3], np.full(700, p0), valid[100:300]]).astype(np.int32)
    out = torch.zeros(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(lst).to(dev())), K, Vv, out, sel=sel)
    # an empty set for block 0
    cnt0 = sel_cnt.clone()
    cnt0[0] = 0
    out0 = torch.zeros(64, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(valid[:64].copy()).to(dev())), K, Vv, out0,
                         sel=V().kvsel(8, 512, sel_idx, cnt0))
    torch.cuda.synchronize()
    out, ref, out0 = out.cpu().numpy(), ref.cpu().numpy(), out0.cpu().numpy()
    assert np.isnan(out[100]) and np.isnan(out[101])
    assert np.array_equal(out[:100], ref[:100])
    assert np.array_equal(out[102:802], np.full(700, ref[3], np.float32))
    assert np.array_equal(out[802:], ref[100:300])
    assert np.all(np.isfinite(out0))
    print("[guard] out-of-grid entries NaN, 700 repeated entries decoded, empty set finite", flush=True)


# ---------------------------------------------------------------- per-head token sets

def run_select_heads(dec, w, K, R, blocks, k, cap, block=8):
    nb = len(blocks)
    sel_idx = torch.empty((nb, w.H, cap), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty((nb, w.H), dtype=torch.int32, device=dev())
    bt = torch.from_numpy(np.asarray(blocks, np.int32)).to(dev())
    V().vdm_select_kv(dec, R, block, k, cap, K, bt, sel_idx, sel_cnt, heads=True)
    torch.cuda.synchronize()
    return sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()


def compare_sets_heads(dec, w, K, R, blocks, k, cap, sel_idx, sel_cnt, block=8):
    Qp = gpu_probe_q(dec, w, R, blocks, block)
    Kh = f64(K)
    n_amb, differ = 0, 0
    for r, b in enumerate(blocks):
        sc = oak.probe_scores_per_head(Qp[r], Kh, w.H)
        ref_sets = [oak.select(sc[h], k, cap) for h in range(w.H)]
        for h in range(w.H):
            got = sel_idx[r, h, : sel_cnt[r, h]]
            assert np.all(np.diff(got) > 0) and np.all(sel_idx[r, h, sel_cnt[r, h]:] == -1)
            sym = np.setxor1d(ref_sets[h], got)
            if sym.size:
                amb = oak.near_tie_tokens(sc[h], k, cap)
                n_amb += sym.size
                assert np.all(np.isin(sym, amb)), (b, h, sym)
        differ += any(not np.array_equal(ref_sets[0], ref_sets[h]) for h in range(1, w.H))
    print(f"[parity] per-head selection R={R} k={k} cap={cap}: {len(blocks)} blocks x {w.H} heads, "
          f"{n_amb} near-tie tokens differ; heads' sets differ in {differ} blocks", flush=True)
    return differ


@pytest.mark.parametrize("R,k,cap", [(75, 64, 512), (75, 64, 100), (150, 32, 512)])
def test_select_per_head_matches_oracle(R, k, cap):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    nb = hv.nblocks(R + 1)
    blocks = np.sort(np.random.default_rng(R + k + cap + 7).choice(nb ** 3, 40, replace=False))
    blocks = np.unique(np.concatenate([blocks, [0, nb ** 3 - 1]]))
    sel_idx, sel_cnt = run_select_heads(dec, w, K, R, blocks, k, cap)
    assert np.all(sel_cnt <= cap) and np.all(sel_cnt >= k)
    if cap == 100:
        assert np.all(sel_cnt == 100)
    assert compare_sets_heads(dec, w, K, R, blocks, k, cap, sel_idx, sel_cnt) > 0


def test_gathered_decode_per_head_sets():
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 30
    nb = hv.nblocks(R + 1)
    sel_idx = torch.empty((nb ** 3, w.H, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty((nb ** 3, w.H), dtype=torch.int32, device=dev())
    V().vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt, heads=True)
    lst = hv.blocked_order(np.ones((R + 1,) * 3, bool)).astype(np.int32)
    out = torch.empty(lst.size, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_list(R, torch.from_numpy(lst).to(dev())), K, Vv, out,
                         sel=V().kvsel(8, 512, sel_idx, sel_cnt, heads=True))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.all(np.isfinite(out))
    si, sc = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    od = oracle_decoder(w)
    Kh, Vh = f64(K), f64(Vv)
    blk = hv.block_of(lst, R + 1)
    worst = 0.0
    for b in range(nb ** 3):
        m = np.nonzero(blk == b)[0]
        m = m[tile_sample(m.size, DECODE_TILE)]
        sets = [si[b, h, : sc[b, h]] for h in range(w.H)]
        ref = oak.sdf_per_head_sets(od, odec.grid_points(R, lst[m]), sets, Kh, Vh)
        worst = max(worst, np.abs(out[m].astype(np.float64) - ref).max())
    report("gathered decode with per-head sets vs per-head restricted attention (every work item)", worst, TOL_BF16)
    assert worst <= TOL_BF16


def test_hier_with_per_head_sets_full_workload():
    # the 75 -> 150 -> 300 workload with one token set per (block, head) at every level
    w = W.make(3)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    q = w.query
    kv = dict(q["kvsel"], heads=True)
    params = V().hier_params(R0=q["R0"], levels=q["levels"], tau=q["tau"], dilation=q["dilation"], kvsel=kv)
    levels = params.levels
    vol = torch.empty(301 ** 3, dtype=torch.float32, device=dev())
    stats = torch.zeros(levels * V().STAT_FIELDS, dtype=torch.int64, device=dev())
    dbg = V().HierDebug(params, with_sel=True, H=w.H)
    V().vdm_decode_hier(dec, params, K, Vv, vol, stats, dbg)
    dense = torch.empty(301 ** 3, dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, V().queries_grid(300), K, Vv, dense)
    torch.cuda.synchronize()
    st = V().stats_dict(stats, levels)
    od = oracle_decoder(w)
    Kh, Vh = f64(K), f64(Vv)
    rng = np.random.default_rng(9)
    cap = kv["cap"]
    for L in range(levels):
        R = 75 << L
        s = st[L]
        d = dbg.levels[L]
        nocc = s["blocks"]
        blocks = d["sel_blocks"][:nocc].cpu().numpy()
        cnt = d["sel_cnt"][: nocc * w.H].cpu().numpy().reshape(nocc, w.H)
        idx = d["sel_idx"][: nocc * w.H * cap].cpu().numpy().reshape(nocc, w.H, cap)
        assert s["selected"] == int(cnt.sum())
        print(f"[akvs heads] R={R}: {nocc} blocks, mean selected per head {cnt.mean():.1f} tokens", flush=True)
        pick = np.sort(rng.choice(nocc, min(nocc, 20), replace=False))
        compare_sets_heads(dec, w, K, R, blocks[pick], kv["k"], cap, idx[pick], cnt[pick])
        lst = d["list"][: s["queries"]].cpu().numpy().astype(np.int64)
        volL = d["vol"].cpu().numpy()
        blk = hv.block_of(lst, R + 1)
        starts = np.searchsorted(blk, blocks)
        ends = np.searchsorted(blk, blocks, side="right")
        worst, n_items = 0.0, 0
        for r in range(nocc):
            m = lst[starts[r]:ends[r]][tile_sample(ends[r] - starts[r], DECODE_TILE)]
            n_items += m.size
            sets = [idx[r, h, : cnt[r, h]] for h in range(w.H)]
            ref = oak.sdf_per_head_sets(od, odec.grid_points(R, m), sets, Kh, Vh)
            worst = max(worst, np.abs(volL[m].astype(np.float64) - ref).max())
        assert n_items == s["items"]
        report(f"per-head selection level {L}: one point per work item ({n_items})", worst, TOL_BF16)
        assert worst <= TOL_BF16
    vol_np, dense_np = vol.cpu().numpy(), dense.cpu().numpy()
    flips = int(np.sum((vol_np < 0) != (dense_np < 0)))
    inter = np.sum((vol_np < 0) & (dense_np < 0))
    union = np.sum((vol_np < 0) | (dense_np < 0))
    print(f"[akvs heads] per-head sets vs dense: sign flips {flips}; occupancy IoU {inter / union:.5f}", flush=True)
