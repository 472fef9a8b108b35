"""The bounds-checked build of the library (libvdm_debug.so, built with
-DVDM_DEBUG=1) on the GPU, through the C ABI.

Its kernels check every data-dependent index: token ids of a selection,
selection rows and counts, decode work items, block ids, query-list and
work-item slots, occupied-block slots, and the support ranges and slots of the
local decoder. On valid inputs each call must return exactly what the default
build returns (the checks change no arithmetic). A token id outside [0, M) in a
caller's selection, and a block id outside the grid, must come back as an error
naming the check; both builds clamp such a token into [0, M) before using it and
use block ids only to place probe points, so no access leaves its buffer in
either build."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from tests.helpers import dev, gpu_decoder, gpu_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def V():
    import shape_vae_decoding_amd as mod

    return mod


@pytest.fixture(scope="module")
def libs(V):
    return V._lib, V.debug_library()


def both(V, libs, fn):
    """fn() through the default build, then through the bounds-checked one."""
    rel, dbg = libs
    out = []
    for lib in (rel, dbg):
        V._lib = lib
        try:
            out.append(fn())
            torch.cuda.synchronize()
        finally:
            V._lib = rel
    return out


def same(a, b):
    if isinstance(a, (tuple, list)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            same(x, y)
        return
    a, b = a.cpu().contiguous(), b.cpu().contiguous()
    assert a.dtype == b.dtype and a.shape == b.shape
    if a.dtype == torch.float32:  # bit for bit (NaN patterns included)
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b)


def test_debug_library_is_a_different_build(V, libs):
    rel, dbg = libs
    assert V.DEBUG_LIB_PATH != V.LIB_PATH
    assert dbg.vdm_version() == rel.vdm_version()


def test_dense_decode_equals_default_build(V, libs):
    for cfg, n in ((0, 1000), (1, 4097)):
        w = W.make(cfg)
        dec = gpu_decoder(w)
        K, Vv = gpu_kv(dec, w)
        xyz = torch.from_numpy(np.random.default_rng(cfg).uniform(-1, 1, (n, 3)).astype(np.float32)).to(dev())

        def run():
            sdf = torch.empty(n, dtype=torch.float32, device=dev())
            V.vdm_decode_dense(dec, V.queries_points(xyz), K, Vv, sdf)
            return sdf

        same(*both(V, libs, run))


@pytest.mark.parametrize("kvsel", [None, dict(k=64, cap=512), dict(k=64, cap=512, heads=True)])
def test_hierarchical_decode_equals_default_build(V, libs, kvsel):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    p = V.hier_params(R0=24, levels=3, tau=float(np.float32(4 / 96)), kvsel=kvsel)
    Pf = 96 + 1

    def run():
        vol = torch.empty(Pf ** 3, dtype=torch.float32, device=dev())
        st = torch.zeros(3 * V.STAT_FIELDS, dtype=torch.int64, device=dev())
        V.vdm_decode_hier(dec, p, K, Vv, vol, st)
        return vol, st

    same(*both(V, libs, run))


def test_batched_hierarchical_decode_equals_default_build(V, libs):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    B = 3
    Kb = torch.stack([K] * B).contiguous()
    Vb = torch.stack([Vv] * B).contiguous()
    p = V.hier_params(R0=20, levels=2, tau=float(np.float32(4 / 40)), kvsel=dict(k=64, cap=512))

    def run():
        vol = torch.empty((B, 41 ** 3), dtype=torch.float32, device=dev())
        st = torch.zeros((B, 2 * V.STAT_FIELDS), dtype=torch.int64, device=dev())
        V.vdm_decode_hier_batch(dec, p, Kb, Vb, vol, st)
        return vol, st

    same(*both(V, libs, run))


def _selection_and_list(V, dec, K, R):
    """Token sets of every block of the R grid and a query list of ragged blocks."""
    nb = -(-(R + 1) // 8)
    sel_idx = torch.empty((nb ** 3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(nb ** 3, dtype=torch.int32, device=dev())
    V.vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt)
    P = R + 1
    i, j, k = np.meshgrid(np.arange(P), np.arange(P), np.arange(P), indexing="ij")
    keep = ((i // 8 + j // 8 + k // 8) % 3 == 0).ravel()  # every third block, whole
    lin = np.flatnonzero(keep).astype(np.int32)
    blk = ((i // 8) * nb + j // 8) * nb + k // 8
    lin = lin[np.argsort(blk.ravel()[lin], kind="stable")]  # the blocks' runs contiguous
    return sel_idx, sel_cnt, torch.from_numpy(lin).to(dev())


def test_selection_and_gathered_decode_equal_default_build(V, libs):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 37

    def run():
        sel_idx, sel_cnt, lin = _selection_and_list(V, dec, K, R)
        sdf = torch.empty(lin.shape[0], dtype=torch.float32, device=dev())
        V.vdm_decode_dense(dec, V.queries_list(R, lin), K, Vv, sdf, sel=V.kvsel(8, 512, sel_idx, sel_cnt))
        return sel_idx, sel_cnt, sdf

    same(*both(V, libs, run))


@pytest.mark.parametrize("heads", [False, True])
def test_chunked_selection_equals_default_build(V, libs, heads):
    # 9,000 tokens: rows searched in 4,096-token chunks; a cap of 100 binds, so the
    # cap ranking over the union's members runs too
    w = W.make(4)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w, Z=w.Z[:9000])
    R = 37
    nb = -(-(R + 1) // 8)
    ns = w.H if heads else 1

    def run():
        sel_idx = torch.empty((nb ** 3 * ns, 100), dtype=torch.int32, device=dev())
        sel_cnt = torch.empty(nb ** 3 * ns, dtype=torch.int32, device=dev())
        V.vdm_select_kv(dec, R, 8, 64, 100, K, None, sel_idx, sel_cnt, heads=heads)
        return sel_idx, sel_cnt

    a, b = both(V, libs, run)
    same(a, b)
    assert torch.all(a[1] == 100)


def test_local_decoder_equals_default_build(V, libs):
    w = W.small_local(seed=3, M=700, C=256, F=1024, n_queries=999)
    d = dev()
    wt = {k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(d) for k, v in w.weights.items()}
    for k in ("B", "W1", "W2"):
        wt[k] = wt[k].to(torch.bfloat16)
    ldec = V.LocalDecoder(wt, w.prims, w.K, w.net_scale)
    P = torch.from_numpy(np.ascontiguousarray(w.xyz, np.float32)).to(d)
    Fe = torch.from_numpy(np.ascontiguousarray(w.feats, np.float32)).to(d).to(torch.bfloat16)
    X = torch.from_numpy(np.ascontiguousarray(w.queries, np.float32)).to(d)

    def run():
        sdf = torch.empty(X.shape[0], dtype=torch.float32, device=d)
        nbr = torch.empty((X.shape[0], w.K), dtype=torch.int32, device=d)
        V.vdm_decode_local(ldec, P, Fe, X, sdf, nbr)
        return sdf, nbr

    same(*both(V, libs, run))


def test_surface_extraction_equals_default_build(V, libs):
    R = 40
    g = np.linspace(-1, 1, R + 1, dtype=np.float32)
    x, y, z = np.meshgrid(g, g, g, indexing="ij")
    vol = torch.from_numpy((np.sqrt(x * x + y * y + z * z) - 0.6).astype(np.float32).ravel()).to(dev())

    def run():
        verts = torch.empty((200000, 3), dtype=torch.float32, device=dev())
        tris = torch.empty((400000, 3), dtype=torch.int32, device=dev())
        counts = torch.empty(2, dtype=torch.int64, device=dev())
        V.vdm_extract_surface(vol, R, verts, tris, counts)
        n = counts.cpu()
        return verts[: n[0]], tris[: n[1]], counts

    same(*both(V, libs, run))


def test_out_of_range_token_id_is_reported(V, libs):
    # one selected token id past M: the bounds-checked build reports it; the
    # default build clamps it to M - 1 like the checked one, so both outputs agree
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 37
    sel_idx, sel_cnt, lin = _selection_and_list(V, dec, K, R)
    sel_idx[0, 3] = w.M + 5
    rel, dbg = libs
    outs = []
    for lib in (rel, dbg):
        V._lib = lib
        sdf = torch.empty(lin.shape[0], dtype=torch.float32, device=dev())
        try:
            if lib is dbg:
                with pytest.raises(V.VdmError, match="selected token id"):
                    V.vdm_decode_dense(dec, V.queries_list(R, lin), K, Vv, sdf, sel=V.kvsel(8, 512, sel_idx, sel_cnt))
            else:
                V.vdm_decode_dense(dec, V.queries_list(R, lin), K, Vv, sdf, sel=V.kvsel(8, 512, sel_idx, sel_cnt))
            torch.cuda.synchronize()
        finally:
            V._lib = rel
        outs.append(sdf)
    same(outs[0], outs[1])
    assert torch.isfinite(outs[0]).all()
    # the next call on the bounds-checked build starts clean
    V._lib = dbg
    try:
        sdf = torch.empty(lin.shape[0], dtype=torch.float32, device=dev())
        sel_idx[0, 3] = 0
        V.vdm_decode_dense(dec, V.queries_list(R, lin), K, Vv, sdf, sel=V.kvsel(8, 512, sel_idx, sel_cnt))
    finally:
        V._lib = rel


def test_block_id_outside_the_grid_is_reported(V, libs):
    w = W.make(1)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w)
    R = 37
    nb = -(-(R + 1) // 8)
    blocks = torch.tensor([0, 7, nb ** 3 + 3], dtype=torch.int32, device=dev())
    sel_idx = torch.empty((3, 512), dtype=torch.int32, device=dev())
    sel_cnt = torch.empty(3, dtype=torch.int32, device=dev())
    rel, dbg = libs
    V.vdm_select_kv(dec, R, 8, 64, 512, K, blocks, sel_idx, sel_cnt)  # default build: no check
    torch.cuda.synchronize()
    V._lib = dbg
    try:
        with pytest.raises(V.VdmError, match="selection block id"):
            V.vdm_select_kv(dec, R, 8, 64, 512, K, blocks, sel_idx, sel_cnt)
    finally:
        V._lib = rel
