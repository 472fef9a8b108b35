"""Guard regions around every output of the C ABI's calls: each output buffer is
cut out of a larger allocation whose bytes before and after it hold a known
pattern, and the pattern must be intact after the call (no call writes outside
the outputs it is given). Covers the embedding, the KV projection, the dense,
batched, gathered and no-allocation decodes, KV selection (one set per block and
per head), the hierarchical decode (volume, counters and inspection exports),
surface extraction (buffers shorter than the mesh included) and the local
decoder."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from tests.helpers import dev, gpu_decoder, gpu_kv, tdtype

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of pattern before and after each output


def V():
    import shape_vae_decoding_amd as mod

    return mod


class Guarded:
    """Output tensors carved from guarded byte buffers."""

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.empty(2 * GUARD + n, dtype=torch.uint8, device=dev())
        pat = torch.arange(raw.numel(), dtype=torch.int64, device=dev()).mul_(131).add_(7).remainder_(251).to(torch.uint8)
        raw.copy_(pat)
        self.bufs.append((raw, pat, n))
        return raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        for raw, pat, n in self.bufs:
            assert torch.equal(raw[:GUARD], pat[:GUARD]), "bytes before an output were written"
            assert torch.equal(raw[GUARD + n:], pat[GUARD + n:]), "bytes after an output were written"


def test_embed_project_and_dense_decodes():
    g = Guarded()
    w = W.make(1)
    dec = gpu_decoder(w)
    Zt = torch.from_numpy(np.ascontiguousarray(w.Z, np.float32)).to(dev()).to(tdtype(w))
    K, Vv = g(Zt.shape, Zt.dtype), g(Zt.shape, Zt.dtype)
    V().vdm_project_kv(dec, Zt, K, Vv)
    xyz = torch.from_numpy(W.gen.random_points(3, 1001, -1, 1)).to(dev())
    Q = g((1001, w.D), tdtype(w))
    V().vdm_embed_queries(dec, xyz, Q)
    sdf = g((1001,), torch.float32)
    V().vdm_decode_dense(dec, V().queries_points(xyz), K, Vv, sdf)
    sdf2 = g((1001,), torch.float32)
    V().vdm_decode_dense_noalloc(dec, V().queries_points(xyz), K, Vv, sdf2)
    R = 20
    grid = g(((R + 1) ** 3,), torch.float32)
    V().vdm_decode_dense(dec, V().queries_grid(R), K, Vv, grid)
    Kb = torch.stack([K, K]).contiguous()
    Vb = torch.stack([Vv, Vv]).contiguous()
    batch = g((2, 1001), torch.float32)
    V().vdm_decode_dense_batch(dec, V().queries_points(xyz), Kb, Vb, batch)
    g.check()


def test_selection_and_gathered_decode():
    g = Guarded()
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = 37
    nb = -(-(R + 1) // 8)
    sel_idx, sel_cnt = g((nb ** 3, 512), torch.int32), g((nb ** 3,), torch.int32)
    V().vdm_select_kv(dec, R, 8, 64, 512, K, None, sel_idx, sel_cnt)
    hs_idx, hs_cnt = g((nb ** 3, w.H, 200), torch.int32), g((nb ** 3, w.H), torch.int32)
    V().vdm_select_kv(dec, R, 8, 32, 200, K, None, hs_idx, hs_cnt, heads=True)
    P = R + 1
    i, j, k = np.meshgrid(np.arange(P), np.arange(P), np.arange(P), indexing="ij")
    blk = (((i // 8) * nb + j // 8) * nb + k // 8).ravel()
    lin = np.flatnonzero(blk % 5 == 1).astype(np.int32)
    lin = lin[np.argsort(blk[lin], kind="stable")]
    lt = torch.from_numpy(lin).to(dev())
    out = g((lin.size,), torch.float32)
    V().vdm_decode_dense(dec, V().queries_list(R, lt), K, Vv, out, sel=V().kvsel(8, 512, sel_idx, sel_cnt))
    out_h = g((lin.size,), torch.float32)
    V().vdm_decode_dense(dec, V().queries_list(R, lt), K, Vv, out_h, sel=V().kvsel(8, 200, hs_idx, hs_cnt, heads=True))
    g.check()


def test_chunked_selection():
    # 9,000 tokens (4,096-token chunks), the cap binding, one set per block and per head
    g = Guarded()
    w = W.make(4)
    dec = gpu_decoder(w)
    K, _ = gpu_kv(dec, w, Z=w.Z[:9000])
    R = 30
    nb = -(-(R + 1) // 8)
    sel_idx, sel_cnt = g((nb ** 3, 100), torch.int32), g((nb ** 3,), torch.int32)
    V().vdm_select_kv(dec, R, 8, 64, 100, K, None, sel_idx, sel_cnt)
    hs_idx, hs_cnt = g((nb ** 3, w.H, 100), torch.int32), g((nb ** 3, w.H), torch.int32)
    V().vdm_select_kv(dec, R, 8, 64, 100, K, None, hs_idx, hs_cnt, heads=True)
    g.check()


@pytest.mark.parametrize("kvsel", [None, dict(k=64, cap=512)])
def test_hierarchical_decode_and_exports(kvsel):
    g = Guarded()
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R0, L = 20, 3
    p = V().hier_params(R0=R0, levels=L, tau=float(np.float32(4 / 80)), kvsel=kvsel)
    vol = g(((R0 * 4 + 1) ** 3,), torch.float32)
    st = g((L * V().STAT_FIELDS,), torch.int64)
    dbg = V().HierDebug(p, with_sel=bool(kvsel), H=w.H)
    for lev, bufs in enumerate(dbg.levels):  # every export moved into a guarded buffer
        for name, t in list(bufs.items()):
            gt = g(tuple(t.shape), t.dtype)
            bufs[name] = gt
            getattr(dbg.struct, name)[lev] = gt.data_ptr()
    V().vdm_decode_hier(dec, p, K, Vv, vol, st, dbg=dbg)
    B = 2
    vb = g((B, (R0 * 4 + 1) ** 3), torch.float32)
    sb = g((B, L * V().STAT_FIELDS), torch.int64)
    V().vdm_decode_hier_batch(dec, p, torch.stack([K] * B).contiguous(), torch.stack([Vv] * B).contiguous(), vb, sb)
    g.check()


def test_surface_extraction_short_and_long_buffers():
    g = Guarded()
    R = 40
    gr = np.linspace(-1, 1, R + 1, dtype=np.float32)
    x, y, z = np.meshgrid(gr, gr, gr, indexing="ij")
    vol = torch.from_numpy((np.sqrt(x * x + y * y + z * z) - 0.6).astype(np.float32).ravel()).to(dev())
    for mv, mt in ((100000, 200000), (300, 500)):  # room for the mesh, then much less
        verts, tris = g((mv, 3), torch.float32), g((mt, 3), torch.int32)
        counts, edges = g((2,), torch.int64), g((mv,), torch.int64)
        V().vdm_extract_surface(vol, R, verts, tris, counts, vert_edges=edges)
    g.check()


def test_local_decoder():
    g = Guarded()
    w = W.small_local(seed=4, M=500, C=256, F=1024, n_queries=777)
    d = dev()
    wt = {k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(d) for k, v in w.weights.items()}
    for k in ("B", "W1", "W2"):
        wt[k] = wt[k].to(torch.bfloat16)
    ldec = V().LocalDecoder(wt, w.prims, w.K, w.net_scale)
    P = torch.from_numpy(np.ascontiguousarray(w.xyz, np.float32)).to(d)
    Fe = torch.from_numpy(np.ascontiguousarray(w.feats, np.float32)).to(d).to(torch.bfloat16)
    X = torch.from_numpy(np.ascontiguousarray(w.queries, np.float32)).to(d)
    sdf, nbr = g((X.shape[0],), torch.float32), g((X.shape[0], w.K), torch.int32)
    V().vdm_decode_local(ldec, P, Fe, X, sdf, nbr)
    g.check()
