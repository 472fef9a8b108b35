"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before any device work."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "vdm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(vdm_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_five_calls():
    fns = header_functions()
    for f in ["vdm_embed_queries", "vdm_project_kv", "vdm_decode_dense", "vdm_decode_hier", "vdm_select_kv"]:
        assert f in fns


def test_library_exports_every_declared_symbol():
    import shape_vae_decoding_amd as V

    lib = C.CDLL(V.LIB_PATH)
    missing = [f for f in header_functions() if not hasattr(lib, f)]
    assert not missing, missing
    assert sorted(V.EXPORTS) == header_functions()
    assert V.vdm_version() == 1


def _decoder(D=256, F=1024, dtype=1, n_prims=1):
    import shape_vae_decoding_amd as V

    d = V._Decoder()
    d.D, d.H, d.F, d.n_freq, d.dtype = D, D // 64, F, 8, dtype
    d.net_scale = 0.05
    for k in ("Wq", "Wk", "Wv", "Wo", "W1", "W2", "w_head"):
        setattr(d, k, 0x100000)  # never dereferenced: every case fails validation first
    d.n_prims = n_prims
    d.prims[0].kind = 0
    return d


def test_status_codes_for_bad_decoders():
    import shape_vae_decoding_amd as V

    lib = V._lib
    assert lib.vdm_embed_queries(None, None, 5, None, None) == V.VDM_ERR_INVALID_ARG
    assert "NULL" in V.vdm_last_error()
    d = _decoder(D=128)
    assert lib.vdm_embed_queries(C.byref(d), None, 5, None, None) == V.VDM_ERR_UNSUPPORTED
    d = _decoder(F=1000)
    assert lib.vdm_embed_queries(C.byref(d), None, 5, None, None) == V.VDM_ERR_UNSUPPORTED
    d = _decoder(D=256, dtype=0)  # fp32 is supported only at D = 64
    assert lib.vdm_embed_queries(C.byref(d), None, 5, None, None) == V.VDM_ERR_UNSUPPORTED
    d = _decoder(n_prims=0)
    assert lib.vdm_embed_queries(C.byref(d), None, 5, None, None) == V.VDM_ERR_INVALID_ARG
    d = _decoder()
    d.n_freq = 6
    assert lib.vdm_embed_queries(C.byref(d), None, 5, None, None) == V.VDM_ERR_UNSUPPORTED
    d = _decoder()
    d.Wk = 0x100002  # misaligned
    assert lib.vdm_project_kv(C.byref(d), 0x1000, 4, 0x2000, 0x3000, None) == V.VDM_ERR_INVALID_ARG


def test_zero_sized_calls_are_noops():
    import shape_vae_decoding_amd as V

    d = _decoder()
    assert V._lib.vdm_embed_queries(C.byref(d), None, 0, None, None) == V.VDM_OK
    assert V._lib.vdm_project_kv(C.byref(d), None, 0, None, None, None) == V.VDM_OK
    q = V._Queries(V.VDM_Q_POINTS, 0, 0, None, None)
    assert V._lib.vdm_decode_dense(C.byref(d), C.byref(q), None, None, 1, None, None, None, 0, None) == V.VDM_OK


def test_decode_argument_checks():
    import shape_vae_decoding_amd as V

    d = _decoder()
    lib = V._lib
    q = V._Queries(V.VDM_Q_GRID, 16, 17 ** 3 - 1, None, None)  # N != (R+1)^3
    assert lib.vdm_decode_dense(C.byref(d), C.byref(q), 0x1000, 0x1000, 10, None, 0x1000, 0x1000, 1 << 30,
                                None) == V.VDM_ERR_INVALID_ARG
    q = V._Queries(V.VDM_Q_GRID, 16, 17 ** 3, None, None)
    assert lib.vdm_decode_dense(C.byref(d), C.byref(q), 0x1000, 0x1000, 0, None, 0x1000, 0x1000, 1 << 30,
                                None) == V.VDM_ERR_INVALID_ARG  # M = 0
    assert lib.vdm_decode_dense(C.byref(d), C.byref(q), 0x1000, 0x1000, 10, None, 0x1000, 0x1000, 16,
                                None) == V.VDM_ERR_WORKSPACE
    sel = V._KvSel(8, 64, 0x1000, 0x1000, None)
    assert lib.vdm_decode_dense(C.byref(d), C.byref(q), 0x1000, 0x1000, 10, C.byref(sel), 0x1000, 0x1000,
                                1 << 30, None) == V.VDM_ERR_INVALID_ARG  # selection needs a list
    need = lib.vdm_dense_workspace_size(C.byref(d), 3072, 1000, 0)
    assert need >= 2 * 3072 * 256 * 2


def test_noalloc_decode_argument_checks():
    # the no-allocation decode validates before touching a GPU: zero queries are a
    # no-op, a token count whose scratch exceeds the fixed array is refused
    import shape_vae_decoding_amd as V

    d = _decoder()
    lib = V._lib
    q0 = V._Queries(V.VDM_Q_POINTS, 0, 0, None, None)
    assert lib.vdm_decode_dense_noalloc(C.byref(d), C.byref(q0), None, None, 1, None, None) == V.VDM_OK
    q = V._Queries(V.VDM_Q_GRID, 16, 17 ** 3, None, None)
    assert lib.vdm_decode_dense_noalloc(C.byref(d), C.byref(q), 0x1000, 0x1000, 0, 0x1000, None) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_decode_dense_noalloc(C.byref(d), C.byref(q), None, 0x1000, 10, 0x1000, None) == V.VDM_ERR_INVALID_ARG
    big = 60000  # 2 x 60000 x 256 x 2 bytes of packed K/V alone exceed 48 MiB
    assert lib.vdm_dense_workspace_size(C.byref(d), big, q.N, 0) > V.NOALLOC_SCRATCH_BYTES
    assert lib.vdm_decode_dense_noalloc(C.byref(d), C.byref(q), 0x1000, 0x1000, big, 0x1000, None) == V.VDM_ERR_WORKSPACE
    assert "scratch" in V.vdm_last_error()
    assert lib.vdm_dense_workspace_size(C.byref(d), 40960, q.N, 0) <= V.NOALLOC_SCRATCH_BYTES


def test_local_decoder_argument_checks():
    import shape_vae_decoding_amd as V

    lib = V._lib
    d = V._LocalDecoder()
    d.C, d.F, d.K, d.hidden, d.net_scale = 256, 1024, 16, 32, 0.05
    for k in ("A", "a", "B", "W1", "W2", "w_head"):
        setattr(d, k, 0x100000)  # never dereferenced: every case fails validation first or does nothing
    d.n_prims = 1
    args = (0x1000, 0x1000, 100, 0x1000, 50, 0x1000, None, 0x1000, 1 << 30, None)
    assert lib.vdm_decode_local(None, *args) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_decode_local(C.byref(d), 0x1000, 0x1000, 100, 0x1000, 0, None, None, None, 0, None) == V.VDM_OK
    d.K = 8
    assert lib.vdm_decode_local(C.byref(d), *args) == V.VDM_ERR_UNSUPPORTED
    d.K = 16
    d.F = 1000
    assert lib.vdm_decode_local(C.byref(d), *args) == V.VDM_ERR_UNSUPPORTED
    d.F = 1024
    assert lib.vdm_decode_local(C.byref(d), 0x1000, 0x1000, 15, 0x1000, 50, 0x1000, None, 0x1000, 1 << 30,
                                None) == V.VDM_ERR_INVALID_ARG  # M < K
    assert lib.vdm_decode_local(C.byref(d), 0x1000, 0x1008, 100, 0x1000, 50, 0x1000, None, 0x1000, 1 << 30,
                                None) == V.VDM_ERR_INVALID_ARG  # feats misaligned
    assert lib.vdm_decode_local(C.byref(d), 0x1000, 0x1000, 100, 0x1000, 50, 0x1000, None, 0x1000, 64,
                                None) == V.VDM_ERR_WORKSPACE
    need = lib.vdm_local_workspace_size(C.byref(d), 40960, 200000)
    assert need >= 200000 * 256 * 2 + 200000 * 16 * 4


def test_select_and_hier_argument_checks():
    import shape_vae_decoding_amd as V

    d = _decoder()
    lib = V._lib
    # k > M, cap < k, M beyond the selection limit
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 65, 512, 0, 0, 0x1000, 64, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 64, 32, 0, 0, 0x1000, 3072, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 64, 512, 0, 0, 0x1000, 65537, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_UNSUPPORTED
    # chunked rows: k * ceil(M / 4096) <= 1024, and 8 k <= 1024 unless cap >= 8 k
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 103, 1024, 0, 0, 0x1000, 40960, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_UNSUPPORTED
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 129, 1000, 0, 0, 0x1000, 8192, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_UNSUPPORTED
    for k, cap in ((102, 1024), (129, 1032), (64, 512)):  # within the limits: only the workspace is missing
        assert lib.vdm_select_kv(C.byref(d), 75, 8, k, cap, 0, 0, 0x1000, 40960 if k != 129 else 8192, None, 1000,
                                 0x1000, 0x1000, None, 0, None) == V.VDM_ERR_WORKSPACE
    assert lib.vdm_select_kv_heads(C.byref(d), 75, 8, 64, 512, 0, 0, 0x1000, 16385, None, 1000, 0x1000, 0x1000,
                                   None, 0, None) == V.VDM_ERR_UNSUPPORTED
    assert lib.vdm_select_kv_heads(C.byref(d), 75, 8, 64, 512, 0, 0, 0x1000, 16384, None, 1000, 0x1000, 0x1000,
                                   None, 0, None) == V.VDM_ERR_WORKSPACE
    assert lib.vdm_select_workspace_size(C.byref(d), 65536) > 0 and lib.vdm_select_workspace_size(C.byref(d), 65537) == 0
    assert lib.vdm_select_heads_workspace_size(C.byref(d), 16384) > 0
    assert lib.vdm_select_heads_workspace_size(C.byref(d), 16385) == 0
    # blocks == NULL requires nblk = NB^3 (76 points per axis -> 10 blocks)
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 64, 512, 0, 0, 0x1000, 3072, None, 999, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_INVALID_ARG
    # probes: 0 (corners) or 1 (random)
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 64, 512, 2, 0, 0x1000, 3072, None, 1000, 0x1000, 0x1000, None, 0,
                             None) == V.VDM_ERR_INVALID_ARG
    # the score scratch is required and sized by vdm_select_workspace_size
    need = lib.vdm_select_workspace_size(C.byref(d), 3072)
    assert need >= 32 * 3072 * 4
    assert lib.vdm_select_kv(C.byref(d), 75, 8, 64, 512, 0, 0, 0x1000, 3072, None, 1000, 0x1000, 0x1000, 0x1000,
                             need - 1, None) == V.VDM_ERR_WORKSPACE
    p = V.hier_params(R0=75, levels=3)
    assert lib.vdm_hier_workspace_size(C.byref(d), C.byref(p), 3072) > 27 * 10 ** 6 * 4
    bad = V.hier_params(R0=75, levels=7)
    assert lib.vdm_hier_workspace_size(C.byref(d), C.byref(bad), 3072) == 0
    bad = V.hier_params(kvsel={"k": 64, "cap": 512})
    bad.probes = 3
    assert lib.vdm_hier_workspace_size(C.byref(d), C.byref(bad), 3072) == 0 and "probes" in V.vdm_last_error()
    bad = V.hier_params(tau=float("nan"))
    assert lib.vdm_decode_hier(C.byref(d), C.byref(bad), 0x1000, 0x1000, 3072, 0x1000, 301 ** 3, None, None,
                               0x1000, 1 << 40, None) == V.VDM_ERR_INVALID_ARG
    p = V.hier_params(kvsel=dict(k=64, cap=512, block=4))
    assert lib.vdm_decode_hier(C.byref(d), C.byref(p), 0x1000, 0x1000, 3072, 0x1000, 301 ** 3, None, None,
                               0x1000, 1 << 40, None) == V.VDM_ERR_UNSUPPORTED
    p = V.hier_params()
    assert lib.vdm_decode_hier(C.byref(d), C.byref(p), 0x1000, 0x1000, 3072, 0x1000, 300 ** 3, None, None,
                               0x1000, 1 << 40, None) == V.VDM_ERR_INVALID_ARG  # volume too small
    assert lib.vdm_decode_hier(C.byref(d), C.byref(p), 0x1000, 0x1000, 3072, 0x1000, 301 ** 3, None, None,
                               0x1000, 1024, None) == V.VDM_ERR_WORKSPACE


def test_timing_api_without_launches():
    import shape_vae_decoding_amd as V

    V.vdm_timing(2)
    V.vdm_timing(1)
    assert V.vdm_timing_read("decode") == (0, 0.0)  # nothing launched: no events to wait for
    V.vdm_timing(0)
    assert V._lib.vdm_timing(3) == V.VDM_ERR_INVALID_ARG
    assert "timing mode" in V.vdm_last_error()
    n, ms = C.c_int64(), C.c_double()
    assert V._lib.vdm_timing_read(len(V.TIME_KINDS), C.byref(n), C.byref(ms)) == V.VDM_ERR_INVALID_ARG
    assert V._lib.vdm_timing_read(0, None, C.byref(ms)) == V.VDM_ERR_INVALID_ARG


def test_surface_extraction_argument_checks():
    import shape_vae_decoding_amd as V

    lib = V._lib
    fake = 0x100000  # never dereferenced: every case fails validation first
    assert lib.vdm_surface_workspace_size(0) == 0 and "R=0" in V.vdm_last_error()
    assert lib.vdm_surface_workspace_size(894) == 0
    n300 = lib.vdm_surface_workspace_size(300)
    # per axis one bit per point (8-byte words of 63 points) and an int32 prefix per
    # word, one more bit plane for the inside test, and small partial sums
    words = 301 * 301 * ((301 + 62) // 63)
    assert 3 * 12 * words + 8 * words <= n300 <= 2 * (3 * 12 * words + 8 * words)
    ok = dict(vol=fake, R=300, mask=None, verts=fake, mv=10, tris=fake, mt=10, edges=None, counts=fake,
              ws=fake, wsb=n300)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.vdm_extract_surface(a["vol"], a["R"], a["mask"], a["verts"], a["mv"], a["tris"], a["mt"],
                                       a["edges"], a["counts"], a["ws"], a["wsb"], None)

    assert call(R=0) == V.VDM_ERR_INVALID_ARG
    assert call(vol=None) == V.VDM_ERR_INVALID_ARG
    assert call(counts=None) == V.VDM_ERR_INVALID_ARG
    assert call(verts=None) == V.VDM_ERR_INVALID_ARG
    assert call(mt=-1) == V.VDM_ERR_INVALID_ARG
    assert call(vol=fake + 2) == V.VDM_ERR_INVALID_ARG and "misaligned" in V.vdm_last_error()
    assert call(edges=fake + 4) == V.VDM_ERR_INVALID_ARG
    assert call(wsb=n300 - 1) == V.VDM_ERR_WORKSPACE
    assert call(ws=fake + 16) == V.VDM_ERR_WORKSPACE


def test_batched_decode_argument_checks():
    import shape_vae_decoding_amd as V

    lib = V._lib
    d = _decoder()
    q = V._Queries(V.VDM_Q_GRID, 16, 17 ** 3, None, None)
    assert lib.vdm_dense_batch_workspace_size(C.byref(d), 0, 3072) == 0
    need = lib.vdm_dense_batch_workspace_size(C.byref(d), 4, 3072)
    one = lib.vdm_dense_batch_workspace_size(C.byref(d), 1, 3072)
    assert need > 3 * (one - 2 * 256)  # per-shape packed K/V dominate
    assert lib.vdm_decode_dense_batch(C.byref(d), C.byref(q), 0, 0x1000, 0x1000, 3072, 0x1000, 0x1000, need,
                                      None) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_decode_dense_batch(C.byref(d), C.byref(q), 4, None, 0x1000, 3072, 0x1000, 0x1000, need,
                                      None) == V.VDM_ERR_INVALID_ARG
    assert lib.vdm_decode_dense_batch(C.byref(d), C.byref(q), 4, 0x1000, 0x1000, 3072, 0x1000, 0x1000, need - 1,
                                      None) == V.VDM_ERR_WORKSPACE


def test_batched_hier_argument_checks():
    import shape_vae_decoding_amd as V

    lib = V._lib
    d = _decoder()
    p = V.hier_params(R0=75, levels=3)
    assert lib.vdm_hier_batch_workspace_size(C.byref(d), C.byref(p), 0, 3072) == 0
    one = lib.vdm_hier_workspace_size(C.byref(d), C.byref(p), 3072)
    need = lib.vdm_hier_batch_workspace_size(C.byref(d), C.byref(p), 4, 3072)
    assert need % 4 == 0 and need // 4 >= one and need // 4 % 256 == 0 and need // 4 - one < 256
    P3 = 301 ** 3

    def call(B=4, K=0x1000, vol_elems=4 * P3, wsb=need, ws=0x1000, params=p):
        return lib.vdm_decode_hier_batch(C.byref(d), C.byref(params), B, K, 0x1000, 3072, 0x1000, vol_elems, None,
                                         ws, wsb, None)

    assert call(B=0) == V.VDM_ERR_INVALID_ARG
    assert call(B=4097) == V.VDM_ERR_INVALID_ARG
    assert call(K=None) == V.VDM_ERR_INVALID_ARG
    assert call(K=0x1008) == V.VDM_ERR_INVALID_ARG
    assert call(vol_elems=4 * P3 - 1) == V.VDM_ERR_INVALID_ARG
    assert call(wsb=need - 1) == V.VDM_ERR_WORKSPACE
    assert call(ws=0x1010) == V.VDM_ERR_WORKSPACE
    bad = V.hier_params(R0=75, levels=7)
    assert call(params=bad) == V.VDM_ERR_INVALID_ARG
