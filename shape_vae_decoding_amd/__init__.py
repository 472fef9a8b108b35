"""Python binding of libvdm.so, the gfx950 vecset SDF decoder (see include/vdm.h).

Argument marshalling only: every step of the decoder runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. Importing this
module raises if the built library is missing; there is no fallback path.

Functions carry the C names: vdm_embed_queries, vdm_project_kv,
vdm_decode_dense, vdm_select_kv, vdm_decode_hier, plus the workspace-size
helpers. ``Decoder`` bundles a vdm_decoder struct with the tensors it points to.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VDM_LIB names another build of the library (e.g. an instrumented one); default: the in-tree build
LIB_PATH = os.environ.get("VDM_LIB") or os.path.join(_HERE, "libvdm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python shape_vae_decoding_amd/build.py`")
_lib = C.CDLL(LIB_PATH)

VDM_OK, VDM_ERR_INVALID_ARG, VDM_ERR_UNSUPPORTED, VDM_ERR_WORKSPACE, VDM_ERR_HIP = 0, -1, -2, -3, -4
VDM_F32, VDM_BF16 = 0, 1
VDM_Q_POINTS, VDM_Q_GRID, VDM_Q_GRID_LIST = 0, 1, 2
MAX_PRIMS, MAX_LEVELS, STAT_FIELDS = 16, 6, 8
STAT_NAMES = ["R", "tested", "active", "kept", "queries", "blocks", "items", "selected"]
EXPORTS = [
    "vdm_embed_queries", "vdm_project_kv", "vdm_decode_dense", "vdm_select_kv", "vdm_decode_hier",
    "vdm_dense_workspace_size", "vdm_select_workspace_size", "vdm_hier_workspace_size", "vdm_timing",
    "vdm_timing_read", "vdm_version", "vdm_last_error", "vdm_extract_surface", "vdm_surface_workspace_size",
    "vdm_decode_dense_batch", "vdm_dense_batch_workspace_size", "vdm_decode_hier_batch",
    "vdm_hier_batch_workspace_size", "vdm_decode_dense_noalloc", "vdm_decode_local", "vdm_local_workspace_size",
    "vdm_select_kv_heads", "vdm_select_heads_workspace_size", "vdm_device_info",
]
TIME_KINDS = ["decode", "decode_gathered", "select", "embed", "project_kv", "cell_test", "dilate", "mark", "scan",
              "emit", "fill", "surface", "local_grid", "local_knn", "local_fuse", "local_head"]


class VdmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"vdm status {status}: {msg}")
        self.status = status


class _Prim(C.Structure):
    _fields_ = [("kind", C.c_int32), ("centre", C.c_float * 3), ("size", C.c_float * 3)]


class _Decoder(C.Structure):
    _fields_ = [
        ("D", C.c_int32), ("H", C.c_int32), ("F", C.c_int32), ("n_freq", C.c_int32), ("dtype", C.c_int32),
        ("net_scale", C.c_float),
        ("Wq", C.c_void_p), ("Wk", C.c_void_p), ("Wv", C.c_void_p), ("Wo", C.c_void_p),
        ("W1", C.c_void_p), ("W2", C.c_void_p), ("w_head", C.c_void_p),
        ("n_prims", C.c_int32), ("prims", _Prim * MAX_PRIMS),
    ]


class _Queries(C.Structure):
    _fields_ = [("mode", C.c_int32), ("R", C.c_int32), ("N", C.c_int64), ("xyz", C.c_void_p), ("list", C.c_void_p)]


class _KvSel(C.Structure):
    _fields_ = [("block", C.c_int32), ("cap", C.c_int32), ("sel_idx", C.c_void_p), ("sel_cnt", C.c_void_p),
                ("block_row", C.c_void_p), ("heads", C.c_int32)]


class _HierParams(C.Structure):
    _fields_ = [("R0", C.c_int32), ("levels", C.c_int32), ("dilation", C.c_int32), ("tau", C.c_float),
                ("use_kvsel", C.c_int32), ("block", C.c_int32), ("k", C.c_int32), ("cap", C.c_int32),
                ("probes", C.c_int32), ("seed", C.c_uint64), ("heads", C.c_int32)]


class _LocalDecoder(C.Structure):
    _fields_ = [
        ("C", C.c_int32), ("F", C.c_int32), ("K", C.c_int32), ("hidden", C.c_int32), ("net_scale", C.c_float),
        ("A", C.c_void_p), ("a", C.c_void_p), ("B", C.c_void_p), ("W1", C.c_void_p), ("W2", C.c_void_p),
        ("w_head", C.c_void_p), ("n_prims", C.c_int32), ("prims", _Prim * MAX_PRIMS),
    ]


_PtrArr = C.c_void_p * MAX_LEVELS


class _HierDebug(C.Structure):
    _fields_ = [("vol", _PtrArr), ("active", _PtrArr), ("kept", _PtrArr), ("list", _PtrArr),
                ("sel_blocks", _PtrArr), ("sel_cnt", _PtrArr), ("sel_idx", _PtrArr)]


_st = C.c_int32


def _bind(lib) -> None:
    """Argument and result types of every entry point of a build of the library."""
    lib.vdm_embed_queries.argtypes = [C.POINTER(_Decoder), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    lib.vdm_embed_queries.restype = _st
    lib.vdm_project_kv.argtypes = [C.POINTER(_Decoder), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.vdm_project_kv.restype = _st
    lib.vdm_decode_dense.argtypes = [C.POINTER(_Decoder), C.POINTER(_Queries), C.c_void_p, C.c_void_p, C.c_int64,
                                      C.POINTER(_KvSel), C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.vdm_decode_dense.restype = _st
    lib.vdm_decode_dense_noalloc.argtypes = [C.POINTER(_Decoder), C.POINTER(_Queries), C.c_void_p, C.c_void_p,
                                              C.c_int64, C.c_void_p, C.c_void_p]
    lib.vdm_decode_dense_noalloc.restype = _st
    lib.vdm_select_kv.argtypes = [C.POINTER(_Decoder), C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                   C.c_uint64, C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_size_t, C.c_void_p]
    lib.vdm_select_kv.restype = _st
    lib.vdm_select_kv_heads.argtypes = lib.vdm_select_kv.argtypes
    lib.vdm_select_kv_heads.restype = _st
    lib.vdm_select_heads_workspace_size.argtypes = [C.POINTER(_Decoder), C.c_int64]
    lib.vdm_select_heads_workspace_size.restype = C.c_size_t
    lib.vdm_decode_hier.argtypes = [C.POINTER(_Decoder), C.POINTER(_HierParams), C.c_void_p, C.c_void_p, C.c_int64,
                                     C.c_void_p, C.c_int64, C.c_void_p, C.POINTER(_HierDebug), C.c_void_p, C.c_size_t,
                                     C.c_void_p]
    lib.vdm_decode_hier.restype = _st
    lib.vdm_dense_workspace_size.argtypes = [C.POINTER(_Decoder), C.c_int64, C.c_int64, C.c_int32]
    lib.vdm_dense_workspace_size.restype = C.c_size_t
    lib.vdm_select_workspace_size.argtypes = [C.POINTER(_Decoder), C.c_int64]
    lib.vdm_select_workspace_size.restype = C.c_size_t
    lib.vdm_hier_workspace_size.argtypes = [C.POINTER(_Decoder), C.POINTER(_HierParams), C.c_int64]
    lib.vdm_hier_workspace_size.restype = C.c_size_t
    lib.vdm_extract_surface.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                                         C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.vdm_extract_surface.restype = _st
    lib.vdm_surface_workspace_size.argtypes = [C.c_int32]
    lib.vdm_surface_workspace_size.restype = C.c_size_t
    lib.vdm_decode_dense_batch.argtypes = [C.POINTER(_Decoder), C.POINTER(_Queries), C.c_int32, C.c_void_p, C.c_void_p,
                                            C.c_int64, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.vdm_decode_dense_batch.restype = _st
    lib.vdm_dense_batch_workspace_size.argtypes = [C.POINTER(_Decoder), C.c_int32, C.c_int64]
    lib.vdm_dense_batch_workspace_size.restype = C.c_size_t
    lib.vdm_decode_hier_batch.argtypes = [C.POINTER(_Decoder), C.POINTER(_HierParams), C.c_int32, C.c_void_p,
                                           C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                           C.c_size_t, C.c_void_p]
    lib.vdm_decode_hier_batch.restype = _st
    lib.vdm_hier_batch_workspace_size.argtypes = [C.POINTER(_Decoder), C.POINTER(_HierParams), C.c_int32, C.c_int64]
    lib.vdm_hier_batch_workspace_size.restype = C.c_size_t
    lib.vdm_decode_local.argtypes = [C.POINTER(_LocalDecoder), C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                                      C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    lib.vdm_decode_local.restype = _st
    lib.vdm_local_workspace_size.argtypes = [C.POINTER(_LocalDecoder), C.c_int64, C.c_int64]
    lib.vdm_local_workspace_size.restype = C.c_size_t
    lib.vdm_timing.argtypes = [C.c_int32]
    lib.vdm_timing.restype = C.c_int
    lib.vdm_timing_read.argtypes = [C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_double)]
    lib.vdm_timing_read.restype = C.c_int
    lib.vdm_version.restype = C.c_int32
    lib.vdm_device_info.argtypes = [C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    lib.vdm_device_info.restype = _st
    lib.vdm_last_error.restype = C.c_char_p


_bind(_lib)

# the bounds-checked build (VDM_DEBUG): every data-dependent index in the kernels
# is checked and each call reports the first failed check (see debug_library)
DEBUG_LIB_PATH = os.path.join(_HERE, "libvdm_debug.so")


def debug_library():
    """The bounds-checked build of the library, bound like the default one.
    Assigning it to this module's ``_lib`` routes every wrapper through it."""
    if not os.path.exists(DEBUG_LIB_PATH):
        raise ImportError(f"{DEBUG_LIB_PATH} is not built; run `python shape_vae_decoding_amd/build.py`")
    lib = C.CDLL(DEBUG_LIB_PATH)
    _bind(lib)
    return lib


def vdm_version() -> int:
    return int(_lib.vdm_version())


def vdm_device_info() -> dict:
    cus, khz = C.c_int32(0), C.c_int32(0)
    _check(_lib.vdm_device_info(C.byref(cus), C.byref(khz)))
    return {"compute_units": cus.value, "peak_clock_khz": khz.value}


def vdm_last_error() -> str:
    return _lib.vdm_last_error().decode()


def _check(status: int) -> None:
    if status != VDM_OK:
        raise VdmError(status, vdm_last_error())


def vdm_timing(mode: int) -> None:
    """1 = record launch events, 0 = stop (records kept), 2 = drop records."""
    _check(_lib.vdm_timing(mode))


def vdm_timing_read(kind: str):
    """(launches, total ms) recorded for one of TIME_KINDS; waits for the events."""
    n, ms = C.c_int64(), C.c_double()
    _check(_lib.vdm_timing_read(TIME_KINDS.index(kind), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class Decoder:
    """A vdm_decoder plus the device tensors it points to.

    weights: Wq [D,51], Wk/Wv/Wo [D,D], W1 [F,D], W2 [D,F] in the decoder dtype
    and w_head [D] float32 (device tensors). prims: objects with .kind, .centre,
    .size (sphere: size[0] = radius; box: half extents)."""

    def __init__(self, weights: Dict[str, torch.Tensor], prims: Sequence, net_scale: float = 0.05):
        wq = weights["Wq"]
        self.torch_dtype = wq.dtype
        dtype = {torch.bfloat16: VDM_BF16, torch.float32: VDM_F32}[wq.dtype]
        D = wq.shape[0]
        F = weights["W1"].shape[0]
        self.tensors = {}
        for k in ("Wq", "Wk", "Wv", "Wo", "W1", "W2"):
            self.tensors[k] = _dev(weights[k], wq.dtype, k)
        self.tensors["w_head"] = _dev(weights["w_head"], torch.float32, "w_head")
        s = _Decoder()
        s.D, s.H, s.F, s.n_freq, s.dtype = D, D // 64, F, 8, dtype
        s.net_scale = float(net_scale)
        for k, t in self.tensors.items():
            setattr(s, k, t.data_ptr())
        if len(prims) > MAX_PRIMS:
            raise ValueError("too many primitives")
        s.n_prims = len(prims)
        for i, p in enumerate(prims):
            s.prims[i].kind = int(p.kind)
            for c in range(3):
                s.prims[i].centre[c] = float(p.centre[c])
                s.prims[i].size[c] = float(p.size[c])
        self.struct = s
        self.D, self.H, self.F, self.dtype = D, D // 64, F, dtype

    @property
    def ref(self):
        return C.byref(self.struct)


class LocalDecoder:
    """A vdm_local_decoder plus the device tensors it points to.

    weights: A [hidden,3], a [hidden] float32; B [C,hidden], W1 [F,C], W2 [C,F]
    bf16; w_head [C] float32 (device tensors). K: neighbours per query."""

    def __init__(self, weights: Dict[str, torch.Tensor], prims: Sequence, K: int = 16, net_scale: float = 0.05):
        self.tensors = {}
        for k in ("A", "a", "w_head"):
            self.tensors[k] = _dev(weights[k], torch.float32, k)
        for k in ("B", "W1", "W2"):
            self.tensors[k] = _dev(weights[k], torch.bfloat16, k)
        s = _LocalDecoder()
        s.C, s.hidden = self.tensors["B"].shape
        s.F = self.tensors["W1"].shape[0]
        s.K = int(K)
        s.net_scale = float(net_scale)
        for k, t in self.tensors.items():
            setattr(s, k, t.data_ptr())
        if len(prims) > MAX_PRIMS:
            raise ValueError("too many primitives")
        s.n_prims = len(prims)
        for i, p in enumerate(prims):
            s.prims[i].kind = int(p.kind)
            for c in range(3):
                s.prims[i].centre[c] = float(p.centre[c])
                s.prims[i].size[c] = float(p.size[c])
        self.struct = s
        self.C, self.F, self.K = s.C, s.F, s.K

    @property
    def ref(self):
        return C.byref(self.struct)


def vdm_local_workspace_size(dec: LocalDecoder, M: int, N: int) -> int:
    n = int(_lib.vdm_local_workspace_size(dec.ref, M, N))
    if n == 0:
        raise VdmError(VDM_ERR_INVALID_ARG, vdm_last_error())
    return n


def vdm_decode_local(dec: LocalDecoder, sup_xyz: torch.Tensor, feats: torch.Tensor, xyz: torch.Tensor,
                     sdf: torch.Tensor, nbr: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    _dev(sup_xyz, torch.float32, "sup_xyz")
    _dev(feats, torch.bfloat16, "feats")
    _dev(xyz, torch.float32, "xyz")
    _dev(sdf, torch.float32, "sdf")
    if nbr is not None:
        _dev(nbr, torch.int32, "nbr")
    M, N = sup_xyz.shape[0], xyz.shape[0]
    if ws is None:
        ws = workspace(vdm_local_workspace_size(dec, M, N), sdf.device)
    _check(_lib.vdm_decode_local(dec.ref, sup_xyz.data_ptr(), feats.data_ptr(), M, xyz.data_ptr(), N,
                                 sdf.data_ptr(), _ptr(nbr), ws.data_ptr(), ws.numel(), _stream(stream)))


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A device byte buffer usable as a workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------- calls

def vdm_embed_queries(dec: Decoder, xyz: torch.Tensor, Q: torch.Tensor, stream=None) -> None:
    _dev(xyz, torch.float32, "xyz")
    _dev(Q, dec.torch_dtype, "Q")
    _check(_lib.vdm_embed_queries(dec.ref, xyz.data_ptr(), xyz.shape[0], Q.data_ptr(), _stream(stream)))


def vdm_project_kv(dec: Decoder, Z: torch.Tensor, K: torch.Tensor, V: torch.Tensor, stream=None) -> None:
    for n, t in (("Z", Z), ("K", K), ("V", V)):
        _dev(t, dec.torch_dtype, n)
    _check(_lib.vdm_project_kv(dec.ref, Z.data_ptr(), Z.shape[0], K.data_ptr(), V.data_ptr(), _stream(stream)))


class Queries:
    """A vdm_queries struct plus the device tensors it points to (kept alive for
    as long as this object is)."""

    def __init__(self, struct: _Queries, *keep: torch.Tensor):
        self.struct = struct
        self.keep = keep

    @property
    def N(self) -> int:
        return int(self.struct.N)


def queries_points(xyz: torch.Tensor) -> Queries:
    _dev(xyz, torch.float32, "xyz")
    return Queries(_Queries(VDM_Q_POINTS, 0, xyz.shape[0], xyz.data_ptr(), None), xyz)


def queries_grid(R: int) -> Queries:
    return Queries(_Queries(VDM_Q_GRID, R, (R + 1) ** 3, None, None))


def queries_list(R: int, lin: torch.Tensor) -> Queries:
    _dev(lin, torch.int32, "list")
    return Queries(_Queries(VDM_Q_GRID_LIST, R, lin.shape[0], None, lin.data_ptr()), lin)


class KvSel:
    """A vdm_kvsel struct plus the device tensors it points to."""

    def __init__(self, struct: _KvSel, *keep: torch.Tensor):
        self.struct = struct
        self.keep = keep


def kvsel(block: int, cap: int, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
          block_row: Optional[torch.Tensor] = None, heads: bool = False) -> KvSel:
    """heads: the sets come from vdm_select_kv_heads (rows [block][H])."""
    _dev(sel_idx, torch.int32, "sel_idx")
    _dev(sel_cnt, torch.int32, "sel_cnt")
    keep = [sel_idx, sel_cnt]
    if block_row is not None:
        _dev(block_row, torch.int32, "block_row")
        keep.append(block_row)
    return KvSel(_KvSel(block, cap, sel_idx.data_ptr(), sel_cnt.data_ptr(), _ptr(block_row), int(heads)), *keep)


def vdm_dense_workspace_size(dec: Decoder, M: int, N: int, with_sel: bool = False) -> int:
    n = int(_lib.vdm_dense_workspace_size(dec.ref, M, N, int(with_sel)))
    if n == 0:
        raise VdmError(VDM_ERR_INVALID_ARG, vdm_last_error())
    return n


def vdm_dense_batch_workspace_size(dec: Decoder, B: int, M: int) -> int:
    n = _lib.vdm_dense_batch_workspace_size(dec.ref, B, M)
    if n == 0:
        raise VdmError(-1, vdm_last_error())
    return n


def vdm_decode_dense_batch(dec: Decoder, q: Queries, K: torch.Tensor, V: torch.Tensor, sdf: torch.Tensor,
                           ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """K, V [B, M, D] in the decoder dtype, sdf [B, N] float32 (see include/vdm.h)."""
    _dev(K, dec.torch_dtype, "K")
    _dev(V, dec.torch_dtype, "V")
    _dev(sdf, torch.float32, "sdf")
    if K.dim() != 3 or V.shape != K.shape or sdf.dim() != 2 or sdf.shape[0] != K.shape[0] or sdf.shape[1] < q.N:
        raise ValueError("K, V must be [B, M, D] and sdf [B, N]")
    if sdf.shape[1] != q.N:
        raise ValueError("sdf rows must hold exactly N values (the batch stride is N)")
    B, M = K.shape[0], K.shape[1]
    if ws is None:
        ws = workspace(vdm_dense_batch_workspace_size(dec, B, M), sdf.device)
    _check(_lib.vdm_decode_dense_batch(dec.ref, C.byref(q.struct), B, K.data_ptr(), V.data_ptr(), M, sdf.data_ptr(),
                                       ws.data_ptr(), ws.numel(), _stream(stream)))


def vdm_select_workspace_size(dec: Decoder, M: int) -> int:
    return int(_lib.vdm_select_workspace_size(dec.ref, M))


def vdm_hier_workspace_size(dec: Decoder, params: _HierParams, M: int) -> int:
    n = int(_lib.vdm_hier_workspace_size(dec.ref, C.byref(params), M))
    if n == 0:
        raise VdmError(VDM_ERR_INVALID_ARG, vdm_last_error())
    return n


def vdm_decode_dense(dec: Decoder, q: Queries, K: torch.Tensor, V: torch.Tensor, sdf: torch.Tensor,
                     sel: Optional[KvSel] = None, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _dev(K, dec.torch_dtype, "K")
    _dev(V, dec.torch_dtype, "V")
    _dev(sdf, torch.float32, "sdf")
    M = K.shape[0]
    if ws is None:
        ws = workspace(vdm_dense_workspace_size(dec, M, q.N, sel is not None), sdf.device)
    _check(_lib.vdm_decode_dense(dec.ref, C.byref(q.struct), K.data_ptr(), V.data_ptr(), M,
                                 C.byref(sel.struct) if sel is not None else None, sdf.data_ptr(), ws.data_ptr(),
                                 ws.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 48 << 20


def vdm_decode_dense_noalloc(dec: Decoder, q: Queries, K: torch.Tensor, V: torch.Tensor, sdf: torch.Tensor,
                             stream=None) -> None:
    """vdm_decode_dense with full attention and no workspace: the library's
    per-GPU scratch array stands in for it (nothing is allocated)."""
    _dev(K, dec.torch_dtype, "K")
    _dev(V, dec.torch_dtype, "V")
    _dev(sdf, torch.float32, "sdf")
    _check(_lib.vdm_decode_dense_noalloc(dec.ref, C.byref(q.struct), K.data_ptr(), V.data_ptr(), K.shape[0],
                                         sdf.data_ptr(), _stream(stream)))


PROBES = {"corners": 0, "random": 1}


def vdm_select_kv(dec: Decoder, R: int, block: int, k: int, cap: int, K: torch.Tensor,
                  blocks: Optional[torch.Tensor], sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                  nblk: Optional[int] = None, ws: Optional[torch.Tensor] = None, stream=None,
                  probes: str = "corners", seed: int = 0, heads: bool = False) -> None:
    """heads: one set per (block, head) (vdm_select_kv_heads): sel_idx [nblk, H, cap], sel_cnt [nblk, H]."""
    _dev(K, dec.torch_dtype, "K")
    _dev(sel_idx, torch.int32, "sel_idx")
    _dev(sel_cnt, torch.int32, "sel_cnt")
    if blocks is not None:
        _dev(blocks, torch.int32, "blocks")
        nblk = blocks.shape[0]
    elif nblk is None:
        nb = -(-(R + 1) // block)
        nblk = nb ** 3
    if ws is None:
        size = _lib.vdm_select_heads_workspace_size if heads else _lib.vdm_select_workspace_size
        ws = workspace(int(size(dec.ref, K.shape[0])), K.device)
    fn = _lib.vdm_select_kv_heads if heads else _lib.vdm_select_kv
    _check(fn(dec.ref, R, block, k, cap, PROBES[probes], seed, K.data_ptr(), K.shape[0], _ptr(blocks), nblk,
              sel_idx.data_ptr(), sel_cnt.data_ptr(), _ptr(ws), ws.numel(), _stream(stream)))


def hier_params(R0=75, levels=3, tau=2 * 2 / 300, dilation=1, kvsel: Optional[dict] = None) -> _HierParams:
    p = _HierParams(R0, levels, dilation, float(tau), 0, 8, 64, 512, 0, 0, 0)
    if kvsel:
        p.use_kvsel, p.block, p.k, p.cap = 1, kvsel.get("block", 8), kvsel["k"], kvsel["cap"]
        p.probes, p.seed = PROBES[kvsel.get("probes", "corners")], kvsel.get("seed", 0)
        p.heads = int(bool(kvsel.get("heads", False)))
    return p


class HierDebug:
    """Device buffers for the inspection outputs of vdm_decode_hier."""

    def __init__(self, params: _HierParams, device=None, with_sel: bool = False, H: int = 4):
        """H: heads of the decoder (per-head sets hold H rows per block)."""
        dev = device or "cuda"
        ns = H if params.heads else 1
        self.levels = []
        s = _HierDebug()
        for L in range(params.levels):
            R = params.R0 << L
            P = R + 1
            nb = -(-P // 8)
            d = {
                "vol": torch.empty(P ** 3, dtype=torch.float32, device=dev),
                "active": torch.empty(R ** 3, dtype=torch.uint8, device=dev),
                "kept": torch.zeros(R ** 3, dtype=torch.uint8, device=dev),
                "list": torch.empty(P ** 3, dtype=torch.int32, device=dev),
            }
            if with_sel:
                d["sel_blocks"] = torch.empty(nb ** 3, dtype=torch.int32, device=dev)
                d["sel_cnt"] = torch.empty(nb ** 3 * ns, dtype=torch.int32, device=dev)
                d["sel_idx"] = torch.empty(nb ** 3 * ns * params.cap, dtype=torch.int32, device=dev)
            for k, t in d.items():
                getattr(s, k)[L] = t.data_ptr()
            self.levels.append(d)
        self.struct = s


def vdm_decode_hier(dec: Decoder, params: _HierParams, K: torch.Tensor, V: torch.Tensor, vol: torch.Tensor,
                    stats: Optional[torch.Tensor] = None, dbg: Optional[HierDebug] = None,
                    ws: Optional[torch.Tensor] = None, stream=None) -> None:
    _dev(K, dec.torch_dtype, "K")
    _dev(V, dec.torch_dtype, "V")
    _dev(vol, torch.float32, "vol")
    if stats is not None:
        _dev(stats, torch.int64, "stats")
    M = K.shape[0]
    if ws is None:
        ws = workspace(vdm_hier_workspace_size(dec, params, M), vol.device)
    _check(_lib.vdm_decode_hier(dec.ref, C.byref(params), K.data_ptr(), V.data_ptr(), M, vol.data_ptr(),
                                vol.numel(), _ptr(stats), C.byref(dbg.struct) if dbg is not None else None,
                                ws.data_ptr(), ws.numel(), _stream(stream)))


def vdm_hier_batch_workspace_size(dec: Decoder, params: _HierParams, B: int, M: int) -> int:
    n = int(_lib.vdm_hier_batch_workspace_size(dec.ref, C.byref(params), B, M))
    if n == 0:
        raise VdmError(VDM_ERR_INVALID_ARG, vdm_last_error())
    return n


def vdm_decode_hier_batch(dec: Decoder, params: _HierParams, K: torch.Tensor, V: torch.Tensor, vol: torch.Tensor,
                          stats: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    """K, V [B, M, D] in the decoder dtype, vol [B, (R+1)^3] float32, stats
    [B, levels * VDM_STAT_FIELDS] int64 or None (see include/vdm.h)."""
    _dev(K, dec.torch_dtype, "K")
    _dev(V, dec.torch_dtype, "V")
    _dev(vol, torch.float32, "vol")
    if K.dim() != 3 or V.shape != K.shape or vol.dim() != 2 or vol.shape[0] != K.shape[0]:
        raise ValueError("K, V must be [B, M, D] and vol [B, (R+1)^3]")
    P = (params.R0 << (params.levels - 1)) + 1
    if vol.shape[1] != P ** 3:
        raise ValueError(f"vol rows must hold exactly (R+1)^3 = {P ** 3} values (the batch stride)")
    B, M = K.shape[0], K.shape[1]
    if stats is not None:
        _dev(stats, torch.int64, "stats")
        if stats.shape != (B, params.levels * STAT_FIELDS):
            raise ValueError("stats must be [B, levels * STAT_FIELDS]")
    if ws is None:
        ws = workspace(vdm_hier_batch_workspace_size(dec, params, B, M), vol.device)
    _check(_lib.vdm_decode_hier_batch(dec.ref, C.byref(params), B, K.data_ptr(), V.data_ptr(), M, vol.data_ptr(),
                                      vol.numel(), _ptr(stats), ws.data_ptr(), ws.numel(), _stream(stream)))


def vdm_surface_workspace_size(R: int) -> int:
    n = _lib.vdm_surface_workspace_size(R)
    if n == 0:
        raise VdmError(-1, vdm_last_error())
    return n


def vdm_extract_surface(vol: torch.Tensor, R: int, verts: torch.Tensor, tris: torch.Tensor, counts: torch.Tensor,
                        cell_mask: Optional[torch.Tensor] = None, vert_edges: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """Marching cubes at SDF = 0 on the (R+1)^3 volume (see include/vdm.h).
    verts [max_verts, 3] float32, tris [max_tris, 3] int32, counts [2] int64,
    cell_mask [R^3] uint8 or None, vert_edges [max_verts] int64 or None."""
    _dev(vol, torch.float32, "vol")
    _dev(verts, torch.float32, "verts")
    _dev(tris, torch.int32, "tris")
    _dev(counts, torch.int64, "counts")
    if vol.numel() < (R + 1) ** 3:
        raise ValueError(f"vol holds {vol.numel()} values, (R+1)^3 = {(R + 1) ** 3} needed")
    if cell_mask is not None:
        _dev(cell_mask, torch.uint8, "cell_mask")
        if cell_mask.numel() < R ** 3:
            raise ValueError(f"cell_mask holds {cell_mask.numel()} cells, R^3 = {R ** 3} needed")
    if vert_edges is not None:
        _dev(vert_edges, torch.int64, "vert_edges")
        if vert_edges.numel() < verts.numel() // 3:
            raise ValueError("vert_edges must hold max_verts entries")
    if ws is None:
        ws = workspace(vdm_surface_workspace_size(R), vol.device)
    _check(_lib.vdm_extract_surface(vol.data_ptr(), R, _ptr(cell_mask), verts.data_ptr(), verts.numel() // 3,
                                    tris.data_ptr(), tris.numel() // 3, _ptr(vert_edges), counts.data_ptr(),
                                    ws.data_ptr(), ws.numel(), _stream(stream)))


def stats_dict(stats: torch.Tensor, levels: int):
    s = stats.view(-1)[: levels * STAT_FIELDS].cpu().view(levels, STAT_FIELDS).tolist()
    return [dict(zip(STAT_NAMES, row)) for row in s]
