"""The no-allocation dense decode (vdm_decode_dense_noalloc) through the C ABI:
its output equals vdm_decode_dense's bit for bit on two calls in a row, the
second with fewer queries and fewer tokens (so it reuses the per-GPU scratch
array with stale contents beyond its own), and on the tiny float32 decoder."""

import numpy as np
import pytest
import torch

import vdm_workloads as W
from tests.helpers import dev, gpu_decoder, gpu_kv

pytestmark = pytest.mark.gpu


def V():
    import shape_vae_decoding_amd as mod

    return mod


def _pair(dec, q, K, Vv, n):
    a = torch.full((n,), float("nan"), dtype=torch.float32, device=dev())
    b = torch.full((n,), float("nan"), dtype=torch.float32, device=dev())
    V().vdm_decode_dense(dec, q, K, Vv, a)
    V().vdm_decode_dense_noalloc(dec, q, K, Vv, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_equals_workspace_decode_twice_second_smaller():
    w = W.make(1)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    # call 1: the 33^3 grid against all 3072 tokens
    R = 32
    a, b = _pair(dec, V().queries_grid(R), K, Vv, (R + 1) ** 3)
    print(f"[noalloc] 33^3 grid, M=3072: {np.count_nonzero(a != b)} differing outputs", flush=True)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)
    # call 2: fewer points (a ragged tile) and fewer tokens (a ragged key tile)
    M2 = 1000
    K2, V2 = K[:M2].contiguous(), Vv[:M2].contiguous()
    xyz = torch.from_numpy(W.gen.random_points(77, 1001)).to(dev())
    a, b = _pair(dec, V().queries_points(xyz), K2, V2, 1001)
    print(f"[noalloc] 1001 points, M=1000: {np.count_nonzero(a != b)} differing outputs", flush=True)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


def test_noalloc_float32_decoder():
    w = W.make(0)
    dec = gpu_decoder(w)
    K, Vv = gpu_kv(dec, w)
    R = w.query["R"]
    a, b = _pair(dec, V().queries_grid(R), K, Vv, (R + 1) ** 3)
    assert np.array_equal(a, b)


def test_noalloc_refuses_a_token_set_beyond_its_scratch():
    w = W.make(1)
    dec = gpu_decoder(w)
    M = 60000
    K = torch.zeros((M, w.D), dtype=torch.bfloat16, device=dev())
    sdf = torch.zeros(10, dtype=torch.float32, device=dev())
    xyz = torch.zeros((10, 3), dtype=torch.float32, device=dev())
    with pytest.raises(V().VdmError):
        V().vdm_decode_dense_noalloc(dec, V().queries_points(xyz), K, K, sdf)
    torch.cuda.synchronize()
    assert torch.all(sdf == 0)
