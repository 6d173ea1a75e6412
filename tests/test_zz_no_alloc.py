"""mq_gemm_noalloc (the GEMM whose K-slice partials live in the library's
per-device scratch array) against mq_gemm (the caller's workspace), through
the C ABI: bit-identical outputs over calls in a row whose partials shrink
(the scratch keeps the previous call's contents), the 64 MiB limit refused
with MQ_ERR_WORKSPACE and nothing written, and no-split shapes."""

import ctypes

import numpy as np
import pytest
import torch

import nested_int_matmul_amd as mq
from nested_int_matmul_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _linear(N, K, group, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(inputs.seed64("mistral_small", inputs.TAG_W, 50, seed))
    codes = torch.randint(0, 256, (N, K), generator=g, device=DEV, dtype=torch.int32)
    codes = codes.to(torch.uint8)
    G = K // group
    alpha = (torch.rand((N, G), generator=g, device=DEV) * 1e-3 + 1e-4).contiguous()
    zero = (torch.rand((N, G), generator=g, device=DEV) * 255.0).contiguous()
    return codes, alpha, zero


def _x(M, K, seed):
    xb = inputs.activations_bf16("mistral_small", M, K, layer=50, matrix=seed, heavy_channels=8)
    return torch.from_numpy(xb.view(np.int16)).to(DEV)


def _call_noalloc(packed, r, alpha, zero, group, N, K, x, M, y):
    L = mq.lib()
    return L.mq_gemm_noalloc(ctypes.c_void_p(packed.data_ptr()), r,
                             ctypes.c_void_p(alpha.data_ptr()), ctypes.c_void_p(zero.data_ptr()),
                             group, N, K, ctypes.c_void_p(x.data_ptr()), M,
                             ctypes.c_void_p(y.data_ptr()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (M, N, K, group, r): the first needs the whole 64 MiB (the prefill down
# projection, K split in 2), then 45.9 MB (mid batch, 4 slices), 14.7 MB and
# 3.7 MB (small batch, 4 and 14 slices), then shapes with no split at all
CASES = [
    (2048, 4096, 14336, 128, 4),
    (200, 14336, 4096, 128, 2),
    (64, 14336, 4096, 128, 8),
    (16, 4096, 14336, 14336, 4),
    (33, 301, 1536, 128, 6),
    (4, 512, 1024, 128, 4),
    (2048, 1024, 1024, 1024, 3),
]


def test_noalloc_matches_gemm_over_shrinking_calls():
    print("mq_gemm_noalloc vs mq_gemm", flush=True)
    prev_need = None
    for i, (M, N, K, group, r) in enumerate(CASES):
        need = mq.gemm_workspace_bytes(M, N, K, group)
        assert need <= mq.GEMM_NOALLOC_MAX_BYTES
        if prev_need is not None and i <= 3:
            assert need < prev_need  # each call's partials are smaller than the last one's
        prev_need = need
        print(f"  case M={M} N={N} K={K} group={group} r={r} partials={need} B", flush=True)
        codes, alpha, zero = _linear(N, K, group, i)
        plane = mq.pack(codes, r)
        x = _x(M, K, i)
        y_ref = mq.gemm(plane, r, alpha, zero, group, N, K, x)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        st = _call_noalloc(plane, r, alpha, zero, group, N, K, x, M, y)
        assert st == 0, mq.lib().mq_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"case {i}: outputs differ"
        # again, right away: the scratch now holds this call's own partials
        y2 = torch.full_like(y, float("nan"))
        assert _call_noalloc(plane, r, alpha, zero, group, N, K, x, M, y2) == 0
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref), f"case {i}: repeated call differs"
        del codes, plane, y, y2, y_ref


def test_noalloc_refuses_more_than_its_scratch():
    """M = 64, K = 16384 (16 slices of partials) and N = 16448: 67.4 MB of
    partials, above the 64 MiB scratch.  The buffers have their full sizes
    (the call must refuse before reading any of them)."""
    print("mq_gemm_noalloc over the limit", flush=True)
    M, N, K, group, r = 64, 16448, 16384, 128, 2
    assert mq.gemm_workspace_bytes(M, N, K, group) > mq.GEMM_NOALLOC_MAX_BYTES
    plane = torch.empty(mq.packed_bytes(N, K, r), dtype=torch.uint8, device=DEV)
    alpha = torch.empty((N, K // group), dtype=torch.float32, device=DEV)
    zero = torch.empty_like(alpha)
    x = torch.zeros((M, K), dtype=torch.int16, device=DEV)
    y = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
    assert _call_noalloc(plane, r, alpha, zero, group, N, K, x, M, y) == 6  # MQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
