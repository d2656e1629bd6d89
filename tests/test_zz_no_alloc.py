"""moe_dense_gemm_bf16_noalloc through the C ABI: the same bits as moe_dense_gemm_bf16 with a
caller workspace, on two calls in a row (the second smaller, so the library's scratch holds
the first call's partial tiles when it starts), no device allocation by the call, and a
refusal of sizes whose partials exceed the scratch."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import bf16_bits_host, bf16_dev

pytestmark = pytest.mark.gpu


def _raw_noalloc(lib, a, b, c):
    m, k = a.shape
    n = b.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.moe_dense_gemm_bf16_noalloc(
        ctypes.c_void_p(a.data_ptr()), a.stride(0), ctypes.c_void_p(b.data_ptr()), b.stride(0),
        ctypes.c_void_p(c.data_ptr()), c.stride(0), m, n, k, stream)


def test_noalloc_matches_the_workspace_form_on_two_calls(hip):
    lib = hip.load()
    rng = np.random.default_rng(61)
    # the shared expert's down projection at 256 rows (25.2 MB of partials), then a smaller
    # problem with ragged rows
    shapes = [(256, 6144, 2048), (40, 512, 1024)]
    cases = []
    for m, n, k in shapes:
        a = bf16_dev(wl.bf16_normal(rng, (m, k)))
        b = bf16_dev(wl.bf16_normal_scaled(rng, (n, k), 1.0 / np.sqrt(k)))
        ref = torch.full((m, n), 5.0, dtype=torch.bfloat16, device="cuda")
        got = torch.full((m, n), -5.0, dtype=torch.bfloat16, device="cuda")
        ws = hip.dense_workspace(m, n, k)
        cases.append((a, b, ref, got, ws))
    torch.cuda.synchronize()
    for i, (a, b, ref, got, ws) in enumerate(cases):
        hip.moe_dense_gemm_bf16(a, b, ref, workspace=ws)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        assert _raw_noalloc(lib, a, b, got) == 0, lib.moe_w4a16_last_error().decode()
        torch.cuda.synchronize()
        if i > 0:  # the first call on a device may load the library's code and its array
            assert torch.cuda.mem_get_info()[0] == free_before
        assert np.array_equal(bf16_bits_host(got), bf16_bits_host(ref)), f"call {i}"


def test_noalloc_refuses_partials_beyond_the_scratch(hip):
    lib = hip.load()
    m, n, k = 1024, 8320, 4096  # 8 x 65 tiles of 64 KB partials, unsplit: 34.1 MB
    assert hip.moe_dense_workspace_bytes(m, n, k) > hip.DENSE_NOALLOC_SCRATCH_BYTES
    a = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
    c = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda")
    assert _raw_noalloc(lib, a, b, c) == 2  # MOE_ECAPACITY, nothing enqueued
    assert b"scratch" in lib.moe_w4a16_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(c == 3.0))
    with pytest.raises(hip.MoeError):
        hip.moe_dense_gemm_bf16_noalloc(a, b, c)
