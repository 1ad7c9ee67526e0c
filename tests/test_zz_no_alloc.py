"""The no-allocation GEMM entry point (mxfp4_gemm_nt_ex_noalloc) through the C
ABI: the split-K scratch lives in the library's static device array.  Its
output must equal mxfp4_gemm_nt_ex's (caller workspace) bit for bit and meet
the oracle's fp32 bar, on two calls in a row (the second smaller, so the array
holds the first call's partial sums and counters when it starts); a call whose
workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import binding
from tests.gpu_common import device, log, poisoned, random_bf16, to_np, upload

pytestmark = pytest.mark.gpu

SPLITK = binding.KERNELS["splitk"]


def _operands(m, n, k, seed, dev):
    a = random_bf16((m, k), seed, spread=3)
    b = random_bf16((n, k), seed + 1, spread=3)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    return (aq, as_, bq, bs), [upload(t, dev) for t in (aq, as_, bq, bs)]


def _noalloc(lib, d, c, m, n, k, kernel, splits):
    code = binding.MXFP4_OUT_F32 if c.dtype == torch.float32 else binding.MXFP4_OUT_BF16
    p = [ctypes.c_void_p(t.data_ptr()) for t in (*d, c)]
    return lib.mxfp4_gemm_nt_ex_noalloc(*p, code, m, n, k, kernel, splits,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _with_workspace(lib, d, c, m, n, k, kernel, splits):
    need = lib.mxfp4_gemm_nt_ex_workspace_size(m, n, k, kernel, splits)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=c.device)
    code = binding.MXFP4_OUT_F32 if c.dtype == torch.float32 else binding.MXFP4_OUT_BF16
    p = [ctypes.c_void_p(t.data_ptr()) for t in (*d, c)]
    st = lib.mxfp4_gemm_nt_ex(*p, code, m, n, k, kernel, splits, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, ws


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    dev = device()
    lib = binding.load_library()
    # first call larger than the second: 4 and 3 K splits, one k % 512 != 0
    for m, n, k, splits in ((100, 640, 4096, 4), (40, 200, 1056, 3)):
        log(f"no-alloc split-K m={m} n={n} k={k} splits={splits}")
        need = lib.mxfp4_gemm_nt_ex_workspace_size(m, n, k, SPLITK, splits)
        assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
        host, d = _operands(m, n, k, m + n + k, dev)
        for dtype in (torch.float32, torch.bfloat16):
            c_all = poisoned((m + 1, n), dtype, dev, 0xFF)
            assert _noalloc(lib, d, c_all[:m], m, n, k, SPLITK, splits) == 0, lib.mxfp4_last_error()
            ref = torch.empty((m, n), dtype=dtype, device=dev)
            st, ws = _with_workspace(lib, d, ref, m, n, k, SPLITK, splits)
            assert st == 0, lib.mxfp4_last_error()
            torch.cuda.synchronize()
            assert torch.all(c_all[m:].view(torch.uint8) == 0xFF), "write past the end of C"
            got = c_all[:m]
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"{dtype} differs from mxfp4_gemm_nt_ex"
            if dtype == torch.float32:
                c64 = oracle.gemm_nt(*host)
                assert oracle.floored_max_rel(to_np(got).astype(np.float64), c64) <= 1e-5
            # the caller's workspace is left zero-filled (its arrival counters reset)
            assert int(ws[:65536].count_nonzero()) == 0


def test_noalloc_tile_kernel_and_refusals():
    dev = device()
    lib = binding.load_library()
    m, n, k = 300, 260, 512
    host, d = _operands(m, n, k, 9, dev)
    c = torch.empty((m, n), dtype=torch.float32, device=dev)
    assert _noalloc(lib, d, c, m, n, k, binding.KERNELS["auto"], 0) == 0, lib.mxfp4_last_error()
    ref = torch.empty((m, n), dtype=torch.float32, device=dev)
    st, _ = _with_workspace(lib, d, ref, m, n, k, binding.KERNELS["auto"], 0)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(c, ref)
    # a workspace larger than the scratch array: refused, nothing launched
    m2, n2, k2, splits = 128, 14336, 1024, 3
    assert lib.mxfp4_gemm_nt_ex_workspace_size(m2, n2, k2, SPLITK, splits) > binding.NOALLOC_SCRATCH_BYTES
    _, d2 = _operands(m2, n2, k2, 11, dev)
    c2 = poisoned((m2, n2), torch.float32, dev, 0xFF)
    assert _noalloc(lib, d2, c2, m2, n2, k2, SPLITK, splits) == 3        # MXFP4_ERR_WORKSPACE
    assert b"scratch" in lib.mxfp4_last_error()
    torch.cuda.synchronize()
    assert torch.all(c2.view(torch.uint8) == 0xFF)
