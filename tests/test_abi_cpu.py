"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the headers in include/ declare, and rejects bad arguments on the
host before any device call (argument validation runs before the device query)."""
import ctypes
import glob
import os
import re

import pytest

from block_scaled_fp4_mxfp4_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
        names.update(re.findall(r"\b((?:mxfp[48]|nvfp4)_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmxfp4.so is not built (build it with: python -m block_scaled_fp4_mxfp4_amd.build)")
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(binding.EXPORTED) == names


def test_abi_version_and_status_strings(lib):
    assert lib.mxfp4_abi_version() == 1
    assert lib.mxfp4_status_string(0) == b"ok"
    assert lib.mxfp4_status_string(1) == b"invalid argument"
    assert lib.mxfp4_status_string(3) == b"workspace too small"
    assert lib.mxfp4_status_string(99) == b"unknown status"


def _fake(addr=0x1000):
    return ctypes.c_void_p(addr)


def test_quantize_rejects_bad_arguments_on_host(lib):
    # k not a multiple of 32, k <= 0, negative rows, null and misaligned pointers
    assert lib.mxfp4_quantize(_fake(), 4, 48, _fake(), _fake(), None) == 1
    assert lib.mxfp4_quantize(_fake(), 4, 0, _fake(), _fake(), None) == 1
    assert lib.mxfp4_quantize(_fake(), -1, 64, _fake(), _fake(), None) == 1
    assert lib.mxfp4_quantize(None, 4, 64, _fake(), _fake(), None) == 1
    assert b"x_bf16 is NULL" in lib.mxfp4_last_error()
    assert lib.mxfp4_quantize(_fake(0x1008), 4, 64, _fake(), _fake(), None) == 1
    assert b"16-byte aligned" in lib.mxfp4_last_error()
    assert lib.mxfp4_quantize(_fake(), 4, 64, _fake(0x1002), _fake(), None) == 1
    assert b"q is not 4-byte aligned" in lib.mxfp4_last_error()
    # zero rows: valid no-op, returns before touching the device
    assert lib.mxfp4_quantize(None, 0, 64, None, None, None) == 0


def test_mxfp8_quantize_rejects_bad_arguments_on_host(lib):
    assert lib.mxfp8_quantize(_fake(), 4, 48, _fake(), _fake(), None) == 1
    assert lib.mxfp8_quantize(_fake(), -1, 64, _fake(), _fake(), None) == 1
    assert lib.mxfp8_quantize(_fake(), 4, (1 << 24) + 32, _fake(), _fake(), None) == 1
    assert lib.mxfp8_quantize(None, 4, 64, _fake(), _fake(), None) == 1
    assert b"x_bf16 is NULL" in lib.mxfp4_last_error()
    assert lib.mxfp8_quantize(_fake(0x1008), 4, 64, _fake(), _fake(), None) == 1
    assert lib.mxfp8_quantize(_fake(), 4, 64, _fake(0x1004), _fake(), None) == 1
    assert b"q8 is not 8-byte aligned" in lib.mxfp4_last_error()
    assert lib.mxfp8_quantize(_fake(), 4, 64, _fake(), None, None) == 1
    assert lib.mxfp8_quantize(None, 0, 64, None, None, None) == 0


def test_gemm_rejects_bad_arguments_on_host(lib):
    f = _fake()
    args = dict(a_q=f, a_s=f, b_q=f, b_s=f, c=f)

    def call(m=64, n=64, k=128, c_type=0, kernel=0, splits=0, **kw):
        a = dict(args, **kw)
        return lib.mxfp4_gemm_nt_ex(a["a_q"], a["a_s"], a["b_q"], a["b_s"], a["c"], c_type, m, n, k,
                                    kernel, splits, None, 0, None)

    assert call(k=100) == 1
    assert call(k=-32) == 1
    assert call(m=-1) == 1
    assert call(c_type=7) == 1
    assert call(kernel=9) == 1
    assert call(kernel=6) == 1
    assert b"unknown kernel id 6" in lib.mxfp4_last_error()
    # forced kernels' requirements are checked before any device call: the stream
    # kernel needs k % 512 == 0, the persistent one k % 1024 == 0
    assert call(kernel=4, k=1056) == 1
    assert b"stream kernel needs" in lib.mxfp4_last_error()
    assert call(kernel=5, k=1536) == 1
    assert b"persistent kernel needs" in lib.mxfp4_last_error()
    assert call(b_s=None) == 1
    assert b"b_s is NULL" in lib.mxfp4_last_error()
    assert call(c=_fake(0x1004)) == 1
    assert call(a_s=_fake(0x1002)) == 1
    assert b"a_s is not 4-byte aligned" in lib.mxfp4_last_error()
    assert call(a_q=_fake(0x1008)) == 1
    # size limits: k at most 2^24, m and n at most 2^30
    assert call(k=(1 << 24) + 32) == 1
    assert b"k too large" in lib.mxfp4_last_error()
    assert call(m=(1 << 30) + 1) == 1
    assert call(n=(1 << 30) + 1) == 1
    assert lib.mxfp4_gemm_nt_workspace_size(64, 64, (1 << 24) + 32) == 0
    # empty problems are no-ops that launch nothing
    assert call(m=0, a_q=None, a_s=None, c=None) == 0
    assert call(n=0, b_q=None, b_s=None, c=None) == 0


def test_w4a8_rejects_bad_arguments_on_host(lib):
    f = _fake()
    assert lib.mxfp8_gemm_w4a8_nt(f, f, f, f, f, 0, 64, 64, 100, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(f, f, f, f, f, 5, 64, 64, 128, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(f, f, f, f, f, 0, -1, 64, 128, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(None, f, f, f, f, 0, 64, 64, 128, None) == 1
    assert b"a_q is NULL" in lib.mxfp4_last_error()
    assert lib.mxfp8_gemm_w4a8_nt(_fake(0x1008), f, f, f, f, 0, 64, 64, 128, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(f, _fake(0x1002), f, f, f, 0, 64, 64, 128, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(f, f, f, f, f, 0, 64, 64, (1 << 24) + 32, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt(None, None, f, f, None, 0, 0, 64, 128, None) == 0
    # forced kernels: only auto (0), tile128 (2) and stream (4); stream needs k % 512 == 0
    assert lib.mxfp8_gemm_w4a8_nt_ex(f, f, f, f, f, 0, 64, 64, 512, 1, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt_ex(f, f, f, f, f, 0, 64, 64, 512, 3, None) == 1
    assert lib.mxfp8_gemm_w4a8_nt_ex(f, f, f, f, f, 0, 64, 64, 256, 4, None) == 1
    assert b"stream kernel needs" in lib.mxfp4_last_error()
    assert lib.mxfp8_gemm_w4a8_nt_ex(None, None, f, f, None, 0, 0, 64, 512, 4, None) == 0
    assert lib.mxfp8_grouped_gemm_w4a8_nt(f, f, f, f, f, 0, 64, f, 0, 64, 128, None) == 1
    assert lib.mxfp8_grouped_gemm_w4a8_nt(f, f, f, f, None, 4, 64, f, 0, 64, 128, None) == 1
    assert lib.mxfp8_grouped_gemm_w4a8_nt(f, f, f, f, f, 4, 64, f, 0, 64, 100, None) == 1
    assert lib.mxfp8_grouped_gemm_w4a8_nt(None, None, f, f, None, 4, 0, None, 0, 64, 128, None) == 0


def test_grouped_rejects_bad_arguments_on_host(lib):
    f = _fake()
    assert lib.mxfp4_grouped_gemm_nt(f, f, f, f, f, 0, 64, f, 0, 64, 128, None, 0, None) == 1
    assert lib.mxfp4_grouped_gemm_nt(f, f, f, f, f, 2000, 64, f, 0, 64, 128, None, 0, None) == 1
    assert lib.mxfp4_grouped_gemm_nt(f, f, f, f, f, 4, 64, f, 0, 64, 100, None, 0, None) == 1
    assert lib.mxfp4_grouped_gemm_nt(f, f, f, f, None, 4, 64, f, 0, 64, 128, None, 0, None) == 1
    assert lib.mxfp4_grouped_gemm_nt(None, None, f, f, None, 4, 0, None, 0, 64, 128, None, 0, None) == 0


def test_interleaved_entry_points_reject_bad_arguments_on_host(lib):
    f = _fake
    # interleaving: k a positive multiple of 512, 16-byte aligned arrays
    assert lib.mxfp4_scales_interleave(f(), 1, 64, 256, f(), None) == 1
    assert b"k % 512" in lib.mxfp4_last_error()
    assert lib.mxfp4_scales_interleave(f(), -1, 64, 512, f(), None) == 1
    assert lib.mxfp4_scales_interleave(f(0x1004), 1, 64, 512, f(), None) == 1
    assert lib.mxfp4_scales_interleave(f(), 1, 64, 512, None, None) == 1
    assert lib.mxfp4_scales_interleave(None, 0, 64, 512, None, None) == 0        # no groups: no-op
    # quantizer: k % 512, rows * k / 32 < 2^31
    assert lib.mxfp4_quantize_interleaved(f(), 4, 1024 + 32, f(), f(), None) == 1
    assert lib.mxfp4_quantize_interleaved(f(), 1 << 27, 512, f(), f(), None) == 1
    assert lib.mxfp4_quantize_interleaved(None, 0, 512, None, None, None) == 0   # no rows: no-op
    # dense GEMM: k % 512, 16-byte aligned scale arrays, rows * k / 32 < 2^31 per operand
    assert lib.mxfp4_gemm_nt_interleaved(f(), f(), f(), f(), f(), 0, 64, 64, 256, None) == 1
    assert lib.mxfp4_gemm_nt_interleaved(f(), f(0x1004), f(), f(), f(), 0, 64, 64, 512, None) == 1
    assert lib.mxfp4_gemm_nt_interleaved(f(), f(), f(), f(0x1004), f(), 0, 64, 64, 512, None) == 1
    assert lib.mxfp4_gemm_nt_interleaved(f(), f(), f(), f(), f(), 0, 1 << 27, 64, 512, None) == 1
    assert lib.mxfp4_gemm_nt_interleaved(f(), f(), f(), f(), f(), 7, 64, 64, 512, None) == 1
    assert lib.mxfp4_gemm_nt_interleaved(None, None, f(), f(), None, 0, 0, 64, 512, None) == 0   # m == 0: no-op
    # grouped GEMM: the same plus the group count and the offsets pointer
    assert lib.mxfp4_grouped_gemm_nt_interleaved(f(), f(), f(), f(), f(), 4, 64, f(), 0, 64, 1536 + 32, None) == 1
    assert lib.mxfp4_grouped_gemm_nt_interleaved(f(), f(), f(), f(), f(), 0, 64, f(), 0, 64, 512, None) == 1
    assert lib.mxfp4_grouped_gemm_nt_interleaved(f(), f(), f(), f(), None, 4, 64, f(), 0, 64, 512, None) == 1
    assert lib.mxfp4_grouped_gemm_nt_interleaved(f(), f(0x1008), f(), f(), f(), 4, 64, f(), 0, 64, 512, None) == 1
    assert lib.mxfp4_grouped_gemm_nt_interleaved(None, None, f(), f(), None, 4, 0, None, 0, 64, 512, None) == 0
    # scatter-quantize: k % 512, total_rows * k / 32 < 2^31
    assert lib.mxfp4_moe_quantize_scatter_interleaved(f(), 4, 256, 2, f(), 8, f(), f(), None) == 1
    assert lib.mxfp4_moe_quantize_scatter_interleaved(f(), 4, 512, 2, f(), (1 << 27), f(), f(), None) == 1
    assert lib.mxfp4_moe_quantize_scatter_interleaved(None, 0, 512, 2, None, 8, None, None, None) == 0
    # the MXFP8 / W4A8 counterparts: the same k % 512 and size rules
    assert lib.mxfp8_quantize_interleaved(f(), 4, 1024 + 32, f(), f(), None) == 1
    assert lib.mxfp8_quantize_interleaved(None, 0, 512, None, None, None) == 0
    for g in (lib.mxfp8_gemm_w4a8_nt_interleaved, lib.mxfp8_gemm_nt_interleaved):
        assert g(f(), f(), f(), f(), f(), 0, 64, 64, 256, None) == 1
        assert g(f(), f(0x1004), f(), f(), f(), 0, 64, 64, 512, None) == 1
        assert g(f(), f(), f(), f(), f(), 0, 1 << 27, 64, 512, None) == 1
        assert g(None, None, f(), f(), None, 0, 0, 64, 512, None) == 0
    assert lib.mxfp8_gemm_nt_interleaved(f(), f(), f(), f(), f(), 0, 64, 64, 1 << 24, None) == 1   # k > 2^23
    gw = lib.mxfp8_grouped_gemm_w4a8_nt_interleaved
    assert gw(f(), f(), f(), f(), f(), 4, 64, f(), 0, 64, 1536 + 32, None) == 1
    assert gw(f(), f(), f(), f(), None, 4, 64, f(), 0, 64, 512, None) == 1
    assert gw(None, None, f(), f(), None, 4, 0, None, 0, 64, 512, None) == 0
    assert lib.mxfp8_moe_quantize_scatter_interleaved(f(), 4, 256, 2, f(), 8, f(), f(), None) == 1
    assert lib.mxfp8_moe_quantize_scatter_interleaved(None, 0, 512, 2, None, 8, None, None, None) == 0


def test_workspace_queries(lib):
    assert lib.mxfp4_grouped_gemm_nt_workspace_size(100, 4, 64, 128) == 0
    # tile kernels need no workspace; split-K with one split needs none either
    assert lib.mxfp4_gemm_nt_ex_workspace_size(512, 512, 256, 1, 0) == 0
    assert lib.mxfp4_gemm_nt_ex_workspace_size(64, 512, 256, 3, 1) == 0
    # split-K with 4 splits: the fixed 64 KiB counter region + 4 fp32 partials of every
    # 32-column tile (the narrower tiling needs the most room)
    expect = 65536 + 4 * (512 // 32) * (64 * 32) * 4
    assert lib.mxfp4_gemm_nt_ex_workspace_size(64, 512, 1024, 3, 4) == expect
    # invalid shapes report 0
    assert lib.mxfp4_gemm_nt_ex_workspace_size(64, 512, 100, 3, 4) == 0
    assert lib.mxfp4_gemm_nt_ex_workspace_size(500, 512, 1024, 3, 4) == 0


def test_probes_reject_bad_arguments_on_host(lib):
    f = _fake()
    assert lib.mxfp4_probe_mfma(f, f, 0, 16, None) == 1
    assert lib.mxfp4_probe_mfma(f, f, 65537, 16, None) == 1
    assert lib.mxfp4_probe_mfma(f, f, 4, 0, None) == 1
    assert lib.mxfp4_probe_mfma(f, f, 4, (1 << 24) + 1, None) == 1
    assert lib.mxfp4_probe_mfma(None, f, 4, 16, None) == 1
    assert b"seed is NULL" in lib.mxfp4_last_error()
    assert lib.mxfp4_probe_mfma(f, _fake(0x1004), 4, 16, None) == 1
    assert lib.mxfp4_probe_read(f, 0, f, 4, None) == 1
    assert lib.mxfp4_probe_read(f, 24, f, 4, None) == 1
    assert lib.mxfp4_probe_read(f, (1 << 40) + 16, f, 4, None) == 1
    assert lib.mxfp4_probe_read(f, 4096, f, 0, None) == 1
    assert lib.mxfp4_probe_read(_fake(0x1008), 4096, f, 4, None) == 1
    assert lib.mxfp4_probe_read(f, 4096, _fake(0x1002), 4, None) == 1
    # 8 waves x iters x 8 MFMAs of 2*32*32*64 flops per workgroup
    assert lib.mxfp4_probe_mfma_flops(3, 5) == 3 * 8 * 5 * 8 * 131072
    assert lib.mxfp4_probe_mfma_flops(0, 5) == 0.0


def test_moe_entry_points_reject_bad_arguments_on_host(lib):
    f = _fake
    # routing: experts 1..256, top_k 1..min(8, experts), tokens 0..2^28
    assert lib.mxfp4_moe_route(f(), 4, 0, 1, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(f(), 4, 257, 1, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(f(), 4, 64, 9, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(f(), 4, 2, 3, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(f(), -1, 64, 4, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(f(), (1 << 28) + 1, 64, 4, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(None, 4, 64, 4, f(), f(), None) == 1
    assert b"logits is NULL" in lib.mxfp4_last_error()
    assert lib.mxfp4_moe_route(f(0x1002), 4, 64, 4, f(), f(), None) == 1
    assert lib.mxfp4_moe_route(None, 0, 64, 4, None, None, None) == 0          # no tokens: no-op
    # permutation: experts 1..1024, top_k 1..256, tokens * top_k <= 2^30
    assert lib.mxfp4_moe_permute(f(), 4, 0, 2, f(), f(), f(), None) == 1
    assert lib.mxfp4_moe_permute(f(), 4, 1025, 2, f(), f(), f(), None) == 1
    assert lib.mxfp4_moe_permute(f(), 4, 8, 0, f(), f(), f(), None) == 1
    assert lib.mxfp4_moe_permute(f(), 1 << 29, 8, 4, f(), f(), f(), None) == 1
    assert lib.mxfp4_moe_permute(f(), 4, 8, 2, None, f(), f(), None) == 1
    assert lib.mxfp4_moe_permute(f(), 4, 8, 2, f(), None, f(), None) == 1
    # scatter-quantize: k a positive multiple of 32, top_k 1..256, alignment of x and q
    for fn in (lib.mxfp4_moe_quantize_scatter, lib.mxfp8_moe_quantize_scatter):
        assert fn(f(), 4, 48, 2, f(), 8, f(), f(), None) == 1
        assert fn(f(), 4, 64, 0, f(), 8, f(), f(), None) == 1
        assert fn(f(), -1, 64, 2, f(), 8, f(), f(), None) == 1
        assert fn(f(), 4, 64, 2, f(), 1 << 31, f(), f(), None) == 1
        assert fn(f(0x1008), 4, 64, 2, f(), 8, f(), f(), None) == 1
        assert fn(None, 0, 64, 2, None, 8, None, None, None) == 0              # no tokens: no-op
        assert fn(None, 4, 64, 2, None, 0, None, None, None) == 0              # no rows: no-op
    assert lib.mxfp4_moe_quantize_scatter(f(), 4, 64, 2, f(), 8, f(0x1002), f(), None) == 1
    assert lib.mxfp8_moe_quantize_scatter(f(), 4, 64, 2, f(), 8, f(0x1004), f(), None) == 1
    # combine: output type, sizes, alignment
    assert lib.mxfp4_moe_combine(f(), 8, 64, f(), f(), 4, 2, f(), 7, None) == 1
    assert lib.mxfp4_moe_combine(f(), 8, -1, f(), f(), 4, 2, f(), 0, None) == 1
    assert lib.mxfp4_moe_combine(f(), 8, 64, f(), f(), 4, 0, f(), 0, None) == 1
    assert lib.mxfp4_moe_combine(f(0x1001), 8, 64, f(), f(), 4, 2, f(), 0, None) == 1
    assert lib.mxfp4_moe_combine(f(), 8, 64, f(), f(), 4, 2, f(0x1002), 1, None) == 1
    assert lib.mxfp4_moe_combine(None, 8, 64, None, None, 0, 2, None, 0, None) == 0   # no tokens: no-op


def test_moe_scatter_block_limit(lib):
    # tokens * k / 32 <= 2^30 (32-bit block indices with room for the unrolled grid stride)
    assert lib.mxfp4_moe_quantize_scatter(_fake(), (1 << 30) // 2 + 1, 64, 1, _fake(), 8, _fake(), _fake(), None) == 1
    assert b"too large" in lib.mxfp4_last_error()


def test_producers_reject_bad_arguments_on_host(lib):
    f = _fake
    rms = lib.mxfp4_rmsnorm_quantize
    assert rms(f(), None, f(), 1e-5, 4, 48, None, None, f(), f(), None) == 1           # k % 32
    assert rms(f(), None, f(), 1e-5, 4, 32768 + 32, None, None, f(), f(), None) == 1   # k too large
    assert rms(f(), None, f(), -1.0, 4, 64, None, None, f(), f(), None) == 1           # eps < 0
    assert rms(f(), None, f(), float("nan"), 4, 64, None, None, f(), f(), None) == 1
    assert rms(f(), None, f(), float("inf"), 4, 64, None, None, f(), f(), None) == 1
    assert rms(f(), None, f(), 1e-5, -1, 64, None, None, f(), f(), None) == 1
    assert rms(None, None, f(), 1e-5, 4, 64, None, None, f(), f(), None) == 1
    assert rms(f(), None, None, 1e-5, 4, 64, None, None, f(), f(), None) == 1
    assert rms(f(), None, f(), 1e-5, 4, 64, f(), None, f(), f(), None) == 1            # residual_out without residual
    assert b"needs residual" in lib.mxfp4_last_error()
    assert rms(f(), f(0x1008), f(), 1e-5, 4, 64, None, None, f(), f(), None) == 1      # misaligned residual
    assert rms(f(), None, f(), 1e-5, 4, 64, None, None, f(0x1002), f(), None) == 1     # misaligned q
    assert rms(None, None, None, 1e-5, 0, 64, None, None, None, None, None) == 0       # no rows: no-op
    sw = lib.mxfp4_swiglu_quantize
    assert sw(f(), f(), 64, 4, 48, None, f(), f(), None) == 1                           # k % 32
    assert sw(f(), f(), 60, 4, 64, None, f(), f(), None) == 1                           # ld < k
    assert sw(f(), f(), 68, 4, 64, None, f(), f(), None) == 1                           # ld % 8
    assert sw(f(), f(0x1008), 64, 4, 64, None, f(), f(), None) == 1                     # misaligned up
    assert sw(f(), f(), 64, (1 << 30) // 2 + 1, 64, None, f(), f(), None) == 1          # rows * k / 32
    assert sw(None, None, 64, 0, 64, None, None, None, None) == 0                       # no rows: no-op


def test_nvfp4_entry_points_reject_bad_arguments_on_host(lib):
    f = _fake
    assert lib.nvfp4_quantize(f(), 4, 48, f(), f(), f(), None) == 1                # k % 32
    assert lib.nvfp4_quantize(f(), 4, 32768 + 32, f(), f(), f(), None) == 1        # k too large
    assert lib.nvfp4_quantize(f(), -1, 64, f(), f(), f(), None) == 1
    assert lib.nvfp4_quantize(f(), 4, 64, f(), f(), None, None) == 1               # null global scales
    assert lib.nvfp4_quantize(f(), 4, 64, f(), f(), f(0x1002), None) == 1          # misaligned global scales
    assert lib.nvfp4_quantize(None, 0, 64, None, None, None, None) == 0            # no rows: no-op
    g = lib.nvfp4_gemm_nt
    assert g(f(), f(), f(), f(), f(), f(), f(), 0, 4, 4, 96, None) == 1             # k % 64
    assert b"multiple of 64" in lib.mxfp4_last_error()
    assert g(f(), f(), f(), f(), f(), f(), f(), 5, 4, 4, 64, None) == 1             # output type
    assert g(f(), f(0x1002), f(), f(), f(), f(), f(), 0, 4, 4, 64, None) == 1       # misaligned a_s
    assert g(f(), f(), f(), f(), f(), None, f(), 0, 4, 4, 64, None) == 1            # null b_gs
    assert g(None, None, None, None, None, None, None, 0, 0, 4, 64, None) == 0      # m == 0: no-op


def test_row_per_workgroup_kernels_cap_rows(lib):
    # RMSNorm producer and NVFP4 quantizer run one 256-thread workgroup per row
    f = _fake
    assert lib.mxfp4_rmsnorm_quantize(f(), None, f(), 1e-5, (1 << 24) + 1, 64, None, None, f(), f(), None) == 1
    assert lib.nvfp4_quantize(f(), (1 << 24) + 1, 64, f(), f(), f(), None) == 1
    assert b"2^24" in lib.mxfp4_last_error()


def test_prepacked_split_k_arguments_on_host(lib):
    f = _fake
    ex = lib.mxfp4_gemm_nt_prepacked_ab_ex
    assert ex(f(), f(), f(), f(), f(), 0, 128, 4096, 1000, 0, None, 0, None) == 1      # k % 512
    assert ex(f(), f(), f(), f(), f(), 0, 128, 4096, 14336, 17, None, 0, None) == 1    # splits 0..16
    assert b"splits must be 0..16" in lib.mxfp4_last_error()
    assert ex(f(), f(), f(), f(), f(), 0, 128, 4096, 14336, -1, None, 0, None) == 1
    assert ex(None, None, f(), f(), None, 0, 0, 4096, 14336, 4, None, 0, None) == 0    # empty: no-op
    size = lib.mxfp4_gemm_nt_prepacked_ab_workspace_size
    # 64 panels x 4 ranges of 7 pairs: the 64 KiB counter region + 4 fp32 128 x 64 tiles per panel
    assert size(128, 4096, 14336, 4) == 65536 + 64 * 4 * 128 * 64 * 4
    assert size(128, 4096, 14336, 1) == 0
    # 2048 = 4 pairs: 3 ranges asked give ranges of 2 pairs, so two
    assert size(64, 640, 2048, 3) == 65536 + 10 * 2 * 64 * 64 * 4
    # automatic with no device: 256 compute units assumed; 224 panels need no split
    assert size(128, 14336, 4096, 0) == 0
    assert size(128, 4096, 14336, 0) == 65536 + 64 * 4 * 128 * 64 * 4
    assert size(128, 4096, 14336, 17) == 0 and size(128, 4096, 1000, 4) == 0
    # split-K needs at most 16384 output tiles (one arrival counter each in the 64 KiB region)
    assert size(128, 64 * 16384, 4096, 4) == 65536 + 16384 * 4 * 128 * 64 * 4
    assert size(128, 64 * 16385, 4096, 4) == 0
    assert ex(f(), f(), f(), f(), f(), 0, 128, 64 * 16385, 4096, 4, None, 0, None) == 1
    assert b"at most 16384 output tiles" in lib.mxfp4_last_error()


def test_w4a8_prepacked_rejects_bad_arguments_on_host(lib):
    f = _fake
    g = lib.mxfp8_gemm_w4a8_nt_prepacked
    assert g(f(), f(), f(), f(), f(), 0, 4, 64, 992, None) == 1           # k % 512
    assert b"multiple of 512" in lib.mxfp4_last_error()
    assert g(f(), f(), f(), f(), f(), 3, 4, 64, 512, None) == 1           # output type
    assert g(f(), f(), None, f(), f(), 0, 4, 64, 512, None) == 1          # null bp_q
    assert g(f(), f(), f(), f(), f(), 0, -1, 64, 512, None) == 1
    assert g(None, None, f(), f(), None, 0, 0, 64, 512, None) == 0        # empty: no-op


def test_interleaved_producers_reject_bad_arguments_on_host(lib):
    f = _fake
    r = lib.mxfp4_rmsnorm_quantize_interleaved
    assert r(f(), None, f(), 1e-5, 4, 1024 + 32, None, None, f(), f(), None) == 1   # k % 512
    assert b"multiple of 512" in lib.mxfp4_last_error()
    assert r(f(), None, f(), -1.0, 4, 512, None, None, f(), f(), None) == 1          # eps
    assert r(None, None, None, 1e-5, 0, 512, None, None, None, None, None) == 0      # no rows: no-op
    w = lib.mxfp4_swiglu_quantize_interleaved
    assert w(f(), f(), 1024 + 32, 4, 1024 + 32, None, f(), f(), None) == 1           # k % 512
    assert w(f(), f(), 500, 4, 512, None, f(), f(), None) == 1                       # ld < k
    assert w(None, None, 512, 0, 512, None, None, None, None) == 0                   # no rows: no-op


def test_w4a8_both_prepacked_rejects_bad_arguments_on_host(lib):
    f = _fake
    q = lib.mxfp8_quantize_prepacked
    assert q(f(), 4, 992, f(), f(), None) == 1                           # k % 512
    assert q(f(), -1, 512, f(), f(), None) == 1
    assert q(f(0x1004), 4, 512, f(), f(), None) == 1                     # x alignment
    assert q(None, 0, 512, None, None, None) == 0                        # no rows: no-op
    g = lib.mxfp8_gemm_w4a8_nt_prepacked_ab
    assert g(f(), f(), f(), f(), f(), 0, 4, 64, 992, None) == 1          # k % 512
    assert b"multiple of 512" in lib.mxfp4_last_error()
    assert g(f(), f(), f(), f(), f(), 3, 4, 64, 512, None) == 1          # output type
    assert g(None, f(), f(), f(), f(), 0, 4, 64, 512, None) == 1         # null ap_q8
    assert g(f(), f(), f(), f(), f(), 0, -1, 64, 512, None) == 1
    assert g(None, None, f(), f(), None, 0, 0, 64, 512, None) == 0       # empty: no-op


def test_prepacked_entry_points_reject_bad_arguments_on_host(lib):
    f = _fake
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    size = lib.mxfp4_prepacked_weight_size
    assert size(100, 1024, ctypes.byref(cb), ctypes.byref(sb)) == 0
    assert (cb.value, sb.value) == (128 * 512, 128 * 32)                       # rows padded to 64
    assert size(64, 992, ctypes.byref(cb), ctypes.byref(sb)) == 1               # k % 512
    assert b"multiple of 512" in lib.mxfp4_last_error()
    assert size(-1, 512, ctypes.byref(cb), ctypes.byref(sb)) == 1
    assert size(64, 512, None, ctypes.byref(sb)) == 1
    assert lib.mxfp4_prepack_weight(f(), f(), 64, 544, f(), f(), None) == 1     # k % 512
    assert lib.mxfp4_prepack_weight(f(), f(), 64, 512, f(0x1004), f(), None) == 1   # misaligned bp_q
    assert lib.mxfp4_prepack_weight(None, None, 0, 512, None, None, None) == 0  # no rows: no-op
    assert lib.mxfp4_quantize_prepacked(f(), 4, 1024 + 32, f(), f(), None) == 1
    assert lib.mxfp4_quantize_prepacked(f(0x1008), 4, 1024, f(), f(), None) == 1     # misaligned x
    assert lib.mxfp4_quantize_prepacked(None, 0, 1024, None, None, None) == 0
    for g in (lib.mxfp4_gemm_nt_prepacked,):
        assert g(f(), f(), f(), f(), f(), 0, 4, 64, 1000, None) == 1           # k % 512
        assert g(f(), f(), f(), f(), f(), 3, 4, 64, 512, None) == 1            # output type
        assert g(f(), f(), None, f(), f(), 0, 4, 64, 512, None) == 1           # null bp_q
        assert g(f(), f(0x1004), f(), f(), f(), 0, 4, 64, 512, None) == 1      # misaligned a_s
        assert g(None, None, f(), f(), None, 0, 0, 64, 512, None) == 0         # m == 0: no-op
    g = lib.mxfp4_gemm_nt_prepacked_ab
    assert g(f(), f(), f(), f(), f(), 0, 4, 64, 1000, None) == 1
    assert g(f(), None, f(), f(), f(), 0, 4, 64, 512, None) == 1               # null ap_s
    assert g(f(), f(), f(), f(), f(), 0, (1 << 30) + 1, 64, 512, None) == 1    # m too large
    assert g(None, None, None, None, None, 0, 4, 0, 512, None) == 0            # n == 0: no-op
