"""ctypes binding of libmxfp4.so (the C ABI in include/mxfp4.h, include/mxfp8.h, include/mxfp4_moe.h,
include/mxfp4_producers.h and include/nvfp4.h).

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
functions carry the C entry points' names.  If the library is missing or the
current device is not gfx950 these calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmxfp4.so")

MXFP4_OK = 0
MXFP4_OUT_BF16 = 0
MXFP4_OUT_F32 = 1
KERNELS = {"auto": 0, "tile256": 1, "tile128": 2, "splitk": 3, "stream": 4, "persistent": 5}

EXPORTED = (
    "mxfp4_abi_version", "mxfp4_status_string", "mxfp4_last_error", "mxfp4_quantize",
    "mxfp4_gemm_nt_workspace_size", "mxfp4_gemm_nt", "mxfp4_grouped_gemm_nt_workspace_size",
    "mxfp4_grouped_gemm_nt", "mxfp4_gemm_nt_ex_workspace_size", "mxfp4_gemm_nt_ex",
    "mxfp4_probe_mfma", "mxfp4_probe_mfma_flops", "mxfp4_probe_read", "mxfp8_quantize",
    "mxfp8_gemm_w4a8_nt", "mxfp8_gemm_w4a8_nt_ex", "mxfp8_grouped_gemm_w4a8_nt", "mxfp4_probe_mfma_w4a8",
    "mxfp4_moe_route", "mxfp4_moe_permute", "mxfp4_moe_quantize_scatter", "mxfp8_moe_quantize_scatter",
    "mxfp4_moe_combine", "mxfp4_rmsnorm_quantize", "mxfp4_swiglu_quantize", "nvfp4_quantize", "nvfp4_gemm_nt",
    "mxfp4_prepacked_weight_size", "mxfp4_prepack_weight", "mxfp4_gemm_nt_prepacked", "mxfp4_gemm_nt_prepacked_ab",
    "mxfp4_gemm_nt_prepacked_ab_ex", "mxfp4_gemm_nt_prepacked_ab_workspace_size",
    "mxfp4_quantize_prepacked", "mxfp8_gemm_nt", "mxfp8_gemm_nt_ex", "mxfp4_gemm_nt_ex_noalloc",
    "mxfp4_rmsnorm_quantize_prepacked", "mxfp4_swiglu_quantize_prepacked", "mxfp8_gemm_w4a8_nt_prepacked",
    "mxfp4_scales_interleave", "mxfp4_quantize_interleaved", "mxfp4_gemm_nt_interleaved",
    "mxfp4_grouped_gemm_nt_interleaved", "mxfp4_moe_quantize_scatter_interleaved",
    "mxfp8_quantize_prepacked", "mxfp8_gemm_w4a8_nt_prepacked_ab", "mxfp4_rmsnorm_quantize_interleaved",
    "mxfp4_swiglu_quantize_interleaved", "mxfp8_quantize_interleaved", "mxfp8_gemm_w4a8_nt_interleaved",
    "mxfp8_grouped_gemm_w4a8_nt_interleaved", "mxfp8_gemm_nt_interleaved", "mxfp8_moe_quantize_scatter_interleaved",
)
NOALLOC_SCRATCH_BYTES = 16 << 20
PROBE_SEED_BYTES = 6144

_lib = None
_lock = threading.Lock()


class MXFP4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"mxfp4 status {status}: {detail}")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Loads libmxfp4.so and declares its signatures (raises if it is absent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; build it with: python -m block_scaled_fp4_mxfp4_amd.build")
        lib = ctypes.CDLL(path)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        lib.mxfp4_abi_version.restype = ctypes.c_int
        lib.mxfp4_abi_version.argtypes = []
        lib.mxfp4_status_string.restype = ctypes.c_char_p
        lib.mxfp4_status_string.argtypes = [ctypes.c_int]
        lib.mxfp4_last_error.restype = ctypes.c_char_p
        lib.mxfp4_last_error.argtypes = []
        lib.mxfp4_quantize.restype = ctypes.c_int
        lib.mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp8_quantize.restype = ctypes.c_int
        lib.mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp8_gemm_w4a8_nt.restype = ctypes.c_int
        lib.mxfp8_gemm_w4a8_nt.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp8_gemm_w4a8_nt_prepacked.restype = ctypes.c_int
        lib.mxfp8_gemm_w4a8_nt_prepacked.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp8_gemm_w4a8_nt_ex.restype = ctypes.c_int
        lib.mxfp8_gemm_w4a8_nt_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, vp]
        lib.mxfp8_gemm_nt.restype = ctypes.c_int
        lib.mxfp8_gemm_nt.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp8_gemm_nt_ex.restype = ctypes.c_int
        lib.mxfp8_gemm_nt_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, vp]
        lib.mxfp8_grouped_gemm_w4a8_nt.restype = ctypes.c_int
        lib.mxfp8_grouped_gemm_w4a8_nt.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, i64, i64, vp]
        lib.mxfp4_gemm_nt_workspace_size.restype = sz
        lib.mxfp4_gemm_nt_workspace_size.argtypes = [i64, i64, i64]
        lib.mxfp4_gemm_nt.restype = ctypes.c_int
        lib.mxfp4_gemm_nt.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp, sz, vp]
        lib.mxfp4_gemm_nt_ex_workspace_size.restype = sz
        lib.mxfp4_gemm_nt_ex_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int, i32]
        lib.mxfp4_gemm_nt_ex.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64,
                                         ctypes.c_int, i32, vp, sz, vp]
        lib.mxfp4_gemm_nt_ex_noalloc.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64,
                                                 ctypes.c_int, i32, vp]
        lib.mxfp4_prepacked_weight_size.restype = ctypes.c_int
        lib.mxfp4_prepacked_weight_size.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.mxfp4_prepack_weight.restype = ctypes.c_int
        lib.mxfp4_prepack_weight.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        lib.mxfp4_gemm_nt_prepacked.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_prepacked.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp4_quantize_prepacked.restype = ctypes.c_int
        lib.mxfp4_quantize_prepacked.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp4_gemm_nt_prepacked_ab.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_prepacked_ab.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp4_gemm_nt_prepacked_ab_ex.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_prepacked_ab_ex.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int32,
                                                      vp, ctypes.c_size_t, vp]
        lib.mxfp4_gemm_nt_prepacked_ab_workspace_size.restype = ctypes.c_size_t
        lib.mxfp4_gemm_nt_prepacked_ab_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int32]
        lib.mxfp4_grouped_gemm_nt_workspace_size.restype = sz
        lib.mxfp4_grouped_gemm_nt_workspace_size.argtypes = [i64, i32, i64, i64]
        lib.mxfp4_grouped_gemm_nt.restype = ctypes.c_int
        lib.mxfp4_grouped_gemm_nt.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, i64, i64,
                                              vp, sz, vp]
        lib.mxfp4_probe_mfma.restype = ctypes.c_int
        lib.mxfp4_probe_mfma.argtypes = [vp, vp, i32, i32, vp]
        lib.mxfp4_probe_mfma_w4a8.restype = ctypes.c_int
        lib.mxfp4_probe_mfma_w4a8.argtypes = [vp, vp, i32, i32, vp]
        lib.mxfp4_probe_mfma_flops.restype = ctypes.c_double
        lib.mxfp4_probe_mfma_flops.argtypes = [i32, i32]
        lib.mxfp4_probe_read.restype = ctypes.c_int
        lib.mxfp4_probe_read.argtypes = [vp, i64, vp, i32, vp]
        lib.mxfp4_moe_route.restype = ctypes.c_int
        lib.mxfp4_moe_route.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        lib.mxfp4_moe_permute.restype = ctypes.c_int
        lib.mxfp4_moe_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        lib.mxfp8_quantize_interleaved.restype = ctypes.c_int
        lib.mxfp8_quantize_interleaved.argtypes = [vp, i64, i64, vp, vp, vp]
        for name in ("mxfp8_gemm_w4a8_nt_interleaved", "mxfp8_gemm_nt_interleaved"):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp8_grouped_gemm_w4a8_nt_interleaved.restype = ctypes.c_int
        lib.mxfp8_grouped_gemm_w4a8_nt_interleaved.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, i64,
                                                               i64, vp]
        lib.mxfp8_quantize_prepacked.restype = ctypes.c_int
        lib.mxfp8_quantize_prepacked.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp8_gemm_w4a8_nt_prepacked_ab.restype = ctypes.c_int
        lib.mxfp8_gemm_w4a8_nt_prepacked_ab.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp4_scales_interleave.restype = ctypes.c_int
        lib.mxfp4_scales_interleave.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.mxfp4_quantize_interleaved.restype = ctypes.c_int
        lib.mxfp4_quantize_interleaved.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.mxfp4_gemm_nt_interleaved.restype = ctypes.c_int
        lib.mxfp4_gemm_nt_interleaved.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp4_grouped_gemm_nt_interleaved.restype = ctypes.c_int
        lib.mxfp4_grouped_gemm_nt_interleaved.argtypes = [vp, vp, vp, vp, vp, i32, i64, vp, ctypes.c_int, i64, i64, vp]
        for name in ("mxfp4_moe_quantize_scatter", "mxfp8_moe_quantize_scatter",
                     "mxfp4_moe_quantize_scatter_interleaved", "mxfp8_moe_quantize_scatter_interleaved"):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name).argtypes = [vp, i64, i64, i32, vp, i64, vp, vp, vp]
        lib.mxfp4_rmsnorm_quantize.restype = ctypes.c_int
        lib.mxfp4_rmsnorm_quantize.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, vp, vp, vp, vp, vp]
        lib.mxfp4_swiglu_quantize.restype = ctypes.c_int
        lib.mxfp4_swiglu_quantize.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp]
        lib.mxfp4_rmsnorm_quantize_prepacked.restype = ctypes.c_int
        lib.mxfp4_rmsnorm_quantize_prepacked.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, vp, vp, vp, vp, vp]
        lib.mxfp4_swiglu_quantize_prepacked.restype = ctypes.c_int
        lib.mxfp4_swiglu_quantize_prepacked.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp]
        lib.mxfp4_rmsnorm_quantize_interleaved.restype = ctypes.c_int
        lib.mxfp4_rmsnorm_quantize_interleaved.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, vp, vp, vp, vp, vp]
        lib.mxfp4_swiglu_quantize_interleaved.restype = ctypes.c_int
        lib.mxfp4_swiglu_quantize_interleaved.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp]
        lib.nvfp4_quantize.restype = ctypes.c_int
        lib.nvfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        lib.nvfp4_gemm_nt.restype = ctypes.c_int
        lib.nvfp4_gemm_nt.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.mxfp4_moe_combine.restype = ctypes.c_int
        lib.mxfp4_moe_combine.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp, ctypes.c_int, vp]
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != MXFP4_OK:
        lib = load_library()
        raise MXFP4Error(status, f"{lib.mxfp4_status_string(status).decode()}: "
                                 f"{lib.mxfp4_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t: torch.Tensor, name: str, dtype, shape):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")


_workspaces: dict = {}


def workspace(nbytes: int, device=None) -> torch.Tensor | None:
    """A zero-filled, reusable per-device workspace of at least `nbytes` bytes.

    The library leaves a workspace zero-filled after every call, so one
    buffer (grown on demand) serves every stream-ordered call on a device.
    """
    if nbytes == 0:
        return None
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index)
    ws = _workspaces.get(dev)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[dev] = ws
    return ws


def mxfp4_quantize(x: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   stream=None):
    """x: bf16 [rows, k] -> (q uint8 [rows, k/2], scales uint8 [rows, k/32])."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, k]")
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(q, "q", torch.uint8, (rows, k // 2))
    _require(scales, "scales", torch.uint8, (rows, k // 32))
    _check(lib.mxfp4_quantize(_ptr(x), rows, k, _ptr(q), _ptr(scales), _stream(stream)))
    return q, scales


def mxfp8_quantize(x: torch.Tensor, q8: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                   stream=None):
    """x: bf16 [rows, k] -> (q8 uint8 [rows, k] E4M3 codes, scales uint8 [rows, k/32])."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, k]")
    rows, k = x.shape
    if q8 is None:
        q8 = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(q8, "q8", torch.uint8, (rows, k))
    _require(scales, "scales", torch.uint8, (rows, k // 32))
    _check(lib.mxfp8_quantize(_ptr(x), rows, k, _ptr(q8), _ptr(scales), _stream(stream)))
    return q8, scales


def _out(c, m, n, out_dtype, device):
    if c is None:
        c = torch.empty((m, n), dtype=out_dtype, device=device)
    code = MXFP4_OUT_F32 if c.dtype == torch.float32 else MXFP4_OUT_BF16
    _require(c, "c", torch.float32 if code == MXFP4_OUT_F32 else torch.bfloat16, (m, n))
    return c, code


def mxfp4_gemm_nt(a_q, a_s, b_q, b_s, c=None, out_dtype=torch.bfloat16, kernel: str = "auto",
                  splits: int = 0, ws: torch.Tensor | None = None, stream=None):
    """C[m, n] = A[m, k] . B[n, k]^T on MXFP4 operands (bf16 or fp32 output)."""
    lib = load_library()
    m, kh = a_q.shape
    n = b_q.shape[0]
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (m, k // 2))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s, "b_s", torch.uint8, (n, k // 32))
    c, code = _out(c, m, n, out_dtype, a_q.device)
    kid = KERNELS[kernel]
    need = lib.mxfp4_gemm_nt_ex_workspace_size(m, n, k, kid, splits)
    if ws is None:
        ws = workspace(need, a_q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxfp4_gemm_nt_ex(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(c), code, m, n, k,
                                kid, splits, _ptr(ws), nbytes, _stream(stream)))
    return c


def mxfp4_gemm_nt_noalloc(a_q, a_s, b_q, b_s, c, kernel: str = "auto", splits: int = 0, stream=None):
    """mxfp4_gemm_nt through the no-allocation entry point: the caller passes C
    (bf16 or fp32); split-K scratch is the library's static device array."""
    lib = load_library()
    m, kh = a_q.shape
    n = b_q.shape[0]
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (m, k // 2))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s, "b_s", torch.uint8, (n, k // 32))
    c, code = _out(c, m, n, c.dtype, a_q.device)
    _check(lib.mxfp4_gemm_nt_ex_noalloc(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(c), code, m, n, k,
                                        KERNELS[kernel], splits, _stream(stream)))
    return c


def mxfp4_prepacked_weight_size(n: int, k: int) -> tuple[int, int]:
    """(code_bytes, scale_bytes) of a prepacked [n, k] MXFP4 weight (k % 512 == 0)."""
    lib = load_library()
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.mxfp4_prepacked_weight_size(n, k, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def mxfp4_prepack_weight(b_q, b_s, bp_q=None, bp_s=None, stream=None):
    """Rearranges an MXFP4 weight [n, k] into the prepacked layout; returns (bp_q, bp_s) as flat uint8."""
    lib = load_library()
    n, kh = b_q.shape
    k = kh * 2
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s, "b_s", torch.uint8, (n, k // 32))
    cb, sb = mxfp4_prepacked_weight_size(n, k)
    if bp_q is None:
        bp_q = torch.empty(cb, dtype=torch.uint8, device=b_q.device)
    if bp_s is None:
        bp_s = torch.empty(sb, dtype=torch.uint8, device=b_q.device)
    _require(bp_q, "bp_q", torch.uint8, (cb,))
    _require(bp_s, "bp_s", torch.uint8, (sb,))
    _check(lib.mxfp4_prepack_weight(_ptr(b_q), _ptr(b_s), n, k, _ptr(bp_q), _ptr(bp_s), _stream(stream)))
    return bp_q, bp_s


def mxfp4_gemm_nt_prepacked(a_q, a_s, bp_q, bp_s, n: int, c=None, out_dtype=torch.bfloat16, stream=None):
    """C[m, n] = A . B^T with B given in the prepacked layout (mxfp4_prepack_weight)."""
    lib = load_library()
    m, kh = a_q.shape
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (m, k // 2))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    cb, sb = mxfp4_prepacked_weight_size(n, k)
    _require(bp_q, "bp_q", torch.uint8, (cb,))
    _require(bp_s, "bp_s", torch.uint8, (sb,))
    c, code = _out(c, m, n, out_dtype, a_q.device)
    _check(lib.mxfp4_gemm_nt_prepacked(_ptr(a_q), _ptr(a_s), _ptr(bp_q), _ptr(bp_s), _ptr(c), code, m, n, k,
                                       _stream(stream)))
    return c


def mxfp4_quantize_prepacked(x, ap_q=None, ap_s=None, stream=None):
    """BF16 [rows, k] -> MXFP4 in the prepacked layout; returns (ap_q, ap_s) as flat uint8."""
    lib = load_library()
    rows, k = x.shape
    _require(x, "x", torch.bfloat16, (rows, k))
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    if ap_q is None:
        ap_q = torch.empty(cb, dtype=torch.uint8, device=x.device)
    if ap_s is None:
        ap_s = torch.empty(sb, dtype=torch.uint8, device=x.device)
    _require(ap_q, "ap_q", torch.uint8, (cb,))
    _require(ap_s, "ap_s", torch.uint8, (sb,))
    _check(lib.mxfp4_quantize_prepacked(_ptr(x), rows, k, _ptr(ap_q), _ptr(ap_s), _stream(stream)))
    return ap_q, ap_s


def mxfp8_quantize_prepacked(x, ap_q8=None, ap_s=None, stream=None):
    """BF16 [rows, k] -> MXFP8 in the FP8 prepacked layout (include/mxfp8.h); returns (ap_q8, ap_s) as flat
    uint8 (ap_q8 twice the MXFP4 prepacked code bytes, ap_s the same scale bytes)."""
    lib = load_library()
    rows, k = x.shape
    _require(x, "x", torch.bfloat16, (rows, k))
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    if ap_q8 is None:
        ap_q8 = torch.empty(2 * cb, dtype=torch.uint8, device=x.device)
    if ap_s is None:
        ap_s = torch.empty(sb, dtype=torch.uint8, device=x.device)
    _require(ap_q8, "ap_q8", torch.uint8, (2 * cb,))
    _require(ap_s, "ap_s", torch.uint8, (sb,))
    _check(lib.mxfp8_quantize_prepacked(_ptr(x), rows, k, _ptr(ap_q8), _ptr(ap_s), _stream(stream)))
    return ap_q8, ap_s


def mxfp8_gemm_w4a8_nt_prepacked_ab(ap_q8, ap_s, bp_q, bp_s, m: int, n: int, k: int, c=None,
                                    out_dtype=torch.bfloat16, stream=None):
    """W4A8 C[m, n] = A . B^T with A in the FP8 prepacked layout and B prepacked (mxfp4_prepack_weight)."""
    lib = load_library()
    cba, sba = mxfp4_prepacked_weight_size(m, k)
    cbb, sbb = mxfp4_prepacked_weight_size(n, k)
    _require(ap_q8, "ap_q8", torch.uint8, (2 * cba,))
    _require(ap_s, "ap_s", torch.uint8, (sba,))
    _require(bp_q, "bp_q", torch.uint8, (cbb,))
    _require(bp_s, "bp_s", torch.uint8, (sbb,))
    c, code = _out(c, m, n, out_dtype, ap_q8.device)
    _check(lib.mxfp8_gemm_w4a8_nt_prepacked_ab(_ptr(ap_q8), _ptr(ap_s), _ptr(bp_q), _ptr(bp_s), _ptr(c), code, m, n,
                                               k, _stream(stream)))
    return c


def mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m: int, n: int, k: int, c=None, out_dtype=torch.bfloat16,
                               splits: int = 0, ws: torch.Tensor | None = None, stream=None):
    """C[m, n] = A . B^T with both A [m, k] and B [n, k] prepacked (mxfp4_prepack_weight).

    splits: 0 = automatic K split over workgroups when the 64-column panels do
    not fill the chip (reduced through a zero-filled workspace), 1 = none."""
    lib = load_library()
    for t, rows, name in ((ap_q, m, "ap_q"), (bp_q, n, "bp_q")):
        cb, _ = mxfp4_prepacked_weight_size(rows, k)
        _require(t, name, torch.uint8, (cb,))
    for t, rows, name in ((ap_s, m, "ap_s"), (bp_s, n, "bp_s")):
        _, sb = mxfp4_prepacked_weight_size(rows, k)
        _require(t, name, torch.uint8, (sb,))
    c, code = _out(c, m, n, out_dtype, ap_q.device)
    need = lib.mxfp4_gemm_nt_prepacked_ab_workspace_size(m, n, k, splits)
    if ws is None:
        ws = workspace(need, ap_q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxfp4_gemm_nt_prepacked_ab_ex(_ptr(ap_q), _ptr(ap_s), _ptr(bp_q), _ptr(bp_s), _ptr(c), code, m, n, k,
                                             splits, _ptr(ws), nbytes, _stream(stream)))
    return c


def mxfp4_grouped_gemm_nt(a_q, a_s, b_q, b_s, offsets, c=None, out_dtype=torch.bfloat16,
                          ws: torch.Tensor | None = None, stream=None):
    """Per-group NT GEMM; `offsets` is a device int32 [groups + 1] tensor."""
    lib = load_library()
    total_m, kh = a_q.shape
    groups, n, _ = b_q.shape
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (total_m, k // 2))
    _require(a_s, "a_s", torch.uint8, (total_m, k // 32))
    _require(b_q, "b_q", torch.uint8, (groups, n, k // 2))
    _require(b_s, "b_s", torch.uint8, (groups, n, k // 32))
    _require(offsets, "offsets", torch.int32, (groups + 1,))
    c, code = _out(c, total_m, n, out_dtype, a_q.device)
    need = lib.mxfp4_grouped_gemm_nt_workspace_size(total_m, groups, n, k)
    if ws is None:
        ws = workspace(need, a_q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.mxfp4_grouped_gemm_nt(_ptr(a_q), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), groups,
                                     total_m, _ptr(c), code, n, k, _ptr(ws), nbytes, _stream(stream)))
    return c


def mxfp4_scales_interleave(scales, out=None, stream=None):
    """Row-major scale bytes [rows, k/32] (or [groups, rows, k/32]) -> the
    interleaved layout [k/512, rows, 16] (or [groups, k/512, rows, 16])."""
    lib = load_library()
    grouped = scales.dim() == 3
    groups, rows, kb = scales.shape if grouped else (1, *scales.shape)
    k = kb * 32
    shape = (groups, k // 512, rows, 16) if grouped else (k // 512, rows, 16)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=scales.device)
    _require(scales, "scales", torch.uint8, scales.shape)
    _require(out, "out", torch.uint8, shape)
    _check(lib.mxfp4_scales_interleave(_ptr(scales), groups, rows, k, _ptr(out), _stream(stream)))
    return out


def mxfp4_quantize_interleaved(x: torch.Tensor, q=None, scales_il=None, stream=None):
    """x: bf16 [rows, k] -> (q uint8 [rows, k/2], scales_il uint8 [k/512, rows, 16])."""
    lib = load_library()
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales_il is None:
        scales_il = torch.empty((k // 512, rows, 16), dtype=torch.uint8, device=x.device)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(q, "q", torch.uint8, (rows, k // 2))
    _require(scales_il, "scales_il", torch.uint8, (k // 512, rows, 16))
    _check(lib.mxfp4_quantize_interleaved(_ptr(x), rows, k, _ptr(q), _ptr(scales_il), _stream(stream)))
    return q, scales_il


def mxfp4_gemm_nt_interleaved(a_q, a_s_il, b_q, b_s_il, c=None, out_dtype=torch.bfloat16, stream=None):
    """mxfp4_gemm_nt with interleaved scales: a_s_il [k/512, m, 16], b_s_il [k/512, n, 16]."""
    lib = load_library()
    m, kh = a_q.shape
    n = b_q.shape[0]
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (m, k // 2))
    _require(a_s_il, "a_s_il", torch.uint8, (k // 512, m, 16))
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s_il, "b_s_il", torch.uint8, (k // 512, n, 16))
    c, code = _out(c, m, n, out_dtype, a_q.device)
    _check(lib.mxfp4_gemm_nt_interleaved(_ptr(a_q), _ptr(a_s_il), _ptr(b_q), _ptr(b_s_il), _ptr(c), code, m, n, k,
                                         _stream(stream)))
    return c


def mxfp4_grouped_gemm_nt_interleaved(a_q, a_s_il, b_q, b_s_il, offsets, c=None, out_dtype=torch.bfloat16,
                                      stream=None):
    """mxfp4_grouped_gemm_nt with interleaved scales: a_s_il [k/512, total_m, 16],
    b_s_il [groups, k/512, n, 16]."""
    lib = load_library()
    total_m, kh = a_q.shape
    groups, n, _ = b_q.shape
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (total_m, k // 2))
    _require(a_s_il, "a_s_il", torch.uint8, (k // 512, total_m, 16))
    _require(b_q, "b_q", torch.uint8, (groups, n, k // 2))
    _require(b_s_il, "b_s_il", torch.uint8, (groups, k // 512, n, 16))
    _require(offsets, "offsets", torch.int32, (groups + 1,))
    c, code = _out(c, total_m, n, out_dtype, a_q.device)
    _check(lib.mxfp4_grouped_gemm_nt_interleaved(_ptr(a_q), _ptr(a_s_il), _ptr(b_q), _ptr(b_s_il), _ptr(offsets),
                                                 groups, total_m, _ptr(c), code, n, k, _stream(stream)))
    return c


def mxfp8_quantize_interleaved(x: torch.Tensor, q8=None, scales_il=None, stream=None):
    """x: bf16 [rows, k] -> (q8 uint8 [rows, k] E4M3 codes, scales_il uint8 [k/512, rows, 16])."""
    lib = load_library()
    rows, k = x.shape
    if q8 is None:
        q8 = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales_il is None:
        scales_il = torch.empty((k // 512, rows, 16), dtype=torch.uint8, device=x.device)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(q8, "q8", torch.uint8, (rows, k))
    _require(scales_il, "scales_il", torch.uint8, (k // 512, rows, 16))
    _check(lib.mxfp8_quantize_interleaved(_ptr(x), rows, k, _ptr(q8), _ptr(scales_il), _stream(stream)))
    return q8, scales_il


def _gemm8_interleaved(fn, a_q8, a_s_il, b_q, b_s_il, b_cols, c, out_dtype, stream):
    m, k = a_q8.shape
    n = b_q.shape[0]
    _require(a_q8, "a_q8", torch.uint8, (m, k))
    _require(a_s_il, "a_s_il", torch.uint8, (k // 512, m, 16))
    _require(b_q, "b_q", torch.uint8, (n, b_cols(k)))
    _require(b_s_il, "b_s_il", torch.uint8, (k // 512, n, 16))
    c, code = _out(c, m, n, out_dtype, a_q8.device)
    _check(fn(_ptr(a_q8), _ptr(a_s_il), _ptr(b_q), _ptr(b_s_il), _ptr(c), code, m, n, k, _stream(stream)))
    return c


def mxfp8_gemm_w4a8_nt_interleaved(a_q8, a_s_il, b_q, b_s_il, c=None, out_dtype=torch.bfloat16, stream=None):
    """W4A8 with interleaved scales: a_s_il [k/512, m, 16], b_s_il [k/512, n, 16] (128 x 256 tiles)."""
    lib = load_library()
    return _gemm8_interleaved(lib.mxfp8_gemm_w4a8_nt_interleaved, a_q8, a_s_il, b_q, b_s_il, lambda k: k // 2, c,
                              out_dtype, stream)


def mxfp8_gemm_nt_interleaved(a_q8, a_s_il, b_q8, b_s_il, c=None, out_dtype=torch.bfloat16, stream=None):
    """MXFP8 x MXFP8 with interleaved scales: a_s_il [k/512, m, 16], b_s_il [k/512, n, 16]."""
    lib = load_library()
    return _gemm8_interleaved(lib.mxfp8_gemm_nt_interleaved, a_q8, a_s_il, b_q8, b_s_il, lambda k: k, c, out_dtype,
                              stream)


def mxfp8_grouped_gemm_w4a8_nt_interleaved(a_q8, a_s_il, b_q, b_s_il, offsets, c=None, out_dtype=torch.bfloat16,
                                           stream=None):
    """Grouped W4A8 with interleaved scales: a_s_il [k/512, total_m, 16], b_s_il [groups, k/512, n, 16]."""
    lib = load_library()
    total_m, k = a_q8.shape
    groups, n, _ = b_q.shape
    _require(a_q8, "a_q8", torch.uint8, (total_m, k))
    _require(a_s_il, "a_s_il", torch.uint8, (k // 512, total_m, 16))
    _require(b_q, "b_q", torch.uint8, (groups, n, k // 2))
    _require(b_s_il, "b_s_il", torch.uint8, (groups, k // 512, n, 16))
    _require(offsets, "offsets", torch.int32, (groups + 1,))
    c, code = _out(c, total_m, n, out_dtype, a_q8.device)
    _check(lib.mxfp8_grouped_gemm_w4a8_nt_interleaved(_ptr(a_q8), _ptr(a_s_il), _ptr(b_q), _ptr(b_s_il),
                                                      _ptr(offsets), groups, total_m, _ptr(c), code, n, k,
                                                      _stream(stream)))
    return c


def mxfp8_gemm_w4a8_nt(a_q8, a_s, b_q, b_s, c=None, out_dtype=torch.bfloat16, kernel: str = "auto", stream=None):
    """C[m, n] = A[m, k] . B[n, k]^T with A in MXFP8 ([m, k] codes) and B in MXFP4.
    kernel: "auto", "tile128" (128 x 256 tiles) or "stream"."""
    lib = load_library()
    m, k = a_q8.shape
    n = b_q.shape[0]
    _require(a_q8, "a_q8", torch.uint8, (m, k))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s, "b_s", torch.uint8, (n, k // 32))
    c, code = _out(c, m, n, out_dtype, a_q8.device)
    _check(lib.mxfp8_gemm_w4a8_nt_ex(_ptr(a_q8), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(c), code, m, n, k,
                                     KERNELS[kernel], _stream(stream)))
    return c


def mxfp8_gemm_w4a8_nt_prepacked(a_q8, a_s, bp_q, bp_s, n: int, c=None, out_dtype=torch.bfloat16, stream=None):
    """W4A8 C[m, n] = A[m, k] . B^T with A in MXFP8 and B prepacked (mxfp4_prepack_weight)."""
    lib = load_library()
    m, k = a_q8.shape
    _require(a_q8, "a_q8", torch.uint8, (m, k))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    cb, sb = mxfp4_prepacked_weight_size(n, k)
    _require(bp_q, "bp_q", torch.uint8, (cb,))
    _require(bp_s, "bp_s", torch.uint8, (sb,))
    c, code = _out(c, m, n, out_dtype, a_q8.device)
    _check(lib.mxfp8_gemm_w4a8_nt_prepacked(_ptr(a_q8), _ptr(a_s), _ptr(bp_q), _ptr(bp_s), _ptr(c), code, m, n, k,
                                            _stream(stream)))
    return c


def mxfp8_gemm_nt(a_q8, a_s, b_q8, b_s, c=None, out_dtype=torch.bfloat16, kernel: str = "auto", stream=None):
    """C[m, n] = A[m, k] . B[n, k]^T with both operands in MXFP8 ([rows, k] E4M3 codes).
    kernel: "auto", "tile256" (256 x 256 tiles) or "tile128"."""
    lib = load_library()
    m, k = a_q8.shape
    n = b_q8.shape[0]
    _require(a_q8, "a_q8", torch.uint8, (m, k))
    _require(a_s, "a_s", torch.uint8, (m, k // 32))
    _require(b_q8, "b_q8", torch.uint8, (n, k))
    _require(b_s, "b_s", torch.uint8, (n, k // 32))
    c, code = _out(c, m, n, out_dtype, a_q8.device)
    _check(lib.mxfp8_gemm_nt_ex(_ptr(a_q8), _ptr(a_s), _ptr(b_q8), _ptr(b_s), _ptr(c), code, m, n, k,
                                KERNELS[kernel], _stream(stream)))
    return c


def mxfp8_grouped_gemm_w4a8_nt(a_q8, a_s, b_q, b_s, offsets, c=None, out_dtype=torch.bfloat16, stream=None):
    """Per-group W4A8 NT GEMM; `offsets` is a device int32 [groups + 1] tensor."""
    lib = load_library()
    total_m, k = a_q8.shape
    groups, n, _ = b_q.shape
    _require(a_q8, "a_q8", torch.uint8, (total_m, k))
    _require(a_s, "a_s", torch.uint8, (total_m, k // 32))
    _require(b_q, "b_q", torch.uint8, (groups, n, k // 2))
    _require(b_s, "b_s", torch.uint8, (groups, n, k // 32))
    _require(offsets, "offsets", torch.int32, (groups + 1,))
    c, code = _out(c, total_m, n, out_dtype, a_q8.device)
    _check(lib.mxfp8_grouped_gemm_w4a8_nt(_ptr(a_q8), _ptr(a_s), _ptr(b_q), _ptr(b_s), _ptr(offsets), groups,
                                          total_m, _ptr(c), code, n, k, _stream(stream)))
    return c


def mxfp4_probe_mfma(seed: torch.Tensor, out: torch.Tensor, blocks: int, iters: int, stream=None,
                     a_fp8: bool = False) -> float:
    """Runs the scaled-MFMA probe (include/mxfp4_probe.h), FP4 x FP4 or, with
    a_fp8, FP4 x FP8; returns the flops of the call."""
    lib = load_library()
    if seed.numel() * seed.element_size() < PROBE_SEED_BYTES or not seed.is_contiguous():
        raise ValueError(f"seed must be a contiguous device tensor of at least {PROBE_SEED_BYTES} bytes")
    if out.dtype != torch.float32 or out.numel() < blocks * 512 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 device tensor of at least blocks * 512 elements")
    fn = lib.mxfp4_probe_mfma_w4a8 if a_fp8 else lib.mxfp4_probe_mfma
    _check(fn(_ptr(seed), _ptr(out), blocks, iters, _stream(stream)))
    return lib.mxfp4_probe_mfma_flops(blocks, iters)


def mxfp4_probe_read(src: torch.Tensor, out: torch.Tensor, blocks: int, stream=None) -> int:
    """Runs the streaming-read probe over all of `src`; returns the bytes read."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    if out.dtype not in (torch.int32, torch.uint32) or out.numel() < blocks * 256 or not out.is_contiguous():
        raise ValueError("out must be a contiguous 32-bit integer device tensor of at least blocks * 256 elements")
    _check(lib.mxfp4_probe_read(_ptr(src), nbytes, _ptr(out), blocks, _stream(stream)))
    return nbytes


# ---------------------------------------------------------------------------
# MoE steps (include/mxfp4_moe.h)
# ---------------------------------------------------------------------------

def mxfp4_moe_route(logits: torch.Tensor, top_k: int, ids=None, weights=None, stream=None):
    """logits float32 [tokens, experts] -> (ids int32 [tokens, top_k], weights float32 [tokens, top_k])."""
    lib = load_library()
    tokens, experts = logits.shape
    if ids is None:
        ids = torch.empty((tokens, top_k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((tokens, top_k), dtype=torch.float32, device=logits.device)
    _require(logits, "logits", torch.float32, (tokens, experts))
    _require(ids, "ids", torch.int32, (tokens, top_k))
    _require(weights, "weights", torch.float32, (tokens, top_k))
    _check(lib.mxfp4_moe_route(_ptr(logits), tokens, experts, top_k, _ptr(ids), _ptr(weights), _stream(stream)))
    return ids, weights


def mxfp4_moe_permute(ids: torch.Tensor, experts: int, offsets=None, row_token=None, token_rows=None,
                      stream=None):
    """ids int32 [tokens, top_k] -> (offsets int32 [experts + 1], row_token int32 [tokens * top_k],
    token_rows int32 [tokens, top_k])."""
    lib = load_library()
    tokens, top_k = ids.shape
    dev = ids.device
    if offsets is None:
        offsets = torch.empty((experts + 1,), dtype=torch.int32, device=dev)
    if row_token is None:
        row_token = torch.empty((tokens * top_k,), dtype=torch.int32, device=dev)
    if token_rows is None:
        token_rows = torch.empty((tokens, top_k), dtype=torch.int32, device=dev)
    _require(ids, "ids", torch.int32, (tokens, top_k))
    _require(offsets, "offsets", torch.int32, (experts + 1,))
    _require(row_token, "row_token", torch.int32, (tokens * top_k,))
    _require(token_rows, "token_rows", torch.int32, (tokens, top_k))
    _check(lib.mxfp4_moe_permute(_ptr(ids), tokens, experts, top_k, _ptr(offsets), _ptr(row_token),
                                 _ptr(token_rows), _stream(stream)))
    return offsets, row_token, token_rows


def _quantize_scatter(fn, x, token_rows, total_rows, q, scales, code_cols, stream, interleaved=False):
    tokens, k = x.shape
    top_k = token_rows.shape[1]
    s_shape = (k // 512, total_rows, 16) if interleaved else (total_rows, k // 32)
    if q is None:
        q = torch.empty((total_rows, code_cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(s_shape, dtype=torch.uint8, device=x.device)
    _require(x, "x", torch.bfloat16, (tokens, k))
    _require(token_rows, "token_rows", torch.int32, (tokens, top_k))
    _require(q, "q", torch.uint8, (total_rows, code_cols))
    _require(scales, "scales", torch.uint8, s_shape)
    _check(fn(_ptr(x), tokens, k, top_k, _ptr(token_rows), total_rows, _ptr(q), _ptr(scales), _stream(stream)))
    return q, scales


def mxfp4_moe_quantize_scatter(x, token_rows, total_rows: int, q=None, scales=None, stream=None):
    """x bf16 [tokens, k] -> MXFP4 rows (q uint8 [total_rows, k/2], scales uint8 [total_rows, k/32]);
    row token_rows[t, j] receives token t's quantized row."""
    lib = load_library()
    return _quantize_scatter(lib.mxfp4_moe_quantize_scatter, x, token_rows, total_rows, q, scales,
                             x.shape[1] // 2, stream)


def mxfp4_moe_quantize_scatter_interleaved(x, token_rows, total_rows: int, q=None, scales_il=None, stream=None):
    """mxfp4_moe_quantize_scatter with the scales interleaved: scales_il [k/512, total_rows, 16]."""
    lib = load_library()
    return _quantize_scatter(lib.mxfp4_moe_quantize_scatter_interleaved, x, token_rows, total_rows, q, scales_il,
                             x.shape[1] // 2, stream, interleaved=True)


def mxfp8_moe_quantize_scatter_interleaved(x, token_rows, total_rows: int, q8=None, scales_il=None, stream=None):
    """mxfp8_moe_quantize_scatter with the scales interleaved: scales_il [k/512, total_rows, 16]."""
    lib = load_library()
    return _quantize_scatter(lib.mxfp8_moe_quantize_scatter_interleaved, x, token_rows, total_rows, q8, scales_il,
                             x.shape[1], stream, interleaved=True)


def mxfp8_moe_quantize_scatter(x, token_rows, total_rows: int, q8=None, scales=None, stream=None):
    """The same with MXFP8 rows (q8 uint8 [total_rows, k])."""
    lib = load_library()
    return _quantize_scatter(lib.mxfp8_moe_quantize_scatter, x, token_rows, total_rows, q8, scales,
                             x.shape[1], stream)


def mxfp4_moe_combine(y, token_rows, weights, out=None, out_dtype=torch.bfloat16, stream=None):
    """y bf16 [total_rows, n], token_rows int32 [tokens, top_k], weights float32 [tokens, top_k]
    -> out [tokens, n] = sum_j weights[t, j] * y[token_rows[t, j]] (bf16 or float32)."""
    lib = load_library()
    total_rows, n = y.shape
    tokens, top_k = token_rows.shape
    _require(y, "y", torch.bfloat16, (total_rows, n))
    _require(token_rows, "token_rows", torch.int32, (tokens, top_k))
    _require(weights, "weights", torch.float32, (tokens, top_k))
    out, code = _out(out, tokens, n, out_dtype, y.device)
    _check(lib.mxfp4_moe_combine(_ptr(y), total_rows, n, _ptr(token_rows), _ptr(weights), tokens, top_k,
                                 _ptr(out), code, _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# Fused producers (include/mxfp4_producers.h)
# ---------------------------------------------------------------------------

def _mxfp4_out(q, scales, rows, k, device, prepacked, interleaved=False):
    """Codes and scales of a [rows, k] MXFP4 output: row-major, the prepacked layout's flat buffers, or
    row-major codes with interleaved scales [k/512, rows, 16]."""
    if prepacked and interleaved:
        raise ValueError("prepacked and interleaved are different layouts: choose one")
    if prepacked:
        cb, sb = mxfp4_prepacked_weight_size(rows, k)
        qs, ss = (cb,), (sb,)
    elif interleaved:
        qs, ss = (rows, k // 2), (k // 512, rows, 16)
    else:
        qs, ss = (rows, k // 2), (rows, k // 32)
    if q is None:
        q = torch.empty(qs, dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty(ss, dtype=torch.uint8, device=device)
    _require(q, "q", torch.uint8, qs)
    _require(scales, "scales", torch.uint8, ss)
    return q, scales


def mxfp4_rmsnorm_quantize(x, gamma, eps: float, residual=None, residual_out=None, y=None, q=None, scales=None,
                           stream=None, prepacked: bool = False, interleaved: bool = False):
    """(x [+ residual]) -> RMSNorm(., gamma, eps) -> MXFP4 (q [rows, k/2], scales [rows, k/32]; with
    prepacked=True the prepacked operand layout of the decode GEMM; with interleaved=True the scales as
    [k/512, rows, 16] for mxfp4_gemm_nt_interleaved).
    residual_out (optional) receives x + residual; y (optional) the BF16 RMSNorm output."""
    lib = load_library()
    rows, k = x.shape
    q, scales = _mxfp4_out(q, scales, rows, k, x.device, prepacked, interleaved)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(gamma, "gamma", torch.bfloat16, (k,))
    for t, name in ((residual, "residual"), (residual_out, "residual_out"), (y, "y")):
        if t is not None:
            _require(t, name, torch.bfloat16, (rows, k))
    fn = (lib.mxfp4_rmsnorm_quantize_prepacked if prepacked else
          lib.mxfp4_rmsnorm_quantize_interleaved if interleaved else lib.mxfp4_rmsnorm_quantize)
    _check(fn(_ptr(x), _ptr(residual), _ptr(gamma), float(eps), rows, k, _ptr(residual_out), _ptr(y), _ptr(q),
              _ptr(scales), _stream(stream)))
    return q, scales


def mxfp4_swiglu_quantize(gate, up, y=None, q=None, scales=None, stream=None, prepacked: bool = False,
                          interleaved: bool = False):
    """silu(gate) * up -> MXFP4 (row-major; with prepacked=True the prepacked operand layout; with
    interleaved=True row-major codes and scales [k/512, rows, 16]).  gate and up
    are [rows, k] views sharing one row stride (for example the two halves of a [rows, 2k] projection output);
    y (optional) receives the BF16 activation."""
    lib = load_library()
    rows, k = gate.shape
    if tuple(up.shape) != (rows, k) or gate.stride() != up.stride() or gate.stride(1) != 1:
        raise ValueError("gate and up must be [rows, k] views with the same row stride and unit column stride")
    if gate.dtype != torch.bfloat16 or up.dtype != torch.bfloat16 or not gate.is_cuda or not up.is_cuda:
        raise TypeError("gate and up must be bfloat16 device tensors")
    ld = gate.stride(0) if rows > 1 else k
    q, scales = _mxfp4_out(q, scales, rows, k, gate.device, prepacked, interleaved)
    if y is not None:
        _require(y, "y", torch.bfloat16, (rows, k))
    fn = (lib.mxfp4_swiglu_quantize_prepacked if prepacked else
          lib.mxfp4_swiglu_quantize_interleaved if interleaved else lib.mxfp4_swiglu_quantize)
    _check(fn(_ptr(gate), _ptr(up), ld, rows, k, _ptr(y), _ptr(q), _ptr(scales), _stream(stream)))
    return q, scales


# ---------------------------------------------------------------------------
# NVFP4 (include/nvfp4.h)
# ---------------------------------------------------------------------------

def nvfp4_quantize(x, q=None, scales=None, gs=None, stream=None):
    """x bf16 [rows, k] -> (q uint8 [rows, k/2], scales uint8 [rows, k/16] UE4M3, gs float32 [rows])."""
    lib = load_library()
    rows, k = x.shape
    if q is None:
        q = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    if gs is None:
        gs = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _require(x, "x", torch.bfloat16, (rows, k))
    _require(q, "q", torch.uint8, (rows, k // 2))
    _require(scales, "scales", torch.uint8, (rows, k // 16))
    _require(gs, "gs", torch.float32, (rows,))
    _check(lib.nvfp4_quantize(_ptr(x), rows, k, _ptr(q), _ptr(scales), _ptr(gs), _stream(stream)))
    return q, scales, gs


def nvfp4_gemm_nt(a_q, a_s, a_gs, b_q, b_s, b_gs, c=None, out_dtype=torch.bfloat16, stream=None):
    """C[m, n] = A[m, k] . B[n, k]^T on NVFP4 operands (codes, UE4M3 scales, per-row global scales)."""
    lib = load_library()
    m, kh = a_q.shape
    n = b_q.shape[0]
    k = kh * 2
    _require(a_q, "a_q", torch.uint8, (m, k // 2))
    _require(a_s, "a_s", torch.uint8, (m, k // 16))
    _require(a_gs, "a_gs", torch.float32, (m,))
    _require(b_q, "b_q", torch.uint8, (n, k // 2))
    _require(b_s, "b_s", torch.uint8, (n, k // 16))
    _require(b_gs, "b_gs", torch.float32, (n,))
    c, code = _out(c, m, n, out_dtype, a_q.device)
    _check(lib.nvfp4_gemm_nt(_ptr(a_q), _ptr(a_s), _ptr(a_gs), _ptr(b_q), _ptr(b_s), _ptr(b_gs), _ptr(c), code,
                             m, n, k, _stream(stream)))
    return c
