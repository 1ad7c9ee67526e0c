"""The interleaved scale layout of include/mxfp4.h, built with NumPy from its
definition (no GPU): the GPU tests compare the interleaving kernel, the
interleaved quantizers and, through them, the GEMMs that read the layout
against it."""
import numpy as np


def interleave_numpy(scales):
    """scales [rows, k/32] -> [k/512, rows, 16]; [groups, rows, k/32] -> [groups, k/512, rows, 16]:
    out[..., g, r, j] = scales[..., r, 16 g + j]."""
    s = np.asarray(scales, dtype=np.uint8)
    *lead, rows, kb = s.shape
    assert kb % 16 == 0, "k must be a multiple of 512"
    return np.ascontiguousarray(np.moveaxis(s.reshape(*lead, rows, kb // 16, 16), -2, -3))


def deinterleave_numpy(scales_il):
    """The inverse: [..., k/512, rows, 16] -> [..., rows, k/32]."""
    s = np.asarray(scales_il, dtype=np.uint8)
    *lead, slabs, rows, _ = s.shape
    return np.ascontiguousarray(np.moveaxis(s, -3, -2).reshape(*lead, rows, slabs * 16))
