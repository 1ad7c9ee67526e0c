"""The prepacked operand layout of include/mxfp4.h, built with NumPy from its
definition (no GPU): used by the GPU tests to check the prepacking kernel, the
prepacked quantizer and, through them, the GEMMs that read the layout."""
import numpy as np


def prepack_numpy(bq, bs):
    """The prepacked layout from its definition: per 64-row panel and 512-K pair,
    codes[w, u=2s+j, l, c] = B code byte c of row 32j + l%32 at 256t + 128s + 32w + 16(l//32),
    scales[w, l, b=2s+j] = B scale of that row for block 16t + 8s + 2w + l//32."""
    n, kh = bq.shape
    k = kh * 2
    panels, pairs = -(-n // 64), k // 512
    qpad = np.zeros((panels * 64, kh), np.uint8)
    qpad[:n] = bq
    spad = np.zeros((panels * 64, k // 32), np.uint8)
    spad[:n] = bs
    codes = np.zeros((panels, pairs, 4, 4, 64, 16), np.uint8)
    scales = np.zeros((panels, pairs, 4, 64, 4), np.uint8)
    for w in range(4):
        for s in range(2):
            for j in range(2):
                for l in range(64):
                    rows = np.arange(panels) * 64 + 32 * j + l % 32
                    for t in range(pairs):
                        off = 256 * t + 128 * s + 32 * w + 16 * (l // 32)
                        codes[:, t, w, 2 * s + j, l, :] = qpad[rows, off:off + 16]
                        scales[:, t, w, l, 2 * s + j] = spad[rows, 16 * t + 8 * s + 2 * w + l // 32]
    return codes.reshape(-1), scales.reshape(-1)


def prepack_fp8_numpy(q8, s):
    """The FP8 prepacked layout of include/mxfp8.h from its definition: per 64-row panel P and 512-K
    pair t, codes[w, u=2s+j, e, l, c] = FP8 code of row 64P + 32j + l%32 at K 512t + 256s + 64w + 32e +
    16(l//32) + c; the scale bytes as in the MXFP4 prepacked layout."""
    n, k = q8.shape
    panels, pairs = -(-n // 64), k // 512
    qpad = np.zeros((panels * 64, k), np.uint8)
    qpad[:n] = q8
    codes = np.zeros((panels, pairs, 4, 4, 2, 64, 16), np.uint8)
    for w in range(4):
        for st in range(2):
            for j in range(2):
                for e in range(2):
                    for l in range(64):
                        rows = np.arange(panels) * 64 + 32 * j + l % 32
                        for t in range(pairs):
                            off = 512 * t + 256 * st + 64 * w + 32 * e + 16 * (l // 32)
                            codes[:, t, w, 2 * st + j, e, l, :] = qpad[rows, off:off + 16]
    _, scales = prepack_numpy(np.zeros((n, k // 2), np.uint8), s)
    return codes.reshape(-1), scales
