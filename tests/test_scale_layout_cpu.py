"""CPU checks of the interleaved scale layout definition the GPU tests compare
against: the byte formula stated in include/mxfp4.h, element by element; a
permutation with an inverse; one 512-K slab of 64 consecutive rows is one
contiguous kilobyte."""
import numpy as np

from tests.scale_layout import deinterleave_numpy, interleave_numpy


def _tagged(rows, k, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(rows, k // 32), dtype=np.uint8)


def test_interleave_matches_the_header_formula():
    """scales_il[(kb / 16) * rows * 16 + r * 16 + kb % 16] = scales[r * k/32 + kb], every byte."""
    for rows, k in [(1, 512), (3, 1024), (64, 512), (70, 2048)]:
        s = _tagged(rows, k, rows + k)
        flat = interleave_numpy(s).reshape(-1)
        kb_n = k // 32
        for r in range(rows):
            for kb in range(kb_n):
                assert flat[(kb // 16) * rows * 16 + r * 16 + kb % 16] == s[r, kb]


def test_interleave_grouped_is_per_group():
    s = np.stack([_tagged(37, 1536, g) for g in range(3)])
    il = interleave_numpy(s)
    assert il.shape == (3, 3, 37, 16)
    for g in range(3):
        assert np.array_equal(il[g], interleave_numpy(s[g]))


def test_interleave_is_a_permutation_with_an_inverse():
    for rows, k in [(5, 512), (129, 4096)]:
        s = _tagged(rows, k, 7 * rows)
        il = interleave_numpy(s)
        assert np.array_equal(np.sort(il.reshape(-1)), np.sort(s.reshape(-1)))
        assert np.array_equal(deinterleave_numpy(il), s)


def test_one_slab_of_64_rows_is_one_contiguous_kilobyte():
    """What the GEMM's scale copy reads with one instruction: rows r0 .. r0+63
    of slab g, in row order, 16 bytes each, at consecutive addresses."""
    rows, k = 200, 2048
    s = _tagged(rows, k, 3)
    flat = interleave_numpy(s).reshape(-1)
    for g in range(k // 512):
        for r0 in (0, 64, 136):
            start = g * rows * 16 + r0 * 16
            want = np.concatenate([s[r, 16 * g:16 * g + 16] for r in range(r0, r0 + 64)])
            assert np.array_equal(flat[start:start + 1024], want)
