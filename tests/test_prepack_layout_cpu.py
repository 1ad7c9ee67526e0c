"""CPU checks of the prepacked-layout definition the GPU tests compare against:
it is a permutation of B's bytes (padding rows zero), and it agrees with the
byte formula stated in include/mxfp4.h at sampled positions."""
import numpy as np

from tests.prepack_layout import prepack_numpy


def _tagged(n, k):
    """Codes and scales whose every byte encodes its own position (mod 256 per field)."""
    rng = np.random.default_rng(n * 7 + k)
    q = rng.integers(1, 256, size=(n, k // 2), dtype=np.uint8)
    s = rng.integers(1, 255, size=(n, k // 32), dtype=np.uint8)
    return q, s


def test_prepack_is_a_permutation_with_zero_padding():
    for n, k in [(1, 512), (64, 512), (100, 1024), (130, 1536)]:
        q, s = _tagged(n, k)
        pq, ps = prepack_numpy(q, s)
        panels = -(-n // 64)
        assert pq.size == panels * 64 * k // 2 and ps.size == panels * 64 * k // 32
        # byte multisets: the input bytes plus one zero per padding byte
        pad = (panels * 64 - n)
        assert np.array_equal(np.sort(pq), np.sort(np.concatenate([q.ravel(), np.zeros(pad * k // 2, np.uint8)])))
        assert np.array_equal(np.sort(ps), np.sort(np.concatenate([s.ravel(), np.zeros(pad * k // 32, np.uint8)])))


def test_prepack_matches_the_header_formula():
    """codes: byte w*4096 + u*1024 + l*16 + c of block (P, t), u = 2s + j, is code byte c of row
    64P + 32j + l%32 at row byte 256t + 128s + 32w + 16(l//32); scales: byte w*256 + l*4 + 2s + j is
    that row's scale for block 16t + 8s + 2w + l//32."""
    n, k = 150, 2048
    q, s = _tagged(n, k)
    pq, ps = prepack_numpy(q, s)
    pairs = k // 512
    rng = np.random.default_rng(3)
    for _ in range(4000):
        P, t = rng.integers(-(-n // 64)), rng.integers(pairs)
        w, u, l, c = rng.integers(4), rng.integers(4), rng.integers(64), rng.integers(16)
        st, j = u // 2, u % 2
        row = 64 * P + 32 * j + l % 32
        want_q = q[row, 256 * t + 128 * st + 32 * w + 16 * (l // 32) + c] if row < n else 0
        assert pq[(P * pairs + t) * 16384 + w * 4096 + u * 1024 + l * 16 + c] == want_q
        want_s = s[row, 16 * t + 8 * st + 2 * w + l // 32] if row < n else 0
        assert ps[(P * pairs + t) * 1024 + w * 256 + l * 4 + u] == want_s


def test_fp8_prepack_is_a_permutation_with_zero_padding():
    from tests.prepack_layout import prepack_fp8_numpy
    for n, k in [(1, 512), (64, 512), (100, 1024)]:
        rng = np.random.default_rng(n + k)
        q8 = rng.integers(1, 256, size=(n, k), dtype=np.uint8)
        s = rng.integers(1, 255, size=(n, k // 32), dtype=np.uint8)
        pq, ps = prepack_fp8_numpy(q8, s)
        panels = -(-n // 64)
        pad = panels * 64 - n
        assert pq.size == panels * 64 * k and ps.size == panels * 64 * k // 32
        assert np.array_equal(np.sort(pq), np.sort(np.concatenate([q8.ravel(), np.zeros(pad * k, np.uint8)])))
        # the scale bytes sit where the MXFP4 layout keeps them
        assert np.array_equal(ps, prepack_numpy(np.zeros((n, k // 2), np.uint8), s)[1])


def test_fp8_prepack_matches_the_header_formula():
    """byte (P*pairs + t)*32768 + w*8192 + u*2048 + e*1024 + l*16 + c is the code of row 64P + 32j + l%32
    at K 512t + 256s + 64w + 32e + 16(l//32) + c (u = 2s + j)."""
    from tests.prepack_layout import prepack_fp8_numpy
    n, k = 150, 1536
    rng = np.random.default_rng(5)
    q8 = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    s = rng.integers(0, 256, size=(n, k // 32), dtype=np.uint8)
    pq, _ = prepack_fp8_numpy(q8, s)
    pairs = k // 512
    for _ in range(4000):
        P, t = rng.integers(-(-n // 64)), rng.integers(pairs)
        w, u, e, l, c = rng.integers(4), rng.integers(4), rng.integers(2), rng.integers(64), rng.integers(16)
        st, j = u // 2, u % 2
        row = 64 * P + 32 * j + l % 32
        want = q8[row, 512 * t + 256 * st + 64 * w + 32 * e + 16 * (l // 32) + c] if row < n else 0
        assert pq[(P * pairs + t) * 32768 + w * 8192 + u * 2048 + e * 1024 + l * 16 + c] == want
