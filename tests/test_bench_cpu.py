"""Host-side checks of bench.py's contract that need no GPU: it refuses more
than one GPU with a message and prints nothing on stdout, and its algorithmic
byte counts match their definitions (each code and scale byte of A and B once,
plus C once; the quantizers' BF16 in, codes and scale bytes out)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    import bench
    # decode 128 x 14336 x 4096: the figure the decode roofline divides by
    assert bench.gemm_algorithmic_bytes(128, 14336, 4096) == 35_143_680
    # prefill 4096^3
    assert bench.gemm_algorithmic_bytes(4096, 4096, 4096) == 51_380_224
    # 2 bytes in, 0.5 + 1/32 out per element
    assert bench.quant_algorithmic_bytes(4096, 4096) == 4096 * 4096 * 2 + 4096 * 2048 + 4096 * 128
    # MXFP8: 2 bytes in, 1 + 1/32 out per element
    assert bench.quant_algorithmic_bytes(4096, 4096, 1.0) == 4096 * 4096 * 3 + 4096 * 128
    # W4A8 decode: A one byte per element + scales, B packed + scales, C bf16
    assert bench.w4a8_algorithmic_bytes(128, 14336, 4096) == (128 * 4096 + 128 * 128 + 14336 * 2048
                                                               + 14336 * 128 + 128 * 14336 * 2)
