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


def test_calls_per_replay_divides_and_leaves_four_samples():
    import bench
    assert bench.calls_per_replay(20) == 5
    assert bench.calls_per_replay(200) == 50
    assert bench.calls_per_replay(64) == 16
    assert bench.calls_per_replay(3) == 1
    for steps in range(1, 400):
        p = bench.calls_per_replay(steps)
        assert steps % p == 0 and 1 <= p <= 64
        if steps >= 4:
            assert steps // p >= 4


def test_summary_statistics_come_from_one_sample_set():
    import bench
    samples = [0.050, 0.048, 0.052, 0.049, 0.051]
    s = bench.summarize(samples, 5)
    assert s["samples"] == 5 and s["calls_per_sample"] == 5
    assert s["min"] <= s["median"] <= s["max"]
    assert s["min"] <= s["mean"] <= s["max"]
    assert abs(s["mean"] - sum(samples) / 5) < 1e-15
    u = bench.us(s)
    assert u["samples"] == 5 and u["mean"] == round(s["mean"] * 1e3, 3)


def test_roofline_fields():
    import bench
    r = bench.roofline("mfma", 3165.5, bench.PEAK_FP4_TFLOPS, "TFLOP/s", None, kernel="gemm_tile_kernel")
    assert set(r) == {"bound", "achieved", "peak", "unit", "frac", "traffic", "kernel"}
    assert r["frac"] == round(3165.5 / 10100.0, 4)


def test_inputs_record_names_seeds_and_digests():
    import bench
    import workloads
    w = workloads.TINY
    rec = bench.dense_inputs_record(w)
    a, b = w.make()
    assert rec["seeds"] == {"a": w.seed + workloads.ROLE_A, "a_outlier_channels": w.seed + workloads.ROLE_OUTLIER,
                            "b": w.seed + workloads.ROLE_B}
    assert rec["sha256"]["a_bf16"] == workloads.sha256_of(a)
    assert rec["sha256"]["b_bf16"] == workloads.sha256_of(b)
    small = workloads.MoEWorkload("moe_small", tokens=16, experts=4, top_k=2, n=32, k=64, seed=900)
    mrec = bench.moe_inputs_record(small)
    assert set(mrec["sha256"]) == {"x_bf16", "logits_f32", "w_bf16", "offsets_i32"}
    assert mrec["seeds"]["route_noise"] == 900 + workloads.ROLE_ROUTE_NOISE


def test_detail_lines_are_timed_over_at_least_200_calls():
    """Only the headline step follows --steps; the other lines time at least
    DETAIL_STEPS calls (so --steps 20 does not time microsecond kernels in
    replays of five calls)."""
    import bench
    assert bench.DETAIL_STEPS >= 200 and bench.DETAIL_WARMUP >= 20
    assert bench.calls_per_replay(max(20, bench.DETAIL_STEPS)) >= 50
