"""The oracle still reproduces the digests stored in tests/golden (written by
tests/golden/make_golden.py from the oracle itself; the pages print no worked
example, so these freeze the oracle's results on the seeded workloads)."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "oracle_digests.txt")):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split()
        vals[k] = v
    return vals


def test_oracle_reproduces_stored_digests():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stored = load_golden()
    fresh = dict(mod.entries())
    assert fresh == stored
