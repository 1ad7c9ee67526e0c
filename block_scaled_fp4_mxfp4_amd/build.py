"""Builds the gfx950 HIP library libmxfp4.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmxfp4.so")
SOURCES = ["api.hip", "quantize.hip", "gemm_tile.hip", "gemm_splitk.hip", "gemm_stream.hip", "probes.hip", "moe.hip", "producers.hip", "nvfp4.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# kernel resource remarks (registers, scratch) are printed for every kernel and checked
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
RESOURCES = os.path.join(BUILD, "resources.txt")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep fp32 arithmetic in scalar/float2 VALU forms, never packed-fp32 VOP3P
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, kernel_resources(src, r.stderr)


def kernel_resources(src: str, remarks: str) -> list:
    """(source, kernel, VGPRs, AGPRs, scratch bytes per lane, VGPRs spilled) for every
    kernel in hipcc's resource-usage remarks."""
    rows, cur = [], {}
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = {"kernel": val}
        elif key in ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "VGPRs Spill") and cur:
            cur[key] = int(val)
            if key == "VGPRs Spill":
                rows.append((src, cur["kernel"], cur.get("VGPRs", 0), cur.get("AGPRs", 0),
                             cur.get("ScratchSize [bytes/lane]", 0), cur["VGPRs Spill"]))
                cur = {}
    return rows


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    resources = [row for _, rows in done for row in rows]
    with open(RESOURCES, "w") as f:
        for row in resources:
            f.write("src=%s kernel=%s vgprs=%d agprs=%d scratch=%d spilled=%d\n" % row)
    spilling = [row for row in resources if row[4] > 0 or row[5] > 0]
    if spilling:
        # every kernel is written to keep its working set in registers: a spill is a build error
        raise RuntimeError("kernels using scratch memory:\n" + "\n".join(f"  {r[0]}: {r[1]} scratch={r[4]} "
                                                                          f"spilled={r[5]}" for r in spilling))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
