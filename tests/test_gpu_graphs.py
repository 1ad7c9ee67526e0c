"""HIP graph capture of the MoE layer and a fused producer.

The calls are stream-ordered and allocate nothing, so a caller may capture
them.  The whole on-device MoE layer (route -> permute -> scatter-quantize ->
grouped GEMM -> combine) and the RMSNorm producer are captured once, replayed
several times with the program's own eager work and synchronisations between
the replays, and every replay is compared with the eager result (bit-exact:
the same kernels on the same inputs).
"""
import pytest
import torch

import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_grouped_gemm_nt, mxfp4_moe_combine, mxfp4_moe_permute,
                                        mxfp4_moe_quantize_scatter, mxfp4_moe_route, mxfp4_quantize,
                                        mxfp4_rmsnorm_quantize)
from tests.gpu_common import device, log

pytestmark = pytest.mark.gpu


def test_moe_layer_and_producer_graph_replays_match_eager():
    dev = device()
    tokens, experts, top_k, n, k = 512, 16, 4, 256, 1024
    log(f"graph: moe layer T={tokens} E={experts} k={top_k} N={n} K={k} + rmsnorm producer")
    x = workloads.activation_bf16(tokens, k, 900, outliers=True).to(dev)
    lg = workloads.gaussian_bf16((tokens, experts), 2.0, 901).float().to(dev)
    wq, ws = mxfp4_quantize(workloads.gaussian_bf16((experts * n, k), 0.02, 902).to(dev))
    wq, ws = wq.view(experts, n, k // 2), ws.view(experts, n, k // 32)
    gamma = workloads.gaussian_bf16((k,), 1.0, 903).to(dev)
    rows = tokens * top_k
    ids = torch.empty((tokens, top_k), dtype=torch.int32, device=dev)
    gate = torch.empty((tokens, top_k), dtype=torch.float32, device=dev)
    off = torch.empty((experts + 1,), dtype=torch.int32, device=dev)
    rt = torch.empty((rows,), dtype=torch.int32, device=dev)
    tr = torch.empty((tokens, top_k), dtype=torch.int32, device=dev)
    aq = torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((rows, k // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
    out = torch.empty((tokens, n), dtype=torch.bfloat16, device=dev)
    pq = torch.empty((tokens, k // 2), dtype=torch.uint8, device=dev)
    ps = torch.empty((tokens, k // 32), dtype=torch.uint8, device=dev)

    def layer():
        mxfp4_moe_route(lg, top_k, ids, gate)
        mxfp4_moe_permute(ids, experts, off, rt, tr)
        mxfp4_moe_quantize_scatter(x, tr, rows, aq, as_)
        mxfp4_grouped_gemm_nt(aq, as_, wq, ws, off, c=y)
        mxfp4_moe_combine(y, tr, gate, out=out)
        mxfp4_rmsnorm_quantize(x, gamma, 1e-5, q=pq, scales=ps)

    layer()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (ids, gate, off, rt, tr, aq, as_, y, out, pq, ps)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(4):
        for t in (ids, gate, off, rt, tr, aq, as_, y, out, pq, ps):   # eager work between replays
            t.view(torch.uint8).fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("ids", "gate", "offsets", "row_token", "token_rows", "a_q", "a_s", "y",
                                    "out", "producer q", "producer scales"),
                                   (ids, gate, off, rt, tr, aq, as_, y, out, pq, ps), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}: {name}"


def test_nvfp4_graph_replays_match_eager():
    from block_scaled_fp4_mxfp4_amd import nvfp4_gemm_nt, nvfp4_quantize
    dev = device()
    m, n, k = 256, 384, 1024
    log(f"graph: nvfp4 quantize + gemm m={m} n={n} k={k}")
    a = workloads.activation_bf16(m, k, 960, outliers=True).to(dev)
    b = workloads.gaussian_bf16((n, k), 0.02, 961).to(dev)
    bq, bs, bg = nvfp4_quantize(b)
    aq = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    ag = torch.empty((m,), dtype=torch.float32, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def step():
        nvfp4_quantize(a, aq, as_, ag)
        nvfp4_gemm_nt(aq, as_, ag, bq, bs, bg, c=c)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (aq, as_, ag, c)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (aq, as_, ag, c):
            t.view(torch.uint8).fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("q", "scales", "global scales", "c"), (aq, as_, ag, c), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}: {name}"
