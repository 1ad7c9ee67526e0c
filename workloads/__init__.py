"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random BF16 operands and expert routings; it holds none
of the quantization or GEMM arithmetic, so the CPU oracle and the HIP path see
the same bytes without sharing any of the method.

Shapes follow the Llama-3-8B GEMM shapes measured on the quadbit README
("Headline result" and the real-shape table: prefill 4096^3, ffn-down
4096/4096/14336, square 8192, decode 128/14336/4096) plus a 64-expert top-4
MoE layer.  Values are Gaussian stand-ins for activations and weights:
activations ~N(0, 1) with 1% of the K channels scaled by 20 (outlier
channels), weights ~N(0, 0.02).  Every draw is a CPU torch generator seeded
per workload and role, so the same seed gives the same bytes everywhere.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch

# role offsets added to a workload's base seed
ROLE_A, ROLE_B, ROLE_OUTLIER, ROLE_ROUTE_BIAS, ROLE_ROUTE_NOISE = 0, 1, 2, 3, 4


def gaussian_bf16(shape, sigma: float, seed: int) -> torch.Tensor:
    """BF16 tensor of N(0, sigma^2) draws: fp32 randn * sigma, one RNE cast to BF16."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def outlier_channels(k: int, seed: int, frac: float = 0.01) -> torch.Tensor:
    """Indices of the round(frac * K) outlier channels, drawn by a seeded permutation."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    count = int(round(frac * k))
    return torch.randperm(k, generator=g)[:count]


def activation_bf16(rows: int, k: int, seed: int, outliers: bool, factor: float = 20.0) -> torch.Tensor:
    """Activation ~N(0,1); with outliers, the chosen K columns are multiplied by `factor` in fp32 first."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn((rows, k), generator=g, dtype=torch.float32)
    if outliers:
        ch = outlier_channels(k, seed - ROLE_A + ROLE_OUTLIER)
        x[:, ch] *= factor
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor):
    """Raw BF16 bit patterns as a numpy uint16 array (the form the oracle takes)."""
    import numpy as np
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def sha256_of(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


@dataclass
class DenseWorkload:
    name: str
    m: int
    n: int
    k: int
    seed: int
    a_outliers: bool
    b_sigma: float
    weight_prequantized: bool   # B quantized once outside the timed step

    def make(self):
        a = activation_bf16(self.m, self.k, self.seed + ROLE_A, self.a_outliers)
        b = gaussian_bf16((self.n, self.k), self.b_sigma, self.seed + ROLE_B)
        return a, b

    @property
    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


@dataclass
class MoEWorkload:
    name: str
    tokens: int
    experts: int
    top_k: int
    n: int
    k: int
    seed: int
    bias_sigma: float = 1.0
    w_sigma: float = 0.02
    extra: dict = field(default_factory=dict)

    def logits(self) -> torch.Tensor:
        """Router logits as float32 [tokens, experts]: z + beta drawn in float64
        from the seeds routing() uses, rounded once to float32 (the input of the
        on-device top-k routing)."""
        gb = torch.Generator(device="cpu").manual_seed(self.seed + ROLE_ROUTE_BIAS)
        beta = torch.randn((self.experts,), generator=gb, dtype=torch.float64) * self.bias_sigma
        gz = torch.Generator(device="cpu").manual_seed(self.seed + ROLE_ROUTE_NOISE)
        z = torch.randn((self.tokens, self.experts), generator=gz, dtype=torch.float64)
        return (z + beta[None, :]).to(torch.float32)

    def tokens_bf16(self) -> torch.Tensor:
        """The layer's token activations [tokens, K], BF16 ~N(0, 1)."""
        return gaussian_bf16((self.tokens, self.k), 1.0, self.seed + ROLE_A)

    def routing(self):
        """Top-k experts per token from Gaussian logits plus a per-expert bias.

        logits[t, e] = z[t, e] + beta[e], z ~ N(0,1), beta ~ N(0, bias_sigma^2).
        The bias makes expert loads uneven (some experts get almost no rows).
        Softmax is monotone, so ranking logits ranks the softmax probabilities;
        equal logits go to the lower expert id.  Returns (token_of_row,
        offsets): routed rows sorted by (expert, token) and the int32 [E+1]
        group offsets.
        """
        gb = torch.Generator(device="cpu").manual_seed(self.seed + ROLE_ROUTE_BIAS)
        beta = torch.randn((self.experts,), generator=gb, dtype=torch.float64) * self.bias_sigma
        gz = torch.Generator(device="cpu").manual_seed(self.seed + ROLE_ROUTE_NOISE)
        z = torch.randn((self.tokens, self.experts), generator=gz, dtype=torch.float64)
        logits = z + beta[None, :]
        # stable descending sort keeps the lower expert id first among equal logits
        order = torch.sort(logits, dim=1, descending=True, stable=True).indices[:, : self.top_k]
        tok = torch.arange(self.tokens).repeat_interleave(self.top_k)
        exp = order.reshape(-1)
        key = exp.to(torch.int64) * self.tokens + tok
        perm = torch.argsort(key)
        token_of_row = tok[perm]
        counts = torch.bincount(exp, minlength=self.experts)
        offsets = torch.zeros(self.experts + 1, dtype=torch.int32)
        offsets[1:] = torch.cumsum(counts, 0).to(torch.int32)
        return token_of_row, offsets

    def make(self):
        """(routed activation rows [tokens*top_k, K] bf16, weights [E, N, K] bf16, offsets int32 [E+1])."""
        x = gaussian_bf16((self.tokens, self.k), 1.0, self.seed + ROLE_A)
        token_of_row, offsets = self.routing()
        a = x[token_of_row].contiguous()
        w = gaussian_bf16((self.experts, self.n, self.k), self.w_sigma, self.seed + ROLE_B)
        return a, w, offsets

    @property
    def total_rows(self) -> int:
        return self.tokens * self.top_k

    @property
    def flops(self) -> int:
        return 2 * self.total_rows * self.n * self.k


TINY = DenseWorkload("tiny_64x256x1024", 64, 256, 1024, seed=100, a_outliers=False,
                     b_sigma=1.0, weight_prequantized=False)
DECODE = DenseWorkload("decode_128x14336x4096", 128, 14336, 4096, seed=200, a_outliers=True,
                       b_sigma=0.02, weight_prequantized=True)
SQUARE4096 = DenseWorkload("prefill_4096x4096x4096", 4096, 4096, 4096, seed=300, a_outliers=False,
                           b_sigma=1.0, weight_prequantized=True)
FFN_DOWN = DenseWorkload("ffn_down_4096x4096x14336", 4096, 4096, 14336, seed=400, a_outliers=True,
                         b_sigma=0.02, weight_prequantized=True)
SQUARE8192 = DenseWorkload("square_8192x8192x8192", 8192, 8192, 8192, seed=450, a_outliers=True,
                           b_sigma=0.02, weight_prequantized=True)
# the ffn-down projection at decode: 128 tokens against the 4096 x 14336 down weight
DECODE_DOWN = DenseWorkload("decode_down_128x4096x14336", 128, 4096, 14336, seed=250, a_outliers=True,
                            b_sigma=0.02, weight_prequantized=True)
MOE = MoEWorkload("moe_8192tok_top4_64x2816x4096", tokens=8192, experts=64, top_k=4,
                  n=2816, k=4096, seed=500)

DENSE = {w.name: w for w in (TINY, DECODE, SQUARE4096, FFN_DOWN, SQUARE8192, DECODE_DOWN)}
ALL = dict(DENSE, **{MOE.name: MOE})
