"""Seeded synthetic inputs for the GEMM -> residual -> RMSNorm -> GEMM chain.

This module is shared by the oracle tests and the HIP-path tests/bench. It draws
random tensors and nothing else: it holds none of the chain's arithmetic.

Recipe (the pages use Llama-3-style layer shapes, no dataset; CODA: Rewriting
Transformer Blocks as GEMM-Epilogue Programs, hotdry blog, "performance
expectations" paragraph, and the kucoin article, "experimental results"):

* every tensor has its own CPU ``torch.Generator`` seeded ``seed*100 + id``
  with ids x=1, W0=2, z=3, gamma=4, W1=5, dY=6 (row sample 7, dgamma column
  sample 8, dW1 column sample 9), and for the backward through the first GEMM
  dh=10 (dW0 column sample 11), and for the SwiGLU block's output projection
  W2=12, dOut=13 (dW2 column sample 14), and for the cross-entropy LM head
  h=15, W=16, targets=17, dloss=18, ignored rows=19 (dW row sample 20);
* each draw is fp32 ``randn`` scaled and then cast to bfloat16 (round to
  nearest even): x, z, dY, dh, dOut ~ N(0, 1); W0 ~ N(0, 1/K0); W1 ~ N(0, 1/D);
  W2 ~ N(0, 1/F) (fan-in = rows of the ``[in, out]`` weight); gamma = 1 + 0.1 N(0, 1);
* LM head: h ~ N(0, 1) (a normalised hidden state), W [V, D] ~ N(0, 4/D) (logits
  of standard deviation 2: a peaked softmax), targets uniform in [0, V) with about
  3 % of the rows set to -100 (ignored), dloss ~ N(0, 1) fp32 per row;
* for the largest row count and the widest D or N, a backward saved set drawn directly
  (ids h=21, g=22, y=23, r=24): h, g ~ N(0, 2) and y ~ N(0, 1) in bf16, r ~ U(0.5, 1)
  in fp32; tensors of 2^30 elements are drawn by a seeded generator on the device;
* eps = 1e-5.

W1's columns are read as interleaved gate/up pairs (column 2f = gate f,
column 2f+1 = up f); for independent draws that is only a relabelling.
"""
from __future__ import annotations

import math

import torch

EPS = 1e-5

IDS = {"x": 1, "W0": 2, "z": 3, "gamma": 4, "W1": 5, "dY": 6,
       "rows": 7, "dgamma_cols": 8, "dw1_cols": 9, "dh": 10, "dw0_cols": 11,
       "W2": 12, "dOut": 13, "dw2_cols": 14,
       "h_lm": 15, "W_lm": 16, "targets": 17, "dloss": 18, "ignored": 19, "dw_lm_rows": 20,
       # the largest-row-count case: the backward's saved set drawn directly (not from a forward)
       "h_s": 21, "g_s": 22, "y_s": 23, "r_s": 24}

# name -> (M tokens, K0, D, N = 2 * ffn); the LM head of each model has V = 128256 outputs
LM_VOCAB = 128256
CONFIGS = {
    "tiny": dict(M=64, K0=256, D=256, N=512),
    "llama3_1b": dict(M=8192, K0=2048, D=2048, N=16384),
    "llama3_8b": dict(M=8192, K0=4096, D=4096, N=28672),
    "llama3_70b": dict(M=8192, K0=8192, D=8192, N=57344),
    # one GPU's share of the 8B batch under 8-way data parallelism
    "llama3_8b_dp8": dict(M=1024, K0=4096, D=4096, N=28672),
}


def generator(seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 100 + IDS[name])
    return g


def device_randn_bf16(shape, seed: int, name: str, device, scale: float = 1.0, shift: float = 0.0) -> torch.Tensor:
    """The same recipe drawn by a generator on ``device`` (for tensors too large to draw on the host;
    its stream differs from the host generator's)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed * 100 + IDS[name])
    return (torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * scale + shift).to(torch.bfloat16)


def device_uniform_f32(shape, seed: int, name: str, device, lo: float, hi: float) -> torch.Tensor:
    """Seeded fp32 U(lo, hi) drawn on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed * 100 + IDS[name])
    return torch.rand(*shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def _randn_bf16(shape, seed, name, scale=1.0, shift=0.0):
    t = torch.randn(*shape, generator=generator(seed, name), dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    if shift != 0.0:
        t.add_(shift)
    return t.to(torch.bfloat16)


def forward_inputs(M: int, K0: int, D: int, N: int, seed: int = 0) -> dict:
    """x [M,K0], W0 [K0,D], z [M,D], gamma [D], W1 [D,N]; bf16, CPU, row-major."""
    return {
        "x": _randn_bf16((M, K0), seed, "x"),
        "W0": _randn_bf16((K0, D), seed, "W0", scale=1.0 / math.sqrt(K0)),
        "z": _randn_bf16((M, D), seed, "z"),
        "gamma": _randn_bf16((D,), seed, "gamma", scale=0.1, shift=1.0),
        "W1": _randn_bf16((D, N), seed, "W1", scale=1.0 / math.sqrt(D)),
    }


def output_grad(M: int, N: int, seed: int = 0) -> torch.Tensor:
    """dY [M,N] bf16 ~ N(0,1)."""
    return _randn_bf16((M, N), seed, "dY")


def upstream_grad(M: int, D: int, seed: int = 0) -> torch.Tensor:
    """dh [M,D] bf16 ~ N(0,1): a gradient of h for the backward through the first GEMM."""
    return _randn_bf16((M, D), seed, "dh")


def swiglu_inputs(M: int, N: int, E: int, seed: int = 0) -> dict:
    """Output projection of the SwiGLU block: W2 [N/2, E] bf16 ~ N(0, 2/N) and its
    upstream gradient dOut [M, E] bf16 ~ N(0, 1)."""
    F = N // 2
    return {"W2": _randn_bf16((F, E), seed, "W2", scale=1.0 / math.sqrt(F)),
            "dOut": _randn_bf16((M, E), seed, "dOut")}


def lm_head_inputs(M: int, D: int, V: int, seed: int = 0) -> dict:
    """h [M, D] bf16, W [V, D] bf16, targets [M] int64 (about 3 % = -100), dloss [M] fp32."""
    t = torch.randint(0, V, (M,), generator=generator(seed, "targets"), dtype=torch.int64)
    ign = torch.rand(M, generator=generator(seed, "ignored")) < 0.03
    t[ign] = -100
    return {"h": _randn_bf16((M, D), seed, "h_lm"),
            "W": _randn_bf16((V, D), seed, "W_lm", scale=2.0 / math.sqrt(D)),
            "targets": t,
            "dloss": torch.randn(M, generator=generator(seed, "dloss"), dtype=torch.float32)}


def sample(n: int, count: int, seed: int, name: str) -> torch.Tensor:
    """Sorted seeded sample of ``count`` distinct indices in [0, n) (all of them if count >= n)."""
    if count >= n:
        return torch.arange(n)
    return torch.randperm(n, generator=generator(seed, name))[:count].sort().values
