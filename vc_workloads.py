"""Seeded synthetic inputs for the VC-Attention hot path.

This module only draws random numbers: it holds none of the method's arithmetic,
so both the HIP path and the CPU oracle can take their inputs from it.

The pages measure on real Wan2.2 / HunyuanVideo activations under MovieGen Bench
prompts (VC-Attention paper digest, results table); neither the models nor the
prompts are available, so these seeded tensors stand in for them with the shapes
the pages give (a 5 s 720p Wan2.2-14B clip is about 70K tokens: 21x45x80 = 75600
latent tokens, d = 128, 40 heads) and with the structure the pages describe for
Value (outliers concentrated in a few tokens whose channels change per head:
"Value Is the Error Source Earlier Methods Underestimated").

Every (batch, head) slice has its own generator, seeded from (seed, b, h), so any
single head can be regenerated alone. Draws happen in float32 in a fixed order;
outliers are applied in float32; the result is rounded to bfloat16 once.
"""
from __future__ import annotations

import torch

D = 128

# workload name -> shape, value recipe, V-Smooth settings, which P paths / V formats run
WORKLOADS = {
    "tiny-8bit": dict(B=1, H=2, N=1024, seed=0, recipe="gauss",
                      k=8, iters=10, v_format="e4m3", p_modes=("expcast",)),
    "expcast-ablation": dict(B=1, H=8, N=8192, seed=1, recipe="qk_outlier",
                             k=32, iters=10, v_format="e4m3", p_modes=("fp32exp_e4m3", "expcast")),
    "wan22-attention": dict(B=1, H=40, N=75600, seed=2, recipe="clustered",
                            k=64, iters=8, v_format="e4m3", p_modes=("expcast",)),
    "wan22-vsmooth": dict(B=1, H=40, N=75600, seed=2, recipe="clustered",
                          k=64, iters=8, v_format="e4m3", p_modes=()),
    "ragged-4bit": dict(B=2, H=24, N=32760, seed=4, recipe="clustered",
                        k=64, iters=8, v_format="nvfp4", p_modes=("fp32_bf16",)),
}


def head_generator(seed: int, b: int, h: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1_000_003 + b * 10_007 + h)


def _outlier_tokens(N: int) -> int:
    return max(1, int(round(0.01 * N)))


def draw_head(recipe: str, N: int, seed: int, b: int, h: int, d: int = D):
    """Return float32 (q, k, v), each [N, d], for one (batch, head)."""
    g = head_generator(seed, b, h)
    q = torch.randn(N, d, generator=g)
    k = torch.randn(N, d, generator=g)
    if recipe == "gauss":
        v = torch.randn(N, d, generator=g)
    elif recipe == "qk_outlier":
        ch4 = torch.randperm(d, generator=g)[:4]
        q[:, ch4] *= 10.0
        k[:, ch4] *= 10.0
        v = torch.randn(N, d, generator=g)
    elif recipe == "clustered":
        centers = torch.randn(64, d, generator=g)
        labels = torch.randint(0, 64, (N,), generator=g)
        v = centers[labels] + torch.randn(N, d, generator=g)
    else:
        raise ValueError(recipe)
    ch16 = torch.randperm(d, generator=g)[:16]
    tok = torch.randperm(N, generator=g)[:_outlier_tokens(N)]
    v[tok.unsqueeze(1), ch16.unsqueeze(0)] *= 20.0
    return q, k, v


def make_inputs(name: str, heads=None, N: int | None = None):
    """bf16 CPU tensors Q, K, V of shape [B, H, N, d] for a named workload.

    heads: optional list of (b, h) to draw; the others stay zero (used to build
    sampled oracle cases without drawing the whole tensor).
    N: optional override of the sequence length (smaller parity cases).
    """
    c = WORKLOADS[name]
    B, H = c["B"], c["H"]
    n = c["N"] if N is None else N
    Q = torch.zeros(B, H, n, D, dtype=torch.bfloat16)
    K = torch.zeros_like(Q)
    V = torch.zeros_like(Q)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in todo:
        q, k, v = draw_head(c["recipe"], n, c["seed"], b, h)
        Q[b, h] = q.to(torch.bfloat16)
        K[b, h] = k.to(torch.bfloat16)
        V[b, h] = v.to(torch.bfloat16)
    return Q, K, V


def custom_inputs(B: int, H: int, N: int, seed: int, recipe: str = "clustered"):
    """Same recipes at an arbitrary shape (edge-case and ragged parity tests)."""
    Q = torch.empty(B, H, N, D, dtype=torch.bfloat16)
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    for b in range(B):
        for h in range(H):
            q, k, v = draw_head(recipe, N, seed, b, h)
            Q[b, h] = q.to(torch.bfloat16)
            K[b, h] = k.to(torch.bfloat16)
            V[b, h] = v.to(torch.bfloat16)
    return Q, K, V
