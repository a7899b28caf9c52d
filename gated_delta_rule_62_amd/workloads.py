"""Seeded synthetic inputs for the KDA prefill forward.

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  Both the GPU path and the CPU oracle consume what it
produces.  Shapes, value distributions and state setups follow the five
workloads the library is measured and checked on (head dim 128 unless stated):

  small     B=1, T=128, H=2, D=32, 16-token chunks, zero bf16 initial state
  batched   B=2, T=1024, H=96, bf16 initial state ~ N(0, 0.1^2)
  varlen3   B=1 packed lengths [300, 700, 1024], H=96, fp32 state in and out
  long      B=1, T=32768, H=96, zero initial state
  many      64 packed sequences, lengths uniform in [1, 512], H=32, bf16 state
            (the lengths from a CPU generator seeded 5, so every device draws the same
            batch: T_total 15,579, longest 496, shortest 6)

q, k, v, g and beta are N(0, 1) drawn in fp32 and rounded to bf16 (round to
nearest even); A_log ~ U(0, 1) [H]; dt_bias ~ U(0, 1) [H, D]; lower_bound = -5;
scale = 1/sqrt(D).  The draw order is: lengths, q, k, v, g, beta, A_log,
dt_bias, initial state.  Random lengths come from torch's CPU generator seeded
``length_seed``; the tensors from torch's generator seeded per workload on the
device requested (a CPU draw and a GPU draw of the same seed differ; each run
hands the same tensors to both sides).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    seed: int
    lengths: Optional[list] = None          # varlen sequence lengths (B == 1)
    n_random_seqs: int = 0                  # draw this many lengths in [1, max_len]
    max_len: int = 0
    length_seed: int = 0                    # CPU generator seed of the random lengths
    state_in: Optional[str] = "bf16"        # None | "zero_bf16" | "bf16" | "fp32"
    state_out: str = "bf16"                 # "bf16" | "fp32"
    lower_bound: float = -5.0
    chunk_size: int = 0                     # 0: the library's choice
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "small": Workload("small", B=1, T=128, H=2, D=32, seed=0, state_in="zero_bf16",
                      chunk_size=16),
    "batched": Workload("batched", B=2, T=1024, H=96, D=128, seed=1, state_in="bf16"),
    "varlen3": Workload("varlen3", B=1, T=0, H=96, D=128, seed=2, lengths=[300, 700, 1024],
                        state_in="fp32", state_out="fp32"),
    "long": Workload("long", B=1, T=32768, H=96, D=128, seed=3, state_in="zero_bf16"),
    "many": Workload("many", B=1, T=0, H=32, D=128, seed=4, n_random_seqs=64, max_len=512,
                     length_seed=5, state_in="bf16"),
}


def _bf16_normal(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None) -> dict:
    """Draws the workload's tensors on ``device``; returns a dict of kda_fwd arguments.

    Keys: q, k, v, g, beta, A_log, dt_bias, initial_state, final_state (an empty
    output buffer of the right dtype), out (empty), cu_seqlens (or None), scale,
    lower_bound, chunk_size, lengths, N, T_total.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    lengths = None
    if w.lengths is not None:
        lengths = list(w.lengths)
    elif w.n_random_seqs:
        lengths = torch.randint(1, w.max_len + 1, (w.n_random_seqs,),
                                generator=torch.Generator().manual_seed(w.length_seed)).tolist()
    if lengths is not None:
        B, T = 1, int(sum(lengths))
        N = len(lengths)
        offsets = [0]
        for n in lengths:
            offsets.append(offsets[-1] + int(n))
        cu = torch.tensor(offsets, dtype=torch.int64, device=device)
    else:
        B, T, N, cu = w.B, w.T, w.B, None
    H, D = w.H, w.D
    q = _bf16_normal(gen, (B, T, H, D), device)
    k = _bf16_normal(gen, (B, T, H, D), device)
    v = _bf16_normal(gen, (B, T, H, D), device)
    g = _bf16_normal(gen, (B, T, H, D), device)
    beta = _bf16_normal(gen, (B, T, H), device)
    A_log = torch.rand((H,), generator=gen, device=device, dtype=torch.float32)
    dt_bias = torch.rand((H, D), generator=gen, device=device, dtype=torch.float32)
    s_in = None
    if w.state_in == "zero_bf16":
        s_in = torch.zeros((N, H, D, D), dtype=torch.bfloat16, device=device)
    elif w.state_in == "bf16":
        s_in = (0.1 * torch.randn((N, H, D, D), generator=gen, device=device)).to(torch.bfloat16)
    elif w.state_in == "fp32":
        s_in = 0.1 * torch.randn((N, H, D, D), generator=gen, device=device)
    out_dtype = torch.float32 if w.state_out == "fp32" else torch.bfloat16
    return dict(
        q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias, initial_state=s_in,
        final_state=torch.empty((N, H, D, D), dtype=out_dtype, device=device),
        out=torch.empty((B, T, H, D), dtype=torch.bfloat16, device=device), cu_seqlens=cu,
        scale=1.0 / math.sqrt(D), lower_bound=w.lower_bound, chunk_size=w.chunk_size,
        lengths=lengths, N=N, T_total=B * T)


def token_heads(inputs: dict) -> int:
    """Number of (token, head) pairs of a drawn workload."""
    B, T, H, _ = inputs["q"].shape
    return B * T * H
