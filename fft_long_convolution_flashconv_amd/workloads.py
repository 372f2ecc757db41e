"""Seeded synthetic inputs shaped like the H3 / FlashConv workloads.

This module only draws random numbers and fixes shapes; it holds none of the
method's arithmetic (no convolution, no FFT, no SSM filter).  Both the GPU
path and the CPU oracle consume exactly the tensors made here: every draw is
taken in fp64 from a seeded CPU ``torch.Generator`` and then rounded
(round-to-nearest-even) to the storage dtype, so both sides see identical
values.

Workloads (shapes follow the pages' model widths and lengths: width 768 and
length 1024 of the 125M model, width 2560 and length 2048 of the 2.7B model,
8K as the fused-block limit and 64K as a state-passing length):

  conv_small   fp32  B=1  H=4    N=256    random filter g*exp(-k/64)
  conv_1k      fp16  B=8  H=768  N=1024   diagonal-SSM filter, 64 modes
  conv_8k      fp16  B=4  H=768  N=8192   diagonal-SSM filter, 64 modes
  state_64k    fp16  B=2  H=1024 N=65536  chunk T=8192, 64 modes
  h3_mix_2k    bf16  B=4  N=2048 Dm=2560  shift taps L=4, 64 modes

and two more for the backward pass and generation (not among the five
parity configurations, timed beside them):

  conv_1k_bwd  fp16  B=8  H=768  N=1024   conv_1k with an upstream gradient
                                          dy ~ N(0, 1)
  decode_125m  fp16  B=64 H=768  K=1      one generated token per row from a
                                          state x ~ CN(0, 1), 64 modes (batch
                                          64 as in the pages' generation runs)
  h3_mix_mh_1k fp16  B=4  N=1024 Dm=768 dh=4  multi-head H3 mixing, heads of
                                          dimension 4, one diagonal-SSM filter
                                          per state entry
  bidir_1k     fp16  B=8  H=768  N=1024   bidirectional copies: a causal and
                                          an anti-causal diagonal-SSM filter
                                          per channel (two parameter draws)

Diagonal-SSM parameters: A_j = -0.5 + i*pi*j (j = 0..S-1), B_j = 1,
C_j ~ CN(0, 0.5) (real and imaginary parts independent N(0, 0.25)),
dt = exp(U(log 1e-3, log 1e-1)) per channel, D ~ N(0, 1) per channel.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fft_conv" | "state_pass" | "h3_mix" | "fft_conv_bwd" | "ssm_step" |
                         # "h3_mix_mh" | "fft_conv_bidir"
    dtype: str           # I/O dtype: "f32" | "f16" | "bf16"
    B: int
    N: int
    H: int = 0           # channels (fft_conv, state_pass)
    Dm: int = 0          # model width (h3_mix)
    S: int = 64          # diagonal-SSM modes
    T: int = 0           # chunk length (state_pass)
    L: int = 4           # shift-SSM taps (h3_mix)
    filt: str = "ssm"    # "ssm" | "random_env"
    seed: int = 0
    dh: int = 1          # head dimension (multi-head H3 mixing)

    @property
    def elements(self) -> int:
        return self.B * (self.H or self.Dm) * self.N


WORKLOADS = {
    "conv_small": Workload("conv_small", "fft_conv", "f32", B=1, H=4, N=256, filt="random_env", seed=0),
    "conv_1k": Workload("conv_1k", "fft_conv", "f16", B=8, H=768, N=1024, seed=1),
    "conv_8k": Workload("conv_8k", "fft_conv", "f16", B=4, H=768, N=8192, seed=2),
    "state_64k": Workload("state_64k", "state_pass", "f16", B=2, H=1024, N=65536, T=8192, seed=3),
    "h3_mix_2k": Workload("h3_mix_2k", "h3_mix", "bf16", B=4, N=2048, Dm=2560, seed=4),
    "conv_1k_bwd": Workload("conv_1k_bwd", "fft_conv_bwd", "f16", B=8, H=768, N=1024, seed=5),
    "decode_125m": Workload("decode_125m", "ssm_step", "f16", B=64, H=768, N=1, seed=6),
    "h3_mix_mh_1k": Workload("h3_mix_mh_1k", "h3_mix_mh", "f16", B=4, N=1024, Dm=768, dh=4, seed=7),
    "bidir_1k": Workload("bidir_1k", "fft_conv_bidir", "f16", B=8, H=768, N=1024, seed=8),
}


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal(shape, g: torch.Generator, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) drawn in fp64, rounded (RNE) to ``dtype``."""
    x = torch.randn(*shape, generator=g, dtype=torch.float64)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def uniform(shape, g: torch.Generator, lo: float, hi: float, dtype=torch.float64) -> torch.Tensor:
    x = torch.rand(*shape, generator=g, dtype=torch.float64)
    return (lo + (hi - lo) * x).to(dtype)


def random_env_filter(H: int, N: int, g: torch.Generator) -> torch.Tensor:
    """f[h,k] = g[h,k] * exp(-k/64), g ~ N(0,1)/sqrt(N); fp32 [H,N]."""
    gg = torch.randn(H, N, generator=g, dtype=torch.float64) / math.sqrt(N)
    env = torch.exp(-torch.arange(N, dtype=torch.float64) / 64.0)
    return (gg * env).to(torch.float32).contiguous()


def diag_ssm_params(H: int, S: int, g: torch.Generator) -> dict:
    """Diagonal complex SSM parameters, fp32; complex as interleaved [.., 2].

    A: [H,S,2] with A_j = -0.5 + i*pi*j; Bm: [H,S,2] = 1 + 0i;
    C: [H,S,2] ~ CN(0, 0.5); dt: [H] log-uniform on [1e-3, 1e-1].
    """
    j = torch.arange(S, dtype=torch.float64)
    A = torch.stack([torch.full((S,), -0.5, dtype=torch.float64), math.pi * j], dim=-1)
    A = A.unsqueeze(0).expand(H, S, 2).to(torch.float32).contiguous()
    Bm = torch.zeros(H, S, 2, dtype=torch.float32)
    Bm[..., 0] = 1.0
    C = normal((H, S, 2), g, std=0.5, dtype=torch.float32)
    dt = torch.exp(uniform((H,), g, math.log(1e-3), math.log(1e-1))).to(torch.float32)
    return {"A": A, "Bm": Bm, "C": C, "dt": dt}


def make_inputs(w: Workload, *, B: int | None = None, H: int | None = None,
                N: int | None = None, seed: int | None = None) -> dict:
    """Seeded CPU tensors for workload ``w`` (shape overrides for tests)."""
    B = w.B if B is None else B
    N = w.N if N is None else N
    seed = w.seed if seed is None else seed
    g = gen(seed)
    io = DTYPES[w.dtype]
    if w.kind == "fft_conv":
        H = w.H if H is None else H
        out = {"u": normal((B, H, N), g, dtype=io)}
        if w.filt == "random_env":
            out["f"] = random_env_filter(H, N, g)
        else:
            out.update(diag_ssm_params(H, w.S, g))
        out["D"] = normal((H,), g, dtype=torch.float32)
        return out
    if w.kind == "fft_conv_bidir":
        # causal filter from (A, Bm, C, dt), anti-causal from (gA, gBm, gC, gdt)
        H = w.H if H is None else H
        out = {"u": normal((B, H, N), g, dtype=io)}
        out.update(diag_ssm_params(H, w.S, g))
        out.update({"g" + k: v for k, v in diag_ssm_params(H, w.S, g).items()})
        out["D"] = normal((H,), g, dtype=torch.float32)
        return out
    if w.kind == "fft_conv_bwd":
        H = w.H if H is None else H
        out = {"u": normal((B, H, N), g, dtype=io)}
        out.update(diag_ssm_params(H, w.S, g))
        out["D"] = normal((H,), g, dtype=torch.float32)
        out["dy"] = normal((B, H, N), g, dtype=io)
        return out
    if w.kind == "ssm_step":
        H = w.H if H is None else H
        out = {"u": normal((B, H, N), g, dtype=io)}
        out.update(diag_ssm_params(H, w.S, g))
        out["D"] = normal((H,), g, dtype=torch.float32)
        out["x"] = normal((B, H, w.S, 2), g, std=math.sqrt(0.5), dtype=torch.float32)
        return out
    if w.kind == "state_pass":
        H = w.H if H is None else H
        out = {"u": normal((B, H, N), g, dtype=io)}
        out.update(diag_ssm_params(H, w.S, g))
        out["D"] = normal((H,), g, dtype=torch.float32)
        return out
    if w.kind == "h3_mix_mh":
        Dm = w.Dm if H is None else H
        out = {
            "q": normal((B, N, Dm), g, dtype=io),
            "k": normal((B, N, Dm), g, dtype=io),
            "v": normal((B, N, Dm), g, dtype=io),
            "w": normal((Dm, w.L), g, std=0.5, dtype=torch.float32),
        }
        out.update(diag_ssm_params(Dm * w.dh, w.S, g))
        out["D"] = normal((Dm * w.dh,), g, dtype=torch.float32)
        return out
    if w.kind == "h3_mix":
        Dm = w.Dm if H is None else H
        out = {
            "q": normal((B, N, Dm), g, dtype=io),
            "k": normal((B, N, Dm), g, dtype=io),
            "v": normal((B, N, Dm), g, dtype=io),
            "w": normal((Dm, w.L), g, std=0.5, dtype=torch.float32),
        }
        out.update(diag_ssm_params(Dm, w.S, g))
        out["D"] = normal((Dm,), g, dtype=torch.float32)
        return out
    raise ValueError(w.kind)
