"""Seeded synthetic inputs for PaTH attention.

This module only draws random tensors; it holds none of the attention
arithmetic. Both the HIP path and the CPU oracle are fed from here, so the
two sides see bit-identical (already rounded) inputs.

Recipe (the workload shapes and distributions of the PaTH configurations):
  * numpy ``default_rng(seed)``, float64 draws in this fixed order:
      q, k, v      ~ N(0, 1), shape [B, H, L_total, d] each
      w            ~ N(0, 1), then every row divided by its L2 norm
      beta         = 2 * sigmoid(N(0, 1)), shape [B, H, L_total];
                     clipped to [0.02, 1.98] for bf16 configurations
      log_f        = logsigmoid(3 + N(0, 1)) (FoX configurations only)
  * then q, k, v, w are rounded (round-to-nearest-even) to the compute dtype;
    beta and log_f are stored as float32.

The pages define beta_t = 2 * sigmoid(u^T x_t + b) in (0, 2) and w_t as an
L2-normalised projection of x_t (PaTH paper notes, "key design" section); the
synthetic draws stand in for those trained projections.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class PathConfig:
    name: str
    B: int
    H: int
    L: int              # prefill length
    d: int
    dtype: str          # "f32" or "bf16"
    gate: bool          # FoX forget gate present
    seed: int
    chunk: int = 64
    decode_steps: int = 0
    clip_beta: bool = True

    @property
    def L_total(self) -> int:
        return self.L + self.decode_steps

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workload configurations (tiny fp32 check, bf16 1K, FoX 4K ~760M
# layer shape, FoX 16K long context, d=128 prefill + 256 decode steps).
CONFIGS = {
    "tiny_f32": PathConfig("tiny_f32", 1, 1, 64, 16, "f32", False, 0, chunk=16,
                           clip_beta=False),
    "bf16_L1k": PathConfig("bf16_L1k", 2, 8, 1024, 64, "bf16", False, 1),
    "fox_L4k": PathConfig("fox_L4k", 8, 24, 4096, 64, "bf16", True, 2),
    "fox_L16k": PathConfig("fox_L16k", 1, 16, 16384, 64, "bf16", True, 3),
    "d128_L8k_decode": PathConfig("d128_L8k_decode", 2, 32, 8192, 128, "bf16",
                                  False, 4, decode_steps=256),
    # beyond the five: the same prefill + decode shape with the PaTH-FoX gate
    "fox_d128_L8k_decode": PathConfig("fox_d128_L8k_decode", 2, 32, 8192, 128, "bf16",
                                      True, 5, decode_steps=256),
}


@dataclasses.dataclass
class PathInputs:
    """CPU tensors. q/k/v/w: [B,H,L_total,d] in the config dtype; beta and
    log_f (or None): [B,H,L_total] float32."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    w: torch.Tensor
    beta: torch.Tensor
    log_f: torch.Tensor | None


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _logsigmoid(x):
    # log(sigmoid(x)) = -log1p(exp(-x)), written to stay finite for x << 0
    return -np.logaddexp(0.0, -x)


def generate(B, H, L_total, d, *, dtype="bf16", gate=False, seed=0,
             clip_beta=True) -> PathInputs:
    rng = np.random.default_rng(seed)
    shape = (B, H, L_total, d)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    w = rng.standard_normal(shape)
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    beta = 2.0 * _sigmoid(rng.standard_normal((B, H, L_total)))
    if clip_beta:
        beta = np.clip(beta, 0.02, 1.98)
    log_f = None
    if gate:
        log_f = _logsigmoid(3.0 + rng.standard_normal((B, H, L_total)))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16

    def cast(a):
        return torch.from_numpy(a).to(tdt).contiguous()

    return PathInputs(
        q=cast(q), k=cast(k), v=cast(v), w=cast(w),
        beta=torch.from_numpy(beta).to(torch.float32).contiguous(),
        log_f=None if log_f is None
        else torch.from_numpy(log_f).to(torch.float32).contiguous(),
    )


def generate_config(cfg: PathConfig, *, B=None, H=None) -> PathInputs:
    """Inputs for a named configuration (optionally with fewer heads: the
    draws are then those of a smaller tensor, not a slice of the full one)."""
    return generate(B or cfg.B, H or cfg.H, cfg.L_total, cfg.d,
                    dtype=cfg.dtype, gate=cfg.gate, seed=cfg.seed,
                    clip_beta=cfg.clip_beta)


# ---------------------------------------------------------------------------
# Transition-parameter inputs: the layer input x and the weights of the
# low-rank map, the short convolution and the beta projection.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TransitionConfig:
    name: str
    B: int
    L: int
    Dm: int             # layer width
    r: int              # rank of the low-rank map
    H: int
    d: int
    seed: int


# The ~760M layer shape (width 1536 = 24 heads x 64) at 4K tokens; the rank
# of the low-rank map is not given on the pages, 64 is taken here.
TRANSITION_CONFIGS = {
    "transition_L4k": TransitionConfig("transition_L4k", 8, 4096, 1536, 64, 24, 64, 6),
}


@dataclasses.dataclass
class TransitionInputs:
    """CPU tensors: x [B,L,Dm], w_down [r,Dm], w_up [H*d,r], u [H,Dm] in bf16;
    conv [H*d,3] and b [H] float32."""
    x: torch.Tensor
    w_down: torch.Tensor
    w_up: torch.Tensor
    conv: torch.Tensor
    u: torch.Tensor
    b: torch.Tensor


def generate_transition(B, L, Dm, r, H, d, *, seed=0) -> TransitionInputs:
    """float64 draws in this order, then rounded: x ~ N(0,1); w_down ~
    N(0,1)/sqrt(Dm); w_up ~ N(0,1)/sqrt(r); conv ~ N(0,1)/sqrt(3);
    u ~ N(0,1)/sqrt(Dm); b ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, Dm))
    w_down = rng.standard_normal((r, Dm)) / math.sqrt(Dm)
    w_up = rng.standard_normal((H * d, r)) / math.sqrt(r)
    conv = rng.standard_normal((H * d, 3)) / math.sqrt(3.0)
    u = rng.standard_normal((H, Dm)) / math.sqrt(Dm)
    b = rng.standard_normal(H)

    def bf(a):
        return torch.from_numpy(a).to(torch.bfloat16).contiguous()

    def f32(a):
        return torch.from_numpy(a).to(torch.float32).contiguous()

    return TransitionInputs(x=bf(x), w_down=bf(w_down), w_up=bf(w_up), conv=f32(conv),
                            u=bf(u), b=f32(b))
