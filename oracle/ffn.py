"""The FFN middle that feeds a down projection (fp64).

Test infrastructure only (see the package docstring).

Sources:
* tensai docs, "画像生成" (image generation), section "何が走るか" (what runs):
  every transformer block is attention followed by a SwiGLU feed-forward.
* same page, section "幅とメモリ" (width and memory): the input of each
  product is rotated per 256 columns on the device before it is used.
* TensorFold pull request #948, first comment: the activations between
  operations are kept in bf16.

Readings (also in the design notes):
  R15 SwiGLU(g, u) = silu(g) * u with silu(x) = x / (1 + e^-x) (the pages name
      SwiGLU without defining it; this is its usual definition). The hidden
      activation h is a bf16 tensor: the real value silu(g) * u, rounded once
      to bf16 (nearest, ties to even). Here the real value is taken as its
      fp64 evaluation, which differs from it by about 2^-52 relative, far
      below any bf16 rounding decision on the inputs used.
  R16 The down projection's input is h, treated exactly like any other
      activation: rotated per 256-group, then per-row int8 (W8A8) or rounded
      to bf16 after the rotation (W8 / W4).
"""

import numpy as np

from .hadamard import rotate_groups
from .quantize import bf16_round, quantize_activations_int8


def silu_mul(g, u):
    """silu(g) * u = g * u / (1 + exp(-g)) in fp64 (not rounded)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        return (g * u) / (1.0 + np.exp(-g))


def swiglu_bf16(g, u):
    """h = bf16(silu(g) * u) (R15), returned as fp64 holding bf16 values."""
    return bf16_round(silu_mul(g, u))


def ffn_middle_int8(g, u):
    """Rotated, per-row int8 down-projection input from gate and up (R15, R16):
    (codes int8 [M, K], scales fp32 [M])."""
    return quantize_activations_int8(swiglu_bf16(g, u), rotate=True)


def ffn_middle_rotated(g, u):
    """Rotated h in fp64, before any rounding of the output (R15, R16)."""
    return rotate_groups(swiglu_bf16(g, u))
