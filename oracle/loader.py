"""Undoing a rotated, quantized weight, and requantizing it (fp64).

Test infrastructure only (see the package docstring).

Source: tensai docs, "画像生成" (image generation), section
"チェックポイントの入手" (getting the checkpoints): the ComfyUI int8 files hold
weights rotated per 256 input columns and then stored as int8 with one scale
per row; the loader undoes both steps and applies its own quantization, so
either checkpoint runs through the same code.

Readings (also in the design notes):
  R19 Undoing the two steps: W_hat = (q * s) . blockdiag(Q). Q = H/16 is
      symmetric and orthogonal, so it is its own inverse; the un-rotation is
      the same transform as the rotation. In fp64 it is exact: the values of a
      group share one scale, so every output is (an integer of at most 2^15
      in magnitude) * s / 16.
  R20 Requantizing to another width: rotating W_hat again gives back q * s
      exactly, so "undo, then quantize" is quantizing q * s in the rotated
      domain (no transform), with the rules of R3-R7.
"""

import numpy as np

from .hadamard import rotate_groups
from .quantize import dequantize_int4, dequantize_int8, quantize_weights_int4, quantize_weights_int8


def dequantize(q, s, bits):
    """q * s in the rotated domain (fp64, exact): int8 codes with per-row
    scales (bits 8) or packed int4 codes with per-(row, group) scales (bits 4)."""
    if bits == 8:
        return dequantize_int8(q, s)
    if bits == 4:
        return dequantize_int4(q, s)
    raise ValueError("bits must be 8 or 4")


def dequantize_unrotate(q, s, bits):
    """W_hat = (q * s) . blockdiag(Q) (R19), fp64."""
    return rotate_groups(dequantize(q, s, bits))


def requantize(q, s, bits_in, bits_out):
    """Codes and scales of width bits_out for the weight held as (q, s) of
    width bits_in (R20): quantize(rotate(dequantize_unrotate(...))), which is
    quantizing q * s without a transform."""
    wr = dequantize(q, s, bits_in)
    if bits_out == 8:
        return quantize_weights_int8(wr, rotate=False)
    if bits_out == 4:
        return quantize_weights_int4(wr, rotate=False)
    raise ValueError("bits must be 8 or 4")
