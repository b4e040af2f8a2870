"""A LoRA side path beside a projection (fp64).

Test infrastructure only (see the package docstring).

Source: kvad-gpu internals ("kvad-gpu — the same model, handed to a
framework"), section "Pictures, which are not tokens": each LoRA is a side
path (x.A).B beside the layer it adapts, with a strength chosen per request,
added into the layer's output when the output is stored; the loaded model
itself is left as it was.

Reading (also in the design notes):
  R21 With the usual (PEFT) layouts, lora_A [r, K] and lora_B [N, r], the
      side path adds alpha * (x . A^T) . B^T to the layer's output
      [M, N], x being the layer's activations in the caller's domain. The
      rotation leaves it unchanged when x and A are rotated alike
      ((x Q)(A Q)^T = x A^T), so a caller that passes rotated activations
      passes A rotated too.
"""

import numpy as np


def lora_delta(x, a, b, alpha):
    """alpha * (x . a^T) . b^T in fp64 ([M, N])."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(alpha) * np.matmul(np.matmul(x, a.T), b.T)


def lora_add(c, x, a, b, alpha):
    """c + alpha * (x . a^T) . b^T in fp64 (R21)."""
    return np.asarray(c, dtype=np.float64) + lora_delta(x, a, b, alpha)
