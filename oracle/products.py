"""The three rotated, quantized products (fp64 / exact integer).

Test infrastructure only (see the package docstring).

Source: tensai docs, "画像生成" (image generation), section "幅とメモリ"
(width and memory): because the per-group rotation is orthogonal, multiplying
the rotated input by the rotated weight gives the original product up to
quantization error; section "GPU": the device quantizes each product's
activations (reading R9 for W8A8). The same section's 4-bit width ("-q4"),
combined with those device-quantized activations, gives W4A8 (reading R18).
"""

import numpy as np

from .hadamard import rotate_groups
from .quantize import (
    bf16_round,
    dequantize_int4,
    dequantize_int8,
    quantize_activations_int8,
    unpack_int4,
)


def _rotated_bf16(x, rotate):
    xr = rotate_groups(x) if rotate else np.asarray(x, dtype=np.float64)
    return bf16_round(xr)


def qgemm_w8(x, q, s, rotate=True):
    """Weight-only int8 product Y = bf16(X') . (q * s[n])^T in fp64 (R8).

    x: [M, K] activations (rotated here unless rotate is False);
    q: int8 [N, K]; s: fp32 [N]. Returns fp64 [M, N].
    """
    xb = _rotated_bf16(x, rotate)
    return np.matmul(xb, dequantize_int8(q, s).T)


def qgemm_w4(x, packed, s, rotate=True):
    """Weight-only int4 product Y = bf16(X') . (q * s[n, g])^T in fp64 (R8).

    packed: uint8 [N, K/2]; s: fp32 [N, K/256]. Returns fp64 [M, N].
    """
    xb = _rotated_bf16(x, rotate)
    return np.matmul(xb, dequantize_int4(packed, s).T)


def int_accumulate(qa, q):
    """Exact integer accumulator ACC[m, n] = sum_k qa[m, k] * q[n, k] (int64).

    Computed with an fp64 matrix product, which is exact because every partial
    sum is an integer below 127^2 * K < 2^53 for the K allowed here.
    """
    qa = np.asarray(qa, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    k = qa.shape[1]
    if 127 * 127 * k >= 2 ** 53:
        raise ValueError("K too large for an exact fp64 integer product")
    acc = np.matmul(qa.astype(np.float64), q.astype(np.float64).T)
    return np.rint(acc).astype(np.int64)


def qgemm_w8a8(x, q, sw, rotate=True):
    """W8A8 product (reading R9).

    The rotated activations get per-row int8 codes qa and scales sa; the int32
    accumulator is the exact integer product; the output is acc * sa[m] * sw[n]
    in fp64. Returns (y fp64 [M, N], acc int64 [M, N], qa int8 [M, K],
    sa fp32 [M]).
    """
    qa, sa = quantize_activations_int8(x, rotate=rotate)
    acc = int_accumulate(qa, q)
    y = acc.astype(np.float64) * sa.astype(np.float64)[:, None] * np.asarray(sw, dtype=np.float64)[None, :]
    return y, acc, qa, sa


def group_accumulate(qa, q, group=256):
    """Exact integer accumulators per K-group, ACC[g, m, n] = sum over k in
    group g of qa[m, k] * q[n, k] (int64, [K/group, M, N])."""
    qa = np.asarray(qa)
    q = np.asarray(q)
    k = qa.shape[1]
    return np.stack([int_accumulate(qa[:, g:g + group], q[:, g:g + group]) for g in range(0, k, group)])


def qgemm_w4a8(x, packed, s, rotate=True):
    """W4A8 product (reading R18): per-row int8 activations as in W8A8 (R9),
    int4 weights with one scale per (row, 256-group) (R3, R6, R7):

        y[m, n] = sa[m] * sum_g s[n, g] * ACC[g, m, n]

    with ACC the exact per-group integer accumulators, in fp64. Returns
    (y fp64 [M, N], acc int64 [K/256, M, N], qa int8 [M, K], sa fp32 [M]).
    """
    qa, sa = quantize_activations_int8(x, rotate=rotate)
    q = unpack_int4(packed)
    acc = group_accumulate(qa, q)
    sg = np.asarray(s, dtype=np.float64).T  # [G, N]
    y = np.einsum("gmn,gn->mn", acc.astype(np.float64), sg) * sa.astype(np.float64)[:, None]
    return y, acc, qa, sa
