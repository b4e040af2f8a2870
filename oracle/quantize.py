"""Weight and activation quantization, int4 packing, bf16 rounding (fp64).

Test infrastructure only (see the package docstring).

Sources:
* tensai docs, "画像生成" (image generation), section "幅とメモリ" (width and
  memory): weights are quantized while loading, 8-bit by default and 4-bit
  with "-q4"; after the per-256-column Hadamard rotation the int8 weights carry
  one scale per row.
* same page, section "GPU": the device quantizes each product's activations
  more finely than the CPU path (reading R9: per-token symmetric int8).
* TensorPencil README, model-format table: the "INT8 ConvRot" and
  "INT4 ConvRot" formats (names only; the layout is readings R3, R6, R7).
"""

import numpy as np

from .hadamard import GROUP, rotate_groups

INT8_QMAX = 127
INT4_QMAX = 7


def bf16_round(x):
    """Round fp64 values to the nearest bfloat16 value, ties to even (R8).

    bfloat16 keeps 8 significant bits and fp32's exponent range. The result is
    returned as fp64 (every bf16 value is exact in fp64). Rounding is done once,
    straight from fp64, so there is no double rounding through fp32.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)  # xf = m * 2**e with 0.5 <= |m| < 1
    # bf16 normals start at 2**-126, i.e. e >= -125; below that the spacing
    # is fixed at the subnormal quantum 2**-133.
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    r = np.rint(xf / quantum) * quantum
    bf16_max = np.ldexp(2.0 - 2.0 ** -7, 127)
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def _codes(xr, scale, qmax):
    """Symmetric codes rint(x / s) clamped to [-qmax, qmax]; zero where s == 0.

    xr: fp64 values; scale: fp32 scales broadcastable to xr. The division uses
    the stored fp32 scale widened to fp64 (reading R4) and rounds half to even.
    """
    s64 = np.broadcast_to(np.asarray(scale, dtype=np.float32).astype(np.float64), xr.shape)
    q = np.zeros(xr.shape, dtype=np.float64)
    nz = s64 > 0
    q[nz] = np.rint(xr[nz] / s64[nz])
    return np.clip(q, -qmax, qmax).astype(np.int64)


def _scale(amax, qmax):
    """fp32(amax / qmax): fp64 division, then one rounding to fp32 (R4)."""
    return (np.asarray(amax, dtype=np.float64) / float(qmax)).astype(np.float32)


def quantize_weights_int8(w, rotate=True):
    """Rotate W [N, K] per 256-group, then per-row symmetric int8 (R3, R7).

    Returns (q int8 [N, K], s fp32 [N]) with q = clamp(rint(W'/s), -127, 127),
    s = fp32(max_k |W'[n, k]| / 127), W' = W . blockdiag(H/16). With
    rotate=False, W is taken as already rotated (W' = W).
    """
    wr = rotate_groups(w) if rotate else np.asarray(w, dtype=np.float64)
    s = _scale(np.max(np.abs(wr), axis=1), INT8_QMAX)
    q = _codes(wr, s[:, None], INT8_QMAX)
    return q.astype(np.int8), s


def quantize_weights_int4(w, rotate=True):
    """Rotate W [N, K] per 256-group, then int4 with one scale per (row, group).

    Returns (packed uint8 [N, K/2], s fp32 [N, K/256]): codes are
    clamp(rint(W'/s), -7, 7) with s = fp32(max |W'| over the group / 7), packed
    two per byte (R6). With rotate=False, W is taken as already rotated.
    """
    wr = rotate_groups(w) if rotate else np.asarray(w, dtype=np.float64)
    n, k = wr.shape
    g = wr.reshape(n, k // GROUP, GROUP)
    s = _scale(np.max(np.abs(g), axis=2), INT4_QMAX)
    q = _codes(g, s[:, :, None], INT4_QMAX).reshape(n, k)
    return pack_int4(q), s


def quantize_activations_int8(x, rotate=True):
    """Per-token (per-row) int8 of the rotated activations (reading R9).

    x: [M, K]. If rotate is False, x is taken as already rotated.
    Returns (qa int8 [M, K], sa fp32 [M]).
    """
    xr = rotate_groups(x) if rotate else np.asarray(x, dtype=np.float64)
    sa = _scale(np.max(np.abs(xr), axis=1), INT8_QMAX)
    qa = _codes(xr, sa[:, None], INT8_QMAX)
    return qa.astype(np.int8), sa


def pack_int4(q):
    """Pack int codes in [-8, 7] two per byte: even column in the low nibble (R6)."""
    q = np.asarray(q, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("need an even number of columns")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(p):
    """Inverse of pack_int4: bytes [.., K/2] -> int64 codes [.., K]."""
    p = np.asarray(p, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize_int8(q, s):
    """W'_hat[n, k] = q[n, k] * s[n], exact in fp64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[:, None]


def dequantize_int4(packed, s):
    """W'_hat[n, k] = q[n, k] * s[n, k // 256], exact in fp64."""
    q = unpack_int4(packed).astype(np.float64)
    s64 = np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1)
    return q * s64
