"""Hadamard matrix and per-256-group row rotation (fp64).

Test infrastructure only (see the package docstring).

Source: tensai docs, "画像生成" (image generation), section "幅とメモリ"
(width and memory): weights are rotated by a Hadamard matrix on every group of
256 input columns, and the product's input gets the same rotation; rows are
treated as groups of 256 and multiplied by H once.
"""

import numpy as np

GROUP = 256


def hadamard_matrix(n=GROUP):
    """Sylvester Hadamard matrix of order n (a power of two), natural order.

    Entry (i, j) is (-1) raised to the number of bits set in (i AND j). This is
    reading R1: the pages name "a Hadamard matrix" of order 256 and nothing
    more; the Sylvester matrix in natural order is the plainest one. It is
    symmetric, so applying it to row vectors from the right or to column
    vectors from the left gives the same numbers.
    """
    if n <= 0 or (n & (n - 1)) != 0:
        raise ValueError("order must be a positive power of two")
    idx = np.arange(n, dtype=np.int64)
    both = idx[:, None] & idx[None, :]
    bits = np.zeros_like(both)
    while np.any(both):
        bits += both & 1
        both >>= 1
    return np.where(bits % 2 == 0, 1.0, -1.0)


def rotate_groups(x):
    """Return x . blockdiag(Q, Q, ...) with Q = H/16 (reading R2), in fp64.

    x: array [rows, K] (any float dtype; converted to fp64), K % 256 == 0.
    Each 256-wide group of a row is multiplied on the right by Q. Q is
    orthonormal (H H^T = 256 I) and symmetric, so rotating both operands of a
    product leaves the product unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("expected a 2-D array [rows, K]")
    rows, k = x.shape
    if k % GROUP != 0:
        raise ValueError("K must be a multiple of 256 (reading R10)")
    q = hadamard_matrix(GROUP) / 16.0
    groups = x.reshape(rows, k // GROUP, GROUP)
    return np.matmul(groups, q).reshape(rows, k)
