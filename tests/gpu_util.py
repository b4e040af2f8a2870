"""Helpers for the GPU parity tests: tensor <-> numpy conversion and the
comparison rules (bit-exact codes, scales and int32; 2e-3 relative Frobenius
for the bf16-operand products; 1e-5 relative for the W8A8 output)."""

import sys

import numpy as np
import torch

import oracle

BF16_PATH_TOL = 2e-3   # relative Frobenius, weight-only (bf16 MFMA) products
W8A8_TOL = 1e-5        # relative, elementwise, W8A8 output after scaling


def dev():
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def host(t):
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_bf16_path(got, ref, what):
    err = rel_fro(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= BF16_PATH_TOL, f"{what}: relative Frobenius error {err:.3e} > {BF16_PATH_TOL}"
    return err


def assert_w8a8_out(got, ref, what):
    scale = np.maximum(np.abs(ref), 1e-30)
    bad = np.abs(got - ref) > W8A8_TOL * scale
    assert not np.any(bad), f"{what}: {bad.sum()} outputs off by more than {W8A8_TOL} relative " \
                            f"(max rel {np.max(np.abs(got - ref) / scale):.3e})"
    err = rel_fro(got, ref)
    assert err <= W8A8_TOL
    return err


def rotation_error_bound(x64):
    """Bound on |fp32 FWHT - exact| per element: 8 butterfly stages, each
    rounding a partial sum bounded by the group's L1 norm, then the exact 1/16
    scaling: 8 * 2^-24 * sum|x| / 16 (plus the fp32 rounding of the inputs,
    which are exact here)."""
    m, k = x64.shape
    l1 = np.abs(x64).reshape(m, k // 256, 256).sum(axis=2)
    return np.repeat(8 * 2.0 ** -24 * l1 / 16.0, 256, axis=1) * 1.0001


def sample_rows(m, count, seed):
    """Rows spread over the whole range: first, last, tile boundaries, random."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, m - 1, m - 2] + [r for r in (127, 128, 255, 256, m - 129, m - 128) if 0 <= r < m]
    rand = rng.choice(m, size=min(count, m), replace=False).tolist()
    return np.array(sorted(set(fixed + rand)))
