"""LoRA side path (tp_lora_add) vs the CPU oracle.

The device works in fp32: T = X . A^T summed over k in order, then
C + alpha * T . B^T summed over the rank in order, rounded once to C's dtype.
The gate is that arithmetic's error bound, element by element, from the
oracle's exact pieces: |dT| <= k 2^-24 (|X| . |A|^T), and
|dC| <= |alpha| (|dT| . |B|^T + (r + 1) 2^-24 |T| . |B|^T) + 2^-24 |C_new|
(+ a bf16 rounding of C_new for bf16 C).
"""

import numpy as np
import pytest
import torch

import int4_quantized_gemm_amd as tp
import oracle
import workloads as W
from tests.gpu_util import announce, dev, f64, host, sample_rows

pytestmark = pytest.mark.gpu


def _lora_inputs(m, n, k, r, seed, xd="bf16", abd="bf16", cd="f32"):
    x = W.random_rows((m, k), seed=seed, dtype=xd)
    a = W.random_rows((r, k), seed=seed + 1, dtype=abd, scale=0.02)
    b = W.random_rows((n, r), seed=seed + 2, dtype=abd, scale=0.02)
    c = W.random_rows((m, n), seed=seed + 3, dtype=cd)
    return x, a, b, c


def _padded_b(b, d):
    """lora_b on the device with 16-byte aligned rows (a padded view)."""
    n, r = b.shape
    per = 16 // b.element_size()
    buf = torch.zeros((n, (r + per - 1) // per * per), dtype=b.dtype, device=d)
    buf[:, :r] = b.to(d)
    return buf[:, :r]


def _check(got, c0, x, a, b, alpha, bf16_out=False):
    x64, a64, b64, c64 = f64(x), f64(a), f64(b), f64(c0)
    ref = oracle.lora_add(c64, x64, a64, b64, alpha)
    k, r = x64.shape[1], a64.shape[0]
    t = x64 @ a64.T
    dt = k * 2.0 ** -24 * (np.abs(x64) @ np.abs(a64).T)
    bound = abs(alpha) * (dt @ np.abs(b64).T + (r + 1) * 2.0 ** -24 * (np.abs(t) @ np.abs(b64).T))
    bound = bound * 1.01 + 2.0 ** -24 * np.abs(ref) * 1.01 + 1e-30
    if bf16_out:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(f64(got) - ref)
    bad = err > bound
    assert not np.any(bad), f"{int(bad.sum())} outside the fp32 bound (max ratio {float(np.max(err / bound)):.2f})"


@pytest.mark.parametrize("xd,abd,cd", [("bf16", "bf16", "f32"), ("f32", "f32", "f32"), ("bf16", "f32", "bf16"),
                                        ("f32", "bf16", "bf16")])
@pytest.mark.parametrize("m,n,k,r", [(1, 256, 256, 1), (37, 300, 768, 7), (100, 513, 1024, 32), (64, 1000, 3072, 64)])
def test_lora_add(xd, abd, cd, m, n, k, r):
    d = dev()
    announce("tp_lora_add", xd, abd, cd, m, n, k, r)
    x, a, b, c = _lora_inputs(m, n, k, r, seed=m + n + r, xd=xd, abd=abd, cd=cd)
    cd_ = c.to(d)
    tp.tp_lora_add(cd_, x.to(d), a.to(d), _padded_b(b, d), 0.8)
    _check(cd_, c, x, a, b, 0.8, bf16_out=cd == "bf16")


def test_lora_on_a_projection_output():
    """A rank-32 LoRA beside the W8A8 qkv projection at full size: the product's
    output, then the side path added in place (sampled rows checked; the side
    path of the other rows must not touch them twice)."""
    d = dev()
    wl = W.DIT_QKV
    announce("W8A8 qkv + LoRA rank 32", wl.m, wl.k, wl.n)
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    xd = x.to(d)
    y = tp.tp_qgemm_w8a8(xd, q, s)
    y0 = y.clone()
    _, a, b, _ = _lora_inputs(1, wl.n, wl.k, 32, seed=7)
    tp.tp_lora_add(y, xd, a.to(d), _padded_b(b, d), 1.25)
    sel = np.arange(0, wl.m, 97)
    _check(y[sel], y0[sel], x[sel], a, b, 1.25)


def test_lora_rotated_domain_and_views():
    """Rotated activations with a rotated lora_a give the same side path
    (within the fp32 bounds of both), on padded views."""
    d = dev()
    announce("tp_lora_add rotated domain, padded views")
    m, n, k, r = 48, 640, 1536, 16
    x, a, b, c = _lora_inputs(m, n, k, r, seed=21, xd="f32", abd="f32", cd="f32")
    xr = tp.tp_hadamard_rotate_rows(x.to(d))
    ar = tp.tp_hadamard_rotate_rows(a.to(d))
    cbuf = torch.full((m + 2, n + 8), 4.0, dtype=torch.float32, device=d)
    cbuf[1:1 + m, 4:4 + n] = c.to(d)
    view = cbuf[1:1 + m, 4:4 + n]
    tp.tp_lora_add(view, xr, ar, _padded_b(b, d), -0.5)
    ref = oracle.lora_add(f64(c), f64(x), f64(a), f64(b), -0.5)
    assert np.allclose(f64(view), ref, rtol=1e-4, atol=1e-5)
    assert torch.all(cbuf[0] == 4.0) and torch.all(cbuf[-1] == 4.0)
    assert torch.all(cbuf[:, :4] == 4.0) and torch.all(cbuf[:, 4 + n:] == 4.0)


@pytest.mark.parametrize("cd,off,pad", [("f32", 1, 9), ("f32", 0, 11), ("bf16", 1, 9), ("bf16", 0, 11)])
def test_lora_matrix_unit_views(cd, off, pad):
    """bf16 operands (the matrix-unit kernels) into C views whose base and
    pitch are aligned to the element only (off 1, pitch n + 9: element by
    element) or to 16 bytes (off 0, pitch n + 11: vector accesses with a
    ragged column tail); ragged m, n and r (partial lora_b vectors)."""
    d = dev()
    m, n, k, r = 37, 301, 512, 13
    announce("tp_lora_add matrix-unit path, C view", cd, off, pad, m, n, k, r)
    x, a, b, c = _lora_inputs(m, n, k, r, seed=50 + off + pad, xd="bf16", abd="bf16", cd=cd)
    dt = torch.float32 if cd == "f32" else torch.bfloat16
    cbuf = torch.full((m + 2, n + pad), 4.0, dtype=dt, device=d)
    cbuf[1:1 + m, off:off + n] = c.to(d)
    view = cbuf[1:1 + m, off:off + n]
    tp.tp_lora_add(view, x.to(d), a.to(d), _padded_b(b, d), 0.6)
    _check(view, c, x, a, b, 0.6, bf16_out=cd == "bf16")
    assert torch.all(cbuf[0] == 4.0) and torch.all(cbuf[-1] == 4.0)
    assert torch.all(cbuf[:, :off] == 4.0) and torch.all(cbuf[:, off + n:] == 4.0)


@pytest.mark.parametrize("m,n,k,r", [
    (4096, 9216, 3072, 32),    # qkv at full size: the single-pass kernel, side path in its store
    (4096, 9216, 3072, 64),
    (2000, 5000, 512, 13),     # ragged M and N on the single-pass kernel, a partial lora_b vector
    (512, 1024, 3072, 40),     # split K: product, then the standalone up half
    (48, 3000, 1024, 7),       # few rows: product, then the standalone up half
])
def test_w8a8_lora_in_store(m, n, k, r):
    """tp_lora_down + tp_qgemm_w8a8_prequantized_lora give the bits of
    tp_qgemm_w8a8_prequantized followed by tp_lora_add (bf16 x, lora_a,
    lora_b), and the side path stays inside the fp32 bound of the oracle's
    (sampled rows, against the product alone)."""
    d = dev()
    announce("tp_qgemm_w8a8_prequantized_lora", m, n, k, r)
    x = W.random_rows((m, k), seed=m + r, dtype="bf16")
    _, a, b, _ = _lora_inputs(1, n, k, r, seed=n + r)
    w = W.random_rows((n, k), seed=k + r, dtype="f32", scale=0.02)
    xd, ad, bd = x.to(d), a.to(d), _padded_b(b, d)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    qa, sa = tp.tp_quantize_rows_int8(xd, rotate=True)
    base = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s)
    sep = base.clone()
    tp.tp_lora_add(sep, xd, ad, bd, 0.7)
    t = tp.tp_lora_down(xd, ad)
    fused = tp.tp_qgemm_w8a8_prequantized_lora(qa, sa, q, s, t, bd, 0.7)
    assert torch.equal(fused, sep), f"{int((fused != sep).sum())} elements differ from product + tp_lora_add"
    sel = sample_rows(m, 16, seed=r)
    _check(fused[sel], base[sel], x[sel], a, b, 0.7)
