"""Fused FFN middle (tp_swiglu_rotate) vs the CPU oracle on the same seeded
gate and up activations.

* int8 output: codes and scales bit-exact against the oracle's
  quantize(rotate(bf16(silu(g) u))), at full size (sampled rows) and on
  ragged shapes, from fp32 and bf16 inputs, with gate and up given as the two
  column halves of one gate+up buffer;
* h itself bit-exact: rows with a single nonzero h have scale
  fp32(|h| / 16 / 127), so every scale checks one h, on inputs that drive the
  fp32 shortcut, its fallback and the fp64-only ranges;
* bf16 output: a bf16 rounding of a value within the fp32 rotation's error
  bound around the exact rotation of h.
"""

import numpy as np
import pytest
import torch

import int4_quantized_gemm_amd as tp
import oracle
import workloads as W
from tests.gpu_util import announce, dev, f64, host, rotation_error_bound, sample_rows

pytestmark = pytest.mark.gpu


def _check_i8(g, u, qa, sa, sel=None):
    g64, u64 = f64(g), f64(u)
    if sel is not None:
        g64, u64 = g64[sel], u64[sel]
    rq, rs = oracle.ffn_middle_int8(g64, u64)
    got_q, got_s = host(qa), host(sa)
    if sel is not None:
        got_q, got_s = got_q[sel], got_s[sel]
    assert np.array_equal(got_s, rs), f"{int(np.sum(got_s != rs))} scales differ"
    assert np.array_equal(got_q, rq), f"{int(np.sum(got_q != rq))} codes differ"


def _check_bf16(g, u, y, sel=None):
    g64, u64 = f64(g), f64(u)
    if sel is not None:
        g64, u64 = g64[sel], u64[sel]
    h = oracle.swiglu_bf16(g64, u64)
    exact = oracle.ffn_middle_rotated(g64, u64)
    bound = rotation_error_bound(h)
    got = f64(y) if sel is None else f64(y)[sel]
    lo, hi = oracle.bf16_round(exact - bound), oracle.bf16_round(exact + bound)
    assert np.all((lo <= got) & (got <= hi)), "not a bf16 rounding of a value within the rotation bound"
    assert np.mean(got != oracle.bf16_round(exact)) < 1e-2


def test_ffn_mid_w8a8_full_sampled():
    w = W.FFN_MID_W8A8
    d = dev()
    announce("tp_swiglu_rotate i8", w.name, w.m, w.k)
    gu = W.gate_up(w, fused=True)
    gud = gu.to(d)
    qa, sa = tp.tp_swiglu_rotate(gud[:, :w.k], gud[:, w.k:], out_kind="i8")
    _check_i8(gu[:, :w.k], gu[:, w.k:], qa, sa, sel=sample_rows(w.m, 24, seed=5))


def test_ffn_mid_w4_full_sampled():
    w = W.FFN_MID_W4
    d = dev()
    announce("tp_swiglu_rotate bf16", w.name, w.m, w.k)
    g, u = W.gate_up(w)
    y = tp.tp_swiglu_rotate(g.to(d), u.to(d), out_kind="bf16")
    _check_bf16(g, u, y, sel=sample_rows(w.m, 24, seed=6))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("m,k", [(1, 256), (37, 768), (300, 3072), (9, 4096), (5, 12800)])
def test_ffn_mid_ragged(dt, m, k):
    d = dev()
    announce("tp_swiglu_rotate ragged", dt, m, k)
    w = W.FFN_MID_W8A8.with_(m=m, k=k, seed=m * 31 + k, in_dtype=dt)
    gu = W.gate_up(w, fused=True)
    gud = gu.to(d)
    g, u = gud[:, :k], gud[:, k:]
    qa, sa = tp.tp_swiglu_rotate(g, u, out_kind="i8")
    _check_i8(gu[:, :k], gu[:, k:], qa, sa)
    y = tp.tp_swiglu_rotate(g, u, out_kind="bf16")
    _check_bf16(gu[:, :k], gu[:, k:], y)


def _single_h_rows(n, seed):
    """n rows of K = 256 with one nonzero (g, u) per row at a varying column:
    wide-range g (fast path, fallback near ties, |g| > 64, huge negative g),
    u with tiny and huge magnitudes, exact bf16 ties (g = 64, u = t / 64)."""
    rng = np.random.default_rng(seed)
    g = np.zeros((n, 256), dtype=np.float32)
    u = np.zeros((n, 256), dtype=np.float32)
    col = rng.integers(0, 256, size=n)
    gv = rng.standard_normal(n).astype(np.float32) * np.float32(4.0)
    uv = rng.standard_normal(n).astype(np.float32)
    part = n // 8
    gv[:part] = rng.uniform(-90, 90, size=part)                       # beyond the fp32 range of the shortcut
    uv[part:2 * part] *= np.float32(1e-30)                            # tiny h
    uv[2 * part:3 * part] *= np.float32(1e30)                         # huge h
    ties = 1.0 + (2 * rng.integers(0, 128, size=part) + 1) * 2.0 ** -8  # bf16 midpoints in [1, 2)
    gv[3 * part:4 * part] = 64.0
    uv[3 * part:4 * part] = (ties * rng.choice([-1.0, 1.0], size=part) / 64.0).astype(np.float32)
    gv[4 * part:5 * part] = rng.uniform(-200, -88, size=part)         # e^-g overflows fp32
    g[np.arange(n), col] = gv
    u[np.arange(n), col] = uv
    return torch.from_numpy(g), torch.from_numpy(u)


def test_ffn_mid_h_exact_through_scales():
    d = dev()
    n = 65536
    announce("tp_swiglu_rotate single-h rows", n)
    g, u = _single_h_rows(n, seed=99)
    qa, sa = tp.tp_swiglu_rotate(g.to(d), u.to(d), out_kind="i8")
    h = oracle.swiglu_bf16(f64(g), f64(u)).sum(axis=1)  # the one nonzero per row
    expect = (np.abs(h) / 16.0 / 127.0).astype(np.float32)
    got = host(sa)
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, f"{bad.size} rows: h differs, e.g. g={f64(g)[bad[0]].sum()} u={f64(u)[bad[0]].sum()}"
    _check_i8(g, u, qa, sa, sel=np.arange(0, n, 97))


def test_ffn_mid_gate_up_overlapping_and_padded():
    """gate and up as the same buffer (h = bf16(silu(x) x)) and padded output views."""
    d = dev()
    announce("tp_swiglu_rotate same buffer / padded views")
    w = W.FFN_MID_W8A8.with_(m=40, k=1024, seed=7, in_dtype="bf16")
    g, _ = W.gate_up(w)
    gd = g.to(d)
    qbuf = torch.full((44, 1024 + 64), 7, dtype=torch.int8, device=d)
    sbuf = torch.full((48,), -1.0, dtype=torch.float32, device=d)
    qa, sa = tp.tp_swiglu_rotate(gd, gd, out_kind="i8", out=qbuf[2:42, 32:32 + 1024], scales=sbuf[4:44])
    _check_i8(g, g, qa, sa)
    assert torch.all(qbuf[:2] == 7) and torch.all(qbuf[42:] == 7) and torch.all(qbuf[:, :32] == 7)
    assert torch.all(sbuf[:4] == -1.0) and torch.all(sbuf[44:] == -1.0)
    ybuf = torch.zeros((42, 1024 + 256), dtype=torch.bfloat16, device=d)
    y = tp.tp_swiglu_rotate(gd, gd, out_kind="bf16", out=ybuf[1:41, 128:128 + 1024])
    _check_bf16(g, g, y)
    assert torch.all(ybuf[0] == 0) and torch.all(ybuf[:, :128] == 0) and torch.all(ybuf[:, 1152:] == 0)
