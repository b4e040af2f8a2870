"""W4A8 (tp_qgemm_w4a8, tp_qgemm_w4a8_prequantized) vs the CPU oracle.

* activation codes and scales bit-exact (they are tp_quantize_rows_int8's);
* output within the bound of its fp32 fold, element by element: the device
  adds fl(s[n,g] * acc_g) in group order (acc_g exact, as is its fp32 value)
  and multiplies by sa[m], so |y - y_exact| <= sa[m] * sum_g |s[n,g] acc_g| *
  (G + 2) * 2^-24 (each product and each partial sum rounded once, the final
  product once more), with the exact y and per-group accumulators from the
  oracle;
* full-size sampled rows of the W8A8 block's down projection with int4
  weights, ragged shapes over the 256x128, 128x192 and split-K paths, codes
  from the fused FFN middle, padded views, bf16 output, determinism.
"""

import numpy as np
import pytest
import torch

import int4_quantized_gemm_amd as tp
import oracle
import workloads as W
from tests.gpu_util import announce, dev, f64, host, sample_rows

pytestmark = pytest.mark.gpu

_W4 = {}


def _weights4(key, w, d):
    """The oracle's own int4 codes and group scales of w (no oracle input
    comes from the device), on the device for the product under test."""
    if key not in _W4:
        _W4[key] = oracle.quantize_weights_int4(w.float().numpy())
    rq4, rs4 = _W4[key]
    return rq4, rs4, torch.from_numpy(rq4).to(d), torch.from_numpy(rs4).to(d)


def _check(y_dev, y, acc, s, sa, what, bf16=False):
    g = acc.shape[0]
    terms = np.abs(acc.astype(np.float64)) * np.abs(np.asarray(s, dtype=np.float64).T)[:, None, :]
    bound = terms.sum(axis=0) * np.asarray(sa, dtype=np.float64)[:, None] * (g + 2) * 2.0 ** -24 * 1.01 + 1e-38
    if bf16:
        bound = bound + np.abs(y) * 2.0 ** -8
    err = np.abs(y_dev - y)
    bad = err > bound
    assert np.all(np.isfinite(y_dev)), f"{what}: non-finite output"
    assert not np.any(bad), f"{what}: {int(bad.sum())} outputs outside the fold bound (max ratio " \
                            f"{float(np.max(err / bound)):.2f})"


def _case(wl, sel=None, out_dtype=torch.float32, rotate=True):
    d = dev()
    x, w = W.generate(wl, rows=None)
    rq4, rs4, q4, s4 = _weights4(wl, w, d)
    y, qa, sa = tp.tp_qgemm_w4a8(x.to(d), q4, s4, rotate=rotate, out_dtype=out_dtype, want_codes=True)
    x64 = f64(x) if sel is None else f64(x)[sel]
    ry, racc, rqa, rsa = oracle.qgemm_w4a8(x64, rq4, rs4, rotate=rotate)
    gq, gs = host(qa), host(sa)
    if sel is not None:
        gq, gs = gq[sel], gs[sel]
    assert np.array_equal(gs, rsa), "activation scales"
    assert np.array_equal(gq, rqa), "activation codes"
    yd = f64(y) if sel is None else f64(y)[sel]
    _check(yd, ry, racc, rs4, rsa, wl.name, bf16=out_dtype == torch.bfloat16)
    return y


def test_w4a8_down_full_sampled():
    wl = W.DIT_DOWN
    announce("tp_qgemm_w4a8", wl.name, wl.m, wl.k, wl.n)
    _case(wl, sel=sample_rows(wl.m, 24, seed=8))


def test_w4a8_ffn_down_shape_sampled():
    wl = W.FFN_DOWN
    announce("tp_qgemm_w4a8 (ffn_down activations)", wl.m, wl.k, wl.n)
    _case(wl, sel=sample_rows(wl.m, 24, seed=9))


@pytest.mark.parametrize("m,n,k", [(1, 256, 256), (5, 1000, 2560), (64, 300, 3072), (100, 200, 768),
                                   (129, 385, 512), (300, 3000, 4096), (2100, 3000, 1024), (4000, 8000, 1024)])
def test_w4a8_ragged(m, n, k):
    announce("tp_qgemm_w4a8 ragged", m, n, k)
    wl = W.PROJ256.with_(name=f"w4a8_{m}_{n}_{k}", m=m, n=n, k=k, seed=m + 3 * n + k, path="w4a8", out_dtype="f32")
    sel = None if m * n <= 400000 else sample_rows(m, 16, seed=k)
    _case(wl, sel=sel)


def test_w4a8_bf16_out_and_prerotated():
    announce("tp_qgemm_w4a8 bf16 out, pre-rotated bf16 input")
    wl = W.PROJ256.with_(name="w4a8_pre", m=300, n=700, k=1536, seed=31, path="w4a8")
    d = dev()
    x, w = W.generate(wl)
    # pre-rotated bf16 rows made by the oracle, the input of both sides
    xr64 = oracle.bf16_round(oracle.rotate_groups(f64(x)))
    xr = torch.from_numpy(xr64.astype(np.float32)).to(torch.bfloat16).to(d)  # exact: bf16 values
    rq4, rs4, q4, s4 = _weights4(wl, w, d)
    y = tp.tp_qgemm_w4a8(xr, q4, s4, rotate=False, out_dtype=torch.bfloat16)
    ry, racc, _, rsa = oracle.qgemm_w4a8(xr64, rq4, rs4, rotate=False)
    _check(f64(y), ry, racc, rs4, rsa, "bf16 out", bf16=True)


def test_w4a8_from_fused_ffn_middle():
    """NEXT-1 feeding NEXT-2: gate/up -> tp_swiglu_rotate (int8) -> W4A8 down
    projection on the prequantized entry point, against the oracle's FFN
    middle and W4A8 product on the same codes."""
    d = dev()
    fm = W.FFN_MID_W8A8.with_(m=512)
    announce("swiglu_rotate -> tp_qgemm_w4a8_prequantized", fm.m, fm.k)
    g, u = W.gate_up(fm)
    qa, sa = tp.tp_swiglu_rotate(g.to(d), u.to(d), out_kind="i8")
    _, w = W.generate(W.DIT_DOWN, rows=1)
    rq4, rs4, q4, s4 = _weights4(W.DIT_DOWN, w, d)
    y = tp.tp_qgemm_w4a8_prequantized(qa, sa, q4, s4)
    rqa, rsa = oracle.ffn_middle_int8(f64(g), f64(u))
    assert np.array_equal(host(qa), rqa) and np.array_equal(host(sa), rsa)
    q = oracle.unpack_int4(rq4)
    acc = oracle.group_accumulate(rqa, q)
    ry = np.einsum("gmn,gn->mn", acc.astype(np.float64), rs4.astype(np.float64).T) * rsa.astype(np.float64)[:, None]
    _check(f64(y), ry, acc, rs4, rsa, "fused middle -> w4a8")


def test_w4a8_padded_views_and_determinism():
    d = dev()
    announce("tp_qgemm_w4a8_prequantized padded views, repeats")
    wl = W.PROJ256.with_(name="w4a8_views", m=40, n=520, k=2048, seed=33, path="w4a8")
    x, w = W.generate(wl)
    qa, sa = tp.tp_quantize_rows_int8(x.to(d))
    rq4, rs4, q4, s4 = _weights4(wl, w, d)
    cbuf = torch.full((44, 520 + 16), 9.0, dtype=torch.float32, device=d)
    out = cbuf[2:42, 8:528]
    y1 = tp.tp_qgemm_w4a8_prequantized(qa, sa, q4, s4, out=out).clone()
    y2 = tp.tp_qgemm_w4a8_prequantized(qa, sa, q4, s4, out=out).clone()
    assert torch.equal(y1, y2), "repeat runs differ"
    assert torch.all(cbuf[:2] == 9.0) and torch.all(cbuf[42:] == 9.0)
    assert torch.all(cbuf[:, :8] == 9.0) and torch.all(cbuf[:, 528:] == 9.0)
    ry, racc, rqa, rsa = oracle.qgemm_w4a8(f64(x), rq4, rs4)
    assert np.array_equal(host(qa), rqa)
    _check(f64(y1), ry, racc, rs4, rsa, "padded views")
