"""Undoing and requantizing rotated, quantized weights on the GPU
(tp_dequantize_unrotate, tp_requantize_weights) vs the CPU oracle.

* W_hat bit-exact: the oracle's fp64 un-rotation is exact, and the device
  rounds the same value once (fp32 or bf16);
* requantized codes and scales bit-exact, for all four width pairs, at full
  size for the two largest workload weights, including the identities
  int8 -> int8 and int4 -> int4 on quantizer outputs;
* the loader's round trip: tp_rotate_quantize_weights of the device's fp32
  W_hat gives back the codes (scales within an ulp where W_hat's rounding
  moved the row maximum).
"""

import numpy as np
import pytest
import torch

import int4_quantized_gemm_amd as tp
import oracle
import workloads as W
from tests.gpu_util import announce, dev, f64, host, sample_rows

pytestmark = pytest.mark.gpu


_CODES = {}


def _weights(wl, bits):
    """The oracle's own codes and scales of a workload weight (no oracle
    input comes from the device), on the device for the call under test."""
    d = dev()
    key = (wl, bits)
    if key not in _CODES:
        _, w = W.generate(wl, rows=1)
        wn = w.float().numpy()
        _CODES[key] = oracle.quantize_weights_int8(wn) if bits == 8 else oracle.quantize_weights_int4(wn)
    q, s = _CODES[key]
    return torch.from_numpy(q).to(d), torch.from_numpy(s).to(d)


def _bf16_bits(x64):
    return oracle.bf16_round(x64)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["tiny", "ffn_down"])
def test_dequantize_unrotate(bits, dt, name):
    wl = W.BY_NAME[name]
    announce("tp_dequantize_unrotate", name, bits, dt)
    q, s = _weights(wl, bits)
    odt = torch.float32 if dt == "f32" else torch.bfloat16
    w = tp.tp_dequantize_unrotate(q, s, bits, out_dtype=odt)
    sel = sample_rows(wl.n, 64, seed=3) if wl.n > 512 else np.arange(wl.n)
    rqn, rsn = _CODES[(wl, bits)]
    ref = oracle.dequantize_unrotate(rqn[sel], rsn[sel], bits)
    want = ref.astype(np.float32).astype(np.float64) if dt == "f32" else _bf16_bits(ref)
    got = f64(w)[sel]
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} elements differ"


@pytest.mark.parametrize("bits_in,bits_out", [(8, 8), (8, 4), (4, 8), (4, 4)])
@pytest.mark.parametrize("name", ["tiny", "dit_gateup", "ffn_down"])
def test_requantize(bits_in, bits_out, name):
    wl = W.BY_NAME[name]
    announce("tp_requantize_weights", name, bits_in, "->", bits_out)
    q, s = _weights(wl, bits_in)
    qo, so = tp.tp_requantize_weights(q, s, bits_in, bits_out)
    sel = sample_rows(wl.n, 64, seed=4) if wl.n > 512 else np.arange(wl.n)
    rqn, rsn = _CODES[(wl, bits_in)]
    rq, rs = oracle.requantize(rqn[sel], rsn[sel], bits_in, bits_out)
    assert np.array_equal(host(so)[sel], rs), "scales"
    assert np.array_equal(host(qo)[sel], rq), "codes"
    if bits_in == bits_out:
        assert torch.equal(qo, q) and torch.equal(so, s), "same width must give the codes back"


@pytest.mark.parametrize("bits", [8, 4])
def test_loader_round_trip(bits):
    """Undo, then the library's own quantizer: the codes come back."""
    wl = W.PROJ256
    announce("loader round trip", bits)
    q, s = _weights(wl, bits)
    w = tp.tp_dequantize_unrotate(q, s, bits)
    q2, s2 = tp.tp_rotate_quantize_weights(w, bits=bits)
    assert torch.equal(q2, q), "codes"
    rel = (s2.double() - s.double()).abs() / s.double().clamp_min(1e-30)
    assert float(rel.max()) <= 2.0 ** -23, "scales move by more than an ulp"


def test_loader_ragged_and_views():
    d = dev()
    announce("loader padded views, ragged rows")
    wl = W.TINY.with_(n=37, k=1280, seed=5)
    q, s = _weights(wl, 4)
    qbuf = torch.zeros((40, 640 + 64), dtype=torch.uint8, device=d)
    qbuf[1:38, 16:656] = q
    out = torch.full((39, 1280 + 32), 3.0, dtype=torch.float32, device=d)
    tp.tp_dequantize_unrotate(qbuf[1:38, 16:656], s, 4, out=out[1:38, 16:1296])
    rqn, rsn = _CODES[(wl, 4)]
    ref = oracle.dequantize_unrotate(rqn, rsn, 4).astype(np.float32)
    assert np.array_equal(host(out[1:38, 16:1296]), ref)
    assert torch.all(out[0] == 3.0) and torch.all(out[38] == 3.0) and torch.all(out[:, :16] == 3.0)
    q8 = torch.zeros((37, 1280 + 128), dtype=torch.int8, device=d)
    s8 = torch.zeros((41,), dtype=torch.float32, device=d)
    tp.tp_requantize_weights(qbuf[1:38, 16:656], s, 4, 8, q_out=q8[:, 64:1344], scales_out=s8[4:41])
    rq, rs = oracle.requantize(rqn, rsn, 4, 8)
    assert np.array_equal(host(q8[:, 64:1344]), rq) and np.array_equal(host(s8[4:41]), rs)
    assert torch.all(q8[:, :64] == 0) and torch.all(s8[:4] == 0)
