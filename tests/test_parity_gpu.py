"""HIP path vs the CPU oracle, element by element, on the same seeded inputs.

* weight rotate-and-quantize: codes (int8, packed int4) and fp32 scales
  bit-exact, at full size for every workload's weight;
* activation rotation: within the fp32 transform's error bound (fp32 out), or
  equal to a correct bf16 rounding of a value within that bound (bf16 out);
* per-token activation quantization: codes and scales bit-exact;
* W8 / W4 products: relative Frobenius error <= 2e-3 against the oracle that
  models the bf16 activation operand;
* W8A8: int32 accumulators, codes and scales bit-exact; output within 1e-5.

Small workloads are compared in full; full-size workloads run in the launch
configuration the benchmark times and are compared on sampled rows (whole
output rows, every column, including tile tails).
"""

import numpy as np
import pytest
import torch

import int4_quantized_gemm_amd as tp
import oracle
import workloads as W
from tests.gpu_util import (announce, assert_bf16_path, assert_w8a8_out, dev, f64, host,
                            rotation_error_bound, sample_rows)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ helpers
_ORACLE_W = {}


def oracle_weights(key, w_cpu, bits):
    """The oracle's own rotated, quantized weights (never the device's)."""
    k = (key, bits)
    if k not in _ORACLE_W:
        wn = w_cpu.float().numpy()
        _ORACLE_W[k] = oracle.quantize_weights_int8(wn) if bits == 8 else oracle.quantize_weights_int4(wn)
    return _ORACLE_W[k]


def _check_weights(w_cpu, bits, d):
    q, s = tp.tp_rotate_quantize_weights(w_cpu.to(d), bits=bits)
    torch.cuda.synchronize()
    if bits == 8:
        rq, rs = oracle.quantize_weights_int8(w_cpu.float().numpy())
        assert np.array_equal(host(q), rq), "int8 codes differ"
    else:
        rq, rs = oracle.quantize_weights_int4(w_cpu.float().numpy())
        assert np.array_equal(host(q), rq), "packed int4 codes differ"
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32)), "scales differ"
    return q, s


# ------------------------------------------------- weight rotate + quantize
@pytest.mark.parametrize("name", ["tiny", "proj256", "ffn_up", "dit_qkv", "dit_out", "dit_gateup", "dit_down"])
def test_rotate_quantize_int8_full(name):
    d = dev()
    wl = W.BY_NAME[name]
    announce("tp_rotate_quantize_weights bits=8", name, wl.n, wl.k, "seed", wl.seed)
    _, w = W.generate(wl, rows=1)
    _check_weights(w, 8, d)


@pytest.mark.parametrize("name", ["tiny", "proj256", "ffn_down", "dit_qkv", "dit_out", "dit_gateup", "dit_down"])
def test_rotate_quantize_int4_full(name):
    d = dev()
    wl = W.BY_NAME[name]
    announce("tp_rotate_quantize_weights bits=4", name, wl.n, wl.k, "seed", wl.seed)
    _, w = W.generate(wl, rows=1)
    _check_weights(w, 4, d)


def test_rotate_quantize_edge_rows():
    d = dev()
    announce("tp_rotate_quantize_weights edge rows")
    w = W.random_rows((7, 768), seed=5, scale=0.02)
    w[2] = 0.0                      # zero row -> scale 0, codes 0
    w[3, 256:512] = 0.0             # zero group (int4)
    w[4, 10] = 1e3                  # one huge outlier
    w[5] = torch.arange(768, dtype=torch.float32) - 384.0   # dyadic values: exact rotation
    for bits in (8, 4):
        _check_weights(w, bits, d)
    # bf16 source weights
    wb = W.random_rows((5, 512), seed=6, dtype="bf16", scale=0.02)
    for bits in (8, 4):
        q, s = tp.tp_rotate_quantize_weights(wb.to(d), bits=bits)
        if bits == 8:
            rq, rs = oracle.quantize_weights_int8(wb.float().numpy())
        else:
            rq, rs = oracle.quantize_weights_int4(wb.float().numpy())
        assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)


def test_rotate_quantize_padded_subview():
    d = dev()
    announce("tp_rotate_quantize_weights padded sub-view")
    big = W.random_rows((40, 1024 + 256), seed=7, scale=0.02).to(d)
    w = big[3:35, 256:1280]        # storage offset, ld = 1280
    qbuf = torch.zeros((32, 1024 + 64), dtype=torch.int8, device=d)
    q = qbuf[:, :1024]             # ld = 1088 bytes
    s = torch.empty(32, dtype=torch.float32, device=d)
    tp.tp_rotate_quantize_weights(w, bits=8, q=q, scales=s)
    rq, rs = oracle.quantize_weights_int8(w.float().cpu().numpy())
    assert np.array_equal(host(q), rq) and np.array_equal(host(s), rs)
    assert torch.all(qbuf[:, 1024:] == 0), "wrote past the row"


# ------------------------------------------------------- activation rotation
@pytest.mark.parametrize("xd,yd", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("m,k", [(64, 512), (37, 768), (1, 256), (288, 3072)])
def test_rotate_rows(xd, yd, m, k):
    d = dev()
    announce("tp_hadamard_rotate_rows", xd, yd, m, k)
    x = W.random_rows((m, k), seed=m + k, dtype=xd)
    x[:, 3] *= 30.0
    ydt = torch.float32 if yd == "f32" else torch.bfloat16
    y = tp.tp_hadamard_rotate_rows(x.to(d), out_dtype=ydt)
    x64 = f64(x)
    exact = oracle.rotate_groups(x64)
    bound = rotation_error_bound(x64)
    got = f64(y)
    if yd == "f32":
        assert np.all(np.abs(got - exact) <= bound), "fp32 rotation outside its error bound"
    else:
        lo = oracle.bf16_round(exact - bound)
        hi = oracle.bf16_round(exact + bound)
        # rounding is monotone: bf16(fp32 result) lies between the roundings
        # of the two ends of the fp32 error interval
        assert np.all((lo <= got) & (got <= hi)), "bf16 rotation is not a rounding of a value within the bound"
        assert np.mean(got != oracle.bf16_round(exact)) < 1e-2


@pytest.mark.parametrize("name", ["ffn_up", "ffn_down"])
def test_rotate_rows_full_size(name):
    """The launches the benchmark times (full 4096x3072 and 4032x12288 bf16
    activations to bf16), each output checked directly against the exact
    rotation on sampled whole rows: a correct bf16 rounding of a value within
    the fp32 transform's error bound."""
    d = dev()
    wl = W.BY_NAME[name]
    announce("tp_hadamard_rotate_rows full size", name, wl.m, wl.k)
    x = W.generate_activations(wl)
    y = tp.tp_hadamard_rotate_rows(x.to(d), out_dtype=torch.bfloat16)
    sel = sample_rows(wl.m, 200, seed=wl.seed)
    x64 = f64(x)[sel]
    exact = oracle.rotate_groups(x64)
    bound = rotation_error_bound(x64)
    got = f64(y)[sel]
    lo, hi = oracle.bf16_round(exact - bound), oracle.bf16_round(exact + bound)
    assert np.all((lo <= got) & (got <= hi)), "bf16 rotation is not a rounding of a value within the bound"
    assert np.mean(got != oracle.bf16_round(exact)) < 1e-2


def test_rotate_rows_in_place_and_subview():
    d = dev()
    announce("tp_hadamard_rotate_rows in place / sub-view")
    base = W.random_rows((50, 1024 + 512), seed=9, dtype="bf16").to(d)
    ref_in = base.clone()
    view = base[5:45, 256:1280]
    tp.tp_hadamard_rotate_rows(view, out=view)          # in place on a padded view
    exact = oracle.rotate_groups(f64(ref_in[5:45, 256:1280]))
    bound = rotation_error_bound(f64(ref_in[5:45, 256:1280]))
    got = f64(view)
    lo, hi = oracle.bf16_round(exact - bound), oracle.bf16_round(exact + bound)
    assert np.all((lo <= got) & (got <= hi))
    # untouched outside the view
    assert torch.equal(base[:5], ref_in[:5]) and torch.equal(base[45:], ref_in[45:])
    assert torch.equal(base[:, :256], ref_in[:, :256]) and torch.equal(base[:, 1280:], ref_in[:, 1280:])


def test_rotate_rows_inverse():
    """Rotating twice gives back the input (Q Q = I) up to fp32 rounding."""
    d = dev()
    announce("tp_hadamard_rotate_rows twice")
    x = W.random_rows((33, 1536), seed=10).to(d)
    y = tp.tp_hadamard_rotate_rows(tp.tp_hadamard_rotate_rows(x))
    assert torch.allclose(y, x, rtol=0, atol=1e-5)


# ------------------------------------------- per-token activation quantization
@pytest.mark.parametrize("name,rows", [("tiny", None), ("dit_qkv", None), ("dit_down", 512), ("proj256", None)])
@pytest.mark.parametrize("rotate", [True, False])
def test_quantize_rows_int8(name, rows, rotate):
    d = dev()
    wl = W.BY_NAME[name]
    announce("tp_quantize_rows_int8", name, rows, "rotate", rotate)
    x = W.generate_activations(wl, rows=rows)
    qa, sa = tp.tp_quantize_rows_int8(x.to(d), rotate=rotate)
    rqa, rsa = oracle.quantize_activations_int8(f64(x), rotate=rotate)
    assert np.array_equal(host(sa).view(np.uint32), rsa.view(np.uint32)), "scales differ"
    assert np.array_equal(host(qa), rqa), f"{int(np.sum(host(qa) != rqa))} codes differ"


@pytest.mark.parametrize("groups", [1, 3, 5, 12, 13, 30, 47, 48, 49])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantize_rows_ragged_groups(groups, dt):
    """Group counts that leave 16-lane rows of a wave without a group (fewer
    than 4, or not a multiple of 4), split unevenly over the four waves of a
    row (13 to 47 groups), fill every slot (12, 48), or take the one-wave-per-
    row fp64 kernel above 48; 7 rows (not a multiple of the block's 4), with
    outlier columns, rotated and not."""
    d = dev()
    k = 256 * groups
    announce("tp_quantize_rows_int8 ragged groups", groups, dt)
    x = W.random_rows((7, k), seed=groups + (100 if dt == "f32" else 0), dtype=dt)
    x[:, min(5, k - 1)] *= 30.0
    x[3] *= 1e-3
    for rotate in (True, False):
        qa, sa = tp.tp_quantize_rows_int8(x.to(d), rotate=rotate)
        rqa, rsa = oracle.quantize_activations_int8(f64(x), rotate=rotate)
        assert np.array_equal(host(sa).view(np.uint32), rsa.view(np.uint32)), "scales differ"
        assert np.array_equal(host(qa), rqa), f"{int(np.sum(host(qa) != rqa))} codes differ"


def test_quantize_rows_zero_and_tiny_rows():
    """Zero and tiny rows, and rows whose scale is a subnormal fp32 with few
    significant bits: there s can sit several tenths of a percent away from
    amax / 127, the largest quotient lands above 127.5 and the code must be
    clamped to 127 (rows 6-11, single nonzero elements from 2e-40 to 2e-43,
    fp32 and bf16 inputs, both widths of K)."""
    d = dev()
    announce("tp_quantize_rows_int8 zero, tiny and subnormal-scale rows")
    for k in (512, 12288):
        x = W.random_rows((12, k), seed=11)
        x[1] = 0.0
        x[2] = 1e-30
        x[3, 7] = -5.0
        for i, (val, col) in enumerate([(2e-40, 0), (-3.3e-41, 5), (7.1e-42, 300), (-2.2e-43, 17), (1.5e-40, 0),
                                        (-9.9e-41, 511)]):
            x[6 + i] = 0.0
            x[6 + i, col] = val
        for xin in (x, x.to(torch.bfloat16)):
            qa, sa = tp.tp_quantize_rows_int8(xin.to(d))
            rqa, rsa = oracle.quantize_activations_int8(f64(xin))
            assert np.array_equal(host(sa), rsa), "scales differ"
            assert np.array_equal(host(qa), rqa), f"{int(np.sum(host(qa) != rqa))} codes differ"
            assert host(sa)[1] == 0 and np.all(host(qa)[1] == 0)
        sub = host(sa)[6:]
        assert np.any((sub > 0) & (sub < 2.0 ** -126)), "no subnormal scale was exercised"


def test_non_finite_rows_stay_local():
    """NaN and infinity are not refused (tp.h, Values): the rows holding them
    get codes inside the code range and the calls succeed, while every other
    row keeps the oracle's codes and scales bit for bit (rows are quantized
    independently), for the activation quantizer and both weight widths."""
    d = dev()
    announce("non-finite rows: activation and weight quantizers")
    for k in (3072, 12288):
        x = W.random_rows((16, k), seed=13)
        bad = {2: [(5, float("nan"))], 5: [(0, float("inf"))], 9: [(100, float("-inf")), (101, float("nan"))],
               13: [(k - 1, float("nan"))]}
        for r, cells in bad.items():
            for c, v in cells:
                x[r, c] = v
        good = [r for r in range(16) if r not in bad]
        for xin in (x, x.to(torch.bfloat16)):
            qa, sa = tp.tp_quantize_rows_int8(xin.to(d))
            torch.cuda.synchronize()
            q = host(qa)
            assert q.min() >= -127 and q.max() <= 127, "a code outside [-127, 127]"
            rqa, rsa = oracle.quantize_activations_int8(f64(xin[good]))
            assert np.array_equal(q[good], rqa), "a finite row's codes changed"
            assert np.array_equal(host(sa)[good].view(np.uint32), rsa.view(np.uint32)), "a finite row's scale changed"
    w = W.random_rows((24, 1024), seed=14)
    w[3, 7] = float("nan")
    w[10, 600] = float("inf")
    w[17, 0] = float("-inf")
    good = [r for r in range(24) if r not in (3, 10, 17)]
    q8, s8 = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    q4, s4 = tp.tp_rotate_quantize_weights(w.to(d), bits=4)
    torch.cuda.synchronize()
    c8 = host(q8)
    assert c8.min() >= -127 and c8.max() <= 127
    nib = host(q4).astype(np.int32)
    lo, hi = ((nib & 0xF) ^ 8) - 8, (((nib >> 4) & 0xF) ^ 8) - 8
    assert lo.min() >= -7 and lo.max() <= 7 and hi.min() >= -7 and hi.max() <= 7, "an int4 code outside [-7, 7]"
    rq8, rs8 = oracle.quantize_weights_int8(w[good].numpy())
    rq4, rs4 = oracle.quantize_weights_int4(w[good].numpy())
    assert np.array_equal(c8[good], rq8) and np.array_equal(host(s8)[good].view(np.uint32), rs8.view(np.uint32))
    assert np.array_equal(host(q4)[good], rq4) and np.array_equal(host(s4)[good].view(np.uint32), rs4.view(np.uint32))


@pytest.mark.parametrize("k", [3072, 12288])
def test_quantize_rows_exact_ties(k):
    """Every rotated value is a half-integer multiple of a power-of-two scale,
    so every code is a rounding tie: the device must round half to even, as
    the reference rule does (the fp32 bound cannot decide any of them, so each
    goes through the exact recomputation). Rotated (fp32 input) and
    pre-rotated (bf16 input) paths."""
    d = dev()
    announce("tp_quantize_rows_int8 exact ties", k)
    rng = np.random.default_rng(40 + k)
    m, c = 24, 2.0 ** -3
    xr = (rng.integers(-127, 127, size=(m, k)) + 0.5) * c      # rotated values: (j + 1/2) c
    xr[:, 17] = 127 * c                                          # the row maximum: s = c exactly
    xr[3] = 0.5 * c                                              # a row of 1/2 ties (all -> 0)
    xr[3, 0] = 127 * c
    H = oracle.hadamard_matrix(256) / 16.0
    unrot = lambda a: np.concatenate([a[:, g * 256:(g + 1) * 256] @ H for g in range(k // 256)], axis=1)
    x = torch.from_numpy(unrot(xr).astype(np.float32))
    assert np.array_equal(oracle.rotate_groups(x.numpy()), xr)  # exact in fp32
    expect = np.rint(xr / c).astype(np.int8)                    # numpy rint: half to even
    for inp, rotate in ((x, True), (torch.from_numpy(xr.astype(np.float32)).to(torch.bfloat16), False)):
        qa, sa = tp.tp_quantize_rows_int8(inp.to(d), rotate=rotate)
        rqa, rsa = oracle.quantize_activations_int8(f64(inp), rotate=rotate)
        assert np.all(host(sa) == np.float32(c)) and np.array_equal(rsa, host(sa))
        assert np.array_equal(rqa, expect)
        assert np.array_equal(host(qa), expect), f"{int(np.sum(host(qa) != expect))} tie codes differ"


# ------------------------------------------------------------- W8 / W4 products
def _w8_case(wl, row_sel=None, out_dtype=None):
    d = dev()
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    odt = out_dtype or (torch.float32 if wl.out_dtype == "f32" else torch.bfloat16)
    y = tp.tp_qgemm_w8(x.to(d), q, s, rotate=True, out_dtype=odt)
    sel = row_sel if row_sel is not None else np.arange(wl.m)
    rq, rs = oracle_weights(wl, w, 8)
    ref = oracle.qgemm_w8(f64(x)[sel], rq, rs)
    return f64(y)[sel], ref


def _w4_case(wl, row_sel=None, out_dtype=None):
    d = dev()
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=4)
    odt = out_dtype or (torch.float32 if wl.out_dtype == "f32" else torch.bfloat16)
    y = tp.tp_qgemm_w4(x.to(d), q, s, rotate=True, out_dtype=odt)
    sel = row_sel if row_sel is not None else np.arange(wl.m)
    rq, rs = oracle_weights(wl, w, 4)
    ref = oracle.qgemm_w4(f64(x)[sel], rq, rs)
    return f64(y)[sel], ref


def test_w8_tiny_full():
    announce("tp_qgemm_w8 tiny 64x512x256 fp32 out")
    got, ref = _w8_case(W.TINY)
    err = assert_bf16_path(got, ref, "w8 tiny")
    assert err < 1e-4, "fp32 output: only A-operand rounding flips and fp32 sums remain"


def test_w8_proj256_full():
    announce("tp_qgemm_w8 proj256 288x3072x3072 bf16 out")
    got, ref = _w8_case(W.PROJ256)
    assert_bf16_path(got, ref, "w8 proj256")


def test_w8_ffn_up_sampled():
    wl = W.FFN_UP
    announce("tp_qgemm_w8 ffn_up 4096x3072x12288 (sampled rows)")
    got, ref = _w8_case(wl, row_sel=sample_rows(wl.m, 48, seed=1))
    assert_bf16_path(got, ref, "w8 ffn_up")


def test_w4_tiny_full():
    announce("tp_qgemm_w4 tiny 64x512x256 fp32 out")
    got, ref = _w4_case(W.TINY.with_(path="w4"))
    err = assert_bf16_path(got, ref, "w4 tiny")
    assert err < 1e-4


def test_w4_ffn_down_sampled():
    wl = W.FFN_DOWN
    announce("tp_qgemm_w4 ffn_down 4032x12288x3072 (sampled rows)")
    got, ref = _w4_case(wl, row_sel=sample_rows(wl.m, 48, seed=2))
    assert_bf16_path(got, ref, "w4 ffn_down")


@pytest.mark.parametrize("kind", ["w8", "w4"])
@pytest.mark.parametrize("m,n,k", [(1, 256, 256), (100, 200, 768), (129, 385, 512), (300, 130, 1280)])
def test_weight_only_ragged(kind, m, n, k):
    d = dev()
    announce("tp_qgemm", kind, "ragged", m, n, k)
    wl = W.TINY.with_(m=m, n=n, k=k, seed=m * 7 + n, act_outliers=2, w_outliers=2)
    x, w = W.generate(wl)
    bits = 8 if kind == "w8" else 4
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=bits)
    fn = tp.tp_qgemm_w8 if kind == "w8" else tp.tp_qgemm_w4
    y = fn(x.to(d), q, s, rotate=True, out_dtype=torch.float32)
    rq, rs = oracle_weights(wl, w, bits)
    ref = (oracle.qgemm_w8 if kind == "w8" else oracle.qgemm_w4)(f64(x), rq, rs)
    err = assert_bf16_path(f64(y), ref, f"{kind} ragged")
    assert err < 1e-4


@pytest.mark.parametrize("m,n,k", [(300, 600, 2048), (2048, 4096, 1024), (4000, 3000, 1024)])
def test_w4_group_scale_edges(m, n, k):
    """Hand-made int4 codes and group scales that the quantizer never emits,
    one pattern per column class, on the split-K, 128x192 and 256x192 paths:
    zero scales over nonzero codes (no contribution), scales 1e28 apart in
    both orders, all-zero scales, columns whose only nonzero codes sit in
    the tiny-scale groups, and a staircase of scales each 2^60 below the one
    before (1, 2^-60, 2^-120, repeated): every step is within 2^64 of the
    previous scale, but the third is 2^120 below the first, so a rescale
    bounded by the previous step alone would overflow the running sum. Each
    class is compared on its own columns."""
    d = dev()
    announce("tp_qgemm_w4 group-scale edges", m, n, k)
    rng = np.random.default_rng(m + n + k)
    g = k // 256
    codes = rng.integers(-7, 8, size=(n, k)).astype(np.int8)
    s = (rng.uniform(0.5, 2.0, size=(n, g)) * 1e-2).astype(np.float32)
    cls = np.arange(n) % 7
    tiny = np.float32(1e-30)
    s[cls == 1, 0] = 0.0                                   # zero scale over nonzero codes
    s[cls == 2, 1::2] = tiny                               # normal, tiny, normal, ...
    s[cls == 3, : g // 2] = tiny                           # tiny first, then normal
    s[cls == 4] = 0.0                                      # every scale zero
    s[cls == 5, 1::2] = tiny                               # codes only where the scale is tiny
    c5 = codes[cls == 5].reshape(-1, g, 256)
    c5[:, 0::2] = 0
    codes[cls == 5] = c5.reshape(-1, k)
    stair = np.ldexp(np.float32(1.0), -60 * (np.arange(g) % 3)).astype(np.float32)
    s[cls == 6] = stair                                    # 1, 2^-60, 2^-120, 1, ...
    packed = oracle.pack_int4(codes)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    y = tp.tp_qgemm_w4(x.to(d), torch.from_numpy(packed).to(d), torch.from_numpy(s).to(d), rotate=False,
                       out_dtype=torch.float32)
    got = f64(y)
    ref = oracle.qgemm_w4(f64(x), packed, s, rotate=False)
    assert np.all(np.isfinite(got))
    assert np.all(got[:, cls == 4] == 0.0)
    for c in (0, 1, 2, 3, 5, 6):
        err = np.linalg.norm(got[:, cls == c] - ref[:, cls == c]) / np.linalg.norm(ref[:, cls == c])
        assert err < 1e-5, f"column class {c}: relative error {err:.3e}"


def test_w8_prerotated_padded_views():
    d = dev()
    announce("tp_qgemm_w8 pre-rotated bf16 A, padded A and C views")
    wl = W.TINY.with_(m=96, n=320, k=1024, seed=12)
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    xr = tp.tp_hadamard_rotate_rows(x.to(d), out_dtype=torch.bfloat16)
    abuf = torch.zeros((100, 1024 + 256), dtype=torch.bfloat16, device=d)
    abuf[2:98, 128:1152] = xr
    cbuf = torch.full((100, 320 + 64), 7.0, dtype=torch.float32, device=d)
    out = cbuf[3:99, 32:352]
    tp.tp_qgemm_w8(abuf[2:98, 128:1152], q, s, rotate=False, out=out)
    rq, rs = oracle_weights(wl, w, 8)
    ref = oracle.qgemm_w8(f64(x), rq, rs)   # the oracle rotates the raw input itself
    assert_bf16_path(f64(out), ref, "w8 prerotated view")
    assert torch.all(cbuf[:3] == 7.0) and torch.all(cbuf[99:] == 7.0)
    assert torch.all(cbuf[:, :32] == 7.0) and torch.all(cbuf[:, 352:] == 7.0)


# ------------------------------------------------------------------ W8A8
def _w8a8_case(wl, row_sel=None):
    d = dev()
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    y, qa, sa, acc = tp.tp_qgemm_w8a8(x.to(d), q, s, rotate=True, want_codes=True, want_acc=True)
    sel = row_sel if row_sel is not None else np.arange(wl.m)
    rq, rs = oracle_weights(wl, w, 8)
    ry, racc, rqa, rsa = oracle.qgemm_w8a8(f64(x)[sel], rq, rs)
    assert np.array_equal(host(sa)[sel], rsa), "activation scales differ"
    assert np.array_equal(host(qa)[sel], rqa), "activation codes differ"
    gacc = host(acc)[sel].astype(np.int64)
    assert np.array_equal(gacc, racc), f"{int(np.sum(gacc != racc))} int32 accumulators differ"
    assert_w8a8_out(f64(y)[sel], ry, f"w8a8 {wl.name}")
    # the caller-visible output without the intermediates is the same bytes
    y2 = tp.tp_qgemm_w8a8(x.to(d), q, s, rotate=True)
    assert torch.equal(y, y2)


def test_w8a8_tiny_full():
    announce("tp_qgemm_w8a8 tiny 64x512x256")
    _w8a8_case(W.TINY.with_(path="w8a8"))


@pytest.mark.parametrize("name", ["dit_qkv", "dit_out", "dit_gateup", "dit_down"])
def test_w8a8_dit_block_sampled(name):
    wl = W.BY_NAME[name]
    announce("tp_qgemm_w8a8", name, wl.m, wl.k, wl.n, "(sampled rows)")
    _w8a8_case(wl, row_sel=sample_rows(wl.m, 40, seed=wl.seed))


@pytest.mark.parametrize("m,n,k", [(4000, 9000, 1024), (4000, 3000, 1024), (4000, 24000, 512)])
def test_w8a8_large_ragged(m, n, k):
    """Ragged M and N on the large-tile paths: 4000x9000 takes 256x288 tiles
    (2 full rounds against 2.25 of 256x256), 4000x3000 256x192 tiles (one
    round), 4000x24000 256x256 tiles. Sampled rows include the last tile-row's
    tail."""
    announce("tp_qgemm_w8a8 large ragged", m, n, k)
    wl = W.TINY.with_(name=f"ragged{m}x{n}", m=m, n=n, k=k, seed=m + n, act_outliers=3, w_outliers=3, path="w8a8")
    _w8a8_case(wl, row_sel=sample_rows(m, 24, seed=n))


@pytest.mark.parametrize("m,n,k", [(1024, 3072, 1024), (600, 1000, 1024), (2000, 5184, 1024), (4096, 9216, 256)])
def test_w8a8_large_output_views(m, n, k):
    """The multi-stage W8A8 epilogue on dense and padded outputs: the int32
    accumulators are exact, the fp32 output is (float(acc) * sa) * s rounded
    as written, an output view with odd row pitches and a base 4 bytes past a
    16-byte boundary gets the same bytes and nothing outside the view, and
    the bf16 output (dense or padded) is the RNE rounding of the fp32 one.
    Shapes: 128x192 tiles, a ragged 600x1000 split along K (partial sums),
    256x192 tiles and 256x288 tiles (4096x9216)."""
    d = dev()
    announce("tp_qgemm_w8a8_prequantized output views", m, n, k)
    g = torch.Generator().manual_seed(m + n)
    qa = torch.randint(-127, 128, (m, k), dtype=torch.int8, generator=g).to(d)
    q = torch.randint(-127, 128, (n, k), dtype=torch.int8, generator=g).to(d)
    sa = (torch.rand(m, generator=g) + 0.5).to(d)
    s = (torch.rand(n, generator=g) + 0.5).to(d)
    acc = torch.empty((m, n), dtype=torch.int32, device=d)
    y = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s, acc=acc)
    racc = (qa.cpu().to(torch.float64) @ q.cpu().to(torch.float64).T).to(torch.int64)  # exact: |sum| < 2^53
    assert torch.equal(acc.cpu().to(torch.int64), racc), "int32 accumulators differ"
    ref = (racc.to(torch.float32) * sa.cpu()[:, None]) * s.cpu()[None, :]
    assert torch.equal(y.cpu(), ref), "fp32 output is not (float(acc) * sa) * s"
    # odd pitches and a base 4 bytes past a 16-byte boundary
    ybuf = torch.full((m, n + 3), -1.0, dtype=torch.float32, device=d)
    abuf = torch.full((m, n + 5), -1, dtype=torch.int32, device=d)
    yv = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s, out=ybuf[:, 1:n + 1], acc=abuf[:, 1:n + 1])
    assert torch.equal(yv, y) and torch.equal(abuf[:, 1:n + 1], acc)
    assert bool((ybuf[:, 0] == -1).all()) and bool((ybuf[:, n + 1:] == -1).all()), "stores outside the view"
    assert bool((abuf[:, 0] == -1).all()) and bool((abuf[:, n + 1:] == -1).all()), "stores outside the view"
    ybf = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s, out_dtype=torch.bfloat16)
    assert torch.equal(ybf, y.to(torch.bfloat16)), "bf16 output is not the RNE rounding of the fp32 one"
    bbuf = torch.zeros((m, n + 1), dtype=torch.bfloat16, device=d)
    ybv = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s, out=bbuf[:, :n])
    assert torch.equal(ybv, ybf)


@pytest.mark.parametrize("kind,m,n,k", [("w8", 3000, 5000, 512), ("w4", 4000, 3100, 1024)])
def test_weight_only_large_ragged(kind, m, n, k):
    """Ragged M and N on the large-tile paths (W8 256x256, W4 256x192), with
    the early/late split of the code widening; fp32 output."""
    announce("tp_qgemm", kind, "large ragged", m, n, k)
    wl = W.TINY.with_(name=f"ragged{m}x{n}", m=m, n=n, k=k, seed=m + 2 * n, act_outliers=3, w_outliers=3,
                      path=kind)
    case = _w8_case if kind == "w8" else _w4_case
    got, ref = case(wl, row_sel=sample_rows(m, 24, seed=k), out_dtype=torch.float32)
    err = assert_bf16_path(got, ref, f"{kind} large ragged")
    assert err < 1e-4


@pytest.mark.parametrize("m,n,k", [(1, 256, 256), (100, 200, 768), (129, 385, 512), (257, 131, 1024)])
def test_w8a8_ragged(m, n, k):
    announce("tp_qgemm_w8a8 ragged", m, n, k)
    _w8a8_case(W.TINY.with_(m=m, n=n, k=k, seed=m + 3 * n, act_outliers=2, w_outliers=2, path="w8a8"))


# ------------------------------------------------------------ few rows (M <= 64)
def _small_m_case(kind, wl, rows=None, out_dtype=torch.float32):
    """One small-M product against the oracle; returns the device output."""
    d = dev()
    x, w = W.generate(wl, rows=rows)
    bits = 4 if kind == "w4" else 8
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=bits)
    rq, rs = oracle_weights(wl, w, bits)
    if kind == "w8a8":
        y, qa, sa, acc = tp.tp_qgemm_w8a8(x.to(d), q, s, rotate=True, out_dtype=out_dtype, want_codes=True,
                                          want_acc=True)
        ry, racc, rqa, rsa = oracle.qgemm_w8a8(f64(x), rq, rs)
        assert np.array_equal(host(sa), rsa), "activation scales differ"
        assert np.array_equal(host(qa), rqa), "activation codes differ"
        gacc = host(acc).astype(np.int64)
        assert np.array_equal(gacc, racc), f"{int(np.sum(gacc != racc))} int32 accumulators differ"
        if out_dtype == torch.float32:
            assert_w8a8_out(f64(y), ry, f"w8a8 small-m {wl.name}")
        # the same codes through the prequantized entry point: the same bytes
        y2 = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, s, out_dtype=out_dtype)
        assert torch.equal(y, y2)
    else:
        fn = tp.tp_qgemm_w8 if kind == "w8" else tp.tp_qgemm_w4
        y = fn(x.to(d), q, s, rotate=True, out_dtype=out_dtype)
        ref = (oracle.qgemm_w8 if kind == "w8" else oracle.qgemm_w4)(f64(x), rq, rs)
        err = assert_bf16_path(f64(y), ref, f"{kind} small-m {wl.name}")
        if out_dtype == torch.float32:
            assert err < 1e-4
        y2 = fn(x.to(d), q, s, rotate=True, out_dtype=out_dtype)
        assert torch.equal(y, y2), "split-K result is not reproducible"
    return y


@pytest.mark.parametrize("kind", ["w8", "w4", "w8a8"])
@pytest.mark.parametrize("m,n,k", [(1, 300, 512), (5, 1000, 2560), (8, 4100, 3840), (9, 333, 1280),
                                   (16, 129, 256), (17, 777, 1536), (33, 4000, 768), (64, 515, 3072),
                                   (64, 128, 12288), (3, 20, 12288), (40, 2000, 3072), (57, 3000, 12288)])
def test_small_m_ragged(kind, m, n, k):
    """Few-row products: split-K with several 256-groups per split, ragged N,
    M not a multiple of 16, a single 256-group (no split), and plans with
    several blocks along M whose last block is partly past M."""
    announce("small-m", kind, m, n, k)
    wl = W.TINY.with_(name=f"smallm_{m}_{n}_{k}", m=m, n=n, k=k, seed=m * 31 + n + k, act_outliers=2,
                      w_outliers=2, path=kind)
    _small_m_case(kind, wl)


@pytest.mark.parametrize("name,kind", [("ffn_up", "w8"), ("ffn_down", "w4"), ("dit_qkv", "w8a8"),
                                       ("dit_gateup", "w8a8")])
@pytest.mark.parametrize("rows", [1, 8, 16, 64])
def test_small_m_full_weights(name, kind, rows):
    """The first rows of the full-size workloads against their full weights
    (the M <= 64 sweep the benchmark times), every output element."""
    wl = W.BY_NAME[name]
    announce("small-m full weights", name, kind, rows)
    out = torch.bfloat16 if kind != "w8a8" else torch.float32
    _small_m_case(kind, wl, rows=rows, out_dtype=out)


def test_small_m_bf16_out_and_views():
    """bf16 output of W8A8 and a padded output view on the split-K path."""
    d = dev()
    announce("small-m bf16 out / padded views")
    wl = W.TINY.with_(name="smallm_views", m=20, n=700, k=2048, seed=77, path="w8a8")
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    rq, rs = oracle_weights(wl, w, 8)
    y32 = tp.tp_qgemm_w8a8(x.to(d), q, s, rotate=True)
    ybf = tp.tp_qgemm_w8a8(x.to(d), q, s, rotate=True, out_dtype=torch.bfloat16)
    assert torch.equal(ybf, y32.to(torch.bfloat16)), "bf16 output is not the RNE rounding of the fp32 one"
    cbuf = torch.full((24, 700 + 40), 5.0, dtype=torch.float32, device=d)
    out = cbuf[2:22, 8:708]
    tp.tp_qgemm_w8(x.to(d), q, s, rotate=True, out=out)
    ref = oracle.qgemm_w8(f64(x), rq, rs)
    assert_bf16_path(f64(out), ref, "w8 small-m view")
    assert torch.all(cbuf[:2] == 5.0) and torch.all(cbuf[22:] == 5.0)
    assert torch.all(cbuf[:, :8] == 5.0) and torch.all(cbuf[:, 708:] == 5.0)


@pytest.mark.parametrize("kind,m,n,k", [("w8a8", 4000, 9000, 768), ("w8a8", 3000, 2900, 512), ("w8", 4000, 8000, 512),
                                        ("w4", 300, 3000, 4096), ("w8a8", 500, 1000, 6144), ("w8", 1000, 700, 2048),
                                        ("w4", 4000, 8000, 1024), ("w8a8", 2100, 9000, 256)])
def test_multistage_path_ragged(kind, m, n, k):
    """Shapes large enough for the 256-wide multi-stage kernels, with M and N
    not multiples of the tile: sampled whole rows incl. the last tile row."""
    wl = W.PROJ256.with_(name=f"ragged_{kind}_{m}_{n}_{k}", m=m, n=n, k=k, seed=m + n + k, path=kind,
                         out_dtype="f32" if kind == "w8a8" else "bf16")
    announce("multistage ragged", kind, m, n, k)
    sel = sample_rows(m, 24, seed=k)
    if kind == "w8a8":
        _w8a8_case(wl, row_sel=sel)
    elif kind == "w8":
        got, ref = _w8_case(wl, row_sel=sel)
        assert_bf16_path(got, ref, "w8 multistage ragged")
    else:
        got, ref = _w4_case(wl, row_sel=sel)
        assert_bf16_path(got, ref, "w4 multistage ragged")


def test_multistage_padded_views():
    """Multi-stage W8A8 on a padded, offset activation view and output view."""
    d = dev()
    announce("multistage padded views")
    wl = W.PROJ256.with_(name="padded_views", m=2100, n=9000, k=512, seed=77, path="w8a8", out_dtype="f32")
    x, w = W.generate(wl)
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    abuf = torch.zeros((wl.m + 3, wl.k + 64), dtype=torch.bfloat16, device=d)
    abuf[1:1 + wl.m, 32:32 + wl.k] = x.to(d)
    cbuf = torch.full((wl.m + 2, wl.n + 8), -3.0, dtype=torch.float32, device=d)
    out = cbuf[1:1 + wl.m, 4:4 + wl.n]
    tp.tp_qgemm_w8a8(abuf[1:1 + wl.m, 32:32 + wl.k], q, s, out=out)
    sel = sample_rows(wl.m, 16, seed=3)
    rq, rs = oracle_weights(wl, w, 8)
    ry, _, _, _ = oracle.qgemm_w8a8(f64(x)[sel], rq, rs)
    assert_w8a8_out(f64(out)[sel], ry, "padded views")
    assert torch.all(cbuf[0] == -3.0) and torch.all(cbuf[-1] == -3.0)
    assert torch.all(cbuf[:, :4] == -3.0) and torch.all(cbuf[:, 4 + wl.n:] == -3.0)


def test_w8a8_planted_integers():
    """X = X'.Q and W = W'.Q with integer X', W' whose row maxima are 127:
    the device must return qa = X', sa = 1, acc = X' W'^T, y = acc."""
    d = dev()
    announce("tp_qgemm_w8a8 planted integers")
    rng = np.random.default_rng(30)
    m, n, k = 40, 72, 512
    xv = rng.integers(-127, 128, size=(m, k))
    wv = rng.integers(-127, 128, size=(n, k))
    xv[:, 5] = 127
    wv[:, 9] = -127
    H = oracle.hadamard_matrix(256) / 16.0
    rot = lambda a: np.concatenate([a[:, g * 256:(g + 1) * 256] @ H for g in range(k // 256)], axis=1)
    x = torch.from_numpy(rot(xv.astype(np.float64)).astype(np.float32))
    w = torch.from_numpy(rot(wv.astype(np.float64)).astype(np.float32))
    assert np.array_equal(oracle.rotate_groups(x.numpy()), xv)  # the planted inputs are exact in fp32
    q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    assert np.array_equal(host(q), wv) and np.all(host(s) == 1.0)
    y, qa, sa, acc = tp.tp_qgemm_w8a8(x.to(d), q, s, want_codes=True, want_acc=True)
    ref = xv @ wv.T
    assert np.array_equal(host(qa), xv) and np.all(host(sa) == 1.0)
    assert np.array_equal(host(acc), ref)
    assert np.array_equal(f64(y), ref.astype(np.float64))


def test_w8a8_max_codes_at_large_k():
    """All codes +-127 at K = 12288: acc = +-127^2 K, inside int32."""
    d = dev()
    announce("tp_qgemm_w8a8 extreme codes K=12288")
    m, n, k = 32, 48, 12288
    ones = torch.ones((m, k), dtype=torch.float32)
    ones[1::2] *= -1
    # rotated operand equal to the all-ones rows: pass it pre-rotated
    q = torch.full((n, k), 127, dtype=torch.int8, device=d)
    s = torch.ones(n, dtype=torch.float32, device=d)
    y, qa, sa, acc = tp.tp_qgemm_w8a8(ones.to(d), q, s, rotate=False, want_codes=True, want_acc=True)
    expect = np.where(np.arange(m)[:, None] % 2 == 0, 1, -1) * 127 * 127 * k * np.ones((1, n), dtype=np.int64)
    assert np.array_equal(host(acc).astype(np.int64), expect)


def test_determinism():
    d = dev()
    announce("determinism: repeated calls give identical bytes")
    wl = W.PROJ256
    x, w = W.generate(wl)
    xd = x.to(d)
    q8, s8 = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    q4, s4 = tp.tp_rotate_quantize_weights(w.to(d), bits=4)
    outs = []
    for _ in range(2):
        outs.append((tp.tp_qgemm_w8(xd, q8, s8), tp.tp_qgemm_w4(xd, q4, s4), tp.tp_qgemm_w8a8(xd, q8, s8),
                     tp.tp_hadamard_rotate_rows(xd)))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_empty_inputs_are_noops():
    d = dev()
    announce("empty m / n")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device=d)
    q = torch.zeros((16, 512), dtype=torch.int8, device=d)
    s = torch.ones(16, dtype=torch.float32, device=d)
    assert tp.tp_qgemm_w8(x, q, s).shape == (0, 16)
    assert tp.tp_qgemm_w8a8(x, q, s).shape == (0, 16)
    assert tp.tp_hadamard_rotate_rows(x).shape == (0, 512)


def test_refusal_reaches_python():
    d = dev()
    announce("refusal surfaces as TPError")
    x = torch.zeros((4, 300), dtype=torch.bfloat16, device=d)
    with pytest.raises(tp.TPError) as e:
        tp.tp_hadamard_rotate_rows(x)
    assert e.value.status_name == "TP_ERR_K_NOT_MULTIPLE_OF_256"


@pytest.mark.parametrize("kind", ["w8", "w4"])
@pytest.mark.parametrize("m,n,k,dt", [(1, 300, 512, "f32"), (8, 1000, 3072, "bf16"), (3, 20, 12288, "f32"),
                                      (9, 333, 1280, "f32"), (16, 4100, 3072, "bf16"), (40, 2000, 3072, "f32"),
                                      (64, 515, 12288, "bf16"), (5, 700, 12288, "bf16")])
def test_small_m_rotation_matches_two_step(kind, m, n, k, dt):
    """Few rows with the rotation requested (fp32 and bf16 operands, GEMV and
    split-K plans): the bytes of rotating first to bf16 and multiplying the
    rotated operand."""
    d = dev()
    announce("small-m rotation", kind, m, n, k, dt)
    g = torch.Generator().manual_seed(m * 7 + n + k)
    x = torch.randn((m, k), generator=g, dtype=torch.float64)
    x[:, :: max(1, k // 13)] *= 30.0
    x = x.to(torch.float32 if dt == "f32" else torch.bfloat16).to(d)
    w = (torch.randn((n, k), generator=g, dtype=torch.float64) * 0.02).to(torch.float32).to(d)
    q, s = tp.tp_rotate_quantize_weights(w, bits=4 if kind == "w4" else 8)
    fn = tp.tp_qgemm_w8 if kind == "w8" else tp.tp_qgemm_w4
    for out in (torch.bfloat16, torch.float32):
        y1 = fn(x, q, s, rotate=True, out_dtype=out)
        xr = tp.tp_hadamard_rotate_rows(x, out_dtype=torch.bfloat16)
        y2 = fn(xr, q, s, rotate=False, out_dtype=out)
        assert torch.equal(y1, y2), f"{int((y1 != y2).sum())} outputs differ from rotate-then-multiply"
