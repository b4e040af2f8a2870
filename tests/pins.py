"""Pins for the CPU oracle: checks against facts the pages and the mathematics
fix, written so that a plausible mistake in the oracle (a dropped term, a wrong
sign or index, a transposed operand, another Hadamard ordering, a swapped
nibble, a wrong clamp) fails at least one of them.

Each check takes the function(s) under test as arguments and raises
AssertionError on failure. tests/test_oracle.py runs them on the oracle;
tests/test_controls.py runs them on deliberately broken copies and expects
them to fail.
"""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


# --------------------------------------------------------------------------- H
def check_hadamard(hadamard_matrix):
    """Closed form and construction of the order-256 Sylvester matrix.

    * the order-8 matrix equals the textbook table in golden/sylvester_h8.txt;
    * the order-256 matrix equals the Sylvester doubling H_2n = [[H, H], [H, -H]]
      built here independently with Kronecker products;
    * it is symmetric, has entries +-1 and H . H^T = 256 I.
    """
    h8 = hadamard_matrix(8)
    assert np.array_equal(h8, _load_matrix("sylvester_h8.txt")), "H8 differs from the textbook table"
    h = np.array([[1.0]])
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    for _ in range(8):
        h = np.kron(h2, h)
    got = hadamard_matrix(256)
    assert got.shape == (256, 256)
    assert np.array_equal(got, h), "order-256 matrix is not the Sylvester doubling"
    assert np.array_equal(got, got.T), "not symmetric"
    assert np.all(np.abs(got) == 1.0), "entries must be +-1"
    assert np.array_equal(got @ got.T, 256.0 * np.eye(256)), "H H^T != 256 I"


# -------------------------------------------------------------------- rotation
def _butterfly_fwht(v):
    """Independent in-place fast Walsh-Hadamard transform of one 256-vector
    (natural order), scaled by 1/16. Used only to cross-check the oracle's
    dense product on dyadic inputs, where both are exact."""
    a = [float(t) for t in v]
    h = 1
    while h < len(a):
        for i in range(0, len(a), 2 * h):
            for j in range(i, i + h):
                x, y = a[j], a[j + h]
                a[j], a[j + h] = x + y, x - y
        h *= 2
    return np.array(a) / 16.0


def check_rotation(rotate_groups, hadamard_matrix, seed=11):
    rng = np.random.default_rng(seed)
    H = hadamard_matrix(256)
    # Special cases with closed forms.
    ones = np.ones((1, 256))
    e0 = np.zeros((1, 256)); e0[0, 0] = 16.0
    assert np.array_equal(rotate_groups(ones), e0), "1 . Q must be 16 e0"
    for j in (0, 1, 5, 128, 255):
        ej = np.zeros((1, 256)); ej[0, j] = 1.0
        assert np.array_equal(rotate_groups(ej)[0], H[j] / 16.0), "e_j . Q must be H[j]/16"
        hi = H[j][None, :]
        ek = np.zeros((1, 256)); ek[0, j] = 16.0
        assert np.array_equal(rotate_groups(hi), ek), "H[j] . Q must be 16 e_j"
    # Exact agreement with an independent butterfly FWHT on dyadic integers.
    x = rng.integers(-1000, 1000, size=(3, 512)).astype(np.float64)
    got = rotate_groups(x)
    for r in range(3):
        for g in range(2):
            ref = _butterfly_fwht(x[r, 256 * g:256 * (g + 1)])
            assert np.array_equal(got[r, 256 * g:256 * (g + 1)], ref), "rotation != butterfly FWHT"
    # Group locality: a vector supported on one group stays in that group.
    v = np.zeros((1, 768)); v[0, 256:512] = rng.standard_normal(256)
    rv = rotate_groups(v)
    assert np.all(rv[0, :256] == 0) and np.all(rv[0, 512:] == 0), "rotation leaks across groups"
    # Involution (Q Q = I) and norm preservation per group.
    y = rng.standard_normal((4, 768))
    back = rotate_groups(rotate_groups(y))
    assert np.max(np.abs(back - y)) <= 1e-13 * np.max(np.abs(y)), "rotating twice must give back x"
    ry = rotate_groups(y).reshape(4, 3, 256)
    assert np.allclose(np.linalg.norm(ry, axis=2), np.linalg.norm(y.reshape(4, 3, 256), axis=2), rtol=1e-13)


def check_product_invariance(rotate_groups, seed=12):
    """Rotating both operands leaves the fp64 product unchanged (1e-12 rel)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((16, 1024))
    w = rng.standard_normal((24, 1024))
    x[:, 7] *= 30.0
    w[:, 300] *= 20.0
    ref = x @ w.T
    got = rotate_groups(x) @ rotate_groups(w).T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 1e-12, f"rotated product differs: {rel}"


# ------------------------------------------------------------------ bf16 round
def check_bf16(bf16_round):
    import torch
    with open(os.path.join(GOLDEN, "bf16_values.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            v, _bits, want = line.split()
            got = bf16_round(np.array([float(v)]))[0]
            assert got == float(want), f"bf16({v}) = {got}, want {want}"
    # Agrees with torch's fp32 -> bf16 conversion (nearest, ties to even) on
    # values that are exact in fp32, ties included.
    rng = np.random.default_rng(13)
    base = rng.standard_normal(20000).astype(np.float32)
    bits = base.view(np.uint32)
    ties = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([base, ties, base * np.float32(1e-30), base * np.float32(1e30)])
    ref = torch.from_numpy(vals).to(torch.bfloat16).double().numpy()
    got = bf16_round(vals.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding differs from torch on fp32-exact values"
    big = np.array([3.3e38, 3.4e38, -3.5e38])
    assert np.isinf(bf16_round(big)[2]) and np.isfinite(bf16_round(big)[0])


# -------------------------------------------------------------- quantization
def check_weight_int8(quantize_weights_int8, rotate_groups, seed=14):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((20, 768))).astype(np.float32)
    w[:, [3, 400]] *= 20.0
    w[5, :] = 0.0
    q, s = quantize_weights_int8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32 and q.shape == w.shape and s.shape == (20,)
    wr = rotate_groups(w)
    amax = np.max(np.abs(wr), axis=1)
    # zero row
    assert s[5] == 0.0 and np.all(q[5] == 0)
    nz = np.arange(20) != 5
    s64 = s.astype(np.float64)
    # the scale is amax/127 rounded once to fp32
    assert np.all(np.abs(s64[nz] - amax[nz] / 127.0) <= 2.0 ** -24 * amax[nz] / 127.0)
    # every element within half a step of its source
    err = np.abs(wr - q.astype(np.float64) * s64[:, None])
    assert np.all(err[nz] <= 0.5 * s64[nz, None] * (1 + 1e-12)), "dequantized weight off by more than s/2"
    # the amax element maps to +-127, and no code exceeds it
    am = np.argmax(np.abs(wr), axis=1)
    assert np.all(np.abs(q[nz, am[nz]]) == 127) and np.max(np.abs(q)) == 127
    # signs agree
    assert np.all((np.sign(q) == np.sign(wr)) | (q == 0))


def check_weight_int4(quantize_weights_int4, unpack_int4, rotate_groups, seed=15):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((12, 768))).astype(np.float32)
    w[:, [10, 600]] *= 20.0
    w[2, 256:512] = 0.0
    p, s = quantize_weights_int4(w)
    assert p.dtype == np.uint8 and p.shape == (12, 384) and s.shape == (12, 3) and s.dtype == np.float32
    q = unpack_int4(p).reshape(12, 3, 256)
    wr = rotate_groups(w).reshape(12, 3, 256)
    amax = np.max(np.abs(wr), axis=2)
    assert s[2, 1] == 0.0 and np.all(q[2, 1] == 0)
    s64 = s.astype(np.float64)
    nz = s64 > 0
    assert np.all(np.abs(s64[nz] - amax[nz] / 7.0) <= 2.0 ** -24 * amax[nz] / 7.0)
    err = np.abs(wr - q * s64[:, :, None])
    assert np.all(err[nz] <= 0.5 * s64[nz][:, None] * (1 + 1e-12)), "int4 dequant off by more than s/2"
    am = np.argmax(np.abs(wr), axis=2)
    qa = np.take_along_axis(np.abs(q), am[:, :, None], axis=2)[:, :, 0]
    assert np.all(qa[nz] == 7) and np.max(np.abs(q)) == 7
    assert np.all((np.sign(q) == np.sign(wr)) | (q == 0))


def _planted(rng, rows, k, qmax, per_group):
    """Integer matrix with |v| <= qmax and the extreme value hit in every row
    (or every 256-group), plus power-of-two multipliers."""
    v = rng.integers(-qmax, qmax + 1, size=(rows, k))
    if per_group:
        for g in range(k // 256):
            v[:, 256 * g + rng.integers(0, 256)] = qmax * rng.choice([-1, 1], size=rows)
        c = 2.0 ** rng.integers(-12, 3, size=(rows, k // 256))
    else:
        v[np.arange(rows), rng.integers(0, k, size=rows)] = qmax * rng.choice([-1, 1], size=rows)
        c = 2.0 ** rng.integers(-12, 3, size=rows)
    return v, c


def check_planted_int8(quantize_weights_int8, hadamard_matrix, seed=16):
    """W = W' . Q with integer W' (amax 127 c, c a power of two): then the
    quantizer must return exactly q = W' and s = c."""
    rng = np.random.default_rng(seed)
    Q = hadamard_matrix(256) / 16.0
    v, c = _planted(rng, 9, 512, 127, per_group=False)
    wprime = v * c[:, None]
    w = np.concatenate([wprime[:, :256] @ Q, wprime[:, 256:] @ Q], axis=1)
    q, s = quantize_weights_int8(w)
    assert np.array_equal(q.astype(np.int64), v), "planted codes not recovered"
    assert np.array_equal(s.astype(np.float64), c), "planted scales not recovered"


def check_planted_int4(quantize_weights_int4, unpack_int4, hadamard_matrix, seed=17):
    rng = np.random.default_rng(seed)
    Q = hadamard_matrix(256) / 16.0
    v, c = _planted(rng, 7, 768, 7, per_group=True)
    wprime = v * np.repeat(c, 256, axis=1)
    w = np.concatenate([wprime[:, 256 * g:256 * (g + 1)] @ Q for g in range(3)], axis=1)
    p, s = quantize_weights_int4(w)
    assert np.array_equal(unpack_int4(p), v), "planted int4 codes not recovered"
    assert np.array_equal(s.astype(np.float64), c), "planted int4 scales not recovered"


def check_pack(pack_int4, unpack_int4):
    """Two's-complement nibbles, even column in the low nibble."""
    table = {(-1, 0): 0x0F, (0, -1): 0xF0, (7, -7): 0x97, (-7, 7): 0x79, (1, 2): 0x21, (-8, 0): 0x08, (3, -4): 0xC3}
    for (a, b), byte in table.items():
        got = pack_int4(np.array([[a, b]]))
        assert got.dtype == np.uint8 and got[0, 0] == byte, f"pack({a},{b}) = {got[0, 0]:#x}, want {byte:#x}"
    pairs = np.array([(a, b) for a in range(-7, 8) for b in range(-7, 8)])
    assert len(pairs) == 225
    codes = pairs.reshape(1, -1)
    assert np.array_equal(unpack_int4(pack_int4(codes)), codes)


# -------------------------------------------------------------------- products
def check_int_accumulate(int_accumulate, seed=18):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, size=(5, 512))
    b = rng.integers(-127, 128, size=(4, 512))
    got = int_accumulate(a.astype(np.int8), b.astype(np.int8))
    for i in range(5):
        for j in range(4):
            assert got[i, j] == sum(int(a[i, t]) * int(b[j, t]) for t in range(512))
    k = 12288
    full = np.full((2, k), 127, dtype=np.int8)
    neg = np.full((3, k), -127, dtype=np.int8)
    got = int_accumulate(full, neg)
    assert np.all(got == -127 * 127 * k) and got.dtype == np.int64


def check_products_bruteforce(qgemm_w8, qgemm_w4, qgemm_w8a8, rotate_groups, bf16_round,
                              quantize_weights_int8, quantize_weights_int4, unpack_int4, seed=19):
    """Pure-Python loops over the quantized operands on tiny shapes."""
    rng = np.random.default_rng(seed)
    for m, n, k in ((3, 5, 256), (6, 4, 512)):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, 2] *= 30.0
        w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
        xr = rotate_groups(x)
        xb = bf16_round(xr)
        q8, s8 = quantize_weights_int8(w)
        y8 = qgemm_w8(x, q8, s8)
        p4, s4 = quantize_weights_int4(w)
        q4 = unpack_int4(p4)
        y4 = qgemm_w4(x, p4, s4)
        y, acc, qa, sa = qgemm_w8a8(x, q8, s8)
        amax = np.max(np.abs(xr), axis=1)
        for i in range(m):
            sai = float(np.float32(amax[i] / 127.0))
            assert float(sa[i]) == sai
            for t in range(k):
                want = 0 if sai == 0 else int(max(-127, min(127, np.rint(xr[i, t] / sai))))
                assert int(qa[i, t]) == want
            for j in range(n):
                ref8 = sum(float(xb[i, t]) * int(q8[j, t]) for t in range(k)) * float(s8[j])
                ref4 = sum(float(xb[i, t]) * int(q4[j, t]) * float(s4[j, t // 256]) for t in range(k))
                refacc = sum(int(qa[i, t]) * int(q8[j, t]) for t in range(k))
                assert abs(y8[i, j] - ref8) <= 1e-12 * max(1.0, abs(ref8)), "w8 product"
                assert abs(y4[i, j] - ref4) <= 1e-12 * max(1.0, abs(ref4)), "w4 product"
                assert acc[i, j] == refacc, "w8a8 accumulator"
                refy = refacc * float(sa[i]) * float(s8[j])
                assert abs(y[i, j] - refy) <= 1e-15 * max(1e-30, abs(refy)) + 1e-300, "w8a8 output"


def check_planted_w8a8(qgemm_w8a8, hadamard_matrix, seed=20):
    """Integer X', W' with power-of-two row scales, X = X'.Q and W = W'.Q:
    qa = X', sa = c_m, acc = X' W'^T exactly, y = acc c_m c_n exactly."""
    rng = np.random.default_rng(seed)
    Q = hadamard_matrix(256) / 16.0
    xv, xc = _planted(rng, 6, 512, 127, per_group=False)
    wv, wc = _planted(rng, 5, 512, 127, per_group=False)
    rot = lambda a: np.concatenate([a[:, :256] @ Q, a[:, 256:] @ Q], axis=1)
    x = rot(xv * xc[:, None])
    w_codes = wv.astype(np.int8)
    y, acc, qa, sa = qgemm_w8a8(x, w_codes, wc.astype(np.float32))
    assert np.array_equal(qa.astype(np.int64), xv), "planted activation codes"
    assert np.array_equal(sa.astype(np.float64), xc), "planted activation scales"
    ref = np.array([[sum(int(xv[i, t]) * int(wv[j, t]) for t in range(512)) for j in range(5)] for i in range(6)])
    assert np.array_equal(acc, ref), "planted accumulator"
    assert np.array_equal(y, ref * xc[:, None] * wc[None, :]), "planted output"


def check_rotation_helps(quantize_weights_int8, dequantize_int8, rotate_groups, seed=21):
    """Sanity of the method's purpose (not parity): with outlier input columns,
    rotating before per-row int8 lowers the weight error measured in the
    original basis (the dequantized rotated weight is rotated back)."""
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((64, 1024))).astype(np.float32)
    w[:, rng.choice(1024, 5, replace=False)] *= 20.0
    q, s = quantize_weights_int8(w)
    back = rotate_groups(dequantize_int8(q, s))
    err_rot = np.linalg.norm(back - w) / np.linalg.norm(w)
    s0 = np.max(np.abs(w), axis=1) / 127.0
    plain = np.clip(np.rint(w / s0[:, None]), -127, 127) * s0[:, None]
    err_plain = np.linalg.norm(plain - w) / np.linalg.norm(w)
    assert err_rot < 0.5 * err_plain, (err_rot, err_plain)


# ------------------------------------------------------------- FFN middle
def check_swiglu(silu_mul, swiglu_bf16, seed=23):
    """SwiGLU h = bf16(silu(g) * u), silu(x) = x / (1 + e^-x) (reading R15).

    * closed forms: sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, so
      silu(ln 3) u = 3/4 ln 3 u and silu(-ln 3) u = -1/4 ln 3 u; silu(0) = 0;
      for g >= 64, 1 + e^-g rounds to 1 in fp64 and silu(g) u = g u exactly;
    * the identity silu(x) - silu(-x) = x on random x;
    * bf16 values worked by hand: bf16(3/2 ln 3) = 211/128 and
      bf16(-1/2 ln 3) = -141/256 (ln 3 = 1.0986...);
    * rounding once, ties to even: with g = 64 and u = v / 64 (both exact),
      h = bf16(v): v = 1 + 2^-8 (a tie) gives 1, v = 1 + 3 2^-8 (a tie) gives
      1 + 2^-6, and v = 1 + 2^-8 + 2^-30 (just above the tie, within an fp32
      half-ulp of it, so rounding through fp32 first would give 1) gives
      1 + 2^-7.
    """
    ln3 = np.log(3.0)
    for u in (1.0, -2.5, 7.0):
        assert abs(silu_mul(ln3, u) - 0.75 * ln3 * u) <= 1e-15 * abs(ln3 * u), "silu(ln 3) != 3/4 ln 3"
        assert abs(silu_mul(-ln3, u) + 0.25 * ln3 * u) <= 1e-15 * abs(ln3 * u), "silu(-ln 3) != -1/4 ln 3"
        assert silu_mul(0.0, u) == 0.0
        assert silu_mul(64.0, u) == 64.0 * u
    x = np.random.default_rng(seed).uniform(-20, 20, size=1000)
    d = silu_mul(x, 1.0) - silu_mul(-x, 1.0)
    assert np.all(np.abs(d - x) <= 1e-14 * (1 + np.abs(x))), "silu(x) - silu(-x) != x"
    assert swiglu_bf16(ln3, 2.0) == 211.0 / 128.0
    assert swiglu_bf16(-ln3, 2.0) == -141.0 / 256.0
    assert swiglu_bf16(64.0, (1 + 2.0 ** -8) / 64) == 1.0, "tie must round to even (down)"
    assert swiglu_bf16(64.0, (1 + 3 * 2.0 ** -8) / 64) == 1 + 2.0 ** -6, "tie must round to even (up)"
    assert swiglu_bf16(64.0, (1 + 2.0 ** -8 + 2.0 ** -30) / 64) == 1 + 2.0 ** -7, "rounded twice"
    g = np.array([[ln3, -ln3], [64.0, 0.0]])
    u = np.array([[2.0, 2.0], [(1 + 2.0 ** -8) / 64, 5.0]])
    assert np.array_equal(swiglu_bf16(g, u), np.array([[211 / 128, -141 / 256], [1.0, 0.0]])), "elementwise"


def check_ffn_middle(ffn_middle_int8, ffn_middle_rotated, quantize_activations_int8, bf16_round,
                     hadamard_matrix, seed=24):
    """The down projection's input from gate and up (reading R16).

    Planted rows: xs with entries in {-1, 0, 1} and a 1 in every row; h = xs Q
    per 256-group (multiples of 1/16 up to 16 in magnitude, so bf16-exact).
    With g = 64 (silu(64) u = 64 u exactly) and u = h / 64, SwiGLU gives h
    back, the rotation gives xs, the row maximum is 1, the scale is
    fp32(1/127) and the codes are 127 xs. A random case must equal rotating
    and quantizing bf16(silu(g) u) directly.
    """
    rng = np.random.default_rng(seed)
    m, k = 4, 512
    xs = rng.integers(-1, 2, size=(m, k)).astype(np.float64)
    xs[:, 3] = 1.0
    q = hadamard_matrix(256) / 16.0
    h = np.concatenate([xs[:, j * 256:(j + 1) * 256] @ q for j in range(k // 256)], axis=1)
    assert np.array_equal(bf16_round(h), h), "planted rows must be bf16-exact"
    g = np.full((m, k), 64.0)
    qa, sa = ffn_middle_int8(g, h / 64.0)
    assert np.all(sa == np.float32(1.0 / 127.0)), "scale of a row whose rotated maximum is 1"
    assert np.array_equal(qa, (127 * xs).astype(np.int8)), "codes of the planted rows"
    assert np.array_equal(ffn_middle_rotated(g, h / 64.0), xs), "rotated planted rows"
    gg = rng.standard_normal((3, 768))
    uu = rng.standard_normal((3, 768))
    q1, s1 = ffn_middle_int8(gg, uu)
    q2, s2 = quantize_activations_int8(bf16_round(gg * uu / (1 + np.exp(-gg))), rotate=True)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2), "not the quantized rotation of bf16(silu(g) u)"


# ------------------------------------------------------------------- W4A8
def check_w4a8(qgemm_w4a8, qgemm_w8a8, quantize_weights_int4, unpack_int4, pack_int4, rotate_groups,
               hadamard_matrix, seed=25):
    """W4A8 (reading R18): y = sa[m] * sum_g s[n, g] * acc_g[m, n].

    * pure-Python loops over the quantized operands on tiny shapes (codes,
      per-group accumulators and output);
    * with one scale for all groups of a weight row, W4A8 is the W8A8 product
      of the same codes with that per-row scale;
    * planted integers: X = X' Q with integer X' (row maximum 127 c, c a power
      of two) and integer int4 codes with power-of-two group scales give
      qa = X', sa = c and y in closed form, exactly.
    """
    rng = np.random.default_rng(seed)
    for m, n, k in ((3, 5, 256), (4, 3, 768)):
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, 5] *= 30.0
        w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
        p4, s4 = quantize_weights_int4(w)
        q4 = unpack_int4(p4)
        y, acc, qa, sa = qgemm_w4a8(x, p4, s4)
        assert acc.shape == (k // 256, m, n)
        for i in range(m):
            for j in range(n):
                tot = 0.0
                for g in range(k // 256):
                    a = sum(int(qa[i, t]) * int(q4[j, t]) for t in range(256 * g, 256 * g + 256))
                    assert acc[g, i, j] == a, "w4a8 group accumulator"
                    tot += float(s4[j, g]) * a
                ref = tot * float(sa[i])
                assert abs(y[i, j] - ref) <= 1e-12 * max(1e-30, abs(ref)) + 1e-300, "w4a8 output"
    # equal group scales: the W8A8 product of the same codes
    x = rng.standard_normal((5, 512))
    codes = rng.integers(-7, 8, size=(4, 512))
    c = np.float32([0.5, 0.003, 1.25, 7.0])
    y4, _, qa4, sa4 = qgemm_w4a8(x, pack_int4(codes), np.repeat(c[:, None], 2, axis=1))
    y8, _, qa8, sa8 = qgemm_w8a8(x, codes.astype(np.int8), c)
    assert np.array_equal(qa4, qa8) and np.array_equal(sa4, sa8)
    assert np.allclose(y4, y8, rtol=1e-14, atol=0), "equal group scales must give the W8A8 product"
    # planted integers
    Q = hadamard_matrix(256) / 16.0
    xv = rng.integers(-127, 128, size=(3, 512)).astype(np.float64)
    xv[:, 7] = 127.0
    cx = np.array([1.0, 0.25, 8.0])
    x = np.concatenate([(xv * cx[:, None])[:, g * 256:(g + 1) * 256] @ Q for g in range(2)], axis=1)
    wq = rng.integers(-7, 8, size=(2, 512))
    ws = np.float32([[0.5, 2.0], [0.125, 4.0]])
    y, acc, qa, sa = qgemm_w4a8(x, pack_int4(wq), ws)
    assert np.array_equal(qa.astype(np.int64), xv.astype(np.int64)), "planted activation codes"
    assert np.array_equal(sa.astype(np.float64), cx), "planted activation scales"
    for i in range(3):
        for j in range(2):
            want = cx[i] * sum(float(ws[j, g]) * sum(int(xv[i, t]) * int(wq[j, t]) for t in range(256 * g, 256 * g + 256))
                               for g in range(2))
            assert y[i, j] == want, "planted W4A8 output"


# ------------------------------------------------------------------ loader
def check_loader(dequantize_unrotate, requantize, quantize_weights_int8, quantize_weights_int4, pack_int4,
                 hadamard_matrix, seed=26):
    """Undoing a rotated, quantized weight and requantizing it (R19, R20).

    * closed form: codes 127 at one position j of a group, scale s, give that
      group's row 127 s H[j, :] / 16 and zeros elsewhere;
    * un-rotation undoes the rotation: for quantizer outputs, every 256-group
      of W_hat is within sqrt(256) s / 2 of W in the 2-norm (the codes' error is
      at most s / 2 per element in the rotated domain and Q is orthonormal);
    * requantizing to the same width is the identity on quantizer outputs
      (int8 and int4);
    * planted int8 -> int4: codes 18 t with t in [-7, 7] (a 7 in every group)
      and a power-of-two scale c give t and 18 c;
    * int4 -> int8 on planted power-of-two group scales, against the R3/R4 rule
      written out here.
    """
    rng = np.random.default_rng(seed)
    h = hadamard_matrix(256)
    q = np.zeros((2, 512), dtype=np.int8)
    q[0, 37] = 127
    q[1, 256 + 200] = -127
    s = np.float32([0.5, 1.0 / 127.0])
    w = dequantize_unrotate(q, s, 8)
    assert np.array_equal(w[0, :256], 127 * float(s[0]) * h[37] / 16.0) and np.all(w[0, 256:] == 0)
    assert np.array_equal(w[1, 256:], -127 * float(s[1]) * h[200] / 16.0) and np.all(w[1, :256] == 0)
    wt = (0.02 * rng.standard_normal((6, 768))).astype(np.float32)
    wt[:, 11] *= 20.0
    q8, s8 = quantize_weights_int8(wt)
    wh = dequantize_unrotate(q8, s8, 8)
    err = np.linalg.norm((wh - wt).reshape(6, 3, 256), axis=2)
    assert np.all(err <= 16.0 * s8[:, None] / 2.0 * (1 + 1e-12)), "un-rotation does not undo the rotation"
    q8b, s8b = requantize(q8, s8, 8, 8)
    assert np.array_equal(q8b, q8) and np.array_equal(s8b, s8), "int8 -> int8 must be the identity"
    p4, s4 = quantize_weights_int4(wt)
    p4b, s4b = requantize(p4, s4, 4, 4)
    assert np.array_equal(p4b, p4) and np.array_equal(s4b, s4), "int4 -> int4 must be the identity"
    t = rng.integers(-7, 8, size=(3, 512))
    t[:, 5] = 7
    t[:, 300] = -7
    c = np.float32([0.25, 1.0, 2.0 ** -10])
    p, sc = requantize((18 * t).astype(np.int8), c, 8, 4)
    assert np.array_equal(p, pack_int4(t)), "planted int8 -> int4 codes"
    assert np.array_equal(sc, np.repeat((18 * c)[:, None], 2, axis=1).astype(np.float32)), "planted int4 scales"
    sg = np.float32([[0.5, 2.0], [0.125, 0.125], [4.0, 1.0]])
    q8c, s8c = requantize(pack_int4(t), sg, 4, 8)
    for r in range(3):
        vals = [int(t[r, j]) * float(sg[r, j // 256]) for j in range(512)]
        sr = np.float32(max(abs(v) for v in vals) / 127.0)
        assert s8c[r] == sr, "int4 -> int8 scale"
        want = [max(-127, min(127, int(np.rint(v / float(sr))))) for v in vals]
        assert list(q8c[r].astype(int)) == want, "int4 -> int8 codes"


# -------------------------------------------------------------------- LoRA
def check_lora(lora_add, rotate_groups, seed=27):
    """The side path c + alpha (x A^T) B^T (reading R21).

    * pure-Python loops on a tiny case;
    * rank one with unit vectors: A = e_i, B = e_j adds alpha x[:, i] to
      column j only;
    * alpha = 0 leaves c unchanged, and the result is linear in alpha;
    * rotating x and A alike leaves it unchanged.
    """
    rng = np.random.default_rng(seed)
    m, n, k, r = 3, 5, 256, 4
    x = rng.standard_normal((m, k))
    a = rng.standard_normal((r, k))
    b = rng.standard_normal((n, r))
    c = rng.standard_normal((m, n))
    y = lora_add(c, x, a, b, 0.75)
    for i in range(m):
        for j in range(n):
            t = [sum(x[i, kk] * a[jj, kk] for kk in range(k)) for jj in range(r)]
            want = c[i, j] + 0.75 * sum(t[jj] * b[j, jj] for jj in range(r))
            assert abs(y[i, j] - want) <= 1e-12 * (1 + abs(want)), "side path loops"
    e_a = np.zeros((1, k))
    e_a[0, 17] = 1.0
    e_b = np.zeros((n, 1))
    e_b[2, 0] = 1.0
    y1 = lora_add(c, x, e_a, e_b, 2.0)
    want = c.copy()
    want[:, 2] += 2.0 * x[:, 17]
    assert np.array_equal(y1, want), "rank one with unit vectors"
    assert np.array_equal(lora_add(c, x, a, b, 0.0), c), "alpha = 0"
    d1 = lora_add(c, x, a, b, 1.0) - c
    d3 = lora_add(c, x, a, b, 3.0) - c
    assert np.allclose(d3, 3.0 * d1, rtol=1e-13, atol=1e-13), "linear in alpha"
    y2 = lora_add(c, rotate_groups(x), rotate_groups(a), b, 0.75)
    assert np.allclose(y2, y, rtol=1e-12, atol=1e-12), "rotation invariance"
