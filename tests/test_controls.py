"""Planted-fault controls: each pin must turn red on a deliberately broken copy
of an oracle function. The faults are planted here, in CPU-only copies of the
oracle's arithmetic; nothing touches a GPU."""

import numpy as np
import pytest

import oracle
from oracle import quantize as oq
from tests import pins


def _walsh_ordered(n=256):
    """Hadamard rows sorted by number of sign changes (sequency order)."""
    h = oracle.hadamard_matrix(n)
    changes = np.sum(h[:, 1:] != h[:, :-1], axis=1)
    return h[np.argsort(changes)][:, np.argsort(changes)]


def _rotate_with(hmat, scale=1.0 / 16.0):
    def rot(x):
        x = np.asarray(x, dtype=np.float64)
        r, k = x.shape
        return np.matmul(x.reshape(r, k // 256, 256), hmat * scale).reshape(r, k)
    return rot


def test_walsh_ordering_caught():
    with pytest.raises(AssertionError):
        pins.check_hadamard(_walsh_ordered)


def test_missing_normalization_caught():
    with pytest.raises(AssertionError):
        pins.check_rotation(_rotate_with(oracle.hadamard_matrix(256), 1.0), oracle.hadamard_matrix)


def test_double_normalization_caught():
    with pytest.raises(AssertionError):
        pins.check_product_invariance(_rotate_with(oracle.hadamard_matrix(256), 1.0 / 256.0))


def test_rotation_across_groups_caught():
    def rot_full(x):
        x = np.asarray(x, dtype=np.float64)
        k = x.shape[1]
        return x @ (oracle.hadamard_matrix(k) / np.sqrt(k))
    with pytest.raises(AssertionError):
        pins.check_rotation(rot_full, oracle.hadamard_matrix)


def test_swapped_nibbles_caught():
    def pack_swapped(q):
        q = np.asarray(q, dtype=np.int64)
        return ((q[..., 1::2] & 0xF) | ((q[..., 0::2] & 0xF) << 4)).astype(np.uint8)
    with pytest.raises(AssertionError):
        pins.check_pack(pack_swapped, oracle.unpack_int4)


def test_wrong_qmax_caught():
    def q8_128(w):
        wr = oracle.rotate_groups(w)
        s = (np.max(np.abs(wr), axis=1) / 128.0).astype(np.float32)
        return oq._codes(wr, s[:, None], 127).astype(np.int8), s
    with pytest.raises(AssertionError):
        pins.check_weight_int8(q8_128, oracle.rotate_groups)


def test_truncating_codes_caught():
    def q8_trunc(w):
        wr = oracle.rotate_groups(w)
        s = (np.max(np.abs(wr), axis=1) / 127.0).astype(np.float32)
        q = np.where(s[:, None] > 0, np.trunc(wr / np.maximum(s[:, None], 1e-38)), 0)
        return np.clip(q, -127, 127).astype(np.int8), s
    with pytest.raises(AssertionError):
        pins.check_weight_int8(q8_trunc, oracle.rotate_groups)


def test_int4_range_8_caught():
    def q4_8(w):
        wr = oracle.rotate_groups(w)
        n, k = wr.shape
        g = wr.reshape(n, k // 256, 256)
        s = (np.max(np.abs(g), axis=2) / 8.0).astype(np.float32)
        return oracle.pack_int4(oq._codes(g, s[:, :, None], 8).reshape(n, k)), s
    with pytest.raises(AssertionError):
        pins.check_weight_int4(q4_8, oracle.unpack_int4, oracle.rotate_groups)


def test_truncating_bf16_caught():
    def bf16_trunc(x):
        x32 = np.asarray(x, dtype=np.float32)
        return (x32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    with pytest.raises(AssertionError):
        pins.check_bf16(bf16_trunc)


def test_w4_scale_index_caught():
    def w4_tiled(x, packed, s, rotate=True):
        xb = oracle.bf16_round(oracle.rotate_groups(x))
        q = oracle.unpack_int4(packed).astype(np.float64)
        return xb @ (q * np.tile(np.asarray(s, np.float64), (1, 256))).T
    with pytest.raises(AssertionError):
        pins.check_products_bruteforce(
            oracle.qgemm_w8, w4_tiled, oracle.qgemm_w8a8, oracle.rotate_groups, oracle.bf16_round,
            oracle.quantize_weights_int8, oracle.quantize_weights_int4, oracle.unpack_int4)


def test_w8_missing_bf16_caught():
    def w8_no_bf16(x, q, s, rotate=True):
        return oracle.rotate_groups(x) @ oracle.dequantize_int8(q, s).T
    with pytest.raises(AssertionError):
        pins.check_products_bruteforce(
            w8_no_bf16, oracle.qgemm_w4, oracle.qgemm_w8a8, oracle.rotate_groups, oracle.bf16_round,
            oracle.quantize_weights_int8, oracle.quantize_weights_int4, oracle.unpack_int4)


def test_w8a8_dropped_weight_scale_caught():
    def w8a8_no_sw(x, q, sw, rotate=True):
        y, acc, qa, sa = oracle.qgemm_w8a8(x, q, sw, rotate)
        return acc * sa.astype(np.float64)[:, None], acc, qa, sa
    with pytest.raises(AssertionError):
        pins.check_planted_w8a8(w8a8_no_sw, oracle.hadamard_matrix)


def test_w8a8_unrotated_activations_caught():
    def w8a8_no_rot(x, q, sw, rotate=True):
        return oracle.qgemm_w8a8(x, q, sw, rotate=False)
    with pytest.raises(AssertionError):
        pins.check_planted_w8a8(w8a8_no_rot, oracle.hadamard_matrix)


# ------------------------------------------------------------ FFN middle
def _silu_mul_sigmoid_only(g, u):  # forgets the factor g
    g = np.asarray(g, dtype=np.float64)
    return np.asarray(u, dtype=np.float64) / (1.0 + np.exp(-g))


def _silu_mul_swapped(g, u):  # silu(u) * g
    return oracle.silu_mul(u, g)


def _silu_mul_sign(g, u):  # e^+g in the denominator
    g = np.asarray(g, dtype=np.float64)
    return g * np.asarray(u, dtype=np.float64) / (1.0 + np.exp(g))


@pytest.mark.parametrize("bad", [_silu_mul_sigmoid_only, _silu_mul_swapped, _silu_mul_sign])
def test_swiglu_formula_faults_caught(bad):
    with pytest.raises(AssertionError):
        pins.check_swiglu(bad, lambda g, u: oracle.bf16_round(bad(g, u)))


def test_swiglu_double_rounding_caught():
    def through_fp32(g, u):
        return oracle.bf16_round(np.asarray(oracle.silu_mul(g, u), dtype=np.float32).astype(np.float64))
    with pytest.raises(AssertionError):
        pins.check_swiglu(oracle.silu_mul, through_fp32)


def test_swiglu_missing_rounding_caught():
    with pytest.raises(AssertionError):
        pins.check_swiglu(oracle.silu_mul, oracle.silu_mul)


def test_ffn_middle_without_rotation_caught():
    def no_rot(g, u):
        return oracle.quantize_activations_int8(oracle.swiglu_bf16(g, u), rotate=False)
    with pytest.raises(AssertionError):
        pins.check_ffn_middle(no_rot, oracle.ffn_middle_rotated, oracle.quantize_activations_int8,
                              oracle.bf16_round, oracle.hadamard_matrix)


def test_ffn_middle_unrounded_caught():
    def unrounded(g, u):
        return oracle.quantize_activations_int8(oracle.silu_mul(g, u), rotate=True)
    with pytest.raises(AssertionError):
        pins.check_ffn_middle(unrounded, oracle.ffn_middle_rotated, oracle.quantize_activations_int8,
                              oracle.bf16_round, oracle.hadamard_matrix)


# ------------------------------------------------------------------ W4A8
def _w4a8_with(fold):
    def f(x, packed, s, rotate=True):
        qa, sa = oracle.quantize_activations_int8(x, rotate=rotate)
        acc = oracle.group_accumulate(qa, oracle.unpack_int4(packed))
        y = fold(acc.astype(np.float64), np.asarray(s, dtype=np.float64), sa.astype(np.float64))
        return y, acc, qa, sa
    return f


@pytest.mark.parametrize("fold", [
    lambda acc, s, sa: np.einsum("gmn,n->mn", acc, s[:, 0]) * sa[:, None],          # first group's scale only
    lambda acc, s, sa: np.einsum("gmn,gn->mn", acc, np.roll(s.T, 1, axis=0)) * sa[:, None],  # group index off by one
    lambda acc, s, sa: np.einsum("gmn,gn->mn", acc, s.T),                            # activation scale dropped
    lambda acc, s, sa: np.einsum("gmn,gn->mn", acc, s.T) * sa[None, :acc.shape[2]] if acc.shape[1] == acc.shape[2]
    else np.einsum("gmn,gn->mn", acc, s.T) * sa.mean(),                              # wrong activation scale
])
def test_w4a8_fold_faults_caught(fold):
    with pytest.raises(AssertionError):
        pins.check_w4a8(_w4a8_with(fold), oracle.qgemm_w8a8, oracle.quantize_weights_int4, oracle.unpack_int4,
                        oracle.pack_int4, oracle.rotate_groups, oracle.hadamard_matrix)


# ---------------------------------------------------------------- loader
def _loader_args():
    return (oracle.quantize_weights_int8, oracle.quantize_weights_int4, oracle.pack_int4, oracle.hadamard_matrix)


def test_unrotation_without_normalization_caught():
    def unrot(q, s, bits):
        x = oracle.dequantize(q, s, bits)
        r, k = x.shape
        return np.matmul(x.reshape(r, k // 256, 256), oracle.hadamard_matrix(256)).reshape(r, k)
    with pytest.raises(AssertionError):
        pins.check_loader(unrot, oracle.requantize, *_loader_args())


def test_requantize_rotating_again_caught():
    def req(q, s, bits_in, bits_out):
        w = oracle.dequantize(q, s, bits_in)
        return (oracle.quantize_weights_int8(w) if bits_out == 8 else oracle.quantize_weights_int4(w))
    with pytest.raises(AssertionError):
        pins.check_loader(oracle.dequantize_unrotate, req, *_loader_args())


def test_requantize_int4_scale_index_caught():
    def req(q, s, bits_in, bits_out):
        if bits_in == 4:
            s = np.roll(np.asarray(s), 1, axis=1)
        return oracle.requantize(q, s, bits_in, bits_out)
    with pytest.raises(AssertionError):
        pins.check_loader(oracle.dequantize_unrotate, req, *_loader_args())


# ------------------------------------------------------------------ LoRA
@pytest.mark.parametrize("bad", [
    lambda c, x, a, b, al: np.asarray(c) + al * (np.asarray(x) @ np.asarray(a).T) @ np.asarray(b),   # B not transposed
    lambda c, x, a, b, al: np.asarray(c) + (np.asarray(x) @ np.asarray(a).T) @ np.asarray(b).T,       # strength dropped
    lambda c, x, a, b, al: al * (np.asarray(x) @ np.asarray(a).T) @ np.asarray(b).T,                  # output replaced
])
def test_lora_faults_caught(bad):
    with pytest.raises((AssertionError, ValueError)):
        pins.check_lora(bad, oracle.rotate_groups)
