"""The CPU oracle against its pins (closed forms, invariants, brute force,
planted integers, textbook tables). CPU only."""

import numpy as np
import pytest

import oracle
from tests import pins


def test_hadamard():
    pins.check_hadamard(oracle.hadamard_matrix)


def test_rotation():
    pins.check_rotation(oracle.rotate_groups, oracle.hadamard_matrix)


def test_product_invariance():
    pins.check_product_invariance(oracle.rotate_groups)


def test_bf16_rounding():
    pins.check_bf16(oracle.bf16_round)


def test_weight_int8_invariants():
    pins.check_weight_int8(oracle.quantize_weights_int8, oracle.rotate_groups)


def test_weight_int4_invariants():
    pins.check_weight_int4(oracle.quantize_weights_int4, oracle.unpack_int4, oracle.rotate_groups)


def test_planted_int8():
    pins.check_planted_int8(oracle.quantize_weights_int8, oracle.hadamard_matrix)


def test_planted_int4():
    pins.check_planted_int4(oracle.quantize_weights_int4, oracle.unpack_int4, oracle.hadamard_matrix)


def test_pack():
    pins.check_pack(oracle.pack_int4, oracle.unpack_int4)


def test_int_accumulate():
    pins.check_int_accumulate(oracle.int_accumulate)


def test_products_bruteforce():
    pins.check_products_bruteforce(
        oracle.qgemm_w8, oracle.qgemm_w4, oracle.qgemm_w8a8, oracle.rotate_groups, oracle.bf16_round,
        oracle.quantize_weights_int8, oracle.quantize_weights_int4, oracle.unpack_int4)


def test_planted_w8a8():
    pins.check_planted_w8a8(oracle.qgemm_w8a8, oracle.hadamard_matrix)


def test_rotation_helps():
    pins.check_rotation_helps(oracle.quantize_weights_int8, oracle.dequantize_int8, oracle.rotate_groups)


def test_activation_quant_zero_row():
    x = np.zeros((2, 256))
    x[1, 3] = 1.0
    qa, sa = oracle.quantize_activations_int8(x)
    assert sa[0] == 0 and np.all(qa[0] == 0)
    assert sa[1] > 0 and np.max(np.abs(qa[1])) == 127


def test_refuses_ragged_k():
    with pytest.raises(ValueError):
        oracle.rotate_groups(np.zeros((1, 300)))


def test_swiglu():
    pins.check_swiglu(oracle.silu_mul, oracle.swiglu_bf16)


def test_ffn_middle():
    pins.check_ffn_middle(oracle.ffn_middle_int8, oracle.ffn_middle_rotated, oracle.quantize_activations_int8,
                          oracle.bf16_round, oracle.hadamard_matrix)


def test_w4a8():
    pins.check_w4a8(oracle.qgemm_w4a8, oracle.qgemm_w8a8, oracle.quantize_weights_int4, oracle.unpack_int4,
                    oracle.pack_int4, oracle.rotate_groups, oracle.hadamard_matrix)


def test_loader():
    pins.check_loader(oracle.dequantize_unrotate, oracle.requantize, oracle.quantize_weights_int8,
                      oracle.quantize_weights_int4, oracle.pack_int4, oracle.hadamard_matrix)


def test_lora():
    pins.check_lora(oracle.lora_add, oracle.rotate_groups)
