"""Plain fp64 CPU oracle for the rotated, quantized linear projection ("ConvRot").

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it. It shares no code, header, table or constant generator with the HIP
library, and it imports nothing from it.

What it computes, and where the pages say so
--------------------------------------------
* tensai docs, "画像生成" (image generation), section "幅とメモリ" (width and
  memory): every weight is rotated by a Hadamard matrix on each 256-wide group
  of input columns and then stored as int8 with one scale per row; the
  product's input gets the same rotation, and because the matrix is orthogonal
  the product is unchanged while the outlier columns that would set a row's
  scale are spread over the group. The same section offers a 4-bit width
  ("-q4") and says the activation rotation is one product with H per 256-group
  of a row, done on the device.
* same page, section "GPU": the device quantizes each product's activations
  more finely (read here as per-token symmetric int8 for the W8A8 product).
* same page, section "チェックポイントの入手" (getting the checkpoints): the
  ComfyUI int8 files are rotated per 256 input columns and stored as per-row
  scaled int8.

Everything is computed in fp64 with numpy; library primitives (matmul, rint,
max) are used as steps, with no blocking, fusion or reordering beyond the
definition.

Readings where the pages are silent (each is also listed with its reason in
the design notes):
  R1  Sylvester Hadamard in natural order, H[i,j] = (-1)^popcount(i & j).
  R2  The orthonormal rotation is Q = H/16, applied to weights and activations.
  R3  Symmetric quantization, no zero point: int8 codes in [-127, 127] with
      s = amax/127; int4 codes in [-7, 7] with s = amax/7.
  R4  Codes are rint(x / s) (round half to even) in fp64 using the STORED
      fp32 scale; the scale itself is fp32(fp64(amax) / 127).
  R5  An all-zero row (or group) has s = 0 and all codes 0.
  R6  int4 packing: two's-complement nibbles, the even column in the low
      nibble of each byte.
  R7  Scales are fp32: one per output row for int8, one per (row, 256-group)
      for int4.
  R8  The weight-only (W8/W4) product feeds bf16 activations to the matrix
      unit: the rotated activations are rounded once to bf16 (nearest, ties
      to even) before the product; the product itself is exact here (fp64).
  R9  W8A8: per-row (per-token) scale sa = fp32(amax/127) of the rotated row,
      codes rint(x'/sa) clamped to [-127, 127]; the int32 accumulator is the
      exact integer dot product; the output is acc * sa[m] * sw[n].
  R10 K must be a multiple of 256 (a group never straddles the end of a row).
  R15 SwiGLU(g, u) = silu(g) * u, silu(x) = x / (1 + e^-x); its output h is
      bf16, rounded once from the real value (oracle/ffn.py).
  R16 h enters the down projection like any other activation.
  R19 Undoing a rotated, quantized weight: W_hat = (q * s) . blockdiag(Q)
      (Q is its own inverse), exact in fp64 (oracle/loader.py).
  R20 Requantizing to another width is quantizing q * s in the rotated
      domain (rotation after un-rotation is the identity).
  R21 LoRA side path: c + alpha * (x . A^T) . B^T with lora_A [r, K] and
      lora_B [N, r] (oracle/lora.py).
  R18 W4A8: the 4-bit weights (one scale per row and 256-group) against the
      per-row int8 activations of R9: exact integer sums per group, then
      y = sa[m] * sum_g s[n, g] * acc_g.

Parity pins live in tests/test_oracle.py; planted-fault controls in
tests/test_controls.py.
"""

from .hadamard import GROUP, hadamard_matrix, rotate_groups
from .quantize import (
    bf16_round,
    quantize_weights_int8,
    quantize_weights_int4,
    quantize_activations_int8,
    pack_int4,
    unpack_int4,
    dequantize_int8,
    dequantize_int4,
)
from .products import qgemm_w8, qgemm_w4, qgemm_w8a8, qgemm_w4a8, int_accumulate, group_accumulate
from .ffn import silu_mul, swiglu_bf16, ffn_middle_int8, ffn_middle_rotated
from .loader import dequantize, dequantize_unrotate, requantize
from .lora import lora_delta, lora_add

__all__ = [
    "GROUP",
    "hadamard_matrix",
    "rotate_groups",
    "bf16_round",
    "quantize_weights_int8",
    "quantize_weights_int4",
    "quantize_activations_int8",
    "pack_int4",
    "unpack_int4",
    "dequantize_int8",
    "dequantize_int4",
    "lora_delta",
    "lora_add",
    "dequantize",
    "dequantize_unrotate",
    "requantize",
    "silu_mul",
    "swiglu_bf16",
    "ffn_middle_int8",
    "ffn_middle_rotated",
    "qgemm_w4a8",
    "group_accumulate",
    "qgemm_w8",
    "qgemm_w4",
    "qgemm_w8a8",
    "int_accumulate",
]
