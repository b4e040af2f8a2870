"""Seeded synthetic inputs for the rotated, quantized projections.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no rotation, no quantization, no product). It is the one
piece shared by the CPU oracle's tests and the HIP library's tests and
benchmark, so both sides see the very same inputs.

Workloads (shapes from the diffusion-transformer projections the pages
describe: 256 latent + 32 prompt rows at a 256x256 image, 4096 latent rows at
1024x1024, 1344x768 = 4032 image rows; tensai docs, "画像生成", sections
"サイズと時間" and "GPU"; TensorFold pull request #948, first comment):

  tiny       M=64,   K=512,   N=256    fp32 acts, 4 outlier cols x30,
                                       fp32 weights, 4 outlier input cols x20
  proj256    M=288,  K=3072,  N=3072   bf16 acts, 0.5% outlier channels x30,
                                       weights N(0, 0.02), 0.5% outlier cols x20
  ffn_up     M=4096, K=3072,  N=12288  as proj256
  ffn_down   M=4032, K=12288, N=3072   acts silu(G)*U, G, U ~ N(0,1) (bf16),
                                       weights as proj256
  dit_qkv / dit_out / dit_gateup / dit_down   M=4096; 3072->9216, 3072->3072,
                                       3072->24576, 12288->3072; as proj256

FFN middle (gate and up of a SwiGLU feed-forward, G then U ~ N(0,1), fp32):
  ffn_mid_w8a8  M=4096, K=12288, seed 404: the fp32 gate+up output of the
                W8A8 block, turned into the int8 input of dit_down
  ffn_mid_w4    M=4032, K=12288, seed 3: ffn_down's G and U (same draws),
                turned into its rotated bf16 input

Recipe: numpy default_rng(seed) (PCG64). Draw order: activations (G then U for
ffn_down), weights, activation outlier columns, weight outlier columns (each a
choice without replacement). Outlier count is round(0.005*K) unless fixed.
Activations are drawn in fp32 and rounded to bf16 where the workload says
bf16; weights stay fp32.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    n: int
    seed: int
    path: str            # "w8", "w4" or "w8a8": the product the workload is quoted for
    act_dtype: str       # "f32" or "bf16"
    out_dtype: str       # "f32" or "bf16"
    act_kind: str = "gauss"   # "gauss" or "swiglu"
    act_outliers: int = -1    # -1: round(0.005*K)
    w_outliers: int = -1
    act_outlier_gain: float = 30.0
    w_outlier_gain: float = 20.0
    w_std: float = 0.02

    def n_act_outliers(self):
        if self.act_kind == "swiglu":
            return 0
        return self.act_outliers if self.act_outliers >= 0 else int(round(0.005 * self.k))

    def n_w_outliers(self):
        return self.w_outliers if self.w_outliers >= 0 else int(round(0.005 * self.k))

    def with_(self, **kw):
        return replace(self, **kw)


TINY = Workload("tiny", 64, 512, 256, 0, "w8", "f32", "f32", act_outliers=4, w_outliers=4)
PROJ256 = Workload("proj256", 288, 3072, 3072, 1, "w8", "bf16", "bf16")
FFN_UP = Workload("ffn_up", 4096, 3072, 12288, 2, "w8", "bf16", "bf16")
FFN_DOWN = Workload("ffn_down", 4032, 12288, 3072, 3, "w4", "bf16", "bf16", act_kind="swiglu")
DIT_QKV = Workload("dit_qkv", 4096, 3072, 9216, 400, "w8a8", "bf16", "f32")
DIT_OUT = Workload("dit_out", 4096, 3072, 3072, 401, "w8a8", "bf16", "f32")
DIT_GATEUP = Workload("dit_gateup", 4096, 3072, 24576, 402, "w8a8", "bf16", "f32")
DIT_DOWN = Workload("dit_down", 4096, 12288, 3072, 403, "w8a8", "bf16", "f32")

DIT_BLOCK = (DIT_QKV, DIT_OUT, DIT_GATEUP, DIT_DOWN)
ALL = (TINY, PROJ256, FFN_UP, FFN_DOWN) + DIT_BLOCK
BY_NAME = {w.name: w for w in ALL}


def _to_dtype(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


def generate(w: Workload, rows=None):
    """Return (activations [M, K], weights fp32 [N, K]) as CPU torch tensors.

    rows: optionally keep only the first `rows` activation rows (the weights
    and the outlier columns are unchanged, the draw order is the same).
    """
    rng = np.random.default_rng(w.seed)
    if w.act_kind == "gauss":
        x = rng.standard_normal((w.m, w.k), dtype=np.float32)
    elif w.act_kind == "swiglu":
        g = rng.standard_normal((w.m, w.k), dtype=np.float32)
        u = rng.standard_normal((w.m, w.k), dtype=np.float32)
        x = (g / (np.float32(1.0) + np.exp(-g))) * u
        del g, u
    else:
        raise ValueError(w.act_kind)
    wt = rng.standard_normal((w.n, w.k), dtype=np.float32)
    wt *= np.float32(w.w_std)
    ca = rng.choice(w.k, size=w.n_act_outliers(), replace=False)
    cw = rng.choice(w.k, size=w.n_w_outliers(), replace=False)
    if len(ca):
        x[:, ca] *= np.float32(w.act_outlier_gain)
    if len(cw):
        wt[:, cw] *= np.float32(w.w_outlier_gain)
    if rows is not None:
        x = x[:rows]
    return _to_dtype(x, w.act_dtype), torch.from_numpy(wt)


def generate_activations(w: Workload, rows=None):
    return generate(w, rows)[0]


def random_rows(shape, seed, dtype="f32", scale=1.0):
    """Plain N(0, scale^2) array of a given shape (edge-case tests)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return _to_dtype(a, dtype)


@dataclass(frozen=True)
class FfnMiddle:
    name: str
    m: int
    k: int
    seed: int
    in_dtype: str   # "f32" or "bf16"
    out: str        # "i8" or "bf16"

    def with_(self, **kw):
        return replace(self, **kw)


FFN_MID_W8A8 = FfnMiddle("ffn_mid_w8a8", 4096, 12288, 404, "f32", "i8")
FFN_MID_W4 = FfnMiddle("ffn_mid_w4", 4032, 12288, 3, "f32", "bf16")


def gate_up(w: FfnMiddle, rows=None, fused=False):
    """Gate and up activations [M, K] (G drawn first, then U, both N(0,1) in
    fp32, rounded to bf16 if in_dtype says so). fused=True returns one
    [M, 2K] tensor holding G in columns [0, K) and U in [K, 2K), the layout a
    gate+up projection writes; otherwise (G, U)."""
    rng = np.random.default_rng(w.seed)
    g = rng.standard_normal((w.m, w.k), dtype=np.float32)
    u = rng.standard_normal((w.m, w.k), dtype=np.float32)
    if rows is not None:
        g, u = g[:rows], u[:rows]
    if fused:
        return _to_dtype(np.concatenate([g, u], axis=1), w.in_dtype)
    return _to_dtype(g, w.in_dtype), _to_dtype(u, w.in_dtype)
