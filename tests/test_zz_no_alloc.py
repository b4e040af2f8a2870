"""The no-allocation W8A8 entry point (tp_qgemm_w8a8_prequantized_noalloc),
called through the C ABI, against tp_qgemm_w8a8_prequantized with a
workspace: two calls in a row, the second with a smaller input, each with
split-K partial sums (in the library's scratch array for the former). The
same kernels add the same partial sums in the same order, so the outputs and
the int32 accumulators must be the same bytes."""

import ctypes

import pytest
import torch

import int4_quantized_gemm_amd as tp
from int4_quantized_gemm_amd import _lib
from tests.gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, seed, d):
    g = torch.Generator(device="cpu").manual_seed(seed)
    qa = torch.randint(-127, 128, (m, k), dtype=torch.int8, generator=g).to(d)
    sa = (torch.rand((m,), generator=g) * 0.02 + 1e-3).to(d)
    q = torch.randint(-127, 128, (n, k), dtype=torch.int8, generator=g).to(d)
    sw = (torch.rand((n,), generator=g) * 0.01 + 1e-4).to(d)
    return qa, sa, q, sw


def _noalloc(lib, qa, sa, q, sw, c, acc):
    m, k = qa.shape
    n = q.shape[0]
    dt = _lib.TP_F32 if c.dtype == torch.float32 else _lib.TP_BF16
    st = lib.tp_qgemm_w8a8_prequantized_noalloc(qa.data_ptr(), k, sa.data_ptr(), q.data_ptr(), k, sw.data_ptr(),
                                                m, n, k, c.data_ptr(), dt, n,
                                                ctypes.c_void_p(acc.data_ptr()) if acc is not None else None,
                                                n if acc is not None else 0,
                                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st)


@pytest.mark.parametrize("first,second", [
    ((64, 9216, 3072, torch.float32), (24, 3072, 3072, torch.bfloat16)),
    ((40, 24576, 3072, torch.bfloat16), (17, 3072, 12288, torch.float32)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    d = dev()
    lib = _lib.load()
    for i, (m, n, k, odt) in enumerate((first, second)):
        announce("tp_qgemm_w8a8_prequantized_noalloc", m, n, k, odt)
        need = lib.tp_workspace_size(_lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, 0)
        assert 0 < need <= 32 << 20, "the case must use split-K partial sums that fit the scratch array"
        qa, sa, q, sw = _inputs(m, n, k, seed=11 + i, d=d)
        want_acc = odt == torch.float32
        ref_acc = torch.empty((m, n), dtype=torch.int32, device=d) if want_acc else None
        ref = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, sw, out_dtype=odt, acc=ref_acc)
        got = torch.full((m, n), float("nan"), dtype=odt, device=d)
        got_acc = torch.full((m, n), -7, dtype=torch.int32, device=d) if want_acc else None
        _noalloc(lib, qa, sa, q, sw, got, got_acc)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if odt == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if odt == torch.bfloat16 else torch.int32)), "outputs differ"
        if want_acc:
            assert torch.equal(got_acc, ref_acc), "int32 accumulators differ"


def test_noalloc_repeat_is_byte_identical():
    """The scratch array keeps the previous call's contents: a second call on
    the same inputs must still give the same bytes."""
    d = dev()
    lib = _lib.load()
    m, n, k = 64, 3072, 12288
    announce("tp_qgemm_w8a8_prequantized_noalloc repeat", m, n, k)
    qa, sa, q, sw = _inputs(m, n, k, seed=5, d=d)
    a = torch.empty((m, n), dtype=torch.float32, device=d)
    b = torch.empty((m, n), dtype=torch.float32, device=d)
    _noalloc(lib, qa, sa, q, sw, a, None)
    _noalloc(lib, qa, sa, q, sw, b, None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    ref = tp.tp_qgemm_w8a8_prequantized(qa, sa, q, sw)
    assert torch.equal(a.view(torch.int32), ref.view(torch.int32))
