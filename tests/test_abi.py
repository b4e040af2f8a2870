"""The C ABI without a GPU: libtp.so loads, exports every entry point that
include/tp.h declares, and refuses every invalid call by name before any HIP
call (so these run on a CPU-only host with made-up device addresses: nothing is
dereferenced or launched)."""

import os
import re

import pytest

from int4_quantized_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A, B, C, D, E = 0x10000, 0x4000000, 0x8000000, 0xC000000, 0x10000000  # disjoint fake addresses


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            names |= set(re.findall(r"^[a-z_ *]+?\b(tp_[a-z0-9_]+)\s*\(", text, flags=re.M))
    return names


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"tp_rotate_quantize_weights", "tp_hadamard_rotate_rows", "tp_qgemm_w8", "tp_qgemm_w4",
            "tp_qgemm_w8a8"} <= names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes declaration"


def test_version_and_strings(lib):
    assert lib.tp_abi_version() == 8
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.tp_status_string(code).decode() == name


def _err(lib):
    return lib.tp_last_error_message().decode()


# ------------------------------------------------------- fused FFN middle
def sw(lib, g=A, ldg=512, u=B, ldu=512, dt=0, m=64, k=512, kind=0, y=C, ldy=512, s=D):
    return lib.tp_swiglu_rotate(g, ldg, u, ldu, dt, m, k, kind, y, ldy, s, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldg=304, ldu=304, ldy=304), 3),
    (dict(k=0), 2),
    (dict(m=-1), 2),
    (dict(g=0), 1),
    (dict(u=0), 1),
    (dict(y=0), 1),
    (dict(s=0), 1),
    (dict(ldg=500), 4),
    (dict(ldu=511), 4),
    (dict(ldy=256), 4),
    (dict(g=A + 8), 5),
    (dict(ldy=513), 5),
    (dict(kind=1, ldy=500), 4),
    (dict(dt=3), 6),
    (dict(kind=2), 11),
    (dict(y=A + 4096), 10),
    (dict(s=C + 64), 10),
    (dict(kind=1, y=B + 1024), 10),
    (dict(ldu=2 ** 62), 8),
])
def test_swiglu_rotate_refusals(lib, kw, status):
    assert sw(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_swiglu_rotate_empty_and_optional_scales(lib):
    assert sw(lib, m=0) == 0
    assert sw(lib, m=0, kind=1, s=0, ldy=512) == 0          # bf16 rows: no scales
    assert sw(lib, m=0, u=A, ldu=512) == 0                  # gate and up may overlap
    assert sw(lib, m=0, dt=1, ldg=1024, u=A + 1024, ldu=1024) == 0  # column halves of one [m, 2k] bf16 buffer


# --------------------------------------------------- rotate-quantize weights
def rq(lib, w=A, dt=0, n=64, k=512, ldw=512, bits=8, q=B, ldq=512, s=C):
    return lib.tp_rotate_quantize_weights(w, dt, n, k, ldw, bits, q, ldq, s, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldw=304, ldq=304), 3),
    (dict(k=0), 2),
    (dict(n=-1), 2),
    (dict(w=0), 1),
    (dict(q=0), 1),
    (dict(s=0), 1),
    (dict(w=A + 8), 5),
    (dict(ldw=500), 4),
    (dict(ldw=513), 5),
    (dict(bits=5), 7),
    (dict(bits=4, ldq=200), 4),
    (dict(dt=7), 6),
    (dict(s=C + 2), 5),
    (dict(q=A + 1024), 10),
    (dict(ldw=2 ** 62), 8),
])
def test_rotate_quantize_refusals(lib, kw, status):
    assert rq(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_rotate_quantize_empty_is_noop(lib):
    assert rq(lib, n=0) == 0


def test_last_error_message_is_per_thread(lib):
    """tp.h: the message belongs to the calling thread. Two threads are
    refused for different reasons, one after the other, and each then reads
    its own message."""
    import threading
    step = threading.Barrier(2)
    got = {}

    def worker(name, kw, status):
        if name == "second":
            step.wait()              # the first thread has been refused
        assert rq(lib, **kw) == status
        if name == "first":
            step.wait()
        step.wait()                  # both refused before either reads
        got[name] = _err(lib)

    t1 = threading.Thread(target=worker, args=("first", dict(bits=5), 7))
    t2 = threading.Thread(target=worker, args=("second", dict(k=300, ldw=304, ldq=304), 3))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert "bits" in got["first"] and "256" not in got["first"], got
    assert "256" in got["second"] and "bits" not in got["second"], got


# ------------------------------------------------------------- rotate rows
def rr(lib, x=A, xd=1, m=8, k=512, ldx=512, y=B, yd=1, ldy=512):
    return lib.tp_hadamard_rotate_rows(x, xd, m, k, ldx, y, yd, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=384, ldx=384, ldy=384), 3),
    (dict(x=0), 1),
    (dict(y=0), 1),
    (dict(yd=3), 6),
    (dict(ldy=256), 4),
    (dict(y=A + 512), 10),              # partial overlap
    (dict(y=A, yd=0, ldy=512), 10),     # same base, other dtype: not in place
    (dict(y=A, ldy=1024), 10),          # same base, other pitch
    (dict(x=A + 4), 5),
])
def test_rotate_rows_refusals(lib, kw, status):
    assert rr(lib, **kw) == status, _err(lib)


def test_rotate_rows_empty_and_inplace_validate(lib):
    assert rr(lib, m=0) == 0
    assert rr(lib, m=0, y=A, ldy=512) == 0


# -------------------------------------------------------- quantize rows int8
@pytest.mark.parametrize("kw,status", [
    (dict(flags=2), 11),
    (dict(k=100, ldx=128, ldqa=128), 3),
    (dict(qa=0), 1),
    (dict(sa=0), 1),
    (dict(ldqa=500), 4),
    (dict(qa=A), 10),
])
def test_quantize_rows_refusals(lib, kw, status):
    a = dict(x=A, xd=1, m=8, k=512, ldx=512, flags=1, qa=B, ldqa=512, sa=C)
    a.update(kw)
    got = lib.tp_quantize_rows_int8(a["x"], a["xd"], a["m"], a["k"], a["ldx"], a["flags"], a["qa"], a["ldqa"],
                                    a["sa"], None)
    assert got == status, _err(lib)


# ------------------------------------------------------------ products
def w8(lib, fn="tp_qgemm_w8", a=A, ad=1, lda=512, flags=1, q=B, ldq=512, s=C, m=64, n=256, k=512, c=D, cd=1,
       ldc=256, ws=E, wsb=None):
    if wsb is None:  # what the library asks for (rotated A' and split-K partial sums)
        wsb = lib.tp_workspace_size(1 if fn == "tp_qgemm_w8" else 2, 64, 256, 512, 1)
    return getattr(lib, fn)(a, ad, lda, flags, q, ldq, s, m, n, k, c, cd, ldc, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=768 + 1, lda=1024, ldq=1024), 3),
    (dict(flags=5), 11),
    (dict(flags=0, ad=0), 6),            # pre-rotated operand must be bf16
    (dict(cd=9), 6),
    (dict(ws=0), 9),
    (dict(wsb=100), 9),
    (dict(ws=E + 8), 5),
    (dict(c=A + 256), 10),
    (dict(ws=B), 10),
    (dict(ldc=100), 4),
    (dict(ldq=256), 4),
    (dict(m=-3), 2),
    (dict(m=2 ** 40), 2),
])
def test_w8_refusals(lib, kw, status):
    assert w8(lib, **kw) == status, _err(lib)


def test_w4_checks_packed_rows(lib):
    assert w8(lib, fn="tp_qgemm_w4", ldq=128, m=0) == 4
    assert w8(lib, fn="tp_qgemm_w4", ldq=256, m=0) == 0


def test_products_empty_are_noops(lib):
    assert w8(lib, m=0) == 0
    assert w8(lib, n=0) == 0
    assert w8(lib, fn="tp_qgemm_w4", ldq=256, n=0) == 0


def w8a8(lib, a=A, ad=1, lda=512, flags=1, q=B, ldq=512, s=C, m=64, n=256, k=512, c=D, cd=0, ldc=256, qa=0, sa=0,
         acc=0, ld_acc=0, ws=E, wsb=1 << 20):
    return lib.tp_qgemm_w8a8(a, ad, lda, flags, q, ldq, s, m, n, k, c, cd, ldc, qa or None, sa or None, acc or None,
                             ld_acc, ws or None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=133376, lda=133376, ldq=133376), 2),     # int32 accumulator could overflow
    (dict(ws=0), 9),
    (dict(wsb=1000), 9),
    (dict(acc=0x20000000, ld_acc=100), 4),
    (dict(acc=D, ld_acc=256), 10),                   # acc_out overlaps c
    (dict(c=B), 10),                                 # c overlaps q
    (dict(flags=-1), 11),
    (dict(qa=0x30000000, sa=0x30000000 + 64 * 512 - 4), 10),
    (dict(m=40, k=3072, lda=3072, ldq=3072, qa=0x30000000, sa=0x38000000, ws=0, wsb=0), 9),  # split-K partials
                                                                                           # still need room
])
def test_w8a8_refusals(lib, kw, status):
    assert w8a8(lib, **kw) == status, _err(lib)


def test_w8a8_own_codes_need_no_workspace(lib):
    assert w8a8(lib, m=0, qa=0x30000000, sa=0x38000000, ws=0, wsb=0) == 0


def test_small_m_workspace_refusals(lib):
    # a pre-rotated product with 9..64 rows that is split over K still needs
    # room for its partial sums; up to 8 rows it needs none (single-launch
    # kernel), and neither does a plan with one split
    big = dict(flags=0, m=40, k=3072, lda=3072, ldq=3072)
    assert w8(lib, ws=0, wsb=0, **big) == 9
    need = lib.tp_workspace_size(1, 40, 256, 3072, 0)
    assert need > 0
    assert w8(lib, wsb=need - 1, **big) == 9
    assert w8(lib, ws=E + 8, wsb=need, **big) == 5
    assert lib.tp_workspace_size(1, 40, 256, 512, 0) == 0
    assert lib.tp_workspace_size(1, 8, 12288, 3072, 0) == 0
    assert lib.tp_workspace_size(4, 1, 24576, 3072, 0) == 0


K3 = dict(k=3072, ldqa=3072, ldq=3072)  # a 64 x 256 x 3072 product is split over K


def pq(lib, qa=A, ldqa=512, sa=C, q=B, ldq=512, s=C + 4096, m=64, n=256, k=512, c=D, cd=0, ldc=256, acc=0, ld_acc=0,
       ws=E, wsb=1 << 20):
    return lib.tp_qgemm_w8a8_prequantized(qa, ldqa, sa, q, ldq, s, m, n, k, c, cd, ldc, acc or None, ld_acc,
                                          ws or None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0, wsb=0, **K3), 9),      # m <= 64, K = 3072: split-K partial sums need a workspace
    (dict(wsb=1000, **K3), 9),
    (dict(ws=E + 4, **K3), 5),
    (dict(ws=A, **K3), 10),            # workspace overlaps qa
    (dict(ws=D, **K3), 10),            # workspace overlaps c
    (dict(k=300, ldqa=512, ldq=512), 3),
    (dict(cd=3), 6),
])
def test_prequantized_refusals(lib, kw, status):
    assert pq(lib, **kw) == status, _err(lib)


def pqn(lib, qa=A, ldqa=512, sa=C, q=B, ldq=512, s=C + 4096, m=64, n=256, k=512, c=D, cd=0, ldc=256, acc=0,
        ld_acc=0):
    return lib.tp_qgemm_w8a8_prequantized_noalloc(qa, ldqa, sa, q, ldq, s, m, n, k, c, cd, ldc, acc or None, ld_acc,
                                                  None)


@pytest.mark.parametrize("kw,status", [
    # 64 x 49152 x 3072 needs 36 MiB of split-K partial sums: more than the
    # 32 MiB scratch array, refused before any HIP call
    (dict(n=49152, k=3072, ldqa=3072, ldq=3072, ldc=49152, s=C + (1 << 20)), 9),
    (dict(qa=0), 1),
    (dict(c=0), 1),
    (dict(k=300, ldqa=512, ldq=512), 3),
    (dict(ldc=200), 4),
    (dict(cd=3), 6),
    (dict(c=A + 256), 10),             # c overlaps qa
])
def test_prequantized_noalloc_refusals(lib, kw, status):
    assert pqn(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_prequantized_noalloc_empty_is_noop(lib):
    assert pqn(lib, m=0) == 0
    assert pqn(lib, n=0) == 0


def test_prequantized_large_m_needs_no_workspace(lib):
    assert lib.tp_workspace_size(4, 4096, 9216, 3072, 0) == 0
    assert pq(lib, m=0, ws=0, wsb=0) == 0


# ---------------------------------------------------------------- LoRA
def lo(lib, x=A, xd=1, ldx=512, la=B, lb=B + 65536, abd=1, lda=512, ldb=32, alpha=0.5, m=64, n=256, k=512, r=32,
       c=D, cd=0, ldc=256, ws=E, wsb=1 << 20):
    return lib.tp_lora_add(x, xd, ldx, la, lb, abd, lda, ldb, alpha, m, n, k, r, c, cd, ldc, ws or None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldx=304, lda=304), 3),
    (dict(r=0), 2),
    (dict(r=65, ldb=65), 2),
    (dict(x=0), 1),
    (dict(la=0), 1),
    (dict(c=0), 1),
    (dict(ldb=16), 4),
    (dict(ldx=500), 4),
    (dict(x=A + 1), 5),
    (dict(xd=2), 6),
    (dict(abd=9), 6),
    (dict(cd=5), 6),
    (dict(ws=0, wsb=0), 9),
    (dict(wsb=64 * 64 * 4 - 4), 9),
    (dict(ldb=33), 5),                 # lora_b rows must be 16-byte aligned
    (dict(ws=E + 8), 5),
    (dict(c=A + 256), 10),             # c overlaps x
    (dict(ws=D + 64), 10),             # workspace overlaps c
])
def test_lora_refusals(lib, kw, status):
    assert lo(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_lora_workspace_and_empty(lib):
    assert lib.tp_lora_workspace_size(4096, 32) == 4096 * 64 * 4
    assert lib.tp_lora_workspace_size(4096, 65) == 0
    assert lo(lib, m=0, ws=0, wsb=0) == 0
    assert lo(lib, n=0, ws=0, wsb=0) == 0


def ld(lib, x=A, xd=1, ldx=512, la=B, ad=1, lda=512, m=64, k=512, r=32, t=D, tb=64 * 64 * 4):
    return lib.tp_lora_down(x, xd, ldx, la, ad, lda, m, k, r, t, tb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldx=304, lda=304), 3),
    (dict(r=0), 2),
    (dict(r=65), 2),
    (dict(x=0), 1),
    (dict(la=0), 1),
    (dict(t=0), 1),
    (dict(ldx=500), 4),
    (dict(x=A + 1), 5),
    (dict(t=D + 8), 5),
    (dict(xd=2), 6),
    (dict(ad=9), 6),
    (dict(tb=64 * 64 * 4 - 4), 9),
    (dict(t=A + 256), 10),             # t overlaps x
])
def test_lora_down_refusals(lib, kw, status):
    assert ld(lib, **kw) == status, _err(lib)
    assert _err(lib)


def lq(lib, qa=A, ldqa=512, sa=B, q=B + 4096, ldq=512, sw=C, m=64, n=256, k=512, c=D, ldc=256, t=E,
       lb=E + 65536, ldb=32, r=32, alpha=0.5, ws=0x20000000, wsb=1 << 26):
    return lib.tp_qgemm_w8a8_prequantized_lora(qa, ldqa, sa, q, ldq, sw, m, n, k, c, ldc, t, lb, ldb, r, alpha,
                                               ws or None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldqa=304, ldq=304), 3),
    (dict(r=0), 2),
    (dict(r=65, ldb=72), 2),
    (dict(t=0), 1),
    (dict(lb=0), 1),
    (dict(ldb=16), 4),                 # lora_b pitch below r
    (dict(ldb=33), 5),                 # lora_b rows must be 16-byte aligned
    (dict(t=E + 8), 5),
    (dict(ldc=255), 4),
    (dict(t=D + 64), 10),              # t overlaps c
    (dict(lb=D + 128), 10),            # lora_b overlaps c
])
def test_w8a8_lora_refusals(lib, kw, status):
    assert lq(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_w8a8_lora_empty(lib):
    assert lq(lib, m=0, ws=0, wsb=0) == 0
    assert lq(lib, n=0, ws=0, wsb=0) == 0


# -------------------------------------------------------------- loader
def du(lib, q=A, bits=8, ldq=512, s=C, n=64, k=512, w=D, wd=0, ldw=512):
    return lib.tp_dequantize_unrotate(q, bits, ldq, s, n, k, w, wd, ldw, None)


def rq8(lib, qi=A, bi=8, ldi=512, si=C, n=64, k=512, bo=4, qo=D, ldo=256, so=E):
    return lib.tp_requantize_weights(qi, bi, ldi, si, n, k, bo, qo, ldo, so, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldq=304, ldw=304), 3),
    (dict(n=-1), 2),
    (dict(q=0), 1),
    (dict(s=0), 1),
    (dict(w=0), 1),
    (dict(bits=2), 7),
    (dict(bits=4, ldq=200), 4),
    (dict(ldw=500), 4),
    (dict(wd=4), 6),
    (dict(w=A + 1024), 10),
    (dict(s=C + 2), 5),
    (dict(ldw=2 ** 61), 8),
])
def test_dequantize_unrotate_refusals(lib, kw, status):
    assert du(lib, **kw) == status, _err(lib)
    assert _err(lib)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, ldi=304, ldo=304), 3),
    (dict(qi=0), 1),
    (dict(so=0), 1),
    (dict(bi=5), 7),
    (dict(bo=16), 7),
    (dict(ldo=200), 4),                # int4 rows are k/2 = 256 bytes
    (dict(bo=8, ldo=256), 4),          # int8 rows are k bytes
    (dict(qo=A + 64), 10),             # q_out overlaps q_in
    (dict(so=D + 128), 10),            # s_out overlaps q_out
])
def test_requantize_refusals(lib, kw, status):
    assert rq8(lib, **kw) == status, _err(lib)
    assert _err(lib)


def test_loader_empty_is_noop(lib):
    assert du(lib, n=0) == 0
    assert rq8(lib, n=0) == 0


# ---------------------------------------------------------------- W4A8
def w4a8(lib, a=A, ad=1, lda=512, flags=1, q=B, ldq=256, s=C, m=4096, n=3072, k=512, c=D, cd=0, ldc=3072, qa=0,
         sa=0, ws=E, wsb=1 << 30):
    return lib.tp_qgemm_w4a8(a, ad, lda, flags, q, ldq, s, m, n, k, c, cd, ldc, qa or None, sa or None, ws or None,
                             wsb, None)


def pq4(lib, qa=A, ldqa=4096, sa=C, q=B, ldq=2048, s=C + 65536, m=64, n=256, k=4096, c=D, cd=0, ldc=256, ws=E,
        wsb=1 << 20):
    # k = 4096 at m = 64 splits K, so every refusal below is reached before a
    # launch could be
    return lib.tp_qgemm_w4a8_prequantized(qa, ldqa, sa, q, ldq, s, m, n, k, c, cd, ldc, ws or None, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=300, lda=304, ldq=256), 3),
    (dict(k=0), 2),
    (dict(a=0), 1),
    (dict(q=0), 1),
    (dict(s=0), 1),
    (dict(c=0), 1),
    (dict(ldq=255), 4),                # packed rows are k/2 bytes
    (dict(ldq=264), 5),
    (dict(flags=2), 11),
    (dict(ad=5), 6),
    (dict(cd=9), 6),
    (dict(ws=0, wsb=0), 9),            # the activation codes need a workspace
    (dict(wsb=100), 9),
    (dict(c=B + 1024), 10),            # c overlaps the weight codes
    (dict(qa=E, sa=E + (1 << 20)), 10),  # qa_out overlaps the workspace
    (dict(ldc=2 ** 61), 8),
])
def test_w4a8_refusals(lib, kw, status):
    assert w4a8(lib, **kw) == status, _err(lib)
    assert _err(lib)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0, wsb=0), 9),            # m <= 64: split-K partial sums need a workspace
    (dict(ldq=2000), 4),
    (dict(k=300, ldqa=304, ldq=256), 3),
    (dict(ws=A), 10),
    (dict(cd=3), 6),
    (dict(sa=0), 1),
])
def test_w4a8_prequantized_refusals(lib, kw, status):
    assert pq4(lib, **kw) == status, _err(lib)


def test_w4a8_workspace_sizes(lib):
    # front part as W8A8 (codes, then scales at the next 256-byte boundary)
    assert lib.tp_workspace_size(5, 4096, 3072, 12288, 1) == 4096 * 12288 + 4096 * 4
    assert lib.tp_workspace_size(6, 4096, 3072, 12288, 0) == 0
    assert lib.tp_workspace_size(6, 64, 3072, 12288, 0) > 0      # no small-M kernel: split K
    assert lib.tp_workspace_size(6, 64, 3072, 12288, 0) % (4 * 64 * 3072) == 0
    assert pq4(lib, m=0, ws=0, wsb=0) == 0
    assert w4a8(lib, m=0, ws=0, wsb=0) == 0


def test_workspace_sizes(lib):
    assert lib.tp_workspace_size(1, 4096, 12288, 3072, 1) == 4096 * 3072 * 2
    assert lib.tp_workspace_size(2, 4032, 3072, 12288, 1) == 4032 * 12288 * 2
    assert lib.tp_workspace_size(1, 4096, 12288, 3072, 0) == 0
    assert lib.tp_workspace_size(3, 4096, 9216, 3072, 1) == 4096 * 3072 + 4096 * 4
    assert lib.tp_workspace_size(3, 3, 9216, 256, 1) == 768 + 12
    assert lib.tp_workspace_size(3, -1, 9, 256, 1) == 0
    assert lib.tp_workspace_size(4, 4096, 9216, 3072, 0) == 0


def test_workspace_sizes_small_m(lib):
    # Few rows: split-K partial sums (4 m n bytes per split) follow the front
    # part, 256-byte aligned; the split count does not depend on a_flags.
    m, n, k = 64, 12288, 3072
    pre = lib.tp_workspace_size(1, m, n, k, 0)
    rot = lib.tp_workspace_size(1, m, n, k, 1)
    assert pre > 0 and pre % (4 * m * n) == 0
    assert rot == (m * k * 2 + 255) // 256 * 256 + pre
    w8a8_pre = lib.tp_workspace_size(4, m, n, k, 0)
    assert w8a8_pre > 0 and w8a8_pre % (4 * m * n) == 0
    front = (m * k + 255) // 256 * 256 + 4 * m
    assert lib.tp_workspace_size(3, m, n, k, 1) == (front + 255) // 256 * 256 + w8a8_pre
    # one 256-group cannot be split
    assert lib.tp_workspace_size(1, 40, 256, 256, 0) == 0
    # above the small-M range: split-K partial sums only while the output has
    # fewer than 128 tiles of 256x256; large outputs need nothing
    mid = lib.tp_workspace_size(1, 65, n, k, 0)
    assert mid > 0 and mid % (4 * 65 * n) == 0
    assert lib.tp_workspace_size(1, 4096, n, k, 0) == 0
    assert lib.tp_workspace_size(1, 3, 9, 255, 0) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    import int4_quantized_gemm_amd as tp
    with pytest.raises(ValueError):
        tp.tp_hadamard_rotate_rows(torch.zeros(4, 256))


def test_small_m_plan_workspace_properties(lib):
    """The 9..64-row plan (fragment height, groups per split) is a pure
    function of the shape: repeated queries agree, and a split plan asks for
    whole planes of M x N 4-byte partial sums, at most one per 256-group."""
    import random
    rnd = random.Random(5)
    for _ in range(400):
        m, n, k = rnd.randint(9, 64), rnd.randint(1, 30000), 256 * rnd.randint(1, 64)
        for op in (1, 2, 4):  # W8, W4 pre-rotated; W8A8 pre-quantized
            a = lib.tp_workspace_size(op, m, n, k, 0)
            assert a == lib.tp_workspace_size(op, m, n, k, 0)
            assert a % (m * n * 4) == 0, (op, m, n, k, a)
            assert a // (m * n * 4) <= k // 256, (op, m, n, k, a)
