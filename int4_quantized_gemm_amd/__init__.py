"""Rotated, quantized linear projections ("ConvRot") on AMD Instinct MI355X.

Thin Python binding of libtp.so (C ABI in include/tp.h). Each function has the
name of the C entry point it calls and only marshals arguments: it takes
device tensors, allocates outputs (and the workspace, unless one is given)
with PyTorch, and passes data pointers and the current HIP stream. Every step
of the computation runs in the library's HIP kernels; there is no CPU path.

    tp_rotate_quantize_weights(w, bits)        -> (q, scales)
    tp_hadamard_rotate_rows(x, out_dtype)      -> y = x . blockdiag(H/16)
    tp_quantize_rows_int8(x, rotate)           -> (qa, sa)
    tp_qgemm_w8(a, q, s, rotate, out_dtype)    -> C
    tp_qgemm_w4(a, q, s, rotate, out_dtype)    -> C
    tp_qgemm_w8a8(a, q, s, rotate, out_dtype, want_codes, want_acc)
                                               -> C (and qa, sa, acc on request)
    tp_qgemm_w8a8_prequantized(qa, sa, q, s)   -> C (codes from tp_quantize_rows_int8)
"""

import torch

from . import _lib
from ._lib import TPError, TP_A_PREROTATED, TP_A_ROTATE, TP_FFN_OUT_BF16, TP_FFN_OUT_I8  # noqa: F401

_DTYPE = {torch.float32: _lib.TP_F32, torch.bfloat16: _lib.TP_BF16}


def _dt(t):
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)") from None


def _mat(t, name):
    """Check a 2-D row-major CUDA tensor; return its row pitch in elements."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _vec(t, name, numel):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous float32 tensor with {numel} elements")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def tp_workspace_size(op, m, n, k, a_flags):
    return int(_lib.load().tp_workspace_size(op, m, n, k, a_flags))


def tp_rotate_quantize_weights(w, bits=8, q=None, scales=None, stream=None):
    """Rotate W [n, k] per 256-group (fp64) and quantize: bits=8 gives int8
    [n, k] and fp32 [n] scales; bits=4 gives packed uint8 [n, k/2] and fp32
    [n, k/256] scales."""
    ldw = _mat(w, "w")
    n, k = w.shape
    if q is None:
        q = torch.empty((n, k if bits == 8 else k // 2), dtype=torch.int8 if bits == 8 else torch.uint8,
                        device=w.device)
    if scales is None:
        scales = torch.empty((n,) if bits == 8 else (n, max(k // 256, 0)), dtype=torch.float32, device=w.device)
    ldq = _mat(q, "q")
    _vec(scales, "scales", n * (1 if bits == 8 else k // 256))
    _lib.check(_lib.load().tp_rotate_quantize_weights(w.data_ptr(), _dt(w), n, k, ldw, bits, q.data_ptr(), ldq,
                                                      scales.data_ptr(), _stream(stream)))
    return q, scales


def tp_hadamard_rotate_rows(x, out_dtype=None, out=None, stream=None):
    """y = x . blockdiag(H/16) in fp32 arithmetic; out may be x (in place)."""
    ldx = _mat(x, "x")
    m, k = x.shape
    if out is None:
        out = torch.empty((m, k), dtype=out_dtype or x.dtype, device=x.device)
    ldy = _mat(out, "out")
    _lib.check(_lib.load().tp_hadamard_rotate_rows(x.data_ptr(), _dt(x), m, k, ldx, out.data_ptr(), _dt(out), ldy,
                                                   _stream(stream)))
    return out


def tp_quantize_rows_int8(x, rotate=True, qa=None, sa=None, stream=None):
    """Rotate (unless rotate=False) and quantize each row to int8 with one fp32
    scale per row."""
    ldx = _mat(x, "x")
    m, k = x.shape
    if qa is None:
        qa = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if sa is None:
        sa = torch.empty((m,), dtype=torch.float32, device=x.device)
    ldqa = _mat(qa, "qa")
    _vec(sa, "sa", m)
    flags = TP_A_ROTATE if rotate else TP_A_PREROTATED
    _lib.check(_lib.load().tp_quantize_rows_int8(x.data_ptr(), _dt(x), m, k, ldx, flags, qa.data_ptr(), ldqa,
                                                 sa.data_ptr(), _stream(stream)))
    return qa, sa


def tp_swiglu_rotate(gate, up, out_kind="i8", out=None, scales=None, stream=None):
    """h = bf16(silu(gate) * up) rotated per 256-group, as int8 codes with one
    fp32 scale per row (out_kind "i8": returns (codes, scales)) or as rotated
    bf16 rows (out_kind "bf16": returns the rows). gate and up: [m, k], both
    fp32 or both bf16 (may be column views of one gate+up output)."""
    if out_kind not in ("i8", "bf16"):
        raise ValueError("out_kind must be 'i8' or 'bf16'")
    if gate.shape != up.shape or gate.dtype != up.dtype:
        raise ValueError("gate and up must have the same shape and dtype")
    ldg = _mat(gate, "gate")
    ldu = _mat(up, "up")
    m, k = gate.shape
    i8 = out_kind == "i8"
    if out is None:
        out = torch.empty((m, k), dtype=torch.int8 if i8 else torch.bfloat16, device=gate.device)
    ldy = _mat(out, "out")
    if i8:
        if scales is None:
            scales = torch.empty((m,), dtype=torch.float32, device=gate.device)
        _vec(scales, "scales", m)
    _lib.check(_lib.load().tp_swiglu_rotate(gate.data_ptr(), ldg, up.data_ptr(), ldu, _dt(gate), m, k,
                                            TP_FFN_OUT_I8 if i8 else TP_FFN_OUT_BF16, out.data_ptr(), ldy,
                                            scales.data_ptr() if i8 else None, _stream(stream)))
    return (out, scales) if i8 else out


def _workspace(op, m, n, k, flags, device, workspace):
    need = tp_workspace_size(op, m, n, k, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _weight_only(fn_name, op, a, q, scales, rotate, out_dtype, out, workspace, stream, bits):
    lda = _mat(a, "a")
    m, k = a.shape
    n = q.shape[0]
    ldq = _mat(q, "q")
    _vec(scales, "w_scales", n * (1 if bits == 8 else k // 256))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    ldc = _mat(out, "out")
    flags = TP_A_ROTATE if rotate else TP_A_PREROTATED
    ws, ws_bytes = _workspace(op, m, n, k, flags, a.device, workspace)
    fn = getattr(_lib.load(), fn_name)
    _lib.check(fn(a.data_ptr(), _dt(a), lda, flags, q.data_ptr(), ldq, scales.data_ptr(), m, n, k, out.data_ptr(),
                  _dt(out), ldc, ws.data_ptr(), ws_bytes, _stream(stream)))
    return out


def tp_qgemm_w8(a, q, scales, rotate=True, out_dtype=torch.bfloat16, out=None, workspace=None, stream=None):
    """C = (bf16(A') . q^T) * s[n]; A' = rotated a (or a itself if rotate=False,
    which must then be bf16)."""
    return _weight_only("tp_qgemm_w8", _lib.TP_OP_QGEMM_W8, a, q, scales, rotate, out_dtype, out, workspace,
                        stream, 8)


def tp_qgemm_w4(a, q, scales, rotate=True, out_dtype=torch.bfloat16, out=None, workspace=None, stream=None):
    """C = sum_g s[n, g] (bf16(A'_g) . q_g^T) with packed int4 q [n, k/2]."""
    return _weight_only("tp_qgemm_w4", _lib.TP_OP_QGEMM_W4, a, q, scales, rotate, out_dtype, out, workspace,
                        stream, 4)


def tp_qgemm_w8a8(a, q, scales, rotate=True, out_dtype=torch.float32, out=None, want_codes=False, want_acc=False,
                  workspace=None, stream=None):
    """Per-token int8 activations x int8 weights; int32 sums; fp32 epilogue
    (float(acc) * sa[m]) * sw[n]. Returns C, or (C, qa, sa, acc) with the
    requested intermediates (None where not requested)."""
    lda = _mat(a, "a")
    m, k = a.shape
    n = q.shape[0]
    ldq = _mat(q, "q")
    _vec(scales, "w_scales", n)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    ldc = _mat(out, "out")
    qa = sa = acc = None
    if want_codes:
        qa = torch.empty((m, k), dtype=torch.int8, device=a.device)
        sa = torch.empty((m,), dtype=torch.float32, device=a.device)
    if want_acc:
        acc = torch.empty((m, n), dtype=torch.int32, device=a.device)
    flags = TP_A_ROTATE if rotate else TP_A_PREROTATED
    if want_codes:
        # the codes go to qa / sa: only the split-K partial sums need scratch
        ws, ws_bytes = _workspace(_lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, flags, a.device, workspace)
    else:
        ws, ws_bytes = _workspace(_lib.TP_OP_QGEMM_W8A8, m, n, k, flags, a.device, workspace)
    ld_acc = _mat(acc, "acc") if acc is not None else 0
    _lib.check(_lib.load().tp_qgemm_w8a8(a.data_ptr(), _dt(a), lda, flags, q.data_ptr(), ldq, scales.data_ptr(), m, n,
                                         k, out.data_ptr(), _dt(out), ldc, _ptr(qa), _ptr(sa), _ptr(acc), ld_acc,
                                         _ptr(ws), ws_bytes, _stream(stream)))
    if want_codes or want_acc:
        return out, qa, sa, acc
    return out


def tp_qgemm_w8a8_prequantized(qa, sa, q, scales, out_dtype=torch.float32, out=None, acc=None, workspace=None,
                               stream=None):
    """C = (float(qa . q^T) * sa[m]) * s[n] on activation codes already made by
    tp_quantize_rows_int8; optionally also writes the int32 accumulators."""
    ldqa = _mat(qa, "qa")
    m, k = qa.shape
    n = q.shape[0]
    ldq = _mat(q, "q")
    _vec(sa, "sa", m)
    _vec(scales, "w_scales", n)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=qa.device)
    ldc = _mat(out, "out")
    ld_acc = _mat(acc, "acc") if acc is not None else 0
    ws, ws_bytes = _workspace(_lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, TP_A_PREROTATED, qa.device, workspace)
    _lib.check(_lib.load().tp_qgemm_w8a8_prequantized(qa.data_ptr(), ldqa, sa.data_ptr(), q.data_ptr(), ldq,
                                                      scales.data_ptr(), m, n, k, out.data_ptr(), _dt(out), ldc,
                                                      _ptr(acc), ld_acc, _ptr(ws), ws_bytes, _stream(stream)))
    return out


def tp_qgemm_w8a8_prequantized_noalloc(qa, sa, q, scales, out_dtype=torch.float32, out=None, acc=None, stream=None):
    """tp_qgemm_w8a8_prequantized without a workspace: the split-K partial sums
    go to the library's own scratch array (32 MiB a GPU). The caller passes the
    output (or lets this binding allocate it with torch); the library
    allocates nothing."""
    ldqa = _mat(qa, "qa")
    m, k = qa.shape
    n = q.shape[0]
    ldq = _mat(q, "q")
    _vec(sa, "sa", m)
    _vec(scales, "w_scales", n)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=qa.device)
    ldc = _mat(out, "out")
    ld_acc = _mat(acc, "acc") if acc is not None else 0
    _lib.check(_lib.load().tp_qgemm_w8a8_prequantized_noalloc(qa.data_ptr(), ldqa, sa.data_ptr(), q.data_ptr(), ldq,
                                                              scales.data_ptr(), m, n, k, out.data_ptr(), _dt(out),
                                                              ldc, _ptr(acc), ld_acc, _stream(stream)))
    return out


def tp_qgemm_w8a8_prequantized_lora(qa, sa, q, scales, t, lora_b, alpha, out=None, workspace=None, stream=None):
    """C = (float(qa . q^T) * sa[m]) * s[n] + alpha * T . lora_b^T in fp32, the
    side path added in the product's store; T from tp_lora_down, lora_b bf16
    [n, r]."""
    ldqa = _mat(qa, "qa")
    m, k = qa.shape
    n = q.shape[0]
    r = lora_b.shape[1]
    ldq = _mat(q, "q")
    _vec(sa, "sa", m)
    _vec(scales, "w_scales", n)
    if t.dtype != torch.float32 or t.shape != (m, 64) or not t.is_contiguous():
        raise ValueError("t must be contiguous fp32 [m, 64] (from tp_lora_down)")
    if lora_b.dtype != torch.bfloat16 or lora_b.shape[0] != n:
        raise ValueError("lora_b must be bf16 [n, r]")
    ldb = _mat(lora_b, "lora_b")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=qa.device)
    ldc = _mat(out, "out")
    ws, ws_bytes = _workspace(_lib.TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, TP_A_PREROTATED, qa.device, workspace)
    _lib.check(_lib.load().tp_qgemm_w8a8_prequantized_lora(qa.data_ptr(), ldqa, sa.data_ptr(), q.data_ptr(), ldq,
                                                           scales.data_ptr(), m, n, k, out.data_ptr(), ldc,
                                                           t.data_ptr(), lora_b.data_ptr(), ldb, r, float(alpha),
                                                           _ptr(ws), ws_bytes, _stream(stream)))
    return out


def tp_qgemm_w4a8(a, q4, scales, rotate=True, out_dtype=torch.float32, out=None, want_codes=False, workspace=None,
                  stream=None):
    """Per-token int8 activations x int4 weights with one scale per (row,
    256-group); exact int32 sums per group, folded in fp32. Returns C, or
    (C, qa, sa) when want_codes."""
    lda = _mat(a, "a")
    m, k = a.shape
    n = q4.shape[0]
    ldq = _mat(q4, "q4")
    _vec(scales, "w_scales", n * (k // 256))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    ldc = _mat(out, "out")
    qa = sa = None
    if want_codes:
        qa = torch.empty((m, k), dtype=torch.int8, device=a.device)
        sa = torch.empty((m,), dtype=torch.float32, device=a.device)
    flags = TP_A_ROTATE if rotate else TP_A_PREROTATED
    op = _lib.TP_OP_QGEMM_W4A8_PREQUANTIZED if want_codes else _lib.TP_OP_QGEMM_W4A8
    ws, ws_bytes = _workspace(op, m, n, k, flags, a.device, workspace)
    _lib.check(_lib.load().tp_qgemm_w4a8(a.data_ptr(), _dt(a), lda, flags, q4.data_ptr(), ldq, scales.data_ptr(), m,
                                         n, k, out.data_ptr(), _dt(out), ldc, _ptr(qa), _ptr(sa), _ptr(ws), ws_bytes,
                                         _stream(stream)))
    return (out, qa, sa) if want_codes else out


def tp_qgemm_w4a8_prequantized(qa, sa, q4, scales, out_dtype=torch.float32, out=None, workspace=None, stream=None):
    """C = (sum_g s[n, g] * float(qa_g . q4_g^T)) * sa[m] on activation codes
    already made (tp_quantize_rows_int8, tp_swiglu_rotate)."""
    ldqa = _mat(qa, "qa")
    m, k = qa.shape
    n = q4.shape[0]
    ldq = _mat(q4, "q4")
    _vec(sa, "sa", m)
    _vec(scales, "w_scales", n * (k // 256))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=qa.device)
    ldc = _mat(out, "out")
    ws, ws_bytes = _workspace(_lib.TP_OP_QGEMM_W4A8_PREQUANTIZED, m, n, k, TP_A_PREROTATED, qa.device, workspace)
    _lib.check(_lib.load().tp_qgemm_w4a8_prequantized(qa.data_ptr(), ldqa, sa.data_ptr(), q4.data_ptr(), ldq,
                                                      scales.data_ptr(), m, n, k, out.data_ptr(), _dt(out), ldc,
                                                      _ptr(ws), ws_bytes, _stream(stream)))
    return out


def tp_dequantize_unrotate(q, scales, bits, out_dtype=torch.float32, out=None, stream=None):
    """W_hat = (q * s) . blockdiag(H/16): the weight a rotated, quantized
    checkpoint stands for (exact, rounded once to out_dtype). q: int8 [n, k]
    with scales [n] (bits 8) or packed uint8 [n, k/2] with scales [n, k/256]
    (bits 4)."""
    ldq = _mat(q, "q")
    n = q.shape[0]
    k = q.shape[1] * (1 if bits == 8 else 2)
    _vec(scales, "scales", n * (1 if bits == 8 else k // 256))
    if out is None:
        out = torch.empty((n, k), dtype=out_dtype, device=q.device)
    ldw = _mat(out, "out")
    _lib.check(_lib.load().tp_dequantize_unrotate(q.data_ptr(), bits, ldq, scales.data_ptr(), n, k, out.data_ptr(),
                                                  _dt(out), ldw, _stream(stream)))
    return out


def tp_requantize_weights(q, scales, bits_in, bits_out, q_out=None, scales_out=None, stream=None):
    """Codes and scales of width bits_out for the weight held as (q, scales)
    of width bits_in (same layouts as tp_rotate_quantize_weights)."""
    ldq = _mat(q, "q")
    n = q.shape[0]
    k = q.shape[1] * (1 if bits_in == 8 else 2)
    _vec(scales, "scales", n * (1 if bits_in == 8 else k // 256))
    if q_out is None:
        q_out = torch.empty((n, k if bits_out == 8 else k // 2), dtype=torch.int8 if bits_out == 8 else torch.uint8,
                            device=q.device)
    if scales_out is None:
        scales_out = torch.empty((n,) if bits_out == 8 else (n, k // 256), dtype=torch.float32, device=q.device)
    ldo = _mat(q_out, "q_out")
    _vec(scales_out, "scales_out", n * (1 if bits_out == 8 else k // 256))
    _lib.check(_lib.load().tp_requantize_weights(q.data_ptr(), bits_in, ldq, scales.data_ptr(), n, k, bits_out,
                                                 q_out.data_ptr(), ldo, scales_out.data_ptr(), _stream(stream)))
    return q_out, scales_out


def tp_lora_workspace_size(m, r):
    """Bytes of workspace tp_lora_add needs for m rows at rank r."""
    return int(_lib.load().tp_lora_workspace_size(m, r))


def tp_lora_down(x, lora_a, t=None, stream=None):
    """T = x . lora_a^T in fp32 rows of 64 (zeros past r): the first half of
    the side path, for tp_qgemm_w8a8_prequantized_lora. Returns T [m, 64]."""
    ldx = _mat(x, "x")
    m, k = x.shape
    r = lora_a.shape[0]
    if lora_a.shape[1] != k:
        raise ValueError("lora_a must be [r, k]")
    lda = _mat(lora_a, "lora_a")
    if t is None:
        t = torch.empty((m, 64), dtype=torch.float32, device=x.device)
    _lib.check(_lib.load().tp_lora_down(x.data_ptr(), _dt(x), ldx, lora_a.data_ptr(), _dt(lora_a), lda, m, k, r,
                                        t.data_ptr(), t.numel() * t.element_size(), _stream(stream)))
    return t


def tp_lora_add(c, x, lora_a, lora_b, alpha, workspace=None, stream=None):
    """c += alpha * (x . lora_a^T) . lora_b^T in place (lora_a [r, k],
    lora_b [n, r], same dtype; r <= 64). Returns c."""
    ldx = _mat(x, "x")
    m, k = x.shape
    r = lora_a.shape[0]
    n = c.shape[1]
    if lora_a.shape[1] != k or lora_b.shape != (n, r) or c.shape[0] != m or lora_a.dtype != lora_b.dtype:
        raise ValueError("shapes/dtypes: x [m, k], lora_a [r, k], lora_b [n, r] (same dtype), c [m, n]")
    lda = _mat(lora_a, "lora_a")
    ldb = _mat(lora_b, "lora_b")
    ldc = _mat(c, "c")
    need = _lib.load().tp_lora_workspace_size(m, r)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    _lib.check(_lib.load().tp_lora_add(x.data_ptr(), _dt(x), ldx, lora_a.data_ptr(), lora_b.data_ptr(), _dt(lora_a),
                                       lda, ldb, float(alpha), m, n, k, r, c.data_ptr(), _dt(c), ldc,
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(stream)))
    return c
