// C ABI of the rotated, quantized projection library (declared in
// include/tp.h). Every argument is validated here before any HIP call, so a
// refused call has enqueued no work (the TensorFold pull request #948 review
// asks for sizes and products to be checked before any device work; kvad-gpu
// internals, "Quantised weights on the GPU", refuses dimensions not divisible
// by 256 up front rather than failing halfway).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/tp.h"
#include "kernels.hpp"

namespace {

thread_local char g_msg[512] = "";

tp_status fail(tp_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tp_status fail(tp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

tp_status ok() {
  g_msg[0] = '\0';
  return TP_OK;
}

tp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

// Byte extent [p, p + bytes) of a row-major matrix: (rows-1)*pitch + row_bytes.
struct Extent {
  uintptr_t lo = 0, hi = 0;
};

Extent extent_of(const void* p, int64_t rows, int64_t pitch_bytes, int64_t row_bytes) {
  Extent e;
  e.lo = (uintptr_t)p;
  e.hi = rows > 0 ? e.lo + (uintptr_t)((rows - 1) * pitch_bytes + row_bytes) : e.lo;
  return e;
}

bool overlaps(const Extent& a, const Extent& b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

int64_t dtype_size(tp_dtype d) { return d == TP_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == TP_F32 || d == TP_BF16; }

// Validate one row-major operand: non-null (unless it is empty), ld >= row
// length, base and pitch aligned to `align` bytes, total extent representable.
// On success stores the extent (empty for an empty operand).
tp_status check_matrix(const char* name, const void* p, int64_t rows, int64_t cols_bytes, int64_t ld,
                       int64_t elem_bytes, Extent* ext, int64_t align = 16) {
  int64_t pitch;
  if (!mul_ok(ld, elem_bytes, &pitch)) return fail(TP_ERR_SIZE_OVERFLOW, "%s: ld * element size overflows", name);
  if (ld < 0 || pitch < cols_bytes)
    return fail(TP_ERR_BAD_LEADING_DIM, "%s: leading dimension %lld is smaller than the row (%lld bytes)", name,
                (long long)ld, (long long)cols_bytes);
  if (rows == 0 || cols_bytes == 0) {  // empty: nothing is read or written
    *ext = Extent{};
    return TP_OK;
  }
  if (!p) return fail(TP_ERR_NULL_POINTER, "%s is NULL", name);
  int64_t span;
  if (!mul_ok(rows - 1, pitch, &span) || !add_ok(span, cols_bytes, &span))
    return fail(TP_ERR_SIZE_OVERFLOW, "%s: byte extent overflows", name);
  if (((uintptr_t)p % (uintptr_t)align) != 0)
    return fail(TP_ERR_MISALIGNED, "%s: base pointer is not %lld-byte aligned", name, (long long)align);
  if (pitch % align != 0)
    return fail(TP_ERR_MISALIGNED, "%s: row pitch of %lld bytes is not a multiple of %lld", name, (long long)pitch,
                (long long)align);
  *ext = extent_of(p, rows, pitch, cols_bytes);
  return TP_OK;
}

tp_status check_vector(const char* name, const void* p, int64_t count, Extent* ext) {
  if (count == 0) {
    *ext = Extent{};
    return TP_OK;
  }
  if (!p) return fail(TP_ERR_NULL_POINTER, "%s is NULL", name);
  if (((uintptr_t)p & 3u) != 0) return fail(TP_ERR_MISALIGNED, "%s: not 4-byte aligned", name);
  int64_t bytes;
  if (!mul_ok(count, 4, &bytes)) return fail(TP_ERR_SIZE_OVERFLOW, "%s: size overflows", name);
  ext->lo = (uintptr_t)p;
  ext->hi = ext->lo + (uintptr_t)bytes;
  return TP_OK;
}

tp_status check_sizes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0) return fail(TP_ERR_BAD_SHAPE, "negative size (m=%lld, n=%lld)", (long long)m, (long long)n);
  if (k <= 0) return fail(TP_ERR_BAD_SHAPE, "k must be positive (k=%lld)", (long long)k);
  if (k % 256 != 0)
    return fail(TP_ERR_K_NOT_MULTIPLE_OF_256, "k=%lld is not a multiple of 256 (the rotation group)", (long long)k);
  if (m > INT_MAX || n > INT_MAX || k > INT_MAX)
    return fail(TP_ERR_BAD_SHAPE, "size above 2^31-1 (m=%lld, n=%lld, k=%lld)", (long long)m, (long long)n,
                (long long)k);
  return TP_OK;
}

#define TP_TRY(expr)                  \
  do {                                \
    tp_status _st = (expr);           \
    if (_st != TP_OK) return _st;     \
  } while (0)

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Workspace layout. Front part: W8/W4 with TP_A_ROTATE, bf16 A' [m, k];
// W8A8 (unless the caller takes the codes), int8 qa [m, k] then (256-byte
// aligned) fp32 sa [m]. Then, 256-byte aligned, the split-K partial sums of
// the small-M products (qgemm_partial_bytes; absent for larger M).
struct WsLayout {
  int64_t front = 0;     // bytes of the front part
  int64_t part_off = 0;  // offset of the partial sums
  int64_t total = 0;     // bytes needed
};

bool workspace_layout(tp_op op, int64_t m, int64_t n, int64_t k, int a_flags, bool own_codes, WsLayout* out) {
  int64_t mk;
  if (!mul_ok(m, k, &mk)) return false;
  int kind;
  WsLayout l;
  switch (op) {
    case TP_OP_QGEMM_W8:
    case TP_OP_QGEMM_W4:
      kind = op == TP_OP_QGEMM_W8 ? tp::GEMM_W8 : tp::GEMM_W4;
      if (a_flags == TP_A_ROTATE && !mul_ok(mk, 2, &l.front)) return false;
      break;
    case TP_OP_QGEMM_W8A8:
    case TP_OP_QGEMM_W4A8: {
      kind = op == TP_OP_QGEMM_W8A8 ? tp::GEMM_W8A8 : tp::GEMM_W4A8;
      if (!own_codes) {
        int64_t sa;
        if (!mul_ok(m, 4, &sa)) return false;
        if (mk > INT64_MAX - 512 - sa) return false;
        l.front = round_up(mk, 256) + sa;
      }
      break;
    }
    case TP_OP_QGEMM_W8A8_PREQUANTIZED:
      kind = tp::GEMM_W8A8;
      break;
    case TP_OP_QGEMM_W4A8_PREQUANTIZED:
      kind = tp::GEMM_W4A8;
      break;
    default:
      return false;
  }
  const int64_t part = tp::qgemm_partial_bytes(kind, m, n, k);
  if (part < 0 || l.front > INT64_MAX - 512 - part) return false;
  l.part_off = part > 0 ? round_up(l.front, 256) : l.front;
  l.total = l.part_off + part;
  *out = l;
  return true;
}

// Checks the caller's workspace against the layout; stores its extent.
tp_status check_workspace(const WsLayout& l, const void* ws, size_t ws_bytes, Extent* ew) {
  *ew = Extent{};
  if (l.total == 0) return TP_OK;
  if (!ws || (uint64_t)ws_bytes < (uint64_t)l.total)
    return fail(TP_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes given, %lld needed", ws_bytes,
                (long long)l.total);
  if (((uintptr_t)ws & 15u) != 0) return fail(TP_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  ew->lo = (uintptr_t)ws;
  ew->hi = ew->lo + (uintptr_t)l.total;
  return TP_OK;
}

}  // namespace

extern "C" {

const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_NULL_POINTER: return "TP_ERR_NULL_POINTER";
    case TP_ERR_BAD_SHAPE: return "TP_ERR_BAD_SHAPE";
    case TP_ERR_K_NOT_MULTIPLE_OF_256: return "TP_ERR_K_NOT_MULTIPLE_OF_256";
    case TP_ERR_BAD_LEADING_DIM: return "TP_ERR_BAD_LEADING_DIM";
    case TP_ERR_MISALIGNED: return "TP_ERR_MISALIGNED";
    case TP_ERR_UNSUPPORTED_DTYPE: return "TP_ERR_UNSUPPORTED_DTYPE";
    case TP_ERR_UNSUPPORTED_BITS: return "TP_ERR_UNSUPPORTED_BITS";
    case TP_ERR_SIZE_OVERFLOW: return "TP_ERR_SIZE_OVERFLOW";
    case TP_ERR_WORKSPACE_TOO_SMALL: return "TP_ERR_WORKSPACE_TOO_SMALL";
    case TP_ERR_BAD_ALIASING: return "TP_ERR_BAD_ALIASING";
    case TP_ERR_BAD_FLAGS: return "TP_ERR_BAD_FLAGS";
    case TP_ERR_HIP: return "TP_ERR_HIP";
  }
  return "TP_ERR_UNKNOWN";
}

const char* tp_last_error_message(void) { return g_msg; }

int tp_abi_version(void) { return TP_ABI_VERSION; }

size_t tp_workspace_size(tp_op op, int64_t m, int64_t n, int64_t k, int a_flags) {
  if (m < 0 || n < 0 || k <= 0 || k % 256 != 0 || m > INT_MAX || n > INT_MAX || k > INT_MAX) return 0;
  WsLayout l;
  if (!workspace_layout(op, m, n, k, a_flags, false, &l)) return 0;
  return (size_t)l.total;
}

tp_status tp_rotate_quantize_weights(const void* w, tp_dtype w_dtype, int64_t n, int64_t k, int64_t ldw, int bits,
                                     void* q, int64_t ldq, float* scales, hipStream_t stream) {
  if (!dtype_ok(w_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "w_dtype %d is not TP_F32 or TP_BF16", (int)w_dtype);
  if (bits != 8 && bits != 4) return fail(TP_ERR_UNSUPPORTED_BITS, "bits=%d (expected 8 or 4)", bits);
  TP_TRY(check_sizes(0, n, k));
  Extent ew, eq, es;
  TP_TRY(check_matrix("w", w, n, k * dtype_size(w_dtype), ldw, dtype_size(w_dtype), &ew));
  TP_TRY(check_matrix("q", q, n, bits == 8 ? k : k / 2, ldq, 1, &eq));
  int64_t ns;
  if (!mul_ok(n, bits == 8 ? 1 : k / 256, &ns)) return fail(TP_ERR_SIZE_OVERFLOW, "scale count overflows");
  TP_TRY(check_vector("scales", scales, ns, &es));
  if (overlaps(ew, eq) || overlaps(ew, es) || overlaps(eq, es))
    return fail(TP_ERR_BAD_ALIASING, "w, q and scales must not overlap");
  if (n == 0) return ok();
  return hip_status(tp::launch_rotq_rows(w, w_dtype == TP_BF16, ldw, n, k, true, bits, q, ldq, scales, stream),
                    "rotate-quantize launch");
}

tp_status tp_hadamard_rotate_rows(const void* x, tp_dtype x_dtype, int64_t m, int64_t k, int64_t ldx, void* y,
                                  tp_dtype y_dtype, int64_t ldy, hipStream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "x_dtype %d is not TP_F32 or TP_BF16", (int)x_dtype);
  if (!dtype_ok(y_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "y_dtype %d is not TP_F32 or TP_BF16", (int)y_dtype);
  TP_TRY(check_sizes(m, 0, k));
  Extent ex, ey;
  TP_TRY(check_matrix("x", x, m, k * dtype_size(x_dtype), ldx, dtype_size(x_dtype), &ex));
  TP_TRY(check_matrix("y", y, m, k * dtype_size(y_dtype), ldy, dtype_size(y_dtype), &ey));
  const bool in_place = (x == y && x_dtype == y_dtype && ldx == ldy);
  if (!in_place && overlaps(ex, ey))
    return fail(TP_ERR_BAD_ALIASING, "x and y overlap without being the same buffer, dtype and ld");
  if (m == 0) return ok();
  return hip_status(tp::launch_rotate_rows(x, x_dtype == TP_BF16, ldx, y, y_dtype == TP_BF16, ldy, m, k, stream),
                    "rotate launch");
}

tp_status tp_quantize_rows_int8(const void* x, tp_dtype x_dtype, int64_t m, int64_t k, int64_t ldx, int a_flags,
                                int8_t* qa, int64_t ldqa, float* sa, hipStream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "x_dtype %d is not TP_F32 or TP_BF16", (int)x_dtype);
  if (a_flags != TP_A_ROTATE && a_flags != TP_A_PREROTATED) return fail(TP_ERR_BAD_FLAGS, "a_flags=%d", a_flags);
  TP_TRY(check_sizes(m, 0, k));
  Extent ex, eq, es;
  TP_TRY(check_matrix("x", x, m, k * dtype_size(x_dtype), ldx, dtype_size(x_dtype), &ex));
  TP_TRY(check_matrix("qa", qa, m, k, ldqa, 1, &eq));
  TP_TRY(check_vector("sa", sa, m, &es));
  if (overlaps(ex, eq) || overlaps(ex, es) || overlaps(eq, es))
    return fail(TP_ERR_BAD_ALIASING, "x, qa and sa must not overlap");
  if (m == 0) return ok();
  return hip_status(tp::launch_rotq_rows(x, x_dtype == TP_BF16, ldx, m, k, a_flags == TP_A_ROTATE, 8, qa, ldqa, sa,
                                         stream),
                    "activation quantize launch");
}

namespace {

tp_status check_codes(const char* name, const void* q, int bits, int64_t n, int64_t k, int64_t ldq, const char* sname,
                      const float* s, Extent* eq, Extent* es) {
  if (bits != 8 && bits != 4) return fail(TP_ERR_UNSUPPORTED_BITS, "%s: bits=%d is neither 8 nor 4", name, bits);
  TP_TRY(check_matrix(name, q, n, bits == 8 ? k : k / 2, ldq, 1, eq));
  int64_t ns;
  if (!mul_ok(n, bits == 8 ? 1 : k / 256, &ns)) return fail(TP_ERR_SIZE_OVERFLOW, "%s: scale count overflows", sname);
  return check_vector(sname, s, ns, es);
}

}  // namespace

size_t tp_lora_workspace_size(int64_t m, int64_t r) {
  if (m < 0 || r < 1 || r > 64 || m > INT_MAX) return 0;
  return (size_t)(m * 64 * 4);  // fp32 rows of 64 (zeros past r)
}

tp_status tp_lora_add(const void* x, tp_dtype x_dtype, int64_t ldx, const void* lora_a, const void* lora_b,
                      tp_dtype ab_dtype, int64_t lda, int64_t ldb, float alpha, int64_t m, int64_t n, int64_t k,
                      int64_t r, void* c, tp_dtype c_dtype, int64_t ldc, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "x_dtype %d is not TP_F32 or TP_BF16", (int)x_dtype);
  if (!dtype_ok(ab_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "ab_dtype %d is not TP_F32 or TP_BF16", (int)ab_dtype);
  if (!dtype_ok(c_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "c_dtype %d is not TP_F32 or TP_BF16", (int)c_dtype);
  TP_TRY(check_sizes(m, n, k));
  if (r < 1 || r > 64) return fail(TP_ERR_BAD_SHAPE, "rank r=%lld outside [1, 64]", (long long)r);
  const int64_t ex = dtype_size(x_dtype), eab = dtype_size(ab_dtype), ec_ = dtype_size(c_dtype);
  Extent e_x, e_a, e_b, e_c, e_w;
  TP_TRY(check_matrix("x", x, m, k * ex, ldx, ex, &e_x));
  TP_TRY(check_matrix("lora_a", lora_a, r, k * eab, lda, eab, &e_a));
  TP_TRY(check_matrix("lora_b", lora_b, n, r * eab, ldb, eab, &e_b));
  TP_TRY(check_matrix("c", c, m, n * ec_, ldc, ec_, &e_c, ec_));
  const int64_t need = m * 64 * 4;
  if (m > 0 && n > 0) {
    if (!workspace || (int64_t)workspace_bytes < need)
      return fail(TP_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %lld needed (tp_lora_workspace_size)",
                  workspace_bytes, (long long)need);
    if (((uintptr_t)workspace & 15u) != 0) return fail(TP_ERR_MISALIGNED, "workspace is not 16-byte aligned");
    e_w.lo = (uintptr_t)workspace;
    e_w.hi = e_w.lo + (uintptr_t)need;
  }
  const Extent* ins[] = {&e_x, &e_a, &e_b};
  for (const Extent* i : ins)
    if (overlaps(e_c, *i) || overlaps(e_w, *i)) return fail(TP_ERR_BAD_ALIASING, "c or the workspace overlaps an input");
  if (overlaps(e_c, e_w)) return fail(TP_ERR_BAD_ALIASING, "c and the workspace overlap");
  if (m == 0 || n == 0) return ok();
  return hip_status(tp::launch_lora_add(x, x_dtype == TP_BF16, ldx, lora_a, lora_b, ab_dtype == TP_BF16, lda, ldb,
                                        alpha, m, n, k, r, c, c_dtype == TP_BF16, ldc, (float*)workspace, stream),
                    "lora launch");
}

tp_status tp_lora_down(const void* x, tp_dtype x_dtype, int64_t ldx, const void* lora_a, tp_dtype a_dtype,
                       int64_t lda, int64_t m, int64_t k, int64_t r, float* t, size_t t_bytes, hipStream_t stream) {
  if (!dtype_ok(x_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "x_dtype %d is not TP_F32 or TP_BF16", (int)x_dtype);
  if (!dtype_ok(a_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "a_dtype %d is not TP_F32 or TP_BF16", (int)a_dtype);
  TP_TRY(check_sizes(m, 0, k));
  if (r < 1 || r > 64) return fail(TP_ERR_BAD_SHAPE, "rank r=%lld outside [1, 64]", (long long)r);
  const int64_t ex = dtype_size(x_dtype), ea = dtype_size(a_dtype);
  Extent e_x, e_a, e_t;
  TP_TRY(check_matrix("x", x, m, k * ex, ldx, ex, &e_x));
  TP_TRY(check_matrix("lora_a", lora_a, r, k * ea, lda, ea, &e_a));
  if (m > 0 && (int64_t)t_bytes < m * 64 * 4)
    return fail(TP_ERR_WORKSPACE_TOO_SMALL, "t of %zu bytes, %lld needed (m rows of 64 floats)", t_bytes,
                (long long)(m * 64 * 4));
  TP_TRY(check_matrix("t", t, m, 64 * 4, 64, 4, &e_t));
  if (overlaps(e_t, e_x) || overlaps(e_t, e_a)) return fail(TP_ERR_BAD_ALIASING, "t overlaps an input");
  if (m == 0) return ok();
  return hip_status(tp::launch_lora_down(x, x_dtype == TP_BF16, ldx, lora_a, a_dtype == TP_BF16, lda, m, k, r, t,
                                         stream),
                    "lora down launch");
}

tp_status tp_dequantize_unrotate(const void* q, int bits, int64_t ldq_bytes, const float* scales, int64_t n,
                                 int64_t k, void* w, tp_dtype w_dtype, int64_t ldw, hipStream_t stream) {
  if (!dtype_ok(w_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "w_dtype %d is not TP_F32 or TP_BF16", (int)w_dtype);
  TP_TRY(check_sizes(0, n, k));
  Extent eq, es, ew;
  TP_TRY(check_codes("q", q, bits, n, k, ldq_bytes, "scales", scales, &eq, &es));
  TP_TRY(check_matrix("w", w, n, k * dtype_size(w_dtype), ldw, dtype_size(w_dtype), &ew));
  if (overlaps(ew, eq) || overlaps(ew, es)) return fail(TP_ERR_BAD_ALIASING, "w must not overlap q or scales");
  if (n == 0) return ok();
  return hip_status(tp::launch_dequant_unrotate(q, bits, ldq_bytes, scales, n, k, w, w_dtype == TP_BF16, ldw, stream),
                    "dequantize launch");
}

tp_status tp_requantize_weights(const void* q_in, int bits_in, int64_t ldq_in, const float* s_in, int64_t n,
                                int64_t k, int bits_out, void* q_out, int64_t ldq_out, float* s_out,
                                hipStream_t stream) {
  TP_TRY(check_sizes(0, n, k));
  Extent eqi, esi, eqo, eso;
  TP_TRY(check_codes("q_in", q_in, bits_in, n, k, ldq_in, "s_in", s_in, &eqi, &esi));
  TP_TRY(check_codes("q_out", q_out, bits_out, n, k, ldq_out, "s_out", s_out, &eqo, &eso));
  if (overlaps(eqo, eqi) || overlaps(eqo, esi) || overlaps(eso, eqi) || overlaps(eso, esi) || overlaps(eqo, eso))
    return fail(TP_ERR_BAD_ALIASING, "q_out and s_out must not overlap the inputs or each other");
  if (n == 0) return ok();
  return hip_status(tp::launch_requantize(q_in, bits_in, ldq_in, s_in, n, k, bits_out, q_out, ldq_out, s_out, stream),
                    "requantize launch");
}

tp_status tp_swiglu_rotate(const void* gate, int64_t ld_gate, const void* up, int64_t ld_up, tp_dtype in_dtype,
                           int64_t m, int64_t k, int out_kind, void* y, int64_t ldy, float* scales,
                           hipStream_t stream) {
  if (!dtype_ok(in_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "in_dtype %d is not TP_F32 or TP_BF16", (int)in_dtype);
  if (out_kind != TP_FFN_OUT_I8 && out_kind != TP_FFN_OUT_BF16) return fail(TP_ERR_BAD_FLAGS, "out_kind=%d", out_kind);
  TP_TRY(check_sizes(m, 0, k));
  const bool i8 = out_kind == TP_FFN_OUT_I8;
  const int64_t es = dtype_size(in_dtype), ys = i8 ? 1 : 2;
  Extent eg, eu, ey, esc;
  TP_TRY(check_matrix("gate", gate, m, k * es, ld_gate, es, &eg));
  TP_TRY(check_matrix("up", up, m, k * es, ld_up, es, &eu));
  TP_TRY(check_matrix("y", y, m, k * ys, ldy, ys, &ey));
  if (i8) {
    TP_TRY(check_vector("scales", scales, m, &esc));
    if (overlaps(esc, eg) || overlaps(esc, eu) || overlaps(esc, ey))
      return fail(TP_ERR_BAD_ALIASING, "scales must not overlap gate, up or y");
  }
  if (overlaps(ey, eg) || overlaps(ey, eu)) return fail(TP_ERR_BAD_ALIASING, "y must not overlap gate or up");
  if (m == 0) return ok();
  return hip_status(tp::launch_swiglu_rotate(gate, ld_gate, up, ld_up, in_dtype == TP_BF16, m, k, i8, y, ldy,
                                             i8 ? scales : nullptr, stream),
                    "swiglu rotate launch");
}

namespace {

// Shared by the two weight-only products.
tp_status weight_only(int kind, const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const void* q,
                      int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype,
                      int64_t ldc, void* ws, size_t ws_bytes, hipStream_t stream) {
  const tp_op op = kind == tp::GEMM_W8 ? TP_OP_QGEMM_W8 : TP_OP_QGEMM_W4;
  if (a_flags != TP_A_ROTATE && a_flags != TP_A_PREROTATED) return fail(TP_ERR_BAD_FLAGS, "a_flags=%d", a_flags);
  if (!dtype_ok(a_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "a_dtype %d is not TP_F32 or TP_BF16", (int)a_dtype);
  if (a_flags == TP_A_PREROTATED && a_dtype != TP_BF16)
    return fail(TP_ERR_UNSUPPORTED_DTYPE, "a pre-rotated operand must be TP_BF16");
  if (!dtype_ok(c_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "c_dtype %d is not TP_F32 or TP_BF16", (int)c_dtype);
  TP_TRY(check_sizes(m, n, k));
  Extent ea, eq, es, ec, ew;
  TP_TRY(check_matrix("a", a, m, k * dtype_size(a_dtype), lda, dtype_size(a_dtype), &ea));
  TP_TRY(check_matrix("q", q, n, kind == tp::GEMM_W8 ? k : k / 2, ldq, 1, &eq));
  int64_t ns;
  if (!mul_ok(n, kind == tp::GEMM_W8 ? 1 : k / 256, &ns)) return fail(TP_ERR_SIZE_OVERFLOW, "scale count overflows");
  TP_TRY(check_vector("w_scales", w_scales, ns, &es));
  TP_TRY(check_matrix("c", c, m, n * dtype_size(c_dtype), ldc, dtype_size(c_dtype), &ec, dtype_size(c_dtype)));
  WsLayout wl;
  if (!workspace_layout(op, m, n, k, a_flags, false, &wl)) return fail(TP_ERR_SIZE_OVERFLOW, "workspace size overflows");
  TP_TRY(check_workspace(wl, ws, ws_bytes, &ew));
  if (overlaps(ec, ea) || overlaps(ec, eq) || overlaps(ec, es) || overlaps(ec, ew) || overlaps(ew, ea) ||
      overlaps(ew, eq) || overlaps(ew, es))
    return fail(TP_ERR_BAD_ALIASING, "c and the workspace must not overlap any other operand");
  if (m == 0 || n == 0) return ok();

  const void* a_rot = a;
  int64_t lda_rot = lda;
  if (a_flags == TP_A_ROTATE) {
    TP_TRY(hip_status(tp::launch_rotate_rows(a, a_dtype == TP_BF16, lda, ws, true, k, m, k, stream), "rotate launch"));
    a_rot = ws;
    lda_rot = k;
  }
  tp::GemmArgs g{};
  g.kind = kind;
  g.a = a_rot;
  g.lda = lda_rot;
  g.b = q;
  g.ldb = ldq;
  g.w_scales = w_scales;
  g.a_scales = nullptr;
  g.m = m;
  g.n = n;
  g.k = k;
  g.c = c;
  g.c_bf16 = c_dtype == TP_BF16;
  g.ldc = ldc;
  g.acc_out = nullptr;
  g.ld_acc = 0;
  g.part = wl.total > wl.part_off ? (uint8_t*)ws + wl.part_off : nullptr;
  return hip_status(tp::launch_qgemm(g, stream), "product launch");
}

}  // namespace

tp_status tp_qgemm_w8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const int8_t* q, int64_t ldq,
                      const float* w_scales, int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype, int64_t ldc,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return weight_only(tp::GEMM_W8, a, a_dtype, lda, a_flags, q, ldq, w_scales, m, n, k, c, c_dtype, ldc, workspace,
                     workspace_bytes, stream);
}

tp_status tp_qgemm_w4(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const uint8_t* q, int64_t ldq,
                      const float* w_scales, int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype, int64_t ldc,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return weight_only(tp::GEMM_W4, a, a_dtype, lda, a_flags, q, ldq, w_scales, m, n, k, c, c_dtype, ldc, workspace,
                     workspace_bytes, stream);
}

namespace {

// The int8 x int8 (W8A8) and int8 x int4 (W4A8) products on activations the
// library quantizes first. acc_out is W8A8 only.
tp_status act8_product(int kind, const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const void* q,
                       int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k, void* c,
                       tp_dtype c_dtype, int64_t ldc, int8_t* qa_out, float* sa_out, int32_t* acc_out,
                       int64_t ld_acc, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool w4 = kind == tp::GEMM_W4A8;
  const tp_op op = w4 ? TP_OP_QGEMM_W4A8 : TP_OP_QGEMM_W8A8;
  if (a_flags != TP_A_ROTATE && a_flags != TP_A_PREROTATED) return fail(TP_ERR_BAD_FLAGS, "a_flags=%d", a_flags);
  if (!dtype_ok(a_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "a_dtype %d is not TP_F32 or TP_BF16", (int)a_dtype);
  if (!dtype_ok(c_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "c_dtype %d is not TP_F32 or TP_BF16", (int)c_dtype);
  TP_TRY(check_sizes(m, n, k));
  if (!w4 && k > INT32_MAX / (127 * 127))
    return fail(TP_ERR_BAD_SHAPE, "k=%lld: the int32 accumulator could overflow (k <= %d)", (long long)k,
                INT32_MAX / (127 * 127));
  Extent ea, eq, es, ec, eqa, esa, eacc, ew;
  TP_TRY(check_matrix("a", a, m, k * dtype_size(a_dtype), lda, dtype_size(a_dtype), &ea));
  TP_TRY(check_matrix("q", q, n, w4 ? k / 2 : k, ldq, 1, &eq));
  int64_t ns;
  if (!mul_ok(n, w4 ? k / 256 : 1, &ns)) return fail(TP_ERR_SIZE_OVERFLOW, "scale count overflows");
  TP_TRY(check_vector("w_scales", w_scales, ns, &es));
  TP_TRY(check_matrix("c", c, m, n * dtype_size(c_dtype), ldc, dtype_size(c_dtype), &ec, dtype_size(c_dtype)));
  const bool own_codes = qa_out && sa_out;
  if (qa_out) TP_TRY(check_matrix("qa_out", qa_out, m, k, k, 1, &eqa));
  if (sa_out) TP_TRY(check_vector("sa_out", sa_out, m, &esa));
  if (acc_out) TP_TRY(check_matrix("acc_out", acc_out, m, n * 4, ld_acc, 4, &eacc, 4));
  WsLayout wl;
  if (!workspace_layout(op, m, n, k, a_flags, own_codes, &wl))
    return fail(TP_ERR_SIZE_OVERFLOW, "workspace size overflows");
  TP_TRY(check_workspace(wl, workspace, workspace_bytes, &ew));
  const Extent* outs[] = {&ec, &eqa, &esa, &eacc, &ew};
  const Extent* ins[] = {&ea, &eq, &es};
  for (const Extent* o : outs) {
    for (const Extent* i : ins)
      if (overlaps(*o, *i)) return fail(TP_ERR_BAD_ALIASING, "an output or the workspace overlaps an input");
    for (const Extent* o2 : outs)
      if (o2 != o && overlaps(*o, *o2)) return fail(TP_ERR_BAD_ALIASING, "two outputs overlap");
  }
  if (m == 0 || n == 0) return ok();

  int8_t* qa = qa_out ? qa_out : (int8_t*)workspace;
  float* sa = sa_out ? sa_out : (float*)((uint8_t*)workspace + round_up(m * k, 256));
  TP_TRY(hip_status(tp::launch_rotq_rows(a, a_dtype == TP_BF16, lda, m, k, a_flags == TP_A_ROTATE, 8, qa, k, sa,
                                         stream),
                    "activation quantize launch"));
  tp::GemmArgs g{};
  g.kind = kind;
  g.a = qa;
  g.lda = k;
  g.b = q;
  g.ldb = ldq;
  g.w_scales = w_scales;
  g.a_scales = sa;
  g.m = m;
  g.n = n;
  g.k = k;
  g.c = c;
  g.c_bf16 = c_dtype == TP_BF16;
  g.ldc = ldc;
  g.acc_out = acc_out;
  g.ld_acc = ld_acc;
  g.part = wl.total > wl.part_off ? (uint8_t*)workspace + wl.part_off : nullptr;
  return hip_status(tp::launch_qgemm(g, stream), "product launch");
}

// The side path of tp_qgemm_w8a8_prequantized_lora: T fp32 [m, 64] (rows of
// 64 floats, zeros past r) and lora_b bf16 [n, r]; fp32 C only.
struct LoraIn {
  const float* t;
  const void* b;
  int64_t ldb;
  int64_t r;
  float alpha;
};

tp_status prequantized_product(int kind, const int8_t* qa, int64_t ldqa, const float* sa, const void* q, int64_t ldq,
                               const float* w_scales, int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype,
                               int64_t ldc, int32_t* acc_out, int64_t ld_acc, void* workspace,
                               size_t workspace_bytes, hipStream_t stream, const LoraIn* lora = nullptr,
                               bool noalloc = false) {
  const bool w4 = kind == tp::GEMM_W4A8;
  const tp_op op = w4 ? TP_OP_QGEMM_W4A8_PREQUANTIZED : TP_OP_QGEMM_W8A8_PREQUANTIZED;
  if (!dtype_ok(c_dtype)) return fail(TP_ERR_UNSUPPORTED_DTYPE, "c_dtype %d is not TP_F32 or TP_BF16", (int)c_dtype);
  TP_TRY(check_sizes(m, n, k));
  if (!w4 && k > INT32_MAX / (127 * 127))
    return fail(TP_ERR_BAD_SHAPE, "k=%lld: the int32 accumulator could overflow (k <= %d)", (long long)k,
                INT32_MAX / (127 * 127));
  Extent eqa, esa, eq, es, ec, eacc;
  TP_TRY(check_matrix("qa", qa, m, k, ldqa, 1, &eqa));
  TP_TRY(check_vector("sa", sa, m, &esa));
  TP_TRY(check_matrix("q", q, n, w4 ? k / 2 : k, ldq, 1, &eq));
  int64_t ns;
  if (!mul_ok(n, w4 ? k / 256 : 1, &ns)) return fail(TP_ERR_SIZE_OVERFLOW, "scale count overflows");
  TP_TRY(check_vector("w_scales", w_scales, ns, &es));
  TP_TRY(check_matrix("c", c, m, n * dtype_size(c_dtype), ldc, dtype_size(c_dtype), &ec, dtype_size(c_dtype)));
  if (acc_out) TP_TRY(check_matrix("acc_out", acc_out, m, n * 4, ld_acc, 4, &eacc, 4));
  Extent et, eb;
  if (lora) {
    if (c_dtype != TP_F32) return fail(TP_ERR_UNSUPPORTED_DTYPE, "the side path adds into fp32 C only");
    if (lora->r < 1 || lora->r > 64) return fail(TP_ERR_BAD_SHAPE, "rank r=%lld outside [1, 64]", (long long)lora->r);
    TP_TRY(check_matrix("t", lora->t, m, 64 * 4, 64, 4, &et));
    TP_TRY(check_matrix("lora_b", lora->b, n, lora->r * 2, lora->ldb, 2, &eb));
  }
  WsLayout wl;
  Extent ew;
  if (!workspace_layout(op, m, n, k, TP_A_PREROTATED, true, &wl))
    return fail(TP_ERR_SIZE_OVERFLOW, "workspace size overflows");
  if (noalloc) {
    // the library's own scratch array instead of a workspace (no overlap with
    // any caller buffer possible)
    if (wl.total > tp::NOALLOC_SCRATCH_BYTES)
      return fail(TP_ERR_WORKSPACE_TOO_SMALL,
                  "this shape needs %lld bytes of split-K partial sums; the no-allocation entry point holds %lld "
                  "(use tp_qgemm_w8a8_prequantized with a workspace)",
                  (long long)wl.total, (long long)tp::NOALLOC_SCRATCH_BYTES);
  } else {
    TP_TRY(check_workspace(wl, workspace, workspace_bytes, &ew));
  }
  const Extent* ins[] = {&eqa, &esa, &eq, &es, &et, &eb};
  for (const Extent* i : ins)
    if (overlaps(ec, *i) || overlaps(eacc, *i) || overlaps(ew, *i))
      return fail(TP_ERR_BAD_ALIASING, "an output or the workspace overlaps an input");
  if (overlaps(ec, eacc) || overlaps(ec, ew) || overlaps(eacc, ew))
    return fail(TP_ERR_BAD_ALIASING, "c, acc_out and the workspace must not overlap");
  if (m == 0 || n == 0) return ok();
  tp::GemmArgs g{};
  g.kind = kind;
  g.a = qa;
  g.lda = ldqa;
  g.b = q;
  g.ldb = ldq;
  g.w_scales = w_scales;
  g.a_scales = sa;
  g.m = m;
  g.n = n;
  g.k = k;
  g.c = c;
  g.c_bf16 = c_dtype == TP_BF16;
  g.ldc = ldc;
  g.acc_out = acc_out;
  g.ld_acc = ld_acc;
  g.part = wl.total > 0 ? workspace : nullptr;
  if (noalloc && wl.total > 0) TP_TRY(hip_status(tp::noalloc_scratch(&g.part), "scratch address"));
  if (lora) {
    g.lora.t = lora->t;
    g.lora.b = (const uint16_t*)lora->b;
    g.lora.ldb = lora->ldb;
    g.lora.r = (int)lora->r;
    g.lora.alpha = lora->alpha;
  }
  return hip_status(tp::launch_qgemm(g, stream), "product launch");
}

}  // namespace

tp_status tp_qgemm_w8a8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const int8_t* q, int64_t ldq,
                        const float* w_scales, int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype,
                        int64_t ldc, int8_t* qa_out, float* sa_out, int32_t* acc_out, int64_t ld_acc,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return act8_product(tp::GEMM_W8A8, a, a_dtype, lda, a_flags, q, ldq, w_scales, m, n, k, c, c_dtype, ldc, qa_out,
                      sa_out, acc_out, ld_acc, workspace, workspace_bytes, stream);
}

tp_status tp_qgemm_w8a8_prequantized(const int8_t* qa, int64_t ldqa, const float* sa, const int8_t* q, int64_t ldq,
                                     const float* w_scales, int64_t m, int64_t n, int64_t k, void* c,
                                     tp_dtype c_dtype, int64_t ldc, int32_t* acc_out, int64_t ld_acc,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prequantized_product(tp::GEMM_W8A8, qa, ldqa, sa, q, ldq, w_scales, m, n, k, c, c_dtype, ldc, acc_out,
                              ld_acc, workspace, workspace_bytes, stream);
}

tp_status tp_qgemm_w8a8_prequantized_noalloc(const int8_t* qa, int64_t ldqa, const float* sa, const int8_t* q,
                                             int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k,
                                             void* c, tp_dtype c_dtype, int64_t ldc, int32_t* acc_out,
                                             int64_t ld_acc, hipStream_t stream) {
  return prequantized_product(tp::GEMM_W8A8, qa, ldqa, sa, q, ldq, w_scales, m, n, k, c, c_dtype, ldc, acc_out,
                              ld_acc, nullptr, 0, stream, nullptr, true);
}

tp_status tp_qgemm_w8a8_prequantized_lora(const int8_t* qa, int64_t ldqa, const float* sa, const int8_t* q,
                                          int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k,
                                          float* c, int64_t ldc, const float* t, const void* lora_b, int64_t ldb,
                                          int64_t r, float alpha, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  const LoraIn lora{t, lora_b, ldb, r, alpha};
  return prequantized_product(tp::GEMM_W8A8, qa, ldqa, sa, q, ldq, w_scales, m, n, k, c, TP_F32, ldc, nullptr, 0,
                              workspace, workspace_bytes, stream, &lora);
}

tp_status tp_qgemm_w4a8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags, const uint8_t* q4,
                        int64_t ldq_bytes, const float* w_scales, int64_t m, int64_t n, int64_t k, void* c,
                        tp_dtype c_dtype, int64_t ldc, int8_t* qa_out, float* sa_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return act8_product(tp::GEMM_W4A8, a, a_dtype, lda, a_flags, q4, ldq_bytes, w_scales, m, n, k, c, c_dtype, ldc,
                      qa_out, sa_out, nullptr, 0, workspace, workspace_bytes, stream);
}

tp_status tp_qgemm_w4a8_prequantized(const int8_t* qa, int64_t ldqa, const float* sa, const uint8_t* q4,
                                     int64_t ldq_bytes, const float* w_scales, int64_t m, int64_t n, int64_t k,
                                     void* c, tp_dtype c_dtype, int64_t ldc, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return prequantized_product(tp::GEMM_W4A8, qa, ldqa, sa, q4, ldq_bytes, w_scales, m, n, k, c, c_dtype, ldc,
                              nullptr, 0, workspace, workspace_bytes, stream);
}

}  // extern "C"

