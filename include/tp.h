/*
 * tp.h -- rotated, quantized linear projections ("ConvRot") for AMD Instinct
 * MI355X (gfx950). C ABI: plain device pointers, sizes and a HIP stream.
 *
 * The method (tensai docs, "画像生成" (image generation), section "幅とメモリ"
 * (width and memory)): every weight matrix is rotated by a 256x256 Hadamard
 * matrix on each 256-wide group of input columns and then quantized (8-bit per
 * row by default, 4-bit optionally); each activation row gets the same
 * rotation on the device before the product, one product with H per 256-group,
 * so that, H being orthogonal, the product equals the float one up to
 * quantization error while outlier columns no longer dominate a row's scale.
 * Section "GPU" of the same page: the device quantizes each product's
 * activations (per token here, for the int8 x int8 product).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Rotation    Q = H / 16 with H the Sylvester Hadamard matrix of order 256 in
 *             natural order, H[i][j] = (-1)^popcount(i & j). Q is orthonormal
 *             and symmetric. A row x of length K is rotated group by group:
 *             x'[256g + j] = sum_i x[256g + i] * Q[i][j].
 * Shapes      Matrices are row-major with an explicit leading dimension (ld, in
 *             ELEMENTS of the stated type, except packed int4 whose ld is in
 *             bytes). Activations A are [m, k]; weights W are [n, k] (output
 *             rows by input columns); outputs C are [m, n]. k must be a
 *             positive multiple of 256. m == 0 or n == 0 is a valid no-op.
 * Pointers    All data pointers are DEVICE pointers owned by the caller. The
 *             library keeps no pointer after a call returns and allocates no
 *             memory: scratch comes from the caller's workspace, sized with
 *             tp_workspace_size(). Base pointers of inputs, codes and the
 *             workspace must be 16-byte aligned and their row pitch (ld *
 *             element size) a multiple of 16 bytes; outputs C and acc_out
 *             need only the alignment of their element type; scale arrays
 *             must be 4-byte aligned. An operand with no elements may be NULL.
 * Streams     Work is enqueued on `stream` (NULL = the default stream) and runs
 *             asynchronously; no call synchronizes or copies to the host.
 *             Calls that overlap on different streams and share buffers race.
 * Errors      Every argument is validated BEFORE any HIP call, so a refused
 *             call has enqueued nothing. A HIP launch failure returns
 *             TP_ERR_HIP. The calling thread's last error message is available
 *             from tp_last_error_message().
 * Results     Deterministic: the same inputs give the same output bytes (no
 *             atomics, fixed reduction orders).
 * Values      Floating-point inputs are expected finite. A row or weight
 *             holding NaN or infinity is not refused: its codes stay in the
 *             code range and nothing faults, but its codes, scale and the
 *             outputs that read it are unspecified.
 */
#ifndef TP_H_
#define TP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 8

typedef enum tp_status {
  TP_OK = 0,
  TP_ERR_NULL_POINTER = 1,          /* a required pointer is NULL              */
  TP_ERR_BAD_SHAPE = 2,             /* negative size, or k <= 0                */
  TP_ERR_K_NOT_MULTIPLE_OF_256 = 3, /* a group would straddle the row end      */
  TP_ERR_BAD_LEADING_DIM = 4,       /* ld smaller than the row length          */
  TP_ERR_MISALIGNED = 5,            /* pointer or row pitch not 16-B aligned   */
  TP_ERR_UNSUPPORTED_DTYPE = 6,     /* dtype code not allowed for this operand */
  TP_ERR_UNSUPPORTED_BITS = 7,      /* bits is neither 8 nor 4                 */
  TP_ERR_SIZE_OVERFLOW = 8,         /* a byte size overflows int64             */
  TP_ERR_WORKSPACE_TOO_SMALL = 9,   /* workspace NULL or below the query       */
  TP_ERR_BAD_ALIASING = 10,         /* partially overlapping in/out buffers    */
  TP_ERR_BAD_FLAGS = 11,            /* unknown a_flags value                   */
  TP_ERR_HIP = 12                   /* a HIP runtime call or launch failed     */
} tp_status;

/* Element types of floating-point operands. */
typedef enum tp_dtype {
  TP_F32 = 0,  /* IEEE binary32                                   */
  TP_BF16 = 1  /* bfloat16 (top half of a binary32), RNE on store */
} tp_dtype;

/* a_flags of the products: what the activation operand already is. */
#define TP_A_PREROTATED 0 /* A already holds rotated rows (x . blockdiag(Q)) */
#define TP_A_ROTATE 1     /* A holds plain rows; the library rotates them    */

/* Operation codes for tp_workspace_size(). */
typedef enum tp_op {
  TP_OP_QGEMM_W8 = 1,
  TP_OP_QGEMM_W4 = 2,
  TP_OP_QGEMM_W8A8 = 3,
  TP_OP_QGEMM_W8A8_PREQUANTIZED = 4,
  TP_OP_QGEMM_W4A8 = 5,
  TP_OP_QGEMM_W4A8_PREQUANTIZED = 6
} tp_op;

/*
 * tp_rotate_quantize_weights -- offline rotate-and-quantize of a weight
 * matrix (tensai docs, "画像生成", section "幅とメモリ": quantize while loading,
 * 8-bit by default or 4-bit, after rotating per 256 input columns; section
 * "チェックポイントの入手": per-row scaled int8 after the rotation).
 *
 *   w       [n, k] weights, dtype w_dtype (TP_F32 or TP_BF16), row pitch ldw
 *           elements.
 *   bits    8: q is int8 [n, k] (row pitch ldq bytes), scales is fp32 [n]:
 *              scales[r] = fp32(max_j |W'[r, j]| / 127) (fp64 divide, one
 *              rounding), q = clamp(rint(W' / scales[r]), -127, 127).
 *           4: q is packed int4 [n, k/2] bytes (row pitch ldq bytes): byte j of
 *              a row holds the code of column 2j in its low nibble and of
 *              column 2j+1 in its high nibble, two's complement, codes in
 *              [-7, 7]; scales is fp32 [n, k/256] (contiguous):
 *              scales[r, g] = fp32(max |W'| over group g of row r / 7).
 *   The rotation W' = W . blockdiag(Q) is computed in fp64 and the codes use
 *   round-half-to-even of W' / (double)scale. A row (or group) of zeros gets
 *   scale 0 and codes 0. w and q/scales must not overlap.
 */
tp_status tp_rotate_quantize_weights(const void* w, tp_dtype w_dtype, int64_t n, int64_t k,
                                     int64_t ldw, int bits, void* q, int64_t ldq,
                                     float* scales, hipStream_t stream);

/*
 * tp_hadamard_rotate_rows -- activation rotation y = x . blockdiag(Q)
 * (tensai docs, "画像生成", section "幅とメモリ": the product's input gets the
 * same rotation, rows taken as 256-groups, one product with H).
 *
 *   x       [m, k], dtype x_dtype (TP_F32 or TP_BF16), row pitch ldx.
 *   y       [m, k], dtype y_dtype (TP_F32 or TP_BF16), row pitch ldy.
 *   Arithmetic is fp32 (a fast Walsh-Hadamard transform per group); a bf16
 *   output is rounded to nearest even once. In place (y == x) is allowed when
 *   the dtypes and leading dimensions match; any other overlap is refused.
 */
tp_status tp_hadamard_rotate_rows(const void* x, tp_dtype x_dtype, int64_t m, int64_t k,
                                  int64_t ldx, void* y, tp_dtype y_dtype, int64_t ldy,
                                  hipStream_t stream);

/*
 * tp_quantize_rows_int8 -- rotate (unless a_flags == TP_A_PREROTATED) and
 * quantize activations per row for the int8 x int8 product (tensai docs,
 * "画像生成", section "GPU": each product's activations are quantized on the
 * device).
 *
 *   x       [m, k], TP_F32 or TP_BF16, row pitch ldx.
 *   qa      int8 [m, k], row pitch ldqa bytes.
 *   sa      fp32 [m]: sa[r] = fp32(max_j |X'[r, j]| / 127).
 *   Codes are clamp(rint(X' / (double)sa[r]), -127, 127), 0 for a zero row.
 *   The rotation is exact fp64 arithmetic, so the codes match an fp64
 *   reference bit for bit.
 */
tp_status tp_quantize_rows_int8(const void* x, tp_dtype x_dtype, int64_t m, int64_t k,
                                int64_t ldx, int a_flags, int8_t* qa, int64_t ldqa, float* sa,
                                hipStream_t stream);

/*
 * tp_dequantize_unrotate -- undo a rotated, quantized weight (tensai docs,
 * "画像生成", section "チェックポイントの入手": the loader undoes the rotation
 * and the per-row int8 of a ConvRot checkpoint before quantizing it its own
 * way). Q = H/16 is its own inverse, so
 *
 *   W_hat = (q * s) . blockdiag(Q),
 *
 * computed in fp64, which is exact (a group's values are integers times one
 * scale), and rounded once to w_dtype (RNE).
 *
 *   q       bits 8: int8 [n, k] codes, scales fp32 [n];
 *           bits 4: packed int4 [n, k/2] (two's complement, even k in the
 *           low nibble), scales fp32 [n, k/256]. Row pitch ldq_bytes.
 *   w       [n, k], TP_F32 or TP_BF16, row pitch ldw; must not overlap q or
 *           scales.
 */
tp_status tp_dequantize_unrotate(const void* q, int bits, int64_t ldq_bytes, const float* scales,
                                 int64_t n, int64_t k, void* w, tp_dtype w_dtype, int64_t ldw,
                                 hipStream_t stream);

/*
 * tp_requantize_weights -- the codes of width bits_out (8 or 4) for the
 * weight held as rotated codes of width bits_in (same section: undo, then
 * quantize). Rotating W_hat again gives q * s back exactly, so this is the
 * quantization of q * s with the rules of tp_rotate_quantize_weights, without
 * a transform, in fp64: bit-identical to tp_rotate_quantize_weights on an
 * exact W_hat. Layouts as in tp_dequantize_unrotate; int8 -> int8 and
 * int4 -> int4 give back quantizer outputs unchanged.
 */
tp_status tp_requantize_weights(const void* q_in, int bits_in, int64_t ldq_in, const float* s_in,
                                int64_t n, int64_t k, int bits_out, void* q_out, int64_t ldq_out,
                                float* s_out, hipStream_t stream);

/*
 * tp_lora_add -- a LoRA side path beside a projection, added into its output
 * (kvad-gpu internals, section "Pictures, which are not tokens": each LoRA is
 * a side path (x.A).B beside the layer it adapts, with a per-request strength;
 * the loaded, quantized weights stay as they are):
 *
 *   C[i, j] += alpha * sum_t (sum_q X[i, q] * lora_a[t, q]) * lora_b[j, t]
 *
 *   x        [m, k] (TP_F32 or TP_BF16), row pitch ldx: the activations in the
 *            domain of lora_a (pass the un-rotated activations, or rotate
 *            lora_a with tp_hadamard_rotate_rows as well: (xQ)(AQ)^T = xA^T).
 *   lora_a   [r, k], lora_b [n, r], both ab_dtype, row pitches lda, ldb
 *            (elements; 16-byte aligned rows, as for every matrix operand, so
 *            lora_b rows are padded to 8 bf16 or 4 fp32); 1 <= r <= 64.
 *   c        [m, n] (TP_F32 or TP_BF16), row pitch ldc: read, added to,
 *            written back (rounded once).
 *   workspace  tp_lora_workspace_size(m, r) bytes (fp32 x . lora_a^T in rows
 *            of 64), 16-byte aligned.
 *   Arithmetic is fp32 (inputs widened exactly), summed in a fixed order.
 *   k must be a multiple of 256, as for the projection.
 */
size_t tp_lora_workspace_size(int64_t m, int64_t r);
tp_status tp_lora_add(const void* x, tp_dtype x_dtype, int64_t ldx, const void* lora_a,
                      const void* lora_b, tp_dtype ab_dtype, int64_t lda, int64_t ldb, float alpha,
                      int64_t m, int64_t n, int64_t k, int64_t r, void* c, tp_dtype c_dtype,
                      int64_t ldc, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_lora_down -- the first half of the LoRA side path on its own (same
 * section), for tp_qgemm_w8a8_prequantized_lora:
 *
 *   T[i, t] = sum_q X[i, q] * lora_a[t, q]   (fp32, summed in a fixed order)
 *
 *   x        [m, k] (TP_F32 or TP_BF16), row pitch ldx; lora_a [r, k]
 *            (a_dtype), row pitch lda; 16-byte aligned rows; 1 <= r <= 64;
 *            k a multiple of 256.
 *   t        fp32 [m, 64], rows of 64 floats (zeros past r), 16-byte aligned,
 *            t_bytes >= m * 256; must not overlap x or lora_a.
 * The same T as tp_lora_add computes internally (bit for bit).
 */
tp_status tp_lora_down(const void* x, tp_dtype x_dtype, int64_t ldx, const void* lora_a,
                       tp_dtype a_dtype, int64_t lda, int64_t m, int64_t k, int64_t r, float* t,
                       size_t t_bytes, hipStream_t stream);

/* out_kind of tp_swiglu_rotate. */
#define TP_FFN_OUT_I8 0   /* int8 codes [m, k] and fp32 scales [m] */
#define TP_FFN_OUT_BF16 1 /* rotated bf16 rows [m, k]              */

/*
 * tp_swiglu_rotate -- the input of an FFN's down projection, fused: the
 * SwiGLU hidden activation h = bf16(silu(gate) * up), silu(x) = x / (1 + e^-x),
 * is rotated per 256-group and written as per-row int8 codes or as rotated
 * bf16 rows, without h ever being stored (tensai docs, "画像生成", section
 * "何が走るか": every block is attention plus a SwiGLU feed-forward; section
 * "幅とメモリ": the product's input is rotated per 256 columns on the device;
 * TensorFold pull request #948: bf16 activations, and the row kernels around
 * the projections as the candidates for fusion).
 *
 *   gate, up  [m, k], both in_dtype (TP_F32 or TP_BF16), row pitches ld_gate
 *             and ld_up (elements). They may be the two column halves of one
 *             [m, 2k] gate+up output, and may overlap each other.
 *   h[r, j]   the real value silu(gate[r, j]) * up[r, j] rounded once to bf16
 *             (nearest even); fp32 shortcuts are taken only where they provably
 *             round the same way.
 *   out_kind  TP_FFN_OUT_I8: y int8 [m, k], row pitch ldy bytes, and scales
 *             fp32 [m]: bit-identical to tp_quantize_rows_int8 of h with
 *             TP_A_ROTATE. TP_FFN_OUT_BF16: y bf16 [m, k], row pitch ldy
 *             elements: identical to tp_hadamard_rotate_rows of h to TP_BF16;
 *             scales is not used and may be NULL.
 *   y and scales must not overlap gate, up or each other.
 */
tp_status tp_swiglu_rotate(const void* gate, int64_t ld_gate, const void* up, int64_t ld_up,
                           tp_dtype in_dtype, int64_t m, int64_t k, int out_kind, void* y,
                           int64_t ldy, float* scales, hipStream_t stream);

/*
 * tp_workspace_size -- bytes of device workspace the product `op` needs for
 * these sizes and a_flags (0 when none is needed). Returns 0 for invalid
 * sizes as well; the product call itself reports the error.
 *
 * The workspace holds, in this order: the rotated bf16 activations (W8, W4
 * with TP_A_ROTATE: 2 m k bytes) or the activation codes and scales (W8A8
 * unless the caller takes them through qa_out / sa_out); then, for products
 * whose output tiles would leave compute units idle (few rows, or a small
 * output), the split-K partial sums (4 m n bytes per split; the split count
 * depends on m, n and k). The size therefore depends on all
 * of op, m, n, k and a_flags. A product given less than it needs returns
 * TP_ERR_WORKSPACE_TOO_SMALL; W8A8 with both qa_out and sa_out needs only the
 * partial-sum part. The contents are scratch: nothing is kept between calls.
 */
size_t tp_workspace_size(tp_op op, int64_t m, int64_t n, int64_t k, int a_flags);

/*
 * tp_qgemm_w8 -- weight-only int8 product (tensai docs, "画像生成", section
 * "幅とメモリ" for the format; the bf16 matrix-unit arithmetic with fp32 sums
 * is the precision the TensorFold pull request #948 describes for its
 * projections).
 *
 *   C[r, c] = s[c] * sum_j bf16(A'[r, j]) * q[c, j]
 *
 *   a        [m, k] activations, row pitch lda. With TP_A_ROTATE, a is TP_F32
 *            or TP_BF16 and is rotated (fp32 arithmetic) and rounded to bf16
 *            into the workspace first. With TP_A_PREROTATED, a must be TP_BF16
 *            and already rotated.
 *   q        int8 [n, k] codes, row pitch ldq bytes; w_scales fp32 [n].
 *   c        [m, n], c_dtype TP_F32 or TP_BF16 (RNE), row pitch ldc.
 *   The product runs on bf16 MFMA with fp32 accumulation; the scale is
 *   applied in fp32 in the epilogue. c must not overlap any input.
 */
tp_status tp_qgemm_w8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags,
                      const int8_t* q, int64_t ldq, const float* w_scales, int64_t m, int64_t n,
                      int64_t k, void* c, tp_dtype c_dtype, int64_t ldc, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * tp_qgemm_w4 -- weight-only int4 product, one scale per (row, 256-group)
 * (tensai docs, "画像生成", section "幅とメモリ": the 4-bit width "-q4";
 * TensorPencil README: the "INT4 ConvRot" format).
 *
 *   C[r, c] = sum_g s[c, g] * sum_{j in group g} bf16(A'[r, j]) * q[c, j]
 *
 *   q        packed int4 [n, k/2] bytes (layout as tp_rotate_quantize_weights
 *            with bits = 4), row pitch ldq bytes; w_scales fp32 [n, k/256].
 *   Other arguments as tp_qgemm_w8. Each group's partial sum is kept in fp32
 *   and folded with its scale at the group boundary.
 */
tp_status tp_qgemm_w4(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags,
                      const uint8_t* q, int64_t ldq, const float* w_scales, int64_t m, int64_t n,
                      int64_t k, void* c, tp_dtype c_dtype, int64_t ldc, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * tp_qgemm_w8a8 -- int8 x int8 product with per-token activation
 * quantization (tensai docs, "画像生成", section "GPU").
 *
 *   acc[r, c] = sum_j qa[r, j] * q[c, j]        (exact, int32)
 *   C[r, c]   = (float(acc[r, c]) * sa[r]) * sw[c]   (fp32, then c_dtype)
 *
 *   a        [m, k] activations (TP_F32 or TP_BF16), row pitch lda; rotated
 *            first unless a_flags == TP_A_PREROTATED; then quantized exactly as
 *            tp_quantize_rows_int8.
 *   q        int8 [n, k] weight codes, row pitch ldq; w_scales fp32 [n].
 *   c        [m, n], TP_F32 or TP_BF16, row pitch ldc.
 *   qa_out   optional int8 [m, k] (pitch k bytes) and sa_out optional fp32
 *            [m]: when both are given the activation codes and scales are
 *            written there (and the workspace is not needed for them).
 *   acc_out  optional int32 [m, n], row pitch ld_acc: the raw accumulators.
 *   k * 127 * 127 must fit in int32 (k <= 133144).
 */
tp_status tp_qgemm_w8a8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags,
                        const int8_t* q, int64_t ldq, const float* w_scales, int64_t m,
                        int64_t n, int64_t k, void* c, tp_dtype c_dtype, int64_t ldc,
                        int8_t* qa_out, float* sa_out, int32_t* acc_out, int64_t ld_acc,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tp_qgemm_w8a8_prequantized -- the int8 x int8 product of tp_qgemm_w8a8 on
 * activation codes the caller already holds (from tp_quantize_rows_int8 or an
 * earlier tp_qgemm_w8a8 with qa_out / sa_out), so that one quantized
 * activation can feed several weight matrices (tensai docs, "画像生成", section
 * "GPU": the feed-forward's projections run as one batch on the device).
 *
 *   qa       int8 [m, k] codes, row pitch ldqa bytes; sa fp32 [m] scales.
 *   q        int8 [n, k] weight codes, row pitch ldq; w_scales fp32 [n].
 *   c        [m, n], TP_F32 or TP_BF16, row pitch ldc:
 *            C[r, c] = (float(acc[r, c]) * sa[r]) * w_scales[c].
 *   acc_out  optional int32 [m, n] raw accumulators, row pitch ld_acc.
 *   workspace  tp_workspace_size(TP_OP_QGEMM_W8A8_PREQUANTIZED, m, n, k, 0)
 *            bytes (0, and NULL allowed, unless m is small enough for the
 *            split-K path). k <= 133144.
 */
tp_status tp_qgemm_w8a8_prequantized(const int8_t* qa, int64_t ldqa, const float* sa, const int8_t* q,
                                     int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k,
                                     void* c, tp_dtype c_dtype, int64_t ldc, int32_t* acc_out,
                                     int64_t ld_acc, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * tp_qgemm_w8a8_prequantized_noalloc -- tp_qgemm_w8a8_prequantized without a
 * workspace, for callers that cannot allocate device memory (code recorded
 * into a HIP graph, tight serving loops, harnesses that forbid allocation):
 * the split-K partial sums of the few-row and small-grid plans go to a
 * scratch array the library holds (32 MiB, one copy on each GPU it runs on,
 * kept until the process ends; its address is looked up on the first call on
 * a device). It calls no allocating routine.
 *
 *   qa, sa, q, w_scales, m, n, k, c, c_dtype, ldc, acc_out, ld_acc: as
 *            tp_qgemm_w8a8_prequantized; the output bytes are the same.
 * Errors: as tp_qgemm_w8a8_prequantized, plus TP_ERR_WORKSPACE_TOO_SMALL when
 * the shape's partial sums (tp_workspace_size(TP_OP_QGEMM_W8A8_PREQUANTIZED,
 * m, n, k, 0) bytes) exceed the 32 MiB, refused before any HIP call.
 * Every call on one GPU shares its array (which keeps the last call's
 * contents; nothing in it needs to start at zero): calls that may run at the
 * same time on one GPU (other streams, other host threads) race and must not
 * be issued.
 */
tp_status tp_qgemm_w8a8_prequantized_noalloc(const int8_t* qa, int64_t ldqa, const float* sa, const int8_t* q,
                                             int64_t ldq, const float* w_scales, int64_t m, int64_t n, int64_t k,
                                             void* c, tp_dtype c_dtype, int64_t ldc, int32_t* acc_out,
                                             int64_t ld_acc, hipStream_t stream);

/*
 * tp_qgemm_w8a8_prequantized_lora -- tp_qgemm_w8a8_prequantized with a LoRA
 * side path added in the product's store (kvad-gpu internals, section
 * "Pictures, which are not tokens": the side path is added into the layer's
 * output, here by the kernel that writes it):
 *
 *   C[i, c] = fl(fl((float(acc[i, c]) * sa[i]) * w_scales[c]) + alpha * L[i, c])
 *   L[i, c] = sum_t T[i, t] * lora_b[c, t]   (fp32)
 *
 *   qa, sa, q, w_scales, m, n, k, workspace: as tp_qgemm_w8a8_prequantized.
 *   c        fp32 [m, n], row pitch ldc (fp32 only).
 *   t        fp32 [m, 64] from tp_lora_down (rows of 64 floats, zeros past r).
 *   lora_b   bf16 [n, r], row pitch ldb elements (16-byte aligned rows);
 *            1 <= r <= 64.
 * Large outputs run it in the product kernel's store; the others (few rows,
 * split K) store the product and then add the side path with the up half of
 * tp_lora_add. Both give the bits of tp_qgemm_w8a8_prequantized followed by
 * tp_lora_add with bf16 x, lora_a and lora_b.
 */
tp_status tp_qgemm_w8a8_prequantized_lora(const int8_t* qa, int64_t ldqa, const float* sa,
                                          const int8_t* q, int64_t ldq, const float* w_scales,
                                          int64_t m, int64_t n, int64_t k, float* c, int64_t ldc,
                                          const float* t, const void* lora_b, int64_t ldb, int64_t r,
                                          float alpha, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * tp_qgemm_w4a8 -- the int4 weights of tp_qgemm_w4 (one fp32 scale per row
 * and 256-group) against per-row int8 activations as in tp_qgemm_w8a8, on the
 * int8 matrix units (tensai docs, "画像生成", section "幅とメモリ": the 4-bit
 * "-q4" width; section "GPU": each product's activations are quantized on the
 * device).
 *
 *   a        [m, k] activations (TP_F32 or TP_BF16), row pitch lda; rotated
 *            first unless a_flags == TP_A_PREROTATED, then quantized exactly as
 *            tp_quantize_rows_int8.
 *   q4       packed int4 [n, k/2] (two's complement, even k in the low
 *            nibble), row pitch ldq_bytes; w_scales fp32 [n, k/256].
 *   c        [m, n], TP_F32 or TP_BF16, row pitch ldc:
 *            C[r, c] = (sum_g w_scales[c, g] * float(acc_g[r, c])) * sa[r],
 *            acc_g the exact int32 sum over group g, the fold in fp32 in group
 *            order.
 *   qa_out / sa_out  as in tp_qgemm_w8a8.
 *   workspace  tp_workspace_size(TP_OP_QGEMM_W4A8, m, n, k, a_flags) bytes.
 */
tp_status tp_qgemm_w4a8(const void* a, tp_dtype a_dtype, int64_t lda, int a_flags,
                        const uint8_t* q4, int64_t ldq_bytes, const float* w_scales, int64_t m,
                        int64_t n, int64_t k, void* c, tp_dtype c_dtype, int64_t ldc,
                        int8_t* qa_out, float* sa_out, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * tp_qgemm_w4a8_prequantized -- tp_qgemm_w4a8 on activation codes and scales
 * the caller already holds (tp_quantize_rows_int8, tp_swiglu_rotate with
 * TP_FFN_OUT_I8, or an earlier call's qa_out / sa_out).
 *
 *   qa       int8 [m, k] codes, row pitch ldqa bytes; sa fp32 [m] scales.
 *   workspace  tp_workspace_size(TP_OP_QGEMM_W4A8_PREQUANTIZED, m, n, k, 0)
 *            bytes (0, and NULL allowed, when the product runs unsplit).
 */
tp_status tp_qgemm_w4a8_prequantized(const int8_t* qa, int64_t ldqa, const float* sa,
                                     const uint8_t* q4, int64_t ldq_bytes, const float* w_scales,
                                     int64_t m, int64_t n, int64_t k, void* c, tp_dtype c_dtype,
                                     int64_t ldc, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* tp_status_string(tp_status status);

/* Message of the calling thread's last failed call ("" if none). */
const char* tp_last_error_message(void);

/* TP_ABI_VERSION of the loaded library. */
int tp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_H_ */
