// Internal launchers of the gfx950 kernels. Callers (api.cpp) validate every
// argument first; the launchers assume valid shapes, k % 256 == 0 and the
// alignment rules of include/tp.h, and return the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

hipError_t launch_rotate_rows(const void* x, bool x_bf16, int64_t ldx, void* y, bool y_bf16, int64_t ldy,
                              int64_t m, int64_t k, hipStream_t stream);

// bits 8: int8 codes with one scale per row; bits 4: packed int4 codes with one
// scale per (row, 256-group). rotate == false quantizes the rows as given.
hipError_t launch_rotq_rows(const void* x, bool x_bf16, int64_t ldx, int64_t rows, int64_t k, bool rotate,
                            int bits, void* q, int64_t ldq, float* scales, hipStream_t stream);

// Rotated weight codes (int8 per-row scales, or packed int4 per-group scales):
// w = (q * s) . blockdiag(H/16) rounded once to fp32 or bf16, and the codes
// of another width for the same q * s (no transform).
hipError_t launch_dequant_unrotate(const void* q, int bits, int64_t ldq, const float* scales, int64_t n, int64_t k,
                                  void* w, bool w_bf16, int64_t ldw, hipStream_t stream);
hipError_t launch_requantize(const void* q_in, int bits_in, int64_t ldq_in, const float* s_in, int64_t n, int64_t k,
                             int bits_out, void* q_out, int64_t ldq_out, float* s_out, hipStream_t stream);

// LoRA side path: c += alpha * (x . a^T) . b^T with a [r, k], b [n, r]
// (r <= 64); t is fp32 [m, 64] (rows of 64, zeros past r): the down half
// writes it, the up half reads it.
hipError_t launch_lora_add(const void* x, bool x_bf16, int64_t ldx, const void* a, const void* b, bool ab_bf16,
                           int64_t lda, int64_t ldb, float alpha, int64_t m, int64_t n, int64_t k, int64_t r, void* c,
                           bool c_bf16, int64_t ldc, float* t, hipStream_t stream);
hipError_t launch_lora_down(const void* x, bool x_bf16, int64_t ldx, const void* a, bool a_bf16, int64_t lda,
                            int64_t m, int64_t k, int64_t r, float* t, hipStream_t stream);
hipError_t launch_lora_up(const float* t, const void* b, bool b_bf16, int64_t ldb, float alpha, int64_t m, int64_t n,
                          int64_t r, void* c, bool c_bf16, int64_t ldc, hipStream_t stream);

// FFN middle: h = bf16(silu(g) * u), rotated per 256-group, then int8 codes
// with one scale per row (out_i8) or bf16 rows (scales unused).
hipError_t launch_swiglu_rotate(const void* g, int64_t ldg, const void* u, int64_t ldu, bool in_bf16, int64_t m,
                                int64_t k, bool out_i8, void* y, int64_t ldy, float* scales, hipStream_t stream);

enum GemmKind { GEMM_W8 = 0, GEMM_W4 = 1, GEMM_W8A8 = 2, GEMM_W4A8 = 3 };

// A LoRA side path added in a product's store (t == nullptr: none):
// C = product + alpha * T . b^T, T fp32 [m, 64] (zeros past r), b bf16 [n, r].
struct LoraEpi {
  const float* t;
  const uint16_t* b;
  int64_t ldb;  // elements
  int r;        // 1 .. 64
  float alpha;
};

struct GemmArgs {
  int kind;                 // GemmKind
  const void* a;            // bf16 [m, k] (W8, W4) or int8 [m, k] (W8A8, W4A8)
  int64_t lda;              // elements
  const void* b;            // int8 [n, k] or packed int4 [n, k/2]
  int64_t ldb;              // bytes
  const float* w_scales;    // [n] or [n, k/256]
  const float* a_scales;    // [m] (W8A8, W4A8) or nullptr
  int64_t m, n, k;
  void* c;                  // [m, n]
  bool c_bf16;
  int64_t ldc;              // elements
  int32_t* acc_out;         // optional int32 [m, n] (W8A8 only)
  int64_t ld_acc;
  void* part;               // split-K partial sums, qgemm_partial_bytes() bytes (may be null when that is 0)
  LoraEpi lora;             // fp32 C only
};

hipError_t launch_qgemm(const GemmArgs& args, hipStream_t stream);

// Tile configuration chosen for a shape (exposed for the benchmark's reports).
void qgemm_tile_for(int kind, int64_t m, int64_t n, int64_t k, int* bm, int* bn);

// Bytes of split-K partial sums launch_qgemm needs for this shape (0 when the
// product runs unsplit); -1 when the size overflows.
int64_t qgemm_partial_bytes(int kind, int64_t m, int64_t n, int64_t k);

// Scratch memory of the no-allocation entry point: a file-scope device array
// of NOALLOC_SCRATCH_BYTES in gemm.hip, one copy per GPU the library runs on
// (held until the process ends). noalloc_scratch returns its device address
// on the current device, looked up once per device.
constexpr int64_t NOALLOC_SCRATCH_BYTES = (int64_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace tp
