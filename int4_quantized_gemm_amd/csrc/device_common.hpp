// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, cross-lane exchange and the fast Walsh-Hadamard transform of one
// 256-wide group (the rotation of tensai docs, "画像生成", section "幅とメモリ":
// one product with the order-256 Hadamard matrix per group of 256 columns).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters unconstrained
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define VMCNT_ENCODE(n) ((((n) & 0xF) | ((((n) >> 4) & 3) << 14)) | 0x0F70)

// s_waitcnt immediate for "all of this wave's LDS operations have completed"
// (lgkmcnt 0, other counters unconstrained).
#define LGKMCNT0_ENCODE 0xC07F

// Workgroup barrier without the memory fence of __syncthreads(): waves wait
// for each other, no outstanding-memory wait is implied (callers wait
// explicitly), and the instruction scheduler may move nothing across it (a
// plain memory clobber would still let it sink matrix instructions past it).
__device__ __forceinline__ void barrier_only() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Two fp32 -> two bf16 (round to nearest even; one v_cvt_pk_bf16_f32 on gfx950),
// packed into one dword, the first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 v = hi + mid + lo exactly, each part bf16 (round to nearest even at
// each step; each residual is exact in fp32 and the last one fits in 8 bits).
__device__ __forceinline__ void split3_bf16(const float (&v)[8], bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
  u32x4_t h, m, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = v[2 * e], a1 = v[2 * e + 1];
    const uint32_t hw = pack_bf16x2(a0, a1);
    const float r0 = a0 - bf16_lo(hw), r1 = a1 - bf16_hi(hw);
    const uint32_t mw = pack_bf16x2(r0, r1);
    const uint32_t lw = pack_bf16x2(r0 - bf16_lo(mw), r1 - bf16_hi(mw));
    h[e] = hw;
    m[e] = mw;
    l[e] = lw;
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  mid = __builtin_bit_cast(bf16x8_t, m);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

// Exchange with the lane whose index differs in bit log2(MASK), inside each
// 32-lane half of the wave (ds_swizzle bit-mask mode: and 0x1f, xor MASK).
template <int MASK>
__device__ __forceinline__ float swz_xor(float v) {
  static_assert(MASK > 0 && MASK < 32, "swizzle xor mask must stay inside 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (MASK << 10) | 0x1f));
}

template <int MASK>
__device__ __forceinline__ double swz_xor(double v) {
  static_assert(MASK > 0 && MASK < 32, "swizzle xor mask must stay inside 32 lanes");
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  int lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)u, (MASK << 10) | 0x1f);
  int hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(u >> 32), (MASK << 10) | 0x1f);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// One butterfly stage across lanes: the pair (a, b) at group positions (p, p + h)
// becomes (a + b, a - b); the lane holding b receives a - b = partner - own.
template <int MASK, typename T>
__device__ __forceinline__ void xlane_stage(T (&v)[8], int lane32) {
  const bool upper = (lane32 & MASK) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    T p = swz_xor<MASK>(v[j]);
    v[j] = upper ? (p - v[j]) : (v[j] + p);
  }
}

// Unnormalized fast Walsh-Hadamard transform of one 256-group held by 32
// lanes, 8 consecutive elements per lane: lane L (0..31 within its half) holds
// elements 8L .. 8L+7. The result is x . H with H the Sylvester matrix in
// natural order (H[i][j] = (-1)^popcount(i & j)); butterflies over each index
// bit, in-lane for bits 0..2 and across lanes for bits 3..7. Every stage only
// adds or subtracts, so in fp64 the result is exact whenever the inputs'
// binades span less than 53 - 8 - (input significand bits).
template <typename T>
__device__ __forceinline__ void fwht256_lane8(T (&v)[8], int lane32) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        T a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  xlane_stage<1>(v, lane32);
  xlane_stage<2>(v, lane32);
  xlane_stage<4>(v, lane32);
  xlane_stage<8>(v, lane32);
  xlane_stage<16>(v, lane32);
}

// Loads of 8 consecutive elements as fp32 / fp64.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x);
  v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z);
  v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

template <typename TIn>
__device__ __forceinline__ void load8d(const TIn* p, double (&v)[8]) {
  float f[8];
  load8(p, f);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (double)f[j];
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  f32x4_t a = {v[0], v[1], v[2], v[3]};
  f32x4_t b = {v[4], v[5], v[6], v[7]};
  *reinterpret_cast<f32x4_t*>(p) = a;
  *reinterpret_cast<f32x4_t*>(p + 4) = b;
}

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  u32x4_t a = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
  *reinterpret_cast<u32x4_t*>(p) = a;
}

// Symmetric quantization code clamp(rint(x / s), -qmax, qmax), bit-identical to
// rounding the correctly rounded fp64 quotient: the quotient is first formed as
// x * (1/s); only when that lands within 1e-9 of a half-integer (where the two
// roundings could differ) is the IEEE fp64 division done. s == 0 gives 0.
__device__ __forceinline__ int quant_code(double x, double s, double inv_s, double qmax) {
  if (!(s > 0.0)) return 0;
  double t = x * inv_s;
  double f = t - floor(t);
  double r = rint(t);
  if (fabs(f - 0.5) < 1e-9) r = rint(x / s);
  r = fmin(fmax(r, -qmax), qmax);
  return (int)r;
}

// Maximum over the 32 lanes of a half-wave / over all 64 lanes.
__device__ __forceinline__ double halfwave_max(double v) {
  v = fmax(v, swz_xor<1>(v));
  v = fmax(v, swz_xor<2>(v));
  v = fmax(v, swz_xor<4>(v));
  v = fmax(v, swz_xor<8>(v));
  v = fmax(v, swz_xor<16>(v));
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
  v = halfwave_max(v);
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  // lanes 0..31 <-> 32..63
  int lo = __builtin_amdgcn_ds_bpermute(((int)(threadIdx.x ^ 32) & 63) << 2, (int)(uint32_t)u);
  int hi = __builtin_amdgcn_ds_bpermute(((int)(threadIdx.x ^ 32) & 63) << 2, (int)(uint32_t)(u >> 32));
  double o = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  return fmax(v, o);
}

}  // namespace tp
