// LoRA side path beside a projection: C += alpha * (X . A^T) . B^T, with the
// usual layouts lora_A [r, k] and lora_B [n, r] (kvad-gpu internals, section
// "Pictures, which are not tokens": each LoRA is a side path (x.A).B beside
// the layer it adapts, with a per-request strength, added into the layer's
// output; the loaded model is left as it was).
//
//  * k_lora_down   T[m, j] = sum_k X[m, k] A[j, k]   (fp32 [m, 64], the workspace;
//                  zeros past r)
//  * k_lora_up_add C[m, n] += alpha * sum_j T[m, j] B[n, j], read-modify-write
//
// Both run on fp32 FMAs (the side path is 2 r / k of the projection's work):
// inputs are widened exactly from fp32 or bf16, sums are fp32 in a fixed
// order, and C is rounded once on store.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tp {

constexpr int LORA_RMAX = 64;   // largest rank; T rows are LORA_RMAX floats apart (zeros past r)
constexpr int LD_BM = 8;        // rows of X per block (down)
constexpr int LD_KC = 256;      // K chunk staged in LDS (down)
constexpr int LD_PAD = 4;       // floats of padding per LDS row
constexpr int LU_BM = 32;       // rows of C per block (up)
constexpr int LU_BN = 256;      // columns of C per block (one per thread)

__device__ __forceinline__ float ld_elem(const float* p) { return *p; }
__device__ __forceinline__ float ld_elem(const uint16_t* p) { return __builtin_bit_cast(float, (uint32_t)*p << 16); }

// 8 consecutive elements (16-byte aligned for bf16, 32 for fp32) as fp32.
__device__ __forceinline__ void ld8f(const float* p, float (&v)[8]) { load8(p, v); }
__device__ __forceinline__ void ld8f(const uint16_t* p, float (&v)[8]) { load8(p, v); }

// R (16, 32 or 64) >= r. 256 threads: thread (i = tid / 32, q = tid % 32)
// owns row i of the block's 8 and ranks q + 32 u (u < R / 32; for R = 16
// only q < 16). K advances in chunks of 256 staged in LDS with 16-byte loads.
template <typename TX, typename TA, int R>
__global__ __launch_bounds__(256) void k_lora_down(const TX* __restrict__ x, int64_t ldx, const TA* __restrict__ a,
                                                   int64_t lda, int M, int K, int r, float* __restrict__ t) {
  constexpr int NU = R >= 32 ? R / 32 : 1;
  __shared__ __align__(16) float xs[LD_BM][LD_KC + LD_PAD];
  __shared__ __align__(16) float as[R][LD_KC + LD_PAD];
  const int tid = threadIdx.x;
  const int i = tid >> 5, q = tid & 31;
  const int m0 = blockIdx.x * LD_BM;
  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
  for (int k0 = 0; k0 < K; k0 += LD_KC) {
    {  // X: 8 rows x 256 = one 8-element vector per thread (zeros past M)
      const int rr = tid >> 5, c = (tid & 31) * 8;
      float v[8];
      if (m0 + rr < M) {
        ld8f(x + (int64_t)(m0 + rr) * ldx + k0 + c, v);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
      }
      *reinterpret_cast<f32x4_t*>(&xs[rr][c]) = f32x4_t{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4_t*>(&xs[rr][c + 4]) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
#pragma unroll
    for (int e = tid; e < R * 32; e += 256) {  // A: R rows x 256 (zeros past r)
      const int rr = e >> 5, c = (e & 31) * 8;
      float v[8];
      if (rr < r) {
        ld8f(a + (int64_t)rr * lda + k0 + c, v);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
      }
      *reinterpret_cast<f32x4_t*>(&as[rr][c]) = f32x4_t{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4_t*>(&as[rr][c + 4]) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();
    if (R >= 32 || q < R) {
#pragma unroll 4
      for (int c = 0; c < LD_KC; c += 4) {
        const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(&xs[i][c]);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const f32x4_t av = *reinterpret_cast<const f32x4_t*>(&as[q + 32 * u][c]);
          acc[u] = fmaf(xv.x, av.x, acc[u]);
          acc[u] = fmaf(xv.y, av.y, acc[u]);
          acc[u] = fmaf(xv.z, av.z, acc[u]);
          acc[u] = fmaf(xv.w, av.w, acc[u]);
        }
      }
    }
    __syncthreads();
  }
  if (m0 + i < M) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j = q + 32 * u;
      if (j < LORA_RMAX && (R >= 32 || q < R)) t[(int64_t)(m0 + i) * LORA_RMAX + j] = j < r ? acc[u] : 0.f;
    }
    if (R < LORA_RMAX) {  // ranks this kernel does not compute are zero in T
      for (int j = R + q; j < LORA_RMAX; j += 32) t[(int64_t)(m0 + i) * LORA_RMAX + j] = 0.f;
    }
  }
}

// Thread n of the block owns column n0 + n of the block's 32 rows; its row of
// B (R values, zeros past r) sits in registers, the 32 rows of T in LDS.
template <typename TB, typename TC, int R>
__global__ __launch_bounds__(256) void k_lora_up_add(const float* __restrict__ t, const TB* __restrict__ b,
                                                     int64_t ldb, float alpha, int M, int N, int r,
                                                     TC* __restrict__ c, int64_t ldc) {
  __shared__ __align__(16) float ts[LU_BM][R];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * LU_BM;
  const int n = blockIdx.x * LU_BN + tid;
  for (int e = tid; e < LU_BM * R / 4; e += 256) {
    const int rr = e / (R / 4), j = (e % (R / 4)) * 4;
    *reinterpret_cast<f32x4_t*>(&ts[rr][j]) =
        (m0 + rr < M) ? *reinterpret_cast<const f32x4_t*>(t + (int64_t)(m0 + rr) * LORA_RMAX + j)
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float bv[R];
  const TB* brow = b + (int64_t)min(n, N - 1) * ldb;
#pragma unroll
  for (int j = 0; j < R; j += 8) {
    if (j < r) {  // whole 8-element vectors: the row pitch is 16-byte aligned
      float v[8];
      if (j + 8 <= r) {
        ld8f(brow + j, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = j + e < r ? (float)ld_elem(brow + j + e) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[j + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[j + e] = 0.f;
    }
  }
  __syncthreads();
  if (n >= N) return;  // after the block's only barrier
  for (int rr = 0; rr < LU_BM && m0 + rr < M; ++rr) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < R; j += 4) {
      const f32x4_t tv = *reinterpret_cast<const f32x4_t*>(&ts[rr][j]);
      s = fmaf(tv.x, bv[j], s);
      s = fmaf(tv.y, bv[j + 1], s);
      s = fmaf(tv.z, bv[j + 2], s);
      s = fmaf(tv.w, bv[j + 3], s);
    }
    TC* p = c + (int64_t)(m0 + rr) * ldc + n;
    if constexpr (std::is_same<TC, float>::value) {
      *p = fmaf(alpha, s, *p);
    } else {
      const float v = fmaf(alpha, s, __builtin_bit_cast(float, (uint32_t)*p << 16));
      *p = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
    }
  }
}

template <int R>
static hipError_t lora_rank(const void* x, bool x_bf16, int64_t ldx, const void* a, const void* b, bool ab_bf16,
                            int64_t lda, int64_t ldb, float alpha, int64_t m, int64_t n, int64_t k, int64_t r,
                            void* c, bool c_bf16, int64_t ldc, float* t, hipStream_t stream) {
  const dim3 gd((unsigned)((m + LD_BM - 1) / LD_BM)), bd(256);
#define TP_DOWN(TX, TA)                                                                                         \
  hipLaunchKernelGGL((k_lora_down<TX, TA, R>), gd, bd, 0, stream, (const TX*)x, ldx, (const TA*)a, lda, (int)m,    \
                     (int)k, (int)r, t)
  if (x_bf16) {
    if (ab_bf16) TP_DOWN(uint16_t, uint16_t); else TP_DOWN(uint16_t, float);
  } else {
    if (ab_bf16) TP_DOWN(float, uint16_t); else TP_DOWN(float, float);
  }
#undef TP_DOWN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gu((unsigned)((n + LU_BN - 1) / LU_BN), (unsigned)((m + LU_BM - 1) / LU_BM)), bu(256);
#define TP_UP(TB, TC)                                                                                           \
  hipLaunchKernelGGL((k_lora_up_add<TB, TC, R>), gu, bu, 0, stream, (const float*)t, (const TB*)b, ldb, alpha,      \
                     (int)m, (int)n, (int)r, (TC*)c, ldc)
  if (ab_bf16) {
    if (c_bf16) TP_UP(uint16_t, uint16_t); else TP_UP(uint16_t, float);
  } else {
    if (c_bf16) TP_UP(float, uint16_t); else TP_UP(float, float);
  }
#undef TP_UP
  return hipGetLastError();
}

hipError_t launch_lora_add(const void* x, bool x_bf16, int64_t ldx, const void* a, const void* b, bool ab_bf16,
                           int64_t lda, int64_t ldb, float alpha, int64_t m, int64_t n, int64_t k, int64_t r, void* c,
                           bool c_bf16, int64_t ldc, float* t, hipStream_t stream) {
  if (r <= 16) return lora_rank<16>(x, x_bf16, ldx, a, b, ab_bf16, lda, ldb, alpha, m, n, k, r, c, c_bf16, ldc, t, stream);
  if (r <= 32) return lora_rank<32>(x, x_bf16, ldx, a, b, ab_bf16, lda, ldb, alpha, m, n, k, r, c, c_bf16, ldc, t, stream);
  return lora_rank<64>(x, x_bf16, ldx, a, b, ab_bf16, lda, ldb, alpha, m, n, k, r, c, c_bf16, ldc, t, stream);
}

}  // namespace tp
