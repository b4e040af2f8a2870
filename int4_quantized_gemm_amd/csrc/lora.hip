// LoRA side path beside a projection: C += alpha * (X . A^T) . B^T, with the
// usual layouts lora_A [r, k] and lora_B [n, r] (kvad-gpu internals, section
// "Pictures, which are not tokens": each LoRA is a side path (x.A).B beside
// the layer it adapts, with a per-request strength, added into the layer's
// output; the loaded model is left as it was).
//
//  * down  T[m, j] = sum_k X[m, k] A[j, k]   (fp32 [m, 64], the workspace;
//          zeros past r)
//  * up    C[m, n] += alpha * sum_j T[m, j] B[n, j], read-modify-write
//
// Sums are fp32 in a fixed order and C is rounded once on store. bf16
// operands go through the matrix units (k_lora_down_mfma with bf16 X and A,
// k_lora_up_mfma with bf16 B; every product is exact in fp32), fp32 operands
// through fp32 FMAs (k_lora_down, k_lora_up_add; inputs widened exactly).
#include <climits>
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
                                                     TC* __restrict__ c, int64_t ldc, int nbn) {
  __shared__ __align__(16) float ts[LU_BM][R];
  const int tid = threadIdx.x;
  const int m0 = (int)(blockIdx.x / nbn) * LU_BM;
  const int n = (int)(blockIdx.x % nbn) * LU_BN + tid;
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

// ------------------------------------------------------- matrix-unit paths
// With bf16 operands the products X[m,k] A[j,k] and T-part x B[n,j] are exact
// in fp32, so bf16 MFMAs with fp32 sums keep the arithmetic above: fp32 sums,
// C rounded once.

// Down, bf16 X and lora_A: one block per LDM_FM x 16 rows of X; its LDM_NW
// waves split the K / 32 steps of 32 as evenly as whole steps allow (some
// waves get none when k < 32 * LDM_NW) and their partial sums are added in
// LDS in wave order. Lane l feeds
// X rows 16 i + l % 16 and lora_A row 16 f + l % 16 (zero past r) with K chunk
// 8 (l / 16) of each step.
constexpr int LDM_FM = 1;  // 16-row fragments of X per block (2 and 4 were slower: fewer waves)
constexpr int LDM_NW = 16;  // waves per block, each with 1 / LDM_NW of K (16: 15% faster than 8 at k = 12288)

template <int R>
__global__ __launch_bounds__(64 * LDM_NW) void k_lora_down_mfma(const uint16_t* __restrict__ x, int64_t ldx,
                                                        const uint16_t* __restrict__ a, int64_t lda, int M, int K,
                                                        int r, float* __restrict__ t) {
  constexpr int NF = R / 16;  // 16-column fragments of T
  constexpr int BR = 16 * LDM_FM;
  __shared__ __align__(16) float part[LDM_NW][BR][R];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int m0 = blockIdx.x * BR;
  // This wave's whole 32-deep steps of K: [s0, s1) of the K / 32.
  const int nk = K / 32, s0 = wave * nk / LDM_NW, s1 = (wave + 1) * nk / LDM_NW;
  const int kb = s0 * 32, kw = (s1 - s0) * 32;
  bool rowok[LDM_FM];
  const uint16_t* xrow[LDM_FM];
#pragma unroll
  for (int i = 0; i < LDM_FM; ++i) {
    rowok[i] = m0 + 16 * i + l16 < M;
    xrow[i] = x + (int64_t)min(m0 + 16 * i + l16, M - 1) * ldx + kb + 8 * g4;
  }
  const uint16_t* arow[NF];
  bool aok[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int j = f * 16 + l16;
    aok[f] = j < r;
    arow[f] = a + (int64_t)min(j, r - 1) * lda + kb + 8 * g4;
  }
  f32x4_t acc[LDM_FM][NF];
#pragma unroll
  for (int i = 0; i < LDM_FM; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int k = 0; k < kw; k += 32) {
    u32x4_t xv[LDM_FM];
#pragma unroll
    for (int i = 0; i < LDM_FM; ++i) xv[i] = rowok[i] ? *reinterpret_cast<const u32x4_t*>(xrow[i] + k) : zero;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const u32x4_t av = aok[f] ? *reinterpret_cast<const u32x4_t*>(arow[f] + k) : zero;
#pragma unroll
      for (int i = 0; i < LDM_FM; ++i)
        acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[i]),
                                                            __builtin_bit_cast(bf16x8_t, av), acc[i][f], 0, 0, 0);
    }
  }
  // lane l holds rows 16 i + 4 (l / 16) + v, column 16 f + l % 16
#pragma unroll
  for (int i = 0; i < LDM_FM; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[wave][16 * i + 4 * g4 + v][f * 16 + l16] = acc[i][f][v];
  __syncthreads();
  for (int e = threadIdx.x; e < BR * LORA_RMAX; e += 64 * LDM_NW) {
    const int i = e / LORA_RMAX, j = e % LORA_RMAX;
    if (m0 + i >= M) continue;
    float sum = 0.f;
    if (j < R && j < r) {
      sum = part[0][i][j];
#pragma unroll
      for (int w = 1; w < LDM_NW; ++w) sum += part[w][i][j];
    }
    t[(int64_t)(m0 + i) * LORA_RMAX + j] = sum;
  }
}

// Up, bf16 lora_B: a block owns 16 rows x 256 columns of C, a wave 64 of the
// columns. T (fp32) is split exactly into three bf16 parts; the two small
// parts are summed first and the large part last, so the result carries
// about r + 1 fp32 roundings of sum |T| |B| like the plain fp32 sum. Lane l
// feeds T row l % 16 and lora_B row n0 + 16 f + l % 16 with ranks
// 32 s + 8 (l / 16) + [0, 8) (zeros past r; T holds zeros there already).
// The products go through LDS so that C is read and written a whole row
// segment (1 KB of fp32) per wave instruction, 16 (fp32) or 8 (bf16) bytes a
// lane when C's base and pitch allow it (cvec), element by element otherwise.
constexpr int LUM_PAD = 4;  // floats of padding per LDS row (rows 4 apart land 16 banks apart)

template <typename TC, int R>
__global__ __launch_bounds__(256) void k_lora_up_mfma(const float* __restrict__ t, const uint16_t* __restrict__ b,
                                                      int64_t ldb, float alpha, int M, int N, int r,
                                                      TC* __restrict__ c, int64_t ldc, int nbn, int cvec) {
  constexpr int KS = (R + 31) / 32;  // 32-deep steps over the rank
  __shared__ __align__(16) float prod[16][256 + LUM_PAD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int m0 = (int)(blockIdx.x / nbn) * 16;
  const int nb0 = (int)(blockIdx.x % nbn) * 256;
  const int n0 = nb0 + wave * 64;
  bf16x8_t th[KS], tm[KS], tl[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float v[8];
    if (m0 + l16 < M) {
      load8(t + (int64_t)(m0 + l16) * LORA_RMAX + 32 * s + 8 * g4, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    split3_bf16(v, th[s], tm[s], tl[s]);
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int n = n0 + 16 * f + l16;
    bf16x8_t bo[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int j0 = 32 * s + 8 * g4;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (n < N && j0 < r) {
        const uint16_t* brow = b + (int64_t)n * ldb + j0;
        if (j0 + 8 <= r) {
          w = *reinterpret_cast<const u32x4_t*>(brow);
        } else {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t lo = j0 + e < r ? brow[e] : 0u, hi = j0 + e + 1 < r ? brow[e + 1] : 0u;
            w[e >> 1] = lo | (hi << 16);
          }
        }
      }
      bo[s] = __builtin_bit_cast(bf16x8_t, w);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl[s], bo[s], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tm[s], bo[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th[s], bo[s], acc, 0, 0, 0);
    // lane l holds rows 4 (l / 16) + v, column 16 f + l % 16 of the wave's 64
#pragma unroll
    for (int v = 0; v < 4; ++v) prod[4 * g4 + v][wave * 64 + 16 * f + l16] = acc[v];
  }
  __syncthreads();
  // Read-modify-write of C: thread tid handles 4 columns of row q / 64, q = tid + 256 u.
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = threadIdx.x + 256 * u;
    const int i = q >> 6, c4 = (q & 63) * 4;
    const int row = m0 + i, col = nb0 + c4;
    if (row >= M || col >= N) continue;
    const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&prod[i][c4]);
    TC* p = c + (int64_t)row * ldc + col;
    if (cvec && col + 4 <= N) {
      if constexpr (std::is_same<TC, float>::value) {
        f32x4_t cv = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) cv[e] = fmaf(alpha, pv[e], cv[e]);
        *reinterpret_cast<f32x4_t*>(p) = cv;
      } else {
        const uint2 cw = *reinterpret_cast<const uint2*>(p);
        const float o0 = fmaf(alpha, pv[0], bf16_lo(cw.x)), o1 = fmaf(alpha, pv[1], bf16_hi(cw.x));
        const float o2 = fmaf(alpha, pv[2], bf16_lo(cw.y)), o3 = fmaf(alpha, pv[3], bf16_hi(cw.y));
        *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= N) break;
        if constexpr (std::is_same<TC, float>::value) {
          p[e] = fmaf(alpha, pv[e], p[e]);
        } else {
          const float o = fmaf(alpha, pv[e], __builtin_bit_cast(float, (uint32_t)p[e] << 16));
          p[e] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xFFFFu);
        }
      }
    }
  }
}

template <int R>
static hipError_t lora_down_r(const void* x, bool x_bf16, int64_t ldx, const void* a, bool a_bf16, int64_t lda,
                              int64_t m, int64_t k, int64_t r, float* t, hipStream_t stream) {
  const dim3 gd((unsigned)((m + LD_BM - 1) / LD_BM)), bd(256);
#define TP_DOWN(TX, TA)                                                                                         \
  hipLaunchKernelGGL((k_lora_down<TX, TA, R>), gd, bd, 0, stream, (const TX*)x, ldx, (const TA*)a, lda, (int)m,    \
                     (int)k, (int)r, t)
  if (x_bf16) {
    if (a_bf16)
      hipLaunchKernelGGL((k_lora_down_mfma<R>), dim3((unsigned)((m + 16 * LDM_FM - 1) / (16 * LDM_FM))), dim3(64 * LDM_NW), 0, stream,
                         (const uint16_t*)x, ldx, (const uint16_t*)a, lda, (int)m, (int)k, (int)r, t);
    else
      TP_DOWN(uint16_t, float);
  } else {
    if (a_bf16) TP_DOWN(float, uint16_t); else TP_DOWN(float, float);
  }
#undef TP_DOWN
  return hipGetLastError();
}

template <int R>
static hipError_t lora_up_r(const float* t, const void* b, bool b_bf16, int64_t ldb, float alpha, int64_t m,
                            int64_t n, int64_t r, void* c, bool c_bf16, int64_t ldc, hipStream_t stream) {
  // One flattened grid of (row block, column block) pairs; both kernels'
  // column blocks are 256 wide.
  const int64_t nbn = (n + 255) / 256;
  const int64_t rows_per = b_bf16 ? 16 : LU_BM;
  const int64_t blocks = (m + rows_per - 1) / rows_per * nbn;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  // C may be aligned to its element only; the vector accesses of the matrix
  // unit path need 16 (fp32) or 8 (bf16) bytes for the base and the pitch.
  const uintptr_t cva = c_bf16 ? 8 : 16;
  const int cvec = ((uintptr_t)c % cva == 0) && ((uintptr_t)(ldc * (c_bf16 ? 2 : 4)) % cva == 0);
  const dim3 gu((unsigned)blocks), bu(256);
#define TP_UP(TB, TC)                                                                                           \
  hipLaunchKernelGGL((k_lora_up_add<TB, TC, R>), gu, bu, 0, stream, t, (const TB*)b, ldb, alpha, (int)m, (int)n,   \
                     (int)r, (TC*)c, ldc, (int)nbn)
  if (b_bf16) {
    if (c_bf16)
      hipLaunchKernelGGL((k_lora_up_mfma<uint16_t, R>), gu, bu, 0, stream, t, (const uint16_t*)b, ldb, alpha, (int)m,
                         (int)n, (int)r, (uint16_t*)c, ldc, (int)nbn, cvec);
    else
      hipLaunchKernelGGL((k_lora_up_mfma<float, R>), gu, bu, 0, stream, t, (const uint16_t*)b, ldb, alpha, (int)m,
                         (int)n, (int)r, (float*)c, ldc, (int)nbn, cvec);
  } else {
    if (c_bf16) TP_UP(float, uint16_t); else TP_UP(float, float);
  }
#undef TP_UP
  return hipGetLastError();
}

hipError_t launch_lora_down(const void* x, bool x_bf16, int64_t ldx, const void* a, bool a_bf16, int64_t lda,
                            int64_t m, int64_t k, int64_t r, float* t, hipStream_t stream) {
  if (r <= 16) return lora_down_r<16>(x, x_bf16, ldx, a, a_bf16, lda, m, k, r, t, stream);
  if (r <= 32) return lora_down_r<32>(x, x_bf16, ldx, a, a_bf16, lda, m, k, r, t, stream);
  return lora_down_r<64>(x, x_bf16, ldx, a, a_bf16, lda, m, k, r, t, stream);
}

hipError_t launch_lora_up(const float* t, const void* b, bool b_bf16, int64_t ldb, float alpha, int64_t m, int64_t n,
                          int64_t r, void* c, bool c_bf16, int64_t ldc, hipStream_t stream) {
  if (r <= 16) return lora_up_r<16>(t, b, b_bf16, ldb, alpha, m, n, r, c, c_bf16, ldc, stream);
  if (r <= 32) return lora_up_r<32>(t, b, b_bf16, ldb, alpha, m, n, r, c, c_bf16, ldc, stream);
  return lora_up_r<64>(t, b, b_bf16, ldb, alpha, m, n, r, c, c_bf16, ldc, stream);
}

hipError_t launch_lora_add(const void* x, bool x_bf16, int64_t ldx, const void* a, const void* b, bool ab_bf16,
                           int64_t lda, int64_t ldb, float alpha, int64_t m, int64_t n, int64_t k, int64_t r, void* c,
                           bool c_bf16, int64_t ldc, float* t, hipStream_t stream) {
  const hipError_t e = launch_lora_down(x, x_bf16, ldx, a, ab_bf16, lda, m, k, r, t, stream);
  if (e != hipSuccess) return e;
  return launch_lora_up(t, b, ab_bf16, ldb, alpha, m, n, r, c, c_bf16, ldc, stream);
}

}  // namespace tp
