// Rotation and quantization kernels for gfx950.
//
//  * k_rotate_rows       y = x . blockdiag(H/16), fp32 arithmetic (tensai docs,
//                        "画像生成", section "幅とメモリ": rows are taken as
//                        groups of 256 and multiplied by H once, on the device).
//  * k_rotq_rows<I8_ROW> rotate in fp64, then per-row symmetric int8 (weights
//                        at load time, same section; activations per token for
//                        the int8 x int8 product, section "GPU").
//  * k_rotq_rows<I4_GRP> rotate in fp64, then int4 with one scale per
//                        (row, 256-group), packed two per byte (the "-q4" width
//                        of section "幅とメモリ").
//
// Work layout: a 256-group is held by 32 lanes (a half wave), 8 consecutive
// elements per lane, so every global access is a 16- or 32-byte vector per
// lane and the transform needs 3 in-lane and 5 cross-lane butterfly stages.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tp {

// ---------------------------------------------------------------- rotate rows
// One (row, group) unit per half wave; 4 waves = 8 units per block.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_rotate_rows(const TIn* x, int64_t ldx, TOut* y, int64_t ldy,
                                                     int64_t units, int groups) {
  const int lane = threadIdx.x & 63;
  const int lane32 = lane & 31;
  const int64_t unit = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  if (unit >= units) return;  // uniform over the half wave that owns the unit
  const int64_t row = unit / groups;
  const int64_t col = (unit - row * groups) * 256 + lane32 * 8;
  float v[8];
  load8(x + row * ldx + col, v);
  fwht256_lane8(v, lane32);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= 0.0625f;
  store8(y + row * ldy + col, v);
}

// ------------------------------------------------------- rotate and quantize
enum { MODE_I8_ROW = 0, MODE_I4_GROUP = 1 };

template <typename TIn>
__device__ __forceinline__ void load_group(const TIn* p, bool rotate, int lane32, double (&v)[8]) {
  load8d(p, v);
  if (rotate) {
    fwht256_lane8(v, lane32);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= 0.0625;
  }
}

// One wave per row. Half wave h of the wave processes groups h, h+2, h+4, ...
template <typename TIn, int MODE>
__global__ __launch_bounds__(256) void k_rotq_rows(const TIn* x, int64_t ldx, int64_t rows, int groups,
                                                   int rotate, uint8_t* q, int64_t ldq, float* scales) {
  const int lane = threadIdx.x & 63;
  const int lane32 = lane & 31;
  const int half = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform over the wave
  const TIn* src = x + row * ldx + lane32 * 8;
  uint8_t* dst = q + row * ldq;

  if (MODE == MODE_I8_ROW) {
    double amax = 0.0;
    for (int g = half; g < groups; g += 2) {
      double v[8];
      load_group(src + (int64_t)g * 256, rotate != 0, lane32, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmax(amax, fabs(v[j]));
    }
    amax = wave_max(amax);
    const float s = (float)(amax / 127.0);
    const double s64 = (double)s;
    const double inv = s > 0.0f ? 1.0 / s64 : 0.0;
    for (int g = half; g < groups; g += 2) {
      double v[8];
      load_group(src + (int64_t)g * 256, rotate != 0, lane32, v);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo |= ((uint32_t)quant_code(v[j], s64, inv, 127.0) & 0xffu) << (8 * j);
        hi |= ((uint32_t)quant_code(v[j + 4], s64, inv, 127.0) & 0xffu) << (8 * j);
      }
      uint2 w = {lo, hi};
      *reinterpret_cast<uint2*>(dst + (int64_t)g * 256 + lane32 * 8) = w;
    }
    if (lane == 0) scales[row] = s;
  } else {
    for (int g = half; g < groups; g += 2) {
      double v[8];
      load_group(src + (int64_t)g * 256, rotate != 0, lane32, v);
      double amax = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmax(amax, fabs(v[j]));
      amax = halfwave_max(amax);
      const float s = (float)(amax / 7.0);
      const double s64 = (double)s;
      const double inv = s > 0.0f ? 1.0 / s64 : 0.0;
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) packed |= ((uint32_t)quant_code(v[j], s64, inv, 7.0) & 0xfu) << (4 * j);
      *reinterpret_cast<uint32_t*>(dst + (int64_t)g * 128 + lane32 * 4) = packed;
      if (lane32 == 0) scales[row * groups + g] = s;
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_rotate_rows(const void* x, bool x_bf16, int64_t ldx, void* y, bool y_bf16, int64_t ldy,
                              int64_t m, int64_t k, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const int64_t units = m * groups;
  const dim3 grid((unsigned)((units + 7) / 8)), block(256);
  if (x_bf16 && y_bf16)
    hipLaunchKernelGGL((k_rotate_rows<uint16_t, uint16_t>), grid, block, 0, stream, (const uint16_t*)x, ldx,
                       (uint16_t*)y, ldy, units, groups);
  else if (x_bf16)
    hipLaunchKernelGGL((k_rotate_rows<uint16_t, float>), grid, block, 0, stream, (const uint16_t*)x, ldx,
                       (float*)y, ldy, units, groups);
  else if (y_bf16)
    hipLaunchKernelGGL((k_rotate_rows<float, uint16_t>), grid, block, 0, stream, (const float*)x, ldx,
                       (uint16_t*)y, ldy, units, groups);
  else
    hipLaunchKernelGGL((k_rotate_rows<float, float>), grid, block, 0, stream, (const float*)x, ldx,
                       (float*)y, ldy, units, groups);
  return hipGetLastError();
}

hipError_t launch_rotq_rows(const void* x, bool x_bf16, int64_t ldx, int64_t rows, int64_t k, bool rotate,
                            int bits, void* q, int64_t ldq, float* scales, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  uint8_t* qb = (uint8_t*)q;
  const int rot = rotate ? 1 : 0;
  if (bits == 8) {
    if (x_bf16)
      hipLaunchKernelGGL((k_rotq_rows<uint16_t, MODE_I8_ROW>), grid, block, 0, stream, (const uint16_t*)x, ldx,
                         rows, groups, rot, qb, ldq, scales);
    else
      hipLaunchKernelGGL((k_rotq_rows<float, MODE_I8_ROW>), grid, block, 0, stream, (const float*)x, ldx, rows,
                         groups, rot, qb, ldq, scales);
  } else {
    if (x_bf16)
      hipLaunchKernelGGL((k_rotq_rows<uint16_t, MODE_I4_GROUP>), grid, block, 0, stream, (const uint16_t*)x,
                         ldx, rows, groups, rot, qb, ldq, scales);
    else
      hipLaunchKernelGGL((k_rotq_rows<float, MODE_I4_GROUP>), grid, block, 0, stream, (const float*)x, ldx,
                         rows, groups, rot, qb, ldq, scales);
  }
  return hipGetLastError();
}

}  // namespace tp
