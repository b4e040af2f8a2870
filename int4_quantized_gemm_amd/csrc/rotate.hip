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
//  * k_rotq_i8_fast      the int8 rows of k_rotq_rows<I8_ROW> in fp32 with an
//                        exact fallback.
//
//  * k_unrotate_rows     y = (q * s) . blockdiag(H/16) in fp64 (exact), rounded
//                        once: undoing a rotated, quantized weight (section
//                        "チェックポイントの入手": the loader undoes the
//                        rotation and the per-row int8 before quantizing
//                        itself).
//
// Every kernel reads its rows through a source (RowSrc: a buffer; DequantSrc:
// q * s of rotated int8 or int4 codes; SwigluSrc:
// the FFN middle h = bf16(silu(g) * u) of a gate and an up buffer, computed on
// the fly, so that the down projection's input is rotated and quantized
// without a round trip through memory).
//
// Work layout: a 256-group is held by 32 lanes (a half wave), 8 consecutive
// elements per lane, so every global access is a 16- or 32-byte vector per
// lane and the transform needs 3 in-lane and 5 cross-lane butterfly stages.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tp {

// ---------------------------------------------------------------- rotate rows
// One (row, group) unit per half wave; 4 waves = 8 units per block.
template <typename Src, typename TOut>
__global__ __launch_bounds__(256) void k_rotate_rows(Src src, TOut* y, int64_t ldy, int64_t units, int groups) {
  const int lane = threadIdx.x & 63;
  const int lane32 = lane & 31;
  const int64_t unit = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  if (unit >= units) return;  // uniform over the half wave that owns the unit
  const int64_t row = unit / groups;
  const int64_t col = (unit - row * groups) * 256 + lane32 * 8;
  float v[8];
  src.load8(row, col, v);
  fwht256_lane8(v, lane32);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] *= 0.0625f;
  store8(y + row * ldy + col, v);
}

// Rounds an fp64 value to bf16 (nearest even) with one rounding: through fp32
// with round-to-odd, which keeps the bits that decide the second rounding.
__device__ __forceinline__ uint32_t bf16_bits_from_double(double d) {
  if (d != d) return 0x7FC0u;
  const float f = __double2float_rz(d);
  uint32_t fb = __builtin_bit_cast(uint32_t, f);
  if ((double)f != d) fb |= 1u;
  return (fb + 0x7FFFu + ((fb >> 16) & 1u)) >> 16;
}

// The rotation in fp64 with one rounding of the result: exact for sources
// whose groups are integers times one scale (DequantSrc).
template <typename Src, typename TOut>
__global__ __launch_bounds__(256) void k_unrotate_rows(Src src, TOut* y, int64_t ldy, int64_t units, int groups) {
  const int lane = threadIdx.x & 63;
  const int lane32 = lane & 31;
  const int64_t unit = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  if (unit >= units) return;  // uniform over the half wave that owns the unit
  const int64_t row = unit / groups;
  const int64_t col = (unit - row * groups) * 256 + lane32 * 8;
  double v[8];
  src.load8d(row, col, v);
  fwht256_lane8(v, lane32);
  TOut* out = y + row * ldy + col;
  if constexpr (std::is_same<TOut, float>::value) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = (float)(v[j] * 0.0625);
    store8(out, f);
  } else {
    u32x4_t a;
    a.x = bf16_bits_from_double(v[0] * 0.0625) | (bf16_bits_from_double(v[1] * 0.0625) << 16);
    a.y = bf16_bits_from_double(v[2] * 0.0625) | (bf16_bits_from_double(v[3] * 0.0625) << 16);
    a.z = bf16_bits_from_double(v[4] * 0.0625) | (bf16_bits_from_double(v[5] * 0.0625) << 16);
    a.w = bf16_bits_from_double(v[6] * 0.0625) | (bf16_bits_from_double(v[7] * 0.0625) << 16);
    *reinterpret_cast<u32x4_t*>(out) = a;
  }
}

// ------------------------------------------------------- rotate and quantize
enum { MODE_I8_ROW = 0, MODE_I4_GROUP = 1 };

template <typename Src>
__device__ __forceinline__ void load_group(const Src& src, int64_t row, int64_t col, bool rotate, int lane32,
                                           double (&v)[8]) {
  src.load8d(row, col, v);
  if (rotate) {
    fwht256_lane8(v, lane32);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= 0.0625;
  }
}

// One wave per row. Half wave h of the wave processes groups h, h+2, h+4, ...
template <typename Src, int MODE>
__global__ __launch_bounds__(256) void k_rotq_rows(Src src, int64_t rows, int groups, int rotate, uint8_t* q,
                                                   int64_t ldq, float* scales) {
  const int lane = threadIdx.x & 63;
  const int lane32 = lane & 31;
  const int half = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform over the wave
  const int64_t col0 = lane32 * 8;
  uint8_t* dst = q + row * ldq;

  if (MODE == MODE_I8_ROW) {
    double amax = 0.0;
    for (int g = half; g < groups; g += 2) {
      double v[8];
      load_group(src, row, col0 + (int64_t)g * 256, rotate != 0, lane32, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmax(amax, fabs(v[j]));
    }
    amax = wave_max(amax);
    const float s = (float)(amax / 127.0);
    const double s64 = (double)s;
    const double inv = s > 0.0f ? 1.0 / s64 : 0.0;
    for (int g = half; g < groups; g += 2) {
      double v[8];
      load_group(src, row, col0 + (int64_t)g * 256, rotate != 0, lane32, v);
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
      load_group(src, row, col0 + (int64_t)g * 256, rotate != 0, lane32, v);
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

// ------------------------------- rotate and quantize rows to int8 (fast path)
// The same codes and scales as k_rotq_rows<MODE_I8_ROW>, computed in fp32 with
// a proven error bound and redone exactly (fp64) only where the bound cannot
// decide.
//
// Layout: a 256-group is held by one 16-lane row of the wave. Lane l loads
// elements 16 l + i (i = 0..15, index bits 0-3 in registers) and applies the
// four butterfly stages of those bits; the row then transposes the group
// through LDS so that lane l holds elements l + 16 r (bits 4-7 in registers)
// and applies the other four stages. Outputs stay in that order; the codes go
// back through LDS to be stored 16 contiguous bytes per lane.
//
// Error bound (unnormalized transform, fp32 round-to-nearest): the rounding
// errors that reach one output are those of the nodes of its butterfly tree;
// at each of the 8 stages these nodes partition the 256 inputs, so each stage
// adds at most 2^-24 * L1 (L1 = sum of |inputs| of the group) and the output
// error is at most 8 * 2^-24 * L1 = 2^-21 L1 (before the exact 1/16).
//   * Row maximum: elements whose fp32 magnitude is within twice the largest
//     bound of the fp32 maximum are the only ones that can be the true
//     maximum; their groups are transformed again in fp64 (exact for these
//     inputs, as in k_rotq_rows) and the scale comes from the exact maximum.
//   * Codes: t = v * (1/(16 s)) in fp32 is within B / (16 s) + 2^-22 (|t| + 1)
//     of the exact quotient; a code whose t is at least that far from every
//     half-integer rounds the same way as the exact one. A group with a code
//     closer than that is redone in fp64 with quant_code (the reference rule).

template <int M>
__device__ __forceinline__ int dpp_xor(int v) {
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  if constexpr (M == 4)  // half mirror (i ^ 7), then quad reverse (i ^ 3)
    return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false), 0x1B, 0xF, 0xF, false);
  if constexpr (M == 8)  // mirror (i ^ 15), then half mirror (i ^ 7)
    return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false), 0x141, 0xF, 0xF, false);
  return v;
}

template <int M>
__device__ __forceinline__ float xor16(float v) {
  return __builtin_bit_cast(float, dpp_xor<M>(__builtin_bit_cast(int, v)));
}

// Sum over the 16 lanes of a row (every lane gets the total).
__device__ __forceinline__ float sum16(float v) {
  v += xor16<1>(v);
  v += xor16<2>(v);
  v += xor16<4>(v);
  v += xor16<8>(v);
  return v;
}

// Bitwise or over the 16 lanes of a row (every lane gets the result).
__device__ __forceinline__ uint32_t or16(uint32_t v) {
  v |= (uint32_t)dpp_xor<1>((int)v);
  v |= (uint32_t)dpp_xor<2>((int)v);
  v |= (uint32_t)dpp_xor<4>((int)v);
  v |= (uint32_t)dpp_xor<8>((int)v);
  return v;
}

// Four butterfly stages over the register index of 16 values.
template <typename T>
__device__ __forceinline__ void fwht16_regs(T (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const T a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

// Orders this wave's LDS writes before its later LDS reads (one wave: the LDS
// unit runs its operations in order; this keeps the compiler from reordering).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Row transpose: lane l gives elements 16 l + i, receives elements l + 16 r.
// buf: this row's LDS area, touched by its 16 lanes only. Element e sits at
// e + PAD * (e / 16) so that neither side of the exchange has bank conflicts.
template <typename T>
__device__ __forceinline__ void transpose16(T (&v)[16], T* buf, int l16) {
  constexpr int PAD = sizeof(T) == 4 ? 4 : 2;
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < 16; ++i) buf[(16 + PAD) * l16 + i] = v[i];
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = buf[l16 + (16 + PAD) * r];
}

// The 16 inputs of one lane for one group, kept as loaded (bf16 pairs or fp32)
// for the exact fallbacks.
template <typename TIn>
struct Raw16;

template <>
struct Raw16<uint16_t> {
  uint32_t w[8];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float get(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
};

template <>
struct Raw16<float> {
  float w[16];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 f = reinterpret_cast<const float4*>(p)[c];
      w[4 * c] = f.x; w[4 * c + 1] = f.y; w[4 * c + 2] = f.z; w[4 * c + 3] = f.w;
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0.f;
  }
  __device__ __forceinline__ float get(int i) const { return w[i]; }
};

// ------------------------------------------------------------- input sources
// A source yields 8 or 16 consecutive elements of a row: as fp32 (load8), as
// fp64 (load8d), or as the raw words the fast int8 kernel keeps for its exact
// fallbacks (load16, into Raw16<raw_elem>).

// Rows of a [rows, k] buffer of fp32 or bf16 (uint16_t) elements.
template <typename T>
struct RowSrc {
  typedef T raw_elem;
  // The fast int8 kernel may load a group's inputs again for its exact
  // fallbacks instead of keeping them in registers.
  static constexpr bool REREAD = true;
  const T* x;
  int64_t ldx;
  __device__ __forceinline__ void load8(int64_t r, int64_t c, float (&v)[8]) const { tp::load8(x + r * ldx + c, v); }
  __device__ __forceinline__ void load8d(int64_t r, int64_t c, double (&v)[8]) const {
    tp::load8d(x + r * ldx + c, v);
  }
  __device__ __forceinline__ void load16(int64_t r, int64_t c, Raw16<T>& raw) const { raw.load(x + r * ldx + c); }
  // Two-phase form of load16: fetch issues the loads, finish produces the
  // raw words (here the loaded words themselves).
  typedef Raw16<T> stash_t;
  __device__ __forceinline__ void fetch(int64_t r, int64_t c, stash_t& st) const { st.load(x + r * ldx + c); }
  __device__ __forceinline__ void finish(int64_t, int64_t, const stash_t& st, Raw16<T>& raw) const { raw = st; }
};

// q * s of rotated weight codes: int8 with one scale per row (BITS 8) or
// packed int4 with one scale per row and 256-group (BITS 4). Exact in fp64
// (an 8-bit integer times an fp32 scale). Only the fp64 loads are provided.
template <int BITS>
struct DequantSrc {
  typedef float raw_elem;
  static constexpr bool REREAD = false;
  const uint8_t* q;
  int64_t ldq;  // bytes
  const float* s;
  int groups;
  __device__ __forceinline__ void load8d(int64_t r, int64_t c, double (&v)[8]) const {
    if constexpr (BITS == 8) {
      const double sc = (double)s[r];
      const uint2 w = *reinterpret_cast<const uint2*>(q + r * ldq + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = (double)(int8_t)(w.x >> (8 * j)) * sc;
        v[4 + j] = (double)(int8_t)(w.y >> (8 * j)) * sc;
      }
    } else {
      const double sc = (double)s[r * groups + c / 256];
      const int32_t w = *reinterpret_cast<const int32_t*>(q + r * ldq + c / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (double)((w << (28 - 4 * j)) >> 28) * sc;
    }
  }
};

// The SwiGLU feed-forward's hidden activation h = bf16(silu(g) * u), silu(x)
// = x / (1 + e^-x), rounded once (to nearest even) from its fp64 evaluation
// (tensai docs, "画像生成", section "何が走るか": every block is attention plus
// a SwiGLU feed-forward; TensorFold pull request #948, first comment: the
// activations between operations are kept in bf16).
//
// fp32 first: e = v_exp_f32(-g * fl(log2 e)), h = (g u) v_rcp_f32(1 + e).
// Relative error, to first order, with u = 2^-24: the exponent argument is
// off by at most |g log2 e| (u + 2^-26.2) (the product and the rounded log2 e),
// which makes e off by |g| (u + 2^-26.2) relative; v_exp_f32 and v_rcp_f32 add
// 2u each, 1 + e, g u and the last product u each: below (1.25 |g| + 8) u in
// all. For a normal h in [2^E, 2^(E+1)) that is under 1.25 |g| + 8 fp32 ulps,
// and bf16 rounding only depends on where the low 16 bits of h sit against the
// midpoint 0x8000: when they are more than 2.5 |g| + 20 ulps away (twice the
// bound, plus 4), h rounds like its fp64 evaluation. swiglu_fast returns the
// bf16 bits and whether that holds (false also for |g| > 64 and for h not a
// normal number); swiglu_exact redoes an element in fp64 and rounds it to bf16
// through fp32 with round-to-odd (no double rounding).
__device__ __forceinline__ uint32_t swiglu_fast(float g, float u, bool& ok) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  const float h = (g * u) * __builtin_amdgcn_rcpf(1.0f + e);
  const uint32_t b = __builtin_bit_cast(uint32_t, h);
  const float dist = (float)((int)(b & 0xFFFFu) - 0x8000);
  ok = __builtin_isnormal(h) && fabsf(g) <= 64.f && fabsf(dist) > fmaf(fabsf(g), 2.5f, 20.f);
  return (b + 0x8000u) >> 16;  // not a tie when ok: no even-rule needed
}

__device__ __noinline__ uint32_t swiglu_exact(float g, float u) {
  const double hd = ((double)g * (double)u) / (1.0 + exp(-(double)g));
  if (hd != hd) return 0x7FC0u;
  const float f = __double2float_rz(hd);
  uint32_t fb = __builtin_bit_cast(uint32_t, f);
  if ((double)f != hd) fb |= 1u;
  return (fb + 0x7FFFu + ((fb >> 16) & 1u)) >> 16;
}

// h = bf16(silu(g) * u) of a gate and an up buffer ([rows, k], both fp32 or
// both bf16), element by element. Elements the fp32 shortcut cannot decide
// are collected in a per-lane mask and redone afterwards, one at a time, from
// reloaded inputs, so a wave pays for the fp64 path once per round of such
// elements rather than once per element position.
template <typename T>
struct SwigluSrc {
  typedef uint16_t raw_elem;
  static constexpr bool REREAD = false;  // h is computed, not loaded: keep it
  const T* g;
  int64_t ldg;
  const T* u;
  int64_t ldu;
  template <int N>
  __device__ __forceinline__ void bits(int64_t r, int64_t c, uint32_t (&hb)[N]) const {
    float gv[N], uv[N];
    const T* gp = g + r * ldg + c;
    const T* up = u + r * ldu + c;
#pragma unroll
    for (int j = 0; j < N; j += 8) {
      tp::load8(gp + j, *reinterpret_cast<float(*)[8]>(&gv[j]));
      tp::load8(up + j, *reinterpret_cast<float(*)[8]>(&uv[j]));
    }
    compute(r, c, gv, uv, hb);
  }
  template <int N>
  __device__ __forceinline__ void compute(int64_t r, int64_t c, const float (&gv)[N], const float (&uv)[N],
                                          uint32_t (&hb)[N]) const {
    const T* gp = g + r * ldg + c;
    const T* up = u + r * ldu + c;
    uint32_t redo = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      bool ok;
      hb[j] = swiglu_fast(gv[j], uv[j], ok);
      redo |= ok ? 0u : (1u << j);
    }
    while (redo) {
      const int j = __builtin_ctz(redo);
      redo &= redo - 1;
      float gj[8], uj[8];
      tp::load8(gp + (j & ~7), gj);
      tp::load8(up + (j & ~7), uj);
      float gs = gj[0], us = uj[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) {
        gs = (t == (j & 7)) ? gj[t] : gs;
        us = (t == (j & 7)) ? uj[t] : us;
      }
      const uint32_t v = swiglu_exact(gs, us);
#pragma unroll
      for (int t = 0; t < N; ++t) hb[t] = (t == j) ? v : hb[t];
    }
  }
  __device__ __forceinline__ void load8(int64_t r, int64_t c, float (&v)[8]) const {
    uint32_t hb[8];
    bits(r, c, hb);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_bit_cast(float, hb[j] << 16);
  }
  __device__ __forceinline__ void load8d(int64_t r, int64_t c, double (&v)[8]) const {
    float f[8];
    load8(r, c, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (double)f[j];
  }
  __device__ __forceinline__ void load16(int64_t r, int64_t c, Raw16<uint16_t>& raw) const {
    uint32_t hb[16];
    bits(r, c, hb);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw.w[i] = hb[2 * i] | (hb[2 * i + 1] << 16);
  }
  // Two-phase form of load16: fetch issues the loads of g and u, finish
  // computes h (so a kernel can have several groups' loads in flight).
  struct stash_t {
    Raw16<T> g, u;
  };
  __device__ __forceinline__ void fetch(int64_t r, int64_t c, stash_t& st) const {
    st.g.load(g + r * ldg + c);
    st.u.load(u + r * ldu + c);
  }
  __device__ __forceinline__ void finish(int64_t r, int64_t c, const stash_t& st, Raw16<uint16_t>& raw) const {
    float gv[16], uv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      gv[j] = st.g.get(j);
      uv[j] = st.u.get(j);
    }
    uint32_t hb[16];
    compute(r, c, gv, uv, hb);
#pragma unroll
    for (int i = 0; i < 8; ++i) raw.w[i] = hb[2 * i] | (hb[2 * i + 1] << 16);
  }
};

template <int M>
__device__ __forceinline__ double xor16d(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_xor<M>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_xor<M>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Exact (fp64) unnormalized rotated element e of a group, summed over the 16
// lanes of the row (lane l holds inputs 16 l .. 16 l + 15 in raw): the sign of
// input i is (-1)^popcount(i & e). Without rotation, input e itself. Every
// lane of the row must be active; all get the value.
template <typename TIn>
__device__ __forceinline__ double exact_elem(const Raw16<TIn>& raw, bool rotate, int e, int l16) {
  double acc = 0.0;
  if (rotate) {
    // Bit i of w: the parity of popcount((16 l16 + i) & e), i.e. the sign of
    // input i of this lane. The parity is linear in e, so the low half is the
    // xor of the Walsh rows of e's low bits (0xAAAA for bit 0, 0xCCCC, 0xF0F0,
    // 0xFF00) and the lane's part flips all sixteen.
    const int el = e & 15;
    uint32_t w = ((el & 1) ? 0xAAAAu : 0u) ^ ((el & 2) ? 0xCCCCu : 0u) ^ ((el & 4) ? 0xF0F0u : 0u) ^
                 ((el & 8) ? 0xFF00u : 0u);
    if (__builtin_popcount((unsigned)(l16 & (e >> 4))) & 1) w ^= 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint64_t xb = __builtin_bit_cast(uint64_t, (double)raw.get(i));
      acc += __builtin_bit_cast(double, xb ^ ((uint64_t)((w >> i) & 1u) << 63));
    }
  } else {
    // input e lives in lane e / 16, register e % 16
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i == (e & 15)) acc = (double)raw.get(i);
    acc = (l16 == (e >> 4)) ? acc : 0.0;
  }
  acc += xor16d<1>(acc);
  acc += xor16d<2>(acc);
  acc += xor16d<4>(acc);
  acc += xor16d<8>(acc);
  return acc;
}

constexpr int RQ_ROW_BYTES = 1280 + 64;  // LDS per 16-lane row: 256 padded floats
constexpr float RQ_MAGIC = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer (RNE)

// WPR = 1: one wave per row, four rows per block (k <= 12 * 256).
// WPR = 4: one block per row, the four waves split the groups (k <= 48 * 256).
// Sources that are plain rows (REREAD) load a group's inputs again for the
// rare exact fallbacks, which fits the kernel in 128 registers: four waves per
// SIMD, so the 4096 one-wave rows of a 4096 x 3072 input are all resident at
// once. Computed sources (SwiGLU) keep their inputs in registers for the
// fallbacks, within the 168 registers of three waves per SIMD.
template <typename Src, int WPR, int WPE = Src::REREAD ? 4 : 3>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void k_rotq_i8_fast(
    Src src, int64_t rows, int groups, int rotate, int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales) {
  typedef typename Src::raw_elem TIn;
  constexpr bool KEEP = !Src::REREAD;
  constexpr int NU = 3;  // groups per 16-lane set
  constexpr int NWB = 4;  // waves per block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int set = lane >> 4, l16 = lane & 15;
  __shared__ __align__(16) uint8_t lds[4 * NWB * RQ_ROW_BYTES];
  __shared__ float red[2][NWB];
  __shared__ double red64[NWB];
  uint8_t* mybuf = lds + (wave * 4 + set) * RQ_ROW_BYTES;
  float* fbuf = reinterpret_cast<float*>(mybuf);
  int64_t row;
  int gb, ge;
  if constexpr (WPR == 1) {
    row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= rows) return;  // uniform over the wave; no block barrier below
    gb = 0;
    ge = groups;
  } else {
    row = blockIdx.x;
    const int gpw = (groups + WPR - 1) / WPR;
    gb = min(groups, wave * gpw);
    ge = min(groups, gb + gpw);
  }

  // Load every group of this wave (up to 3 per 16-lane row) and transform it.
  Raw16<TIn> raw[KEEP ? NU : 1];  // the inputs, kept for the exact fallbacks
  float v[NU][16];
  float bnd[NU];
  bool has[NU];
  {
    typename Src::stash_t st[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      has[u] = gb + set + 4 * u < ge;
      if (has[u]) src.fetch(row, (int64_t)(gb + set + 4 * u) * 256 + l16 * 16, st[u]);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      Raw16<TIn> r0;
      if (has[u])
        src.finish(row, (int64_t)(gb + set + 4 * u) * 256 + l16 * 16, st[u], r0);
      else
        r0.zero();
#pragma unroll
      for (int i = 0; i < 16; ++i) v[u][i] = r0.get(i);
      if constexpr (KEEP) raw[u] = r0;
    }
  }
  // The inputs of unit U for an exact fallback (every lane of the row takes
  // part; lanes without the group read zeros).
  auto inputs = [&](auto uc) -> Raw16<TIn> {
    constexpr int U = decltype(uc)::value;
    if constexpr (KEEP) {
      return raw[U];
    } else {
      Raw16<TIn> r;
      if (has[U])
        src.load16(row, (int64_t)(gb + set + 4 * U) * 256 + l16 * 16, r);
      else
        r.zero();
      return r;
    }
  };
  float amax = 0.f, bmax = 0.f;
  float umax[NU];  // this lane's largest |value| of each unit
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    bnd[u] = 0.f;
    if (rotate) {
      float l1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) l1 += fabsf(v[u][i]);
      l1 = sum16(l1);  // rows without a group hold zeros
      fwht16_regs(v[u]);
      transpose16(v[u], fbuf, l16);
      fwht16_regs(v[u]);
      bnd[u] = l1 * 0x1.00004p-21f;  // 2^-21 L1, rounded up
    } else {
      transpose16(v[u], fbuf, l16);
    }
    umax[u] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) umax[u] = fmaxf(umax[u], fabsf(v[u][i]));
    amax = fmaxf(amax, umax[u]);
    bmax = fmaxf(bmax, bnd[u]);
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
  if constexpr (WPR > 1) {
    if (lane == 0) {
      red[0][wave] = amax;
      red[1][wave] = bmax;
    }
    __syncthreads();
    amax = red[0][0];
    bmax = red[1][0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) {
      amax = fmaxf(amax, red[0][w]);
      bmax = fmaxf(bmax, red[1][w]);
    }
  }

  // Exact row maximum (unnormalized): the exact value of every element that
  // could be the maximum. Candidates are kept as per-lane register bitmasks,
  // so the loops below index no register array.
  double amax_ex = (double)amax;
  if (bmax > 0.f) {
    const float thr = amax - 2.f * bmax;
    double m_ex = 0.0;
    auto scan = [&](auto uc) {
      constexpr int U = decltype(uc)::value;
      // units with no lane reaching the threshold hold no candidate
      if (!__ballot(has[U] && umax[U] >= thr)) return;
      uint32_t bits = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) bits |= (uint32_t)(has[U] && fabsf(v[U][r]) >= thr) << r;
      uint32_t rmask = or16(bits);  // registers that hold a candidate in some lane of this row
      if (!__ballot(rmask != 0u)) return;
      const Raw16<TIn> xin = inputs(uc);
      while (rmask) {               // uniform over this 16-lane row
        const int r = __builtin_ctz(rmask);
        rmask &= rmask - 1;
        uint32_t lmask = (uint32_t)(__ballot((bits >> r) & 1u) >> (16 * set)) & 0xFFFFu;
        while (lmask) {
          const int lc = __builtin_ctz(lmask);
          lmask &= lmask - 1;
          m_ex = fmax(m_ex, fabs(exact_elem(xin, true, lc + 16 * r, l16)));
        }
      }
    };
    scan(std::integral_constant<int, 0>{});
    if constexpr (NU > 1) scan(std::integral_constant<int, 1>{});
    if constexpr (NU > 2) scan(std::integral_constant<int, 2>{});
    m_ex = wave_max(m_ex);
    if constexpr (WPR > 1) {
      if (lane == 0) red64[wave] = m_ex;
      __syncthreads();
      m_ex = red64[0];
#pragma unroll
      for (int w = 1; w < WPR; ++w) m_ex = fmax(m_ex, red64[w]);
    }
    amax_ex = m_ex;
  }
  const double unscale = rotate ? 0.0625 : 1.0;  // outputs above are 16 x the rotation (exact)
  const float s = (float)(amax_ex * unscale / 127.0);
  const double s64 = (double)s;
  const double inv64 = s > 0.0f ? 1.0 / s64 : 0.0;
  const float inv = (float)(inv64 * unscale);  // applied to the unnormalized outputs

  // Codes, one group at a time. f = v * inv + 1.5 * 2^23 in one fused
  // rounding holds the nearest integer to the exact product v * inv in its
  // low bits (two's complement in the low byte), and d = v * inv - (f - 1.5 *
  // 2^23), again fused, its distance from that integer. A code is decided when
  // |d| < lim: the fp32 transform (within bnd of the exact value, times inv),
  // the rounding of inv and of d stay below 0.5 - lim, so the exact quotient
  // rounds to the same integer, which is then within [-127, 127] (|exact| <=
  // 127.5 - ...). A lane flag collects undecided codes; only a wave holding one
  // rebuilds the per-element bits and takes the exact path (the reference
  // rule on the exact value). A scale so small that inv overflows to
  // infinity makes d NaN: such codes are undecided too.
  int8_t* qr = q + row * ldq;
  auto codes = [&](auto uc) {
    constexpr int U = decltype(uc)::value;
    uint32_t code[16];
    const float lim = 0.5f - (bnd[U] * inv * 1.0001f + 129.f * 0x1p-22f);
    bool undecided = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float f = fmaf(v[U][r], inv, RQ_MAGIC);
      const float d = fmaf(v[U][r], inv, RQ_MAGIC - f);
      undecided |= !(fabsf(d) < lim);  // NaN (inv overflowed for a tiny scale): undecided
      code[r] = __builtin_bit_cast(uint32_t, f);
    }
    if (__ballot(undecided && has[U])) {
      uint32_t bits = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float f = fmaf(v[U][r], inv, RQ_MAGIC);
        const float d = fmaf(v[U][r], inv, RQ_MAGIC - f);
        bits |= (uint32_t)(has[U] && !(fabsf(d) < lim)) << r;
      }
      uint32_t rmask = or16(bits);
      const Raw16<TIn> xin = inputs(uc);
      while (rmask) {  // uniform over this 16-lane row
        const int r = __builtin_ctz(rmask);
        rmask &= rmask - 1;
        uint32_t lmask = (uint32_t)(__ballot((bits >> r) & 1u) >> (16 * set)) & 0xFFFFu;
        while (lmask) {
          const int lc = __builtin_ctz(lmask);
          lmask &= lmask - 1;
          const double xe = exact_elem(xin, rotate != 0, lc + 16 * r, l16);
          const uint32_t c = (uint32_t)quant_code(xe * unscale, s64, inv64, 127.0);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) code[rr] = (rr == r && l16 == lc) ? c : code[rr];
        }
      }
    }
    // element l16 + 16 r -> byte l16 + 16 r of this row's buffer, then 16
    // contiguous bytes per lane out
    wave_lds_sync();
#pragma unroll
    for (int r = 0; r < 16; ++r) mybuf[l16 + 16 * r] = (uint8_t)code[r];
    wave_lds_sync();
    const uint4 w4 = *reinterpret_cast<const uint4*>(mybuf + 16 * l16);
    if (has[U]) *reinterpret_cast<uint4*>(qr + (int64_t)(gb + set + 4 * U) * 256 + l16 * 16) = w4;
  };
  codes(std::integral_constant<int, 0>{});
  if constexpr (NU > 1) codes(std::integral_constant<int, 1>{});
  if constexpr (NU > 2) codes(std::integral_constant<int, 2>{});
  if (lane == 0 && (WPR == 1 || wave == 0)) scales[row] = s;
}

// ------------------------------------------------------------------ launchers
template <typename Src, typename TOut>
static hipError_t rotate_from(const Src& src, TOut* y, int64_t ldy, int64_t m, int64_t k, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const int64_t units = m * groups;
  const dim3 grid((unsigned)((units + 7) / 8)), block(256);
  hipLaunchKernelGGL((k_rotate_rows<Src, TOut>), grid, block, 0, stream, src, y, ldy, units, groups);
  return hipGetLastError();
}

// int8 rows: the fast kernel up to 48 groups, the fp64 one above.
template <typename Src>
static hipError_t rotq_i8_from(const Src& src, int64_t rows, int groups, int rot, int8_t* q8, int64_t ldq,
                               float* scales, hipStream_t stream) {
  const dim3 block(256);
  if (groups <= 12)
    hipLaunchKernelGGL((k_rotq_i8_fast<Src, 1>), dim3((unsigned)((rows + 3) / 4)), block, 0, stream, src, rows,
                       groups, rot, q8, ldq, scales);
  else if (groups <= 48)
    hipLaunchKernelGGL((k_rotq_i8_fast<Src, 4>), dim3((unsigned)rows), block, 0, stream, src, rows, groups, rot, q8,
                       ldq, scales);
  else
    hipLaunchKernelGGL((k_rotq_rows<Src, MODE_I8_ROW>), dim3((unsigned)((rows + 3) / 4)), block, 0, stream, src,
                       rows, groups, rot, (uint8_t*)q8, ldq, scales);
  return hipGetLastError();
}

hipError_t launch_rotate_rows(const void* x, bool x_bf16, int64_t ldx, void* y, bool y_bf16, int64_t ldy,
                              int64_t m, int64_t k, hipStream_t stream) {
  if (x_bf16) {
    const RowSrc<uint16_t> src{(const uint16_t*)x, ldx};
    return y_bf16 ? rotate_from(src, (uint16_t*)y, ldy, m, k, stream) : rotate_from(src, (float*)y, ldy, m, k, stream);
  }
  const RowSrc<float> src{(const float*)x, ldx};
  return y_bf16 ? rotate_from(src, (uint16_t*)y, ldy, m, k, stream) : rotate_from(src, (float*)y, ldy, m, k, stream);
}

hipError_t launch_rotq_rows(const void* x, bool x_bf16, int64_t ldx, int64_t rows, int64_t k, bool rotate,
                            int bits, void* q, int64_t ldq, float* scales, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const int rot = rotate ? 1 : 0;
  if (bits == 8) {
    if (x_bf16) return rotq_i8_from(RowSrc<uint16_t>{(const uint16_t*)x, ldx}, rows, groups, rot, (int8_t*)q, ldq,
                                    scales, stream);
    return rotq_i8_from(RowSrc<float>{(const float*)x, ldx}, rows, groups, rot, (int8_t*)q, ldq, scales, stream);
  }
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (x_bf16)
    hipLaunchKernelGGL((k_rotq_rows<RowSrc<uint16_t>, MODE_I4_GROUP>), grid, block, 0, stream,
                       RowSrc<uint16_t>{(const uint16_t*)x, ldx}, rows, groups, rot, (uint8_t*)q, ldq, scales);
  else
    hipLaunchKernelGGL((k_rotq_rows<RowSrc<float>, MODE_I4_GROUP>), grid, block, 0, stream,
                       RowSrc<float>{(const float*)x, ldx}, rows, groups, rot, (uint8_t*)q, ldq, scales);
  return hipGetLastError();
}

hipError_t launch_dequant_unrotate(const void* q, int bits, int64_t ldq, const float* scales, int64_t n, int64_t k,
                                  void* w, bool w_bf16, int64_t ldw, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const int64_t units = n * groups;
  const dim3 grid((unsigned)((units + 7) / 8)), block(256);
#define TP_UNROT(B, TO)                                                                                        \
  hipLaunchKernelGGL((k_unrotate_rows<DequantSrc<B>, TO>), grid, block, 0, stream,                               \
                     DequantSrc<B>{(const uint8_t*)q, ldq, scales, groups}, (TO*)w, ldw, units, groups)
  if (bits == 8) {
    if (w_bf16) TP_UNROT(8, uint16_t); else TP_UNROT(8, float);
  } else {
    if (w_bf16) TP_UNROT(4, uint16_t); else TP_UNROT(4, float);
  }
#undef TP_UNROT
  return hipGetLastError();
}

hipError_t launch_requantize(const void* q_in, int bits_in, int64_t ldq_in, const float* s_in, int64_t n, int64_t k,
                             int bits_out, void* q_out, int64_t ldq_out, float* s_out, hipStream_t stream) {
  const int groups = (int)(k / 256);
  const dim3 grid((unsigned)((n + 3) / 4)), block(256);
#define TP_REQ(B, MODE)                                                                                        \
  hipLaunchKernelGGL((k_rotq_rows<DequantSrc<B>, MODE>), grid, block, 0, stream,                                 \
                     DequantSrc<B>{(const uint8_t*)q_in, ldq_in, s_in, groups}, n, groups, 0, (uint8_t*)q_out,   \
                     ldq_out, s_out)
  if (bits_in == 8) {
    if (bits_out == 8) TP_REQ(8, MODE_I8_ROW); else TP_REQ(8, MODE_I4_GROUP);
  } else {
    if (bits_out == 8) TP_REQ(4, MODE_I8_ROW); else TP_REQ(4, MODE_I4_GROUP);
  }
#undef TP_REQ
  return hipGetLastError();
}

hipError_t launch_swiglu_rotate(const void* g, int64_t ldg, const void* u, int64_t ldu, bool in_bf16, int64_t m,
                                int64_t k, bool out_i8, void* y, int64_t ldy, float* scales, hipStream_t stream) {
  const int groups = (int)(k / 256);
  if (in_bf16) {
    const SwigluSrc<uint16_t> src{(const uint16_t*)g, ldg, (const uint16_t*)u, ldu};
    if (out_i8) return rotq_i8_from(src, m, groups, 1, (int8_t*)y, ldy, scales, stream);
    return rotate_from(src, (uint16_t*)y, ldy, m, k, stream);
  }
  const SwigluSrc<float> src{(const float*)g, ldg, (const float*)u, ldu};
  if (out_i8) return rotq_i8_from(src, m, groups, 1, (int8_t*)y, ldy, scales, stream);
  return rotate_from(src, (uint16_t*)y, ldy, m, k, stream);
}

}  // namespace tp
