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
//  * k_rotq_i8_d         the int8 rows of k_rotq_rows<I8_ROW> for up to 48
//                        groups a row, 16 lanes a group (the same fp64
//                        transform; several groups of a row in flight).
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

// --------------------------------------------- group layout of the int8 rows
// A 256-group is held by one 16-lane row of the wave: lane l loads elements
// 16 l + i (i = 0..15, index bits 0-3 in registers) and applies the four
// butterfly stages of those bits; the row then transposes the group through
// LDS so that lane l holds elements l + 16 r (bits 4-7 in registers) and
// applies the other four stages. Outputs stay in that order; the codes go back
// through LDS to be stored 16 contiguous bytes per lane.

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

// The 16 inputs of one lane for one group, as loaded (bf16 pairs or fp32).
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
// fp64 (load8d), or as raw words (fetch then finish, into Raw16<raw_elem>)
// for the int8 rows.

// Rows of a [rows, k] buffer of fp32 or bf16 (uint16_t) elements.
template <typename T>
struct RowSrc {
  typedef T raw_elem;
  const T* x;
  int64_t ldx;
  __device__ __forceinline__ void load8(int64_t r, int64_t c, float (&v)[8]) const { tp::load8(x + r * ldx + c, v); }
  __device__ __forceinline__ void load8d(int64_t r, int64_t c, double (&v)[8]) const {
    tp::load8d(x + r * ldx + c, v);
  }
  // Two-phase load of 16 elements for the int8 rows: fetch issues the loads,
  // finish produces the raw words (here the loaded words themselves).
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
  // Two-phase load of 16 elements for the int8 rows: fetch issues the loads of
  // g and u, finish computes h (so a kernel can have several groups' loads in
  // flight).
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

// Largest magnitude of 16 doubles: a tree of v_max_f64 with both operands
// taken as magnitudes (one instruction per pair; written out because the
// compiler adds a canonicalizing max per element to fmax(., fabs(.))).
__device__ __forceinline__ double absmax2(double a, double b) {
  double r;
  asm("v_max_f64 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ double absmax16(const double (&v)[16]) {
  double m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = absmax2(v[2 * i], v[2 * i + 1]);
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) m[i] = absmax2(m[i], m[i + w]);  // operands already >= 0
  return m[0];
}

// ------------------------- rotate and quantize rows to int8 (fp64 transform)
// The same codes and scales as k_rotq_rows<MODE_I8_ROW> (the transform in
// fp64, whose values are the exact ones whenever k_rotq_rows' are: every stage
// only adds or subtracts), on the group layout above: a 16-lane row of the
// wave per 256-group, 16 elements a lane, a row transpose through LDS between
// the butterflies of index bits 0-3 and 4-7. The row maximum and the codes are
// read off the exact values directly.
//
// Code of an element v (unnormalized, 16 x the rotation): f = fma(v, invu,
// 1.5 * 2^52) holds in its low bits the integer nearest the exact product v *
// invu (invu = (1/s) / 16, exact from 1/s), and d = fma(v, invu, 1.5 * 2^52 -
// f) its distance from that integer. The product is within 2^-45 of the exact
// quotient, so when |d| < 0.5 - 1e-9 the quotient rounds to the same integer,
// which is what quant_code gives; the rare others take quant_code itself, as
// do rows whose scale is subnormal (see below).
template <typename Src, int WPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_rotq_i8_d(
    Src src, int64_t rows, int groups, int rotate, int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales) {
  typedef typename Src::raw_elem TIn;
  constexpr int NU = 3;   // groups per 16-lane row
  constexpr int NWB = 4;  // waves per block
  constexpr int ROWB = 16 * (16 + 2) * 8;  // one row's transpose buffer (transpose16<double>'s padded layout)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int set = lane >> 4, l16 = lane & 15;
  __shared__ __align__(16) uint8_t lds[NWB * 4 * ROWB];
  __shared__ double red64[NWB];
  double* dbuf = reinterpret_cast<double*>(lds + (wave * 4 + set) * ROWB);
  uint8_t* bbuf = lds + (wave * 4 + set) * ROWB;
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

  bool has[NU];
  typename Src::stash_t st[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    has[u] = gb + set + 4 * u < ge;
    if (has[u]) src.fetch(row, (int64_t)(gb + set + 4 * u) * 256 + l16 * 16, st[u]);
  }
  double v[NU][16];
  double amax = 0.0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    Raw16<TIn> r0;
    if (has[u])
      src.finish(row, (int64_t)(gb + set + 4 * u) * 256 + l16 * 16, st[u], r0);
    else
      r0.zero();
#pragma unroll
    for (int i = 0; i < 16; ++i) v[u][i] = (double)r0.get(i);
    if (rotate) {
      fwht16_regs(v[u]);
      transpose16(v[u], dbuf, l16);
      fwht16_regs(v[u]);
    } else {
      transpose16(v[u], dbuf, l16);  // the same output order either way
    }
    amax = fmax(amax, absmax16(v[u]));
    __builtin_amdgcn_sched_barrier(0);  // one group at a time: the next one's registers are not live yet
  }
  amax = wave_max(amax);  // rows without a group hold zeros
  if constexpr (WPR > 1) {
    if (lane == 0) red64[wave] = amax;
    __syncthreads();
    amax = red64[0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) amax = fmax(amax, red64[w]);
  }
  const double unscale = rotate ? 0.0625 : 1.0;  // the values above are 16 x the rotation (exact)
  const float s = (float)(amax * unscale / 127.0);
  const double s64 = (double)s;
  const double inv64 = s > 0.0f ? 1.0 / s64 : 0.0;
  const double invu = inv64 * unscale;
  constexpr double MAGIC = 6755399441055744.0;  // 1.5 * 2^52: adding it rounds to an integer (RNE)
  // A normal s is within 2^-24 of amax / 127 (relative), so no quotient
  // exceeds 127.5 and no code needs the clamp; a subnormal s can be much
  // further off, and such rows take quant_code (which clamps) throughout.
  const bool direct = s == 0.0f || s >= 0x1p-126f;

  int8_t* qr = q + row * ldq;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    // element l16 + 16 r -> byte l16 + 16 r of this row's buffer, then 16
    // contiguous bytes per lane out
    wave_lds_sync();
    bool tie = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const double f = fma(v[u][r], invu, MAGIC);
      const double d = fma(v[u][r], invu, MAGIC - f);
      tie |= !(fabs(d) < 0.5 - 1e-9);
      bbuf[l16 + 16 * r] = (uint8_t)__builtin_bit_cast(uint64_t, f);
    }
    if (__ballot((tie || !direct) && has[u])) {
      // (recomputed from an opaque copy of invu: sharing the first pass's f
      // and d would keep 64 registers live across the branch)
      double invr = invu;
      asm volatile("" : "+v"(invr));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const double f = fma(v[u][r], invr, MAGIC);
        const double d = fma(v[u][r], invr, MAGIC - f);
        if (!direct || !(fabs(d) < 0.5 - 1e-9))
          bbuf[l16 + 16 * r] = (uint8_t)quant_code(v[u][r] * unscale, s64, inv64, 127.0);
      }
    }
    wave_lds_sync();
    const uint4 w4 = *reinterpret_cast<const uint4*>(bbuf + 16 * l16);
    if (has[u]) *reinterpret_cast<uint4*>(qr + (int64_t)(gb + set + 4 * u) * 256 + l16 * 16) = w4;
    __builtin_amdgcn_sched_barrier(0);
  }
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

// int8 rows: k_rotq_i8_d up to 48 groups, k_rotq_rows above.
template <typename Src>
static hipError_t rotq_i8_from(const Src& src, int64_t rows, int groups, int rot, int8_t* q8, int64_t ldq,
                               float* scales, hipStream_t stream) {
  const dim3 block(256);
  if (groups <= 12)
    hipLaunchKernelGGL((k_rotq_i8_d<Src, 1>), dim3((unsigned)((rows + 3) / 4)), block, 0, stream, src, rows,
                       groups, rot, q8, ldq, scales);
  else if (groups <= 48)
    hipLaunchKernelGGL((k_rotq_i8_d<Src, 4>), dim3((unsigned)rows), block, 0, stream, src, rows, groups, rot, q8,
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
