// Quantized products on the gfx950 matrix cores: two-group ("ping-pong")
// schedule over a multi-stage LDS ring.
//
//   W8    C = (bf16(A') . q^T) * s[n]              bf16 MFMA 16x16x32, fp32 sums
//   W4    C = sum_g s[n,g] * (bf16(A'_g) . q_g^T)  bf16 MFMA, per-group fp32 rescale
//   W8A8  acc = qa . q^T (int32, exact); C = (float(acc) * sa[m]) * sw[n]
//                                                   i8 MFMA 16x16x64, int32 sums
//   W4A8  acc_g = qa_g . q_g^T (int32, exact per 256-group);
//         C = (sum_g s[n,g] * float(acc_g)) * sa[m]   i8 MFMA, per-group fp32 fold
//
// (tensai docs, "画像生成", section "幅とメモリ": int8 weights with one scale per
// row and the 4-bit "-q4" width; section "GPU": activations quantized on the
// device. TensorFold pull request #948: bf16 activations, fp32 sums.)
//
// Schedule. A block of 8 waves (two per SIMD) computes a BM x BN tile; the
// waves form two groups of four, one wave of each group per SIMD. K advances
// in stages of 64 elements through an LDS ring of NSTAGE stages filled with
// global_load_lds_dwordx4 (no register staging). Each stage is two half-steps
// separated by barriers; in every half-step one group runs its memory phase
// (read the stage's operand fragments from LDS into registers, issue the
// direct loads of stage k + NSTAGE - 1) while the other runs its compute phase
// (back-to-back MFMAs on fragments already in registers). Group 1 trails group
// 0 by one half-step, so on every SIMD one wave feeds the matrix unit while
// the other waits on LDS. Stage k is read by group 0 in half-step 2k and by
// group 1 in half-step 2k+1; its buffer is refilled (with stage k + NSTAGE)
// only from half-step 2k+2 on.
//
// LDS layouts (per stage; 16-byte granules; every wave-level direct load fills
// 1 KB, lane p writing granule p, so the swizzle is applied by choosing which
// global granule each lane loads). LDS has 64 banks of 4 bytes. Measured on
// gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT on probe patterns): ds_read_b128
// serves a wave in four passes of 16 lanes; lanes 0-31 and 32-63 never share
// a pass, and within a half, lane l goes with the lanes whose 4-lane block
// (l >> 2) & 7 has the same bit parity: {0-3, 12-15, 20-27} and
// {4-11, 16-19, 28-31}. A pass is conflict-free when its 16 granules are
// distinct modulo 256 bytes. In a fragment read, lane l reads row l & 15 at
// logical granule (chunk) l >> 4 (i8) or 2 * (l >> 4) + kk (bf16), so a pass
// holds rows {0-3, 12-15} at one chunk and rows {4-11} at the next; the
// swizzles below (XOR of the chunk with a function of the row) keep those
// 16 granules apart, which the plain "distinct per 16 consecutive rows"
// swizzles do not (they cost one extra pass per read, measured):
//   int8 rows of 64 B (A of W8A8, B of W8A8 and W8): granule c of row r at
//     c ^ ((r >> 2) & 2);
//   bf16 rows of 128 B (A of W8, W4): granule c of row r at c ^ ((r >> 1) & 5);
//   int4 rows of 32 B (B of W4, read 8 bytes at a time; ds_read_b64 serves
//     32 lanes per pass): granule c of row r at c ^ ((r >> 3) & 1).
// K order inside a stage: MFMA k-step kk (0, 1) of the bf16 kinds gives lane
// group g = lane/16 the K positions 16g + 8kk + [0, 8); A and B use the same
// order, so one 16-byte int8 (8-byte int4) weight read serves both k-steps.
// The i8 kind has one k-step per stage: 16g + [0, 16).
//
// W4A8 widening: the same top-nibble bytes (16 * code, exact in int8), put in
// K order by two byte permutes per 8 codes; the int32 sums of a group are
// exact (below 2^24 even with the factor 16, so also exact as fp32) and are
// folded into fp32 with s[n,g] when the group ends. The first MFMA of a group
// starts from a zero accumulator, so nothing is cleared.
//
// W4 widening: one masked AND per 8 codes moves each code to the top nibble of
// a byte and a signed-byte convert gives 16 * code, so the MFMAs sum 16x the
// products (exact in bf16 and removed by an exact 1/16 at the end). The group
// scales are applied by rescaling the single set of accumulators at group
// boundaries (see cu in the kernel).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tp {

// Row-dependent granule XORs of the LDS layouts above (load and read side).
__device__ __forceinline__ int swz_i8(int row) { return (row >> 2) & 2; }
__device__ __forceinline__ int swz_bf16(int row) { return (row >> 1) & 5; }
__device__ __forceinline__ int swz_i4(int row) { return (row >> 3) & 1; }

// Fixed-order sum of split-K partial sums plus the epilogue (gemm_skinny.hpp).
template <int KIND>
static hipError_t launch_reduce(const GemmArgs& g, int splits, hipStream_t stream);

typedef __attribute__((address_space(3))) void lds_void_t;

// Block -> tile map: each of the 8 XCDs owns one contiguous range of logical
// tiles (hardware deals blocks round-robin over XCDs), walked in groups of GM
// tile-rows so that blocks resident together on one XCD share A rows and B
// columns in that XCD's L2.
__device__ __forceinline__ void pp_map_tile(int pid, int nblk, int tiles_m, int tiles_n, int GM, int& tm, int& tn) {
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = pid & 7, idx = pid >> 3;
  const int logical = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  const int width = GM * tiles_n;
  const int group = logical / width;
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int within = logical - group * width;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

// 8 int8 codes (two dwords) -> 8 bf16 (four dwords), exact.
__device__ __forceinline__ bf16x8_t pp_widen_i8x8(uint32_t lo, uint32_t hi) {
  u32x4_t o;
  o.x = pack_bf16x2((float)(int8_t)(lo), (float)(int8_t)(lo >> 8));
  o.y = pack_bf16x2((float)(int8_t)(lo >> 16), (float)(int8_t)(lo >> 24));
  o.z = pack_bf16x2((float)(int8_t)(hi), (float)(int8_t)(hi >> 8));
  o.w = pack_bf16x2((float)(int8_t)(hi >> 16), (float)(int8_t)(hi >> 24));
  return __builtin_bit_cast(bf16x8_t, o);
}

// 8 int4 codes (one dword, code j in bits 4j..4j+3) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8_t pp_widen_i4x8(uint32_t w) {
  const int32_t v = (int32_t)w;
  u32x4_t o;
  o.x = pack_bf16x2((float)((v << 28) >> 28), (float)((v << 24) >> 28));
  o.y = pack_bf16x2((float)((v << 20) >> 28), (float)((v << 16) >> 28));
  o.z = pack_bf16x2((float)((v << 12) >> 28), (float)((v << 8) >> 28));
  o.w = pack_bf16x2((float)((v << 4) >> 28), (float)(v >> 28));
  return __builtin_bit_cast(bf16x8_t, o);
}

// 16 int4 codes (code j of w.x in bits 4j..4j+3, codes 8.. in w.y) -> 16
// int8 holding 16 * code, in code order.
__device__ __forceinline__ u32x4_t pp_widen_i4_i8x16(uint2 w) {
  const uint32_t xh = w.x & 0xF0F0F0F0u, xl = (w.x << 4) & 0xF0F0F0F0u;  // byte j: code 2j+1 / 2j, top nibble
  const uint32_t yh = w.y & 0xF0F0F0F0u, yl = (w.y << 4) & 0xF0F0F0F0u;
  u32x4_t o;
  o.x = __builtin_amdgcn_perm(xh, xl, 0x05010400u);  // bytes xl.0 xh.0 xl.1 xh.1
  o.y = __builtin_amdgcn_perm(xh, xl, 0x07030602u);  // bytes xl.2 xh.2 xl.3 xh.3
  o.z = __builtin_amdgcn_perm(yh, yl, 0x05010400u);
  o.w = __builtin_amdgcn_perm(yh, yl, 0x07030602u);
  return o;
}

// 8 int4 codes (one dword, code j in bits 4j..4j+3) -> 8 bf16 holding 16 *
// code, exact. Each code is moved to the top nibble of a byte, so a signed
// byte convert (one SDWA instruction) yields 16 * code. mk is 0xF0F0F0F0, or
// 0 to drop the codes of a group that does not take part.
__device__ __forceinline__ bf16x8_t pp_widen_i4x8_x16(uint32_t w, uint32_t mk) {
  const uint32_t hi = w & mk;         // byte j: code 2j+1 in the top nibble
  const uint32_t lo = (w << 4) & mk;  // byte j: code 2j in the top nibble
  u32x4_t o;
  o.x = pack_bf16x2((float)(int8_t)(lo), (float)(int8_t)(hi));
  o.y = pack_bf16x2((float)(int8_t)(lo >> 8), (float)(int8_t)(hi >> 8));
  o.z = pack_bf16x2((float)(int8_t)(lo >> 16), (float)(int8_t)(hi >> 16));
  o.w = pack_bf16x2((float)(int8_t)(lo >> 24), (float)(int8_t)(hi >> 24));
  return __builtin_bit_cast(bf16x8_t, o);
}

template <int KIND, int BM, int BN, int WM, int WN, int NSTAGE>
struct PPCfg {
  static constexpr bool I8 = KIND == GEMM_W8A8 || KIND == GEMM_W4A8;  // int8 activations, i8 MFMA
  static constexpr bool B4 = KIND == GEMM_W4 || KIND == GEMM_W4A8;    // packed int4 weights
  static constexpr int NW = 8, NT = 512;
  static constexpr int NWN = BN / WN;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int AROW = I8 ? 64 : 128;              // A bytes per row per stage
  static constexpr int BROW = B4 ? 32 : 64;               // B bytes per row per stage
  static constexpr int A_STAGE = BM * AROW, B_STAGE = BN * BROW, STAGE = A_STAGE + B_STAGE;
  static constexpr int A_LOADS = A_STAGE / 1024, LOADS = (A_STAGE + B_STAGE) / 1024;
  static constexpr int HALF = (LOADS + 1) / 2;            // loads owned by each group per stage
  static constexpr int LPW = (HALF + 3) / 4;              // loads per wave per stage
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static_assert((BM / WM) * (BN / WN) == NW, "the tile must split into 8 waves");
  static_assert(A_STAGE % 1024 == 0 && B_STAGE % 1024 == 0, "a stage must be whole 1 KB loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KB");
  static_assert(NSTAGE >= 3, "the two-group schedule needs at least three stages");
  static_assert(LPW * (NSTAGE - 2) < 64, "vmcnt range");
};

// PARTIAL: the block computes the K stages [blockIdx.y * sps, ...) of its
// tile and writes the raw sums (int32 for W8A8, unscaled fp32 for W8, scaled
// fp32 for W4 and W4A8, the latter before the activation scale) to part[blockIdx.y][m][n] instead of C; k_qgemm_reduce adds the
// splits in order and applies the epilogue. sps is a multiple of 4 (whole
// 256-groups).
template <int KIND, int BM, int BN, int WM, int WN, int NSTAGE, bool OUT_BF16, bool ACC_OUT, bool PARTIAL,
          int EWN = 0, bool LORA = false>
__global__ __launch_bounds__(512, 1) void k_qgemm_pp(
    const uint8_t* __restrict__ A, int64_t lda_bytes, const uint8_t* __restrict__ B, int64_t ldb_bytes,
    const float* __restrict__ sw, const float* __restrict__ sa, int M, int N, int K, void* __restrict__ Cv,
    int64_t ldc, int32_t* __restrict__ acc_out, int64_t ld_acc, int tiles_m, int tiles_n, int gm, int sps,
    void* __restrict__ part, LoraEpi lora) {
  using Cfg = PPCfg<KIND, BM, BN, WM, WN, NSTAGE>;
  constexpr bool I8 = Cfg::I8;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, NWN = Cfg::NWN;
  constexpr int AROW = Cfg::AROW, BROW = Cfg::BROW, STAGE = Cfg::STAGE, A_STAGE = Cfg::A_STAGE;
  constexpr int LOADS = Cfg::LOADS, A_LOADS = Cfg::A_LOADS, HALF = Cfg::HALF, LPW = Cfg::LPW;

  __shared__ __align__(1024) uint8_t ring[Cfg::LDS_BYTES];

  int tm, tn;
  pp_map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, gm, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // waves 0-3: group 0, 4-7: group 1 (one of each per SIMD)
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;

  // Direct-load slots of this wave: group g owns loads [g*HALF, g*HALF + HALF)
  // of each stage; surplus slots repeat the group's last load (same bytes to
  // the same place).
  const uint8_t* src[LPW];
  int dst[LPW];
  int kbytes[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int lim = min(grp * HALF + HALF, LOADS) - 1;
    const int L = min(grp * HALF + (wave & 3) * LPW + i, lim);
    if (L < A_LOADS) {
      if constexpr (I8) {  // 16 rows x 64 B
        const int row = L * 16 + (lane >> 2), c = (lane & 3) ^ swz_i8(row);
        src[i] = A + (int64_t)min(m0 + row, M - 1) * lda_bytes + c * 16;
      } else {  // 8 rows x 128 B
        const int row = L * 8 + (lane >> 3), c = (lane & 7) ^ swz_bf16(row);
        src[i] = A + (int64_t)min(m0 + row, M - 1) * lda_bytes + c * 16;
      }
      dst[i] = L * 1024;
      kbytes[i] = AROW;
    } else {
      const int LB = L - A_LOADS;
      if constexpr (Cfg::B4) {  // 32 rows x 32 B
        const int row = LB * 32 + (lane >> 1), c = (lane & 1) ^ swz_i4(row);
        src[i] = B + (int64_t)min(n0 + row, N - 1) * ldb_bytes + c * 16;
      } else {  // 16 rows x 64 B
        const int row = LB * 16 + (lane >> 2), c = (lane & 3) ^ swz_i8(row);
        src[i] = B + (int64_t)min(n0 + row, N - 1) * ldb_bytes + c * 16;
      }
      dst[i] = A_STAGE + LB * 1024;
      kbytes[i] = BROW;
    }
  }
  const int ks0 = PARTIAL ? blockIdx.y * sps : 0;             // first stage of this block's K range
  const int KS = PARTIAL ? min(sps, (K >> 6) - ks0) : K >> 6;  // stages of 64 K in the range
#pragma unroll
  for (int i = 0; i < LPW; ++i) src[i] += (int64_t)ks0 * kbytes[i];
  auto issue_stage = [&](int ks) {
    uint8_t* base = ring + (ks % NSTAGE) * STAGE;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + (int64_t)ks * kbytes[i]), (lds_void_t*)(base + dst[i]),
                                       16, 0, 0);
  };

  typedef typename std::conditional<I8, i32x4_t, f32x4_t>::type acc_t;
  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  // W4 keeps one accumulator per output, expressed in units of the scale of
  // the group being summed (cu, per column): the raw products of group g are
  // added as they come, and on entering group g+1 the accumulator is
  // multiplied by s[g]/s[g+1]. A group whose scale is zero, or more than 2^64
  // times smaller than the largest scale taken so far in the column (cmx:
  // every earlier group's sum is then held at most 2^64 times its own size,
  // so the running sum cannot overflow through the rescales however the
  // scales step down), has its codes masked off; a column with a skipped
  // nonzero scale is recomputed exactly in the epilogue (fix bit).
  float cu[KIND == GEMM_W4 ? FN : 1];
  float cmx[KIND == GEMM_W4 ? FN : 1];
  uint32_t mk[KIND == GEMM_W4 ? FN : 1];
  int fix = 0;
  // W4A8: the fp32 sum of the folded groups (the int32 acc holds one group).
  f32x4_t tot[KIND == GEMM_W4A8 ? FM : 1][KIND == GEMM_W4A8 ? FN : 1];
  if constexpr (KIND == GEMM_W4A8) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) tot[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int r16 = lane & 15, g4 = lane >> 4;
  const int groups = K >> 8;

  // Fragments of one stage, held in registers between the memory phase and
  // the compute phase.
  constexpr int NKK = I8 ? 1 : 2;
  u32x4_t fa[NKK][FM];
  typedef typename std::conditional<Cfg::B4, uint2, u32x4_t>::type braw_t;
  braw_t fb[FN];
  // Early widening (W8, W4, W4A8): the first EWF weight fragments are widened
  // at the end of the memory phase, where this wave's VALU work runs beside
  // the other group's MFMAs; the rest in the compute phase, where it
  // serializes with this wave's own. EWN balances the two phases.
  constexpr int EWF = (KIND == GEMM_W8 || KIND == GEMM_W4 || KIND == GEMM_W4A8) ? (EWN < FN ? EWN : FN) : 0;
  constexpr bool EW = EWF > 0 && KIND != GEMM_W4A8;
  bf16x8_t wb[EW ? EWF : 1][2];
  u32x4_t wq[KIND == GEMM_W4A8 && EWF > 0 ? EWF : 1];  // W4A8: int8 (16 * code) fragments
  float s_nx[KIND == GEMM_W4 ? FN : 1];  // W4: scales of the next group
  float s_grp[KIND == GEMM_W4A8 ? FN : 1];  // W4A8: scales of the group being folded
  // W4A8: fold the int32 sums of the group that just ended into tot, in the
  // memory phase of the next group's first stage (beside the other group's
  // MFMAs), and once after the loop.
  auto fold = [&]() {
    if constexpr (KIND == GEMM_W4A8) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) tot[i][j] += s_grp[j] * __builtin_convertvector(acc[i][j], f32x4_t);
    }
  };

  // W4: switch the accumulators to the units of the group whose scales are
  // in s_nx (see cu above).
  auto enter_group = [&]() {
    if constexpr (KIND == GEMM_W4) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float s = s_nx[j];
      const bool use = (s != 0.f) && (cmx[j] <= s * 0x1p64f);  // false for NaN
      const float r = use ? cu[j] / s : 1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] *= r;
      cu[j] = use ? s : cu[j];
      cmx[j] = use ? fmaxf(cmx[j], s) : cmx[j];
      mk[j] = use ? 0xF0F0F0F0u : 0u;
      fix |= (!use && s != 0.f) ? (1 << j) : 0;
    }
    }
  };

  auto mem_phase = [&](int ks) {
    if constexpr (KIND == GEMM_W4A8) {
      if ((ks & 3) == 0 && ks > 0) fold();
    }
    const uint8_t* as = ring + (ks % NSTAGE) * STAGE;
    const uint8_t* bs = as + A_STAGE;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn0 + j * 16 + r16;
      if constexpr (Cfg::B4)
        fb[j] = *reinterpret_cast<const uint2*>(bs + row * 32 + ((((g4 >> 1) ^ swz_i4(row)) << 4) | ((g4 & 1) << 3)));
      else
        fb[j] = *reinterpret_cast<const u32x4_t*>(bs + row * 64 + ((g4 ^ swz_i8(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm0 + i * 16 + r16;
      if constexpr (I8) {
        fa[0][i] = *reinterpret_cast<const u32x4_t*>(as + row * 64 + ((g4 ^ swz_i8(row)) << 4));
      } else {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          fa[kk][i] = *reinterpret_cast<const u32x4_t*>(as + row * 128 + (((2 * g4 + kk) ^ swz_bf16(row)) << 4));
      }
    }
    if constexpr (KIND == GEMM_W4) {
      if ((ks & 3) == 3 && ks + 1 < KS) {  // last stage of a 256-group: fetch the next group's scales
        const int g = ((ks0 + ks) >> 2) + 1;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = min(n0 + wn0 + j * 16 + r16, N - 1);
          s_nx[j] = sw[(int64_t)col * groups + g];
        }
      }
    }
    if constexpr (KIND == GEMM_W4A8) {
      if ((ks & 3) == 3) {  // last stage of a 256-group: its scales, for the fold
        const int g = (ks0 + ks) >> 2;
#pragma unroll
        for (int j = 0; j < FN; ++j) s_grp[j] = sw[(int64_t)min(n0 + wn0 + j * 16 + r16, N - 1) * groups + g];
      }
    }
    if (ks + NSTAGE - 1 < KS) issue_stage(ks + NSTAGE - 1);
    if constexpr (KIND == GEMM_W4A8 && EWF > 0) {
#pragma unroll
      for (int j = 0; j < EWF; ++j) wq[j] = pp_widen_i4_i8x16(fb[j]);
    }
    if constexpr (EW) {
      __builtin_amdgcn_s_waitcnt(LGKMCNT0_ENCODE);
#pragma unroll
      for (int j = 0; j < EWF; ++j) {
        if constexpr (KIND == GEMM_W4) {
          wb[j][0] = pp_widen_i4x8_x16(fb[j].x, mk[j]);
          wb[j][1] = pp_widen_i4x8_x16(fb[j].y, mk[j]);
        } else {
          wb[j][0] = pp_widen_i8x8(fb[j].x, fb[j].y);
          wb[j][1] = pp_widen_i8x8(fb[j].z, fb[j].w);
        }
      }
    }
  };

  auto compute_phase = [&](int ks) {
    if constexpr (KIND == GEMM_W8A8) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, fa[0][i]),
                                                             __builtin_bit_cast(i32x4_t, fb[j]), acc[i][j], 0, 0, 0);
    } else if constexpr (KIND == GEMM_W4A8) {
      // A group's first stage starts its sums from zero (the previous group's
      // were folded in this stage's memory phase).
      const bool first = (ks & 3) == 0;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        u32x4_t bw;
        if (j < EWF)
          bw = wq[j];
        else
          bw = pp_widen_i4_i8x16(fb[j]);
        const i32x4_t b = __builtin_bit_cast(i32x4_t, bw);
        if (first) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, fa[0][i]), b,
                                                               i32x4_t{0, 0, 0, 0}, 0, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < FM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, fa[0][i]), b, acc[i][j],
                                                               0, 0, 0);
        }
      }
    } else if constexpr (EW) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bf16x8_t b0, b1;
        if (j < EWF) {
          b0 = wb[j][0];
          b1 = wb[j][1];
        } else if constexpr (KIND == GEMM_W4) {
          b0 = pp_widen_i4x8_x16(fb[j].x, mk[j]);
          b1 = pp_widen_i4x8_x16(fb[j].y, mk[j]);
        } else {
          b0 = pp_widen_i8x8(fb[j].x, fb[j].y);
          b1 = pp_widen_i8x8(fb[j].z, fb[j].w);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[0][i]), b0, acc[i][j],
                                                               0, 0, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[1][i]), b1, acc[i][j],
                                                               0, 0, 0);
      }
    } else {
      // W8: the widening of fragment j+1 is interleaved with the MFMAs of
      // fragment j, so one wave's VALU work runs while its matrix
      // instructions execute (measured 3% faster at 4096x12288x3072; the same
      // interleave made the int4 kernel slower, which keeps the plain order).
      auto widen = [&](int j, bf16x8_t& b0, bf16x8_t& b1) {
        if constexpr (KIND == GEMM_W4) {
          b0 = pp_widen_i4x8_x16(fb[j].x, mk[j]);
          b1 = pp_widen_i4x8_x16(fb[j].y, mk[j]);
        } else {
          b0 = pp_widen_i8x8(fb[j].x, fb[j].y);
          b1 = pp_widen_i8x8(fb[j].z, fb[j].w);
        }
      };
      bf16x8_t nb0, nb1;
      widen(0, nb0, nb1);
      if constexpr (KIND == GEMM_W8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bf16x8_t b0 = nb0, b1 = nb1;
        if constexpr (KIND == GEMM_W8) {
          if (j + 1 < FN) widen(j + 1, nb0, nb1);
        } else if (j > 0) {
          widen(j, b0, b1);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[0][i]), b0, acc[i][j],
                                                               0, 0, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[1][i]), b1, acc[i][j],
                                                               0, 0, 0);
      }
      if constexpr (KIND == GEMM_W8) {
#pragma unroll
        for (int t = 0; t < 2 * FM * FN; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // then up to two VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (KIND == GEMM_W4) {
      if ((ks & 3) == 3 && ks + 1 < KS) enter_group();
    }
  };

  // Epilogue scales, fetched before the main loop: their latency is hidden by
  // the loop, and no load is left to interleave with the output stores (on
  // gfx9 loads and stores share one completion counter, so a load waited on
  // between stores would drain every store before it).
  float ep_sw[Cfg::B4 ? 1 : FN];
  float ep_sa[I8 ? FM : 1][4];
  if constexpr (!Cfg::B4 && !PARTIAL) {
#pragma unroll
    for (int j = 0; j < FN; ++j) ep_sw[j] = sw[min(n0 + wn0 + j * 16 + r16, N - 1)];
  }
  if constexpr (I8 && !PARTIAL) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ep_sa[i][r] = sa[min(m0 + wm0 + i * 16 + g4 * 4 + r, M - 1)];
  }

  if constexpr (KIND == GEMM_W4) {  // scales of the first group of the K range
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      cu[j] = 0.f;
      cmx[j] = 0.f;
      s_nx[j] = sw[(int64_t)min(n0 + wn0 + j * 16 + r16, N - 1) * groups + (ks0 >> 2)];
    }
  }

  // Stage ks+1 has landed once at most the loads of stages ks+2 .. ks+NSTAGE-1
  // (issued after it by this wave) are outstanding.
  auto wait_next = [&](int ks) {
    if (ks + 1 >= KS) return;
    if (ks + NSTAGE - 1 < KS) {
      __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(LPW * (NSTAGE - 2)));
    } else {
      __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(0));
    }
  };

  // Prologue: stages 0 .. NSTAGE-2 in flight, stage 0 landed everywhere.
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KS) issue_stage(s);
  if (NSTAGE - 2 < KS) {
    __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(LPW * (NSTAGE - 2)));
  } else {
    __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(0));
  }
  barrier_only();
  if constexpr (KIND == GEMM_W4) enter_group();

  // Both groups run the same body (memory phase, barrier, compute phase,
  // barrier); group 1 starts one barrier later and group 0 ends one barrier
  // later, so in every half-step the groups are in opposite phases. Barrier
  // 2ks+1 separates group 0's M(ks) from its C(ks) and group 1's C(ks-1) from
  // its M(ks); stage ks+1 must have landed (in both groups' halves) before
  // barrier 2ks+2, after which group 0 reads it.
  if (grp == 1) barrier_only();
  for (int ks = 0; ks < KS; ++ks) {
    mem_phase(ks);
    if (grp == 1) wait_next(ks);
    // The LDS reads of the memory phase must be complete before any wave can
    // pass the barrier and refill the buffer they read.
    __builtin_amdgcn_s_waitcnt(LGKMCNT0_ENCODE);
    barrier_only();
    compute_phase(ks);
    if (grp == 0) wait_next(ks);
    barrier_only();
  }
  if (grp == 0) barrier_only();
  fold();

  // W4 output of accumulator element (i, j, r): back from units of cu[j]
  // (and from the 16x codes); a column with a skipped group is summed again
  // exactly, group by group, straight from A and the codes (never taken for
  // scales within 2^64 of each other along a row).
  auto w4_value = [&](int i, int j, int r) -> float {
    if (!((fix >> j) & 1)) return (acc[i][j][r] * 0.0625f) * cu[j];
    const int row = m0 + wm0 + i * 16 + g4 * 4 + r, col = n0 + wn0 + j * 16 + r16;
    const uint16_t* arow = reinterpret_cast<const uint16_t*>(A + (int64_t)row * lda_bytes);
    const uint8_t* brow = B + (int64_t)col * ldb_bytes;
    float total = 0.f;
    for (int g = ks0 >> 2; g < (ks0 + KS) >> 2; ++g) {
      const float sg = sw[(int64_t)col * groups + g];
      if (sg == 0.f) continue;
      float dot = 0.f;
      for (int k = g * 256; k < g * 256 + 256; ++k) {
        const int code = ((int)((uint32_t)brow[k >> 1] << ((k & 1) ? 24 : 28))) >> 28;
        dot += __builtin_bit_cast(float, (uint32_t)arow[k] << 16) * (float)code;
      }
      total += sg * dot;
    }
    return total;
  };

  if constexpr (PARTIAL) {
    // Raw sums of this K range, [split][m][n] with row pitch N.
    __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(0));
    typedef typename std::conditional<KIND == GEMM_W8A8, int32_t, float>::type part_t;
    part_t* pbase = reinterpret_cast<part_t*>(part) + (int64_t)blockIdx.y * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm0 + i * 16 + g4 * 4 + r;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn0 + j * 16 + r16;
          if (col >= N) continue;
          if constexpr (KIND == GEMM_W4)
            pbase[(int64_t)row * N + col] = w4_value(i, j, r);
          else if constexpr (KIND == GEMM_W4A8)
            pbase[(int64_t)row * N + col] = tot[i][j][r] * 0.0625f;
          else
            pbase[(int64_t)row * N + col] = acc[i][j][r];
        }
      }
    return;
  }

  // Epilogue: lane l of a 16x16 tile holds rows 4*(l/16)+r, column l%16.
  // Every load this wave issued has completed here; waiting once up front
  // keeps the compiler from re-waiting on the preloaded scales between
  // stores. Interior tiles store without bounds checks.
  __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(0));
  auto value = [&](int i, int j, int r) -> float {
    if constexpr (KIND == GEMM_W8A8) {
      return ((float)acc[i][j][r] * ep_sa[i][r]) * ep_sw[j];
    } else if constexpr (KIND == GEMM_W4A8) {
      return (tot[i][j][r] * 0.0625f) * ep_sa[i][r];
    } else if constexpr (KIND == GEMM_W8) {
      return acc[i][j][r] * ep_sw[j];
    } else {
      return w4_value(i, j, r);
    }
  };
  typedef typename std::conditional<OUT_BF16, __bf16, float>::type out_t;
  if constexpr (LORA) {
    // LoRA side path in the store (fp32 C): out = fma(alpha, L, value) with
    // L = T . lora_b^T for this fragment, on the same MFMA sequence as the
    // standalone up-projection (T split exactly into three bf16 parts; the
    // two small parts first), so both paths give the same bits. The wave's
    // lora_b fragments are loaded once; T rows are fetched one fragment row
    // ahead so that no load latency sits between two fragments.
    static_assert(KIND == GEMM_W8A8, "the side path rides in the W8A8 store only");
    const bool two = lora.r > 32;  // 32-deep steps over the rank: 1 or 2
    // The product's values first, into the accumulators' registers (the
    // epilogue scales are then dead, which makes room for the side path).
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_bit_cast(acc_t, f32x4_t{value(i, j, 0), value(i, j, 1), value(i, j, 2), value(i, j, 3)});
    bf16x8_t lb[FN][2];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn0 + j * 16 + r16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int j0 = 32 * s + 8 * g4;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (col < N && j0 < lora.r) {
          const uint16_t* brow = lora.b + (int64_t)col * lora.ldb + j0;
          if (j0 + 8 <= lora.r) {
            w = *reinterpret_cast<const u32x4_t*>(brow);
          } else {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const uint32_t lo = j0 + e < lora.r ? brow[e] : 0u, hi = j0 + e + 1 < lora.r ? brow[e + 1] : 0u;
              w[e >> 1] = lo | (hi << 16);
            }
          }
        }
        lb[j][s] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    auto fetch_t = [&](int i, float (&v)[2][8]) {
      const int trow = m0 + wm0 + i * 16 + r16;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (trow < M && (s == 0 || two)) {
          load8(lora.t + (int64_t)trow * 64 + 32 * s + 8 * g4, v[s]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[s][e] = 0.f;
        }
      }
    };
    float tv[2][8];
    fetch_t(0, tv);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      bf16x8_t th[2], tm[2], tl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) split3_bf16(tv[s], th[s], tm[s], tl[s]);
      if (i + 1 < FM) fetch_t(i + 1, tv);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn0 + j * 16 + r16;
        f32x4_t L = {0.f, 0.f, 0.f, 0.f};
        L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl[0], lb[j][0], L, 0, 0, 0);
        L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tm[0], lb[j][0], L, 0, 0, 0);
        if (two) {
          L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl[1], lb[j][1], L, 0, 0, 0);
          L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tm[1], lb[j][1], L, 0, 0, 0);
        }
        L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th[0], lb[j][0], L, 0, 0, 0);
        if (two) L = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th[1], lb[j][1], L, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm0 + i * 16 + g4 * 4 + r;
          if (row < M && col < N)
            reinterpret_cast<float*>(Cv)[(int64_t)row * ldc + col] =
                fmaf(lora.alpha, L[r], __builtin_bit_cast(f32x4_t, acc[i][j])[r]);
        }
      }
    }
    return;
  }
  const int row0 = m0 + wm0 + g4 * 4, col0 = n0 + wn0 + r16;
  out_t* cbase = reinterpret_cast<out_t*>(Cv) + (int64_t)row0 * ldc + col0;
  int32_t* abase = ACC_OUT ? acc_out + (int64_t)row0 * ld_acc + col0 : nullptr;
  if ((m0 + BM <= M) && (n0 + BN <= N)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        out_t* crow = cbase + (int64_t)(i * 16 + r) * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          crow[j * 16] = (out_t)value(i, j, r);
          if constexpr (ACC_OUT) abase[(int64_t)(i * 16 + r) * ld_acc + j * 16] = acc[i][j][r];
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (row0 + i * 16 + r >= M) continue;
        out_t* crow = cbase + (int64_t)(i * 16 + r) * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (col0 + j * 16 >= N) continue;
          crow[j * 16] = (out_t)value(i, j, r);
          if constexpr (ACC_OUT) abase[(int64_t)(i * 16 + r) * ld_acc + j * 16] = acc[i][j][r];
        }
      }
  }
}

// splits > 1: K split over blockIdx.y into ranges of sps stages, partial sums
// in g.part, then k_qgemm_reduce (gemm_skinny.hpp).
template <int KIND, int BM, int BN, int WM, int WN, int NSTAGE, int EWN = 0>
static hipError_t launch_pp(const GemmArgs& g, hipStream_t stream, int gm = 8, int splits = 1, int sps = 0) {
  const int tiles_m = (int)((g.m + BM - 1) / BM), tiles_n = (int)((g.n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)splits), block(512);
  const int64_t lda_bytes = g.lda * (PPCfg<KIND, BM, BN, WM, WN, NSTAGE>::I8 ? 1 : 2);
  const uint8_t* a = (const uint8_t*)g.a;
  const uint8_t* b = (const uint8_t*)g.b;
#define TP_LAUNCH_PP(OB, AO, PA)                                                                                  \
  hipLaunchKernelGGL((k_qgemm_pp<KIND, BM, BN, WM, WN, NSTAGE, OB, AO, PA, EWN>), grid, block, 0, stream, a, lda_bytes, b, \
                     g.ldb, g.w_scales, g.a_scales, (int)g.m, (int)g.n, (int)g.k, g.c, g.ldc, g.acc_out, g.ld_acc,    \
                     tiles_m, tiles_n, gm, sps, g.part, g.lora)
  if (splits > 1) {
    TP_LAUNCH_PP(false, false, true);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce<KIND>(g, splits, stream);
  }
  if constexpr (KIND == GEMM_W8A8) {
    if (g.lora.t) {  // fp32 C, no int32 output (checked by the caller)
      hipLaunchKernelGGL((k_qgemm_pp<KIND, BM, BN, WM, WN, NSTAGE, false, false, false, EWN, true>), grid, block, 0,
                         stream, a, lda_bytes, b, g.ldb, g.w_scales, g.a_scales, (int)g.m, (int)g.n, (int)g.k, g.c,
                         g.ldc, g.acc_out, g.ld_acc, tiles_m, tiles_n, gm, sps, g.part, g.lora);
      return hipGetLastError();
    }
  }
  if (KIND == GEMM_W8A8 && g.acc_out) {
    if (g.c_bf16) TP_LAUNCH_PP(true, true, false); else TP_LAUNCH_PP(false, true, false);
  } else {
    if (g.c_bf16) TP_LAUNCH_PP(true, false, false); else TP_LAUNCH_PP(false, false, false);
  }
#undef TP_LAUNCH_PP
  return hipGetLastError();
}

}  // namespace tp
