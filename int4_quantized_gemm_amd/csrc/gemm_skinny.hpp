// Quantized products with few activation rows (small M).
//
// With M up to a few dozen rows the product is bound by reading the weight
// codes once from HBM, so the codes skip LDS: every wave loads its 16-row
// weight fragments straight into registers in MFMA operand order and keeps two
// 256-groups of them in flight. The block's activation rows for its K range
// are staged once in LDS (rows past M are zero). K is split across blocks so
// that all CUs stream a share of the weights; each split writes its partial
// sums (fp32, or int32 for W8A8) to the workspace, and k_qgemm_reduce adds the
// splits in split order (a fixed order, so the bytes of C do not depend on
// timing) and applies the epilogue of the method:
//   W8    C = (bf16(A') . q^T) * s[n]
//   W4    C = sum_g s[n,g] * (bf16(A'_g) . q_g^T), folded per 256-group
//   W8A8  acc = qa . q^T (int32, exact); C = (float(acc) * sa[m]) * sw[n]
//   W4A8  (multi-stage kernel only) C = (sum_g s[n,g] * float(acc_g)) * sa[m]
// (tensai docs, "画像生成", section "幅とメモリ" for the weight formats,
// section "GPU" for the per-token activation codes.)
//
// Lane l of a wave owns weight row 16j + l % 16 of fragment j and the 16
// bytes at 64t + 16 (l / 16) of each 64-byte piece t of that row's 256-group.
// The two MFMA operands only need to agree on which K index each lane holds,
// so the K order inside a piece follows the load:
//   W8A8 (i8 16x16x64):  piece t, lane group g: K 64t + 16g + [0, 16).
//   W8 (bf16 16x16x32):  the 16 codes split in halves h, one MFMA each:
//                        K 64t + 16g + 8h + [0, 8).
//   W4 (bf16 16x16x32):  a piece holds nibbles K 128t + 32g + [0, 32); dword d
//                        feeds one MFMA with K 128t + 32g + 8d + [0, 8).
// The activation fragment of the same MFMA reads those K indices from LDS.
#pragma once

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "gemm_pp.hpp"
#include "kernels.hpp"

namespace tp {

template <int KIND>
struct SkTraits {
  static constexpr int AB = KIND == GEMM_W8A8 ? 1 : 2;     // activation bytes per element
  static constexpr int WBG = KIND == GEMM_W4 ? 128 : 256;  // code bytes per weight row per 256-group
  static constexpr int LPG = WBG / 64;                     // 16-byte loads per lane per fragment per group
};

// Column XOR of activation row r (0-15) in LDS: r with bit 3 flipped when
// bit 2 is set (see the activation staging in k_qgemm_skinny).
__device__ __forceinline__ int sk_swz(int r) { return r ^ ((r << 1) & 8); }

constexpr int SK_NW = 4;                    // waves per block
constexpr int SK_FNW = 2;                   // 16-row weight fragments per wave
constexpr int SK_BN = SK_NW * 16 * SK_FNW;  // weight rows per block
constexpr int SK_DG = 2;                // 256-groups of codes in flight per wave

template <int KIND, int FM, bool OUT_BF16, bool ACC_OUT, bool PARTIAL>
__global__ __launch_bounds__(SK_NW * 64) void k_qgemm_skinny(const uint8_t* __restrict__ A, int64_t lda_bytes,
                                                      const uint8_t* __restrict__ B, int64_t ldb,
                                                      const float* __restrict__ sw, const float* __restrict__ sa,
                                                      int M, int N, int K, void* __restrict__ C, int64_t ldc,
                                                      int32_t* __restrict__ acc_out, int64_t ld_acc,
                                                      void* __restrict__ part, int nb, int splits, int gps) {
  using T = SkTraits<KIND>;
  constexpr int MR = 16 * FM;
  constexpr bool I8 = KIND == GEMM_W8A8;
  using acc_t = typename std::conditional<I8, i32x4_t, f32x4_t>::type;
  extern __shared__ __align__(16) uint8_t sk_lds[];

  const int pid = blockIdx.x;
  const int nbi = pid % nb;
  const int rest = pid / nb;
  const int ks = rest % splits;
  const int mbi = rest / splits;
  const int G = K >> 8;
  const int g0 = ks * gps;
  const int ng = min(gps, G - g0);
  const int m0 = mbi * MR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nw0 = nbi * SK_BN + wave * 16 * SK_FNW;

  const uint8_t* wrow[SK_FNW];
  int ncol[SK_FNW];
#pragma unroll
  for (int j = 0; j < SK_FNW; ++j) {
    ncol[j] = nw0 + 16 * j + r16;
    const int n = min(ncol[j], N - 1);
    wrow[j] = B + (int64_t)n * ldb + (int64_t)g0 * T::WBG + 16 * g4;
  }

  u32x4_t wr[SK_DG][SK_FNW][T::LPG];
  auto load_group = [&](u32x4_t (&dst)[SK_FNW][T::LPG], int gi) {
#pragma unroll
    for (int j = 0; j < SK_FNW; ++j)
#pragma unroll
      for (int t = 0; t < T::LPG; ++t)
        dst[j][t] = *reinterpret_cast<const u32x4_t*>(wrow[j] + (int64_t)gi * T::WBG + 64 * t);
  };

  // Activation rows m0 .. m0+MR-1 (clamped to M-1: rows past M only feed
  // output rows that are never stored), K range of this split, into LDS with
  // direct-to-LDS loads. LDS slot (row r, 16-byte column c) sits at
  // r * cpr + (c ^ sk_swz(r & 15)). Rows are whole multiples of 256 bytes, so a
  // slot's bank group is its column modulo 16. A fragment read has lane l
  // read row l & 15 at a column that grows by 1 (W8A8), 2 (W8) or 4 (W4)
  // from lane group l >> 4 to the next, and ds_read_b128 serves rows
  // {0-3, 12-15} of one lane group with rows {4-11} of the next in one pass
  // (gfx950, measured): sk_swz sends the first set to bank groups 0-7 and the
  // second to 8-15 for all three steps. Each wave instruction fills 64
  // consecutive slots; the total is a multiple of 256 slots, so every wave
  // instruction is whole.
  const int cpr = ng * 256 * T::AB / 16;  // 16-byte columns per row, a multiple of 16
  {
    const int total = MR * cpr;  // a multiple of 256
    const uint8_t* abase = A + (int64_t)g0 * 256 * T::AB;
    const int s = wave * 64 + lane;
    int r = s / cpr, p = s - r * cpr;
    for (int s0 = wave * 64; s0 < total; s0 += SK_NW * 64) {
      const int c = p ^ sk_swz(r & 15);
      const int m = min(m0 + r, M - 1);
      __builtin_amdgcn_global_load_lds((const void*)(abase + (int64_t)m * lda_bytes + c * 16),
                                       (lds_void_t*)(sk_lds + s0 * 16), 16, 0, 0);
      p += SK_NW * 64;
      while (p >= cpr) {
        p -= cpr;
        ++r;
      }
    }
    // W4: the split's group scales of the block's SK_BN weight rows join the
    // stage (slot col * ng + g after the activations, one dword per lane), so
    // no group waits on a scale load of its own. SK_BN * ng is a multiple of
    // 64, so every wave instruction is whole.
    if constexpr (KIND == GEMM_W4) {
      const int nsc = SK_BN * ng;
      for (int s0 = wave * 64; s0 < nsc; s0 += SK_NW * 64) {
        const int e = s0 + lane, col = e / ng, gg = e - col * ng;
        const int n = min(nbi * SK_BN + col, N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(sw + (int64_t)n * G + g0 + gg),
                                         (lds_void_t*)(sk_lds + (int64_t)total * 16 + s0 * 4), 4, 0, 0);
      }
    }
  }
  // The first weight groups go out after the activation stage, so the wait
  // for the stage leaves them in flight (a wave's loads complete in issue
  // order) until the first products need them.
#pragma unroll
  for (int d = 0; d < SK_DG; ++d)
    if (d < ng) load_group(wr[d], d);
  constexpr int GL = SK_FNW * T::LPG;  // loads per weight group
  static_assert(SK_DG == 2 && 2 * GL < 64, "vmcnt range");
  if (ng >= 2)
    __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(2 * GL));
  else
    __builtin_amdgcn_s_waitcnt(VMCNT_ENCODE(GL));
  barrier_only();  // no fence: it would wait for the weight loads too

  acc_t acc[FM][SK_FNW];
  f32x4_t tot[KIND == GEMM_W4 ? FM : 1][SK_FNW];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < SK_FNW; ++j) {
      acc[i][j] = acc_t{};
      if constexpr (KIND == GEMM_W4) tot[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // Fragment rows 16i + r16: all of a lane's reads share r16 & 15 = r16.
  const int rowbytes = cpr * 16;
  const uint8_t* arow = sk_lds + r16 * rowbytes;
  auto afrag = [&](int i, int elem) -> u32x4_t {
    const int c = (elem * T::AB) >> 4;
    return *reinterpret_cast<const u32x4_t*>(arow + i * 16 * rowbytes + ((c ^ sk_swz(r16)) << 4));
  };

  auto compute_group = [&](const u32x4_t (&w)[SK_FNW][T::LPG], int gi) {
    const int kl = gi * 256;
    if constexpr (I8) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4_t a[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = afrag(i, kl + 64 * t + 16 * g4);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < SK_FNW; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a[i]),
                                                               __builtin_bit_cast(i32x4_t, w[j][t]), acc[i][j], 0, 0,
                                                               0);
      }
    } else if constexpr (KIND == GEMM_W8) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8_t b[SK_FNW];
#pragma unroll
          for (int j = 0; j < SK_FNW; ++j) {
            // Opaque copies: without them the compiler splits the in-flight
            // code words into one register per byte.
            uint32_t lo = h == 0 ? w[j][t].x : w[j][t].z, hi = h == 0 ? w[j][t].y : w[j][t].w;
            asm volatile("" : "+v"(lo), "+v"(hi));
            b[j] = pp_widen_i8x8(lo, hi);
          }
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const u32x4_t a = afrag(i, kl + 64 * t + 16 * g4 + 8 * h);
#pragma unroll
            for (int j = 0; j < SK_FNW; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b[j], acc[i][j],
                                                                   0, 0, 0);
          }
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bf16x8_t b[SK_FNW];
#pragma unroll
          for (int j = 0; j < SK_FNW; ++j) {
            const uint32_t word = d == 0 ? w[j][t].x : d == 1 ? w[j][t].y : d == 2 ? w[j][t].z : w[j][t].w;
            b[j] = pp_widen_i4x8_x16(word, 0xF0F0F0F0u);  // 16 x code (exact)
          }
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const u32x4_t a = afrag(i, kl + 128 * t + 32 * g4 + 8 * d);
#pragma unroll
            for (int j = 0; j < SK_FNW; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), b[j], acc[i][j],
                                                                   0, 0, 0);
          }
        }
    }
  };

  for (int gb = 0; gb < ng; gb += SK_DG) {
#pragma unroll
    for (int d = 0; d < SK_DG; ++d) {
      const int gi = gb + d;
      if (gi < ng) {
        float sg[SK_FNW];
        if constexpr (KIND == GEMM_W4) {
          const float* ssc = reinterpret_cast<const float*>(sk_lds + MR * cpr * 16);
#pragma unroll
          for (int j = 0; j < SK_FNW; ++j) sg[j] = ssc[(ncol[j] - nbi * SK_BN) * ng + gi];
        }
        compute_group(wr[d], gi);
        if (gi + SK_DG < ng) load_group(wr[d], gi + SK_DG);
        if constexpr (KIND == GEMM_W4) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < SK_FNW; ++j) {
              tot[i][j] += (sg[j] * 0.0625f) * acc[i][j];  // acc holds 16 x the sums
              acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
    }
  }

  // Output: lane holds column ncol[j] and rows m0 + 16i + 4 g4 + r.
#pragma unroll
  for (int j = 0; j < SK_FNW; ++j) {
    const int n = ncol[j];
    if (n >= N) continue;
    float scol = 1.f;
    if constexpr (!PARTIAL && KIND != GEMM_W4) scol = sw[n];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * g4 + r;
        if (m >= M) continue;
        if constexpr (PARTIAL) {
          const int64_t off = ((int64_t)ks * M + m) * N + n;
          if constexpr (I8)
            reinterpret_cast<int32_t*>(part)[off] = acc[i][j][r];
          else if constexpr (KIND == GEMM_W4)
            reinterpret_cast<float*>(part)[off] = tot[i][j][r];
          else
            reinterpret_cast<float*>(part)[off] = acc[i][j][r];
        } else {
          float y;
          if constexpr (I8) {
            if constexpr (ACC_OUT) acc_out[(int64_t)m * ld_acc + n] = acc[i][j][r];
            y = ((float)acc[i][j][r] * sa[m]) * scol;
          } else if constexpr (KIND == GEMM_W4) {
            y = tot[i][j][r];
          } else {
            y = acc[i][j][r] * scol;
          }
          if constexpr (OUT_BF16)
            reinterpret_cast<__bf16*>(C)[(int64_t)m * ldc + n] = (__bf16)y;
          else
            reinterpret_cast<float*>(C)[(int64_t)m * ldc + n] = y;
        }
      }
  }
}

// ------------------------------------------------------- M <= GV_MAX_M rows
// One activation fragment (rows 0..15, rows past M clamped to M-1: they only
// feed output rows that are never stored). A block owns 16 weight rows and the
// whole K range; its waves split K by 256-groups (contiguous ranges), so
// each weight byte is read once and every wave streams two groups ahead. The
// activation fragments come straight from global memory (the same few rows are
// read by every block, so they stay in L2); their K order is the weights' (see
// the lane layout above). The waves' partial sums are added in LDS in wave
// order (fixed, so the result does not depend on timing) and wave 0 applies the
// epilogue. No workspace, one launch.
// Waves per block. W8 (about 120 VGPRs a lane without the activation stage)
// keeps all blocks of a 12288-row weight resident only with four waves a block
// (M = 1: 11.2 -> 10.9 us, M = 8: 14.8 -> 12.8 us); W4 and W8A8 are faster
// with eight (W4 at M = 1: 10.3 us with eight, 12.9 with four).
template <int KIND>
constexpr int gv_waves() {
  return KIND == GEMM_W8 ? 4 : 8;
}
constexpr int GV_MAX_M = 8;  // rows up to which k_qgemv is used (measured: from 16 rows on, the
                             // split-K kernel's shared activation tile wins)
constexpr int GV_LDS_MAX = 48 * 1024;  // activation bytes (M rows x K) staged in LDS when they fit (with
                                       // the 8 KB of partial sums, within the default 64 KB a block)

// ALDS (W8A8, W4): the block first copies the M activation rows into LDS
// (dynamic shared memory, M * K * AB bytes) and the waves read their
// fragments there. Every lane of a 16-lane group needs the same activation bytes (rows
// past M are clamped copies), so read from global memory the fragments cost as
// many load instructions as the weights; from LDS they are broadcast reads.
template <int KIND, bool OUT_BF16, bool ACC_OUT, bool ALDS>
__global__ __launch_bounds__(gv_waves<KIND>() * 64) void k_qgemv(const uint8_t* __restrict__ A, int64_t lda_bytes,
                                                      const uint8_t* __restrict__ B, int64_t ldb,
                                                      const float* __restrict__ sw, const float* __restrict__ sa,
                                                      int M, int N, int K, void* __restrict__ C, int64_t ldc,
                                                      int32_t* __restrict__ acc_out, int64_t ld_acc) {
  using T = SkTraits<KIND>;
  constexpr bool I8 = KIND == GEMM_W8A8;
  constexpr int ALD = I8 ? 4 : 8;  // 16-byte activation loads per lane per group
  using acc_t = typename std::conditional<I8, i32x4_t, f32x4_t>::type;
  constexpr int GV_NW = gv_waves<KIND>();
  __shared__ __align__(16) uint8_t red[GV_NW][64][16];
  extern __shared__ __align__(16) uint8_t gv_act[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int G = K >> 8;
  const int gpw = (G + GV_NW - 1) / GV_NW;
  const int gb = min(G, wave * gpw), ge = min(G, gb + gpw);
  const int ncol = blockIdx.x * 16 + r16;
  const uint8_t* wrow = B + (int64_t)min(ncol, N - 1) * ldb + 16 * g4;
  const uint8_t* arow = A + (int64_t)min(r16, M - 1) * lda_bytes;
  const int64_t kab = (int64_t)K * T::AB;  // activation bytes per row
  const uint8_t* alds = gv_act + (ALDS ? (int64_t)min(r16, M - 1) * kab : 0);

  struct Stage {
    u32x4_t w[T::LPG];
    u32x4_t a[ALD];
  };
  // K index (within a group) of activation fragment j of this lane.
  auto a_elem = [&](int j) -> int {
    if constexpr (I8) return 64 * j + 16 * g4;
    else if constexpr (KIND == GEMM_W8) return 64 * (j >> 1) + 16 * g4 + 8 * (j & 1);
    else return 128 * (j >> 2) + 32 * g4 + 8 * (j & 3);
  };
  auto load = [&](Stage& st, int g) {
#pragma unroll
    for (int t = 0; t < T::LPG; ++t)
      st.w[t] = *reinterpret_cast<const u32x4_t*>(wrow + (int64_t)g * T::WBG + 64 * t);
    if constexpr (!ALDS) {
      const uint8_t* ag = arow + (int64_t)g * 256 * T::AB;
#pragma unroll
      for (int j = 0; j < ALD; ++j) st.a[j] = *reinterpret_cast<const u32x4_t*>(ag + a_elem(j) * T::AB);
    }
  };
  // Activation fragments of group g from LDS (ALDS), read just before use.
  auto load_a_lds = [&](Stage& st, int g) {
    const uint8_t* ag = alds + (int64_t)g * 256 * T::AB;
#pragma unroll
    for (int j = 0; j < ALD; ++j) st.a[j] = *reinterpret_cast<const u32x4_t*>(ag + a_elem(j) * T::AB);
  };

  acc_t acc = acc_t{};
  f32x4_t tot = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Stage& st) {
    if constexpr (I8) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, st.a[t]),
                                                    __builtin_bit_cast(i32x4_t, st.w[t]), acc, 0, 0, 0);
    } else if constexpr (KIND == GEMM_W8) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t lo = h == 0 ? st.w[t].x : st.w[t].z, hi = h == 0 ? st.w[t].y : st.w[t].w;
          asm volatile("" : "+v"(lo), "+v"(hi));  // keep the code words whole (see k_qgemm_skinny)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, st.a[2 * t + h]),
                                                        pp_widen_i8x8(lo, hi), acc, 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t word = d == 0 ? st.w[t].x : d == 1 ? st.w[t].y : d == 2 ? st.w[t].z : st.w[t].w;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, st.a[4 * t + d]),
                                                        pp_widen_i4x8_x16(word, 0xF0F0F0F0u), acc, 0, 0, 0);
        }
    }
  };

  // Groups of weight codes in flight per wave. W4 with the activations in
  // LDS: a stage is only its 32 bytes of codes a lane, so all 6 groups of a
  // 48-group K split 8 ways are loaded ahead (M = 1, 3072 x 12288: 10.7 ->
  // 9.9 us). For W8A8 the extra registers cost a resident block per CU and
  // were slower (gate+up 14.8 -> 17.5 us).
  constexpr int DEPTH = ALDS && KIND == GEMM_W4 ? 6 : 2;
  Stage ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (gb + d < ge) load(ring[d], gb + d);
  if constexpr (ALDS) {
    // The M activation rows into LDS, 16 bytes per thread per step (the
    // weight loads above are already in flight).
    const int64_t total = (int64_t)M * kab;
    for (int64_t o = (int64_t)tid * 16; o < total; o += GV_NW * 64 * 16) {
      const int64_t row = o / kab, col = o - row * kab;
      *reinterpret_cast<u32x4_t*>(gv_act + o) = *reinterpret_cast<const u32x4_t*>(A + row * lda_bytes + col);
    }
    __syncthreads();
  }
  for (int g = gb; g < ge; g += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (g + d < ge) {
        float sg = 0.f;
        if constexpr (KIND == GEMM_W4) sg = sw[(int64_t)min(ncol, N - 1) * G + g + d];
        if constexpr (ALDS) load_a_lds(ring[d], g + d);
        compute(ring[d]);
        if (g + d + DEPTH < ge) load(ring[d], g + d + DEPTH);
        if constexpr (KIND == GEMM_W4) {
          tot += (sg * 0.0625f) * acc;  // acc holds 16 x the sums (16 x code, exact)
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }

  // Fixed-order sum over the waves, then the epilogue (wave 0).
  if constexpr (KIND == GEMM_W4)
    *reinterpret_cast<f32x4_t*>(red[wave][lane]) = tot;
  else
    *reinterpret_cast<acc_t*>(red[wave][lane]) = acc;
  __syncthreads();
  if (wave != 0) return;
  acc_t sum = *reinterpret_cast<const acc_t*>(red[0][lane]);
#pragma unroll
  for (int w = 1; w < GV_NW; ++w) sum += *reinterpret_cast<const acc_t*>(red[w][lane]);
  if (ncol >= N) return;
  const float scol = KIND == GEMM_W4 ? 1.f : sw[ncol];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g4 + r;
    if (m >= M) continue;
    float y;
    if constexpr (I8) {
      if constexpr (ACC_OUT) acc_out[(int64_t)m * ld_acc + ncol] = sum[r];
      y = ((float)sum[r] * sa[m]) * scol;
    } else {
      y = sum[r] * scol;
    }
    if constexpr (OUT_BF16)
      reinterpret_cast<__bf16*>(C)[(int64_t)m * ldc + ncol] = (__bf16)y;
    else
      reinterpret_cast<float*>(C)[(int64_t)m * ldc + ncol] = y;
  }
}

template <int KIND>
static hipError_t launch_gemv(const GemmArgs& g, hipStream_t stream) {
  const int64_t lda_bytes = g.lda * (KIND == GEMM_W8A8 ? 1 : 2);
  const uint8_t* a = (const uint8_t*)g.a;
  const uint8_t* b = (const uint8_t*)g.b;
  const dim3 grid((unsigned)((g.n + 15) / 16)), block(gv_waves<KIND>() * 64);
  const int64_t act_bytes = g.m * g.k * (KIND == GEMM_W8A8 ? 1 : 2);
  // Staging measured at M = 1: W8A8 qkv 10.3 -> 8.3 us and gate+up 18.3 -> 14.7 us;
  // W4 (with the deeper prefetch it allows) 10.7 -> 9.9 us; no gain for W8.
  const bool alds = (KIND == GEMM_W8A8 || KIND == GEMM_W4) && act_bytes <= GV_LDS_MAX;
#define TP_LAUNCH_GV(OB, AO, AL)                                                                              \
  hipLaunchKernelGGL((k_qgemv<KIND, OB, AO, AL>), grid, block, AL ? (size_t)act_bytes : 0, stream, a, lda_bytes, \
                     b, g.ldb, g.w_scales, g.a_scales, (int)g.m, (int)g.n, (int)g.k, g.c, g.ldc, g.acc_out,   \
                     g.ld_acc)
  if (KIND == GEMM_W8A8 && g.acc_out) {
    if (g.c_bf16) {
      if (alds) TP_LAUNCH_GV(true, true, true); else TP_LAUNCH_GV(true, true, false);
    } else {
      if (alds) TP_LAUNCH_GV(false, true, true); else TP_LAUNCH_GV(false, true, false);
    }
  } else {
    if (g.c_bf16) {
      if (alds) TP_LAUNCH_GV(true, false, true); else TP_LAUNCH_GV(true, false, false);
    } else {
      if (alds) TP_LAUNCH_GV(false, false, true); else TP_LAUNCH_GV(false, false, false);
    }
  }
#undef TP_LAUNCH_GV
  return hipGetLastError();
}

// Sum of the split partials in split order, then the epilogue. One thread per
// output element; blockIdx.y is the row. The scales and each run of up to
// eight partials are loaded before any of them is added, so the loads are in
// flight together instead of each waiting on the previous add (the additions
// themselves keep split order).
template <int KIND, bool OUT_BF16, bool ACC_OUT>
__global__ __launch_bounds__(256) void k_qgemm_reduce(const void* __restrict__ part, int splits, int M, int N,
                                                      const float* __restrict__ sw, const float* __restrict__ sa,
                                                      void* __restrict__ C, int64_t ldc,
                                                      int32_t* __restrict__ acc_out, int64_t ld_acc) {
  constexpr int RUN = 8;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  if (n >= N) return;
  const int64_t plane = (int64_t)M * N;
  const int64_t off = (int64_t)m * N + n;
  const float scol = (KIND == GEMM_W8A8 || KIND == GEMM_W8) ? sw[n] : 1.f;
  const float srow = (KIND == GEMM_W8A8 || KIND == GEMM_W4A8) ? sa[m] : 1.f;
  typedef typename std::conditional<KIND == GEMM_W8A8, int32_t, float>::type part_t;
  const part_t* p = reinterpret_cast<const part_t*>(part) + off;
  part_t s = p[0];
  for (int sp0 = 1; sp0 < splits; sp0 += RUN) {
    part_t v[RUN];
#pragma unroll
    for (int u = 0; u < RUN; ++u) v[u] = sp0 + u < splits ? p[(sp0 + u) * plane] : part_t(0);
#pragma unroll
    for (int u = 0; u < RUN; ++u)
      if (sp0 + u < splits) s += v[u];
  }
  float y;
  if constexpr (KIND == GEMM_W8A8) {
    if constexpr (ACC_OUT) acc_out[(int64_t)m * ld_acc + n] = s;
    y = ((float)s * srow) * scol;
  } else {
    y = KIND == GEMM_W8 ? s * scol : (KIND == GEMM_W4A8 ? s * srow : s);
  }
  if constexpr (OUT_BF16)
    reinterpret_cast<__bf16*>(C)[(int64_t)m * ldc + n] = (__bf16)y;
  else
    reinterpret_cast<float*>(C)[(int64_t)m * ldc + n] = y;
}

// The same sums and epilogue, four consecutive outputs a thread: 16-byte
// partial loads and whole-vector stores (used when N, the output pitches and
// the base addresses allow them). Each output adds its splits in split order
// and is rounded exactly as in k_qgemm_reduce.
template <int KIND, bool OUT_BF16, bool ACC_OUT>
__global__ __launch_bounds__(256) void k_qgemm_reduce4(const void* __restrict__ part, int splits, int M, int N,
                                                       const float* __restrict__ sw, const float* __restrict__ sa,
                                                       void* __restrict__ C, int64_t ldc,
                                                       int32_t* __restrict__ acc_out, int64_t ld_acc) {
  constexpr int RUN = 8;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int m = blockIdx.y;
  if (n >= N) return;
  const int64_t plane = (int64_t)M * N;
  const int64_t off = (int64_t)m * N + n;
  float scol[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) scol[e] = (KIND == GEMM_W8A8 || KIND == GEMM_W8) ? sw[n + e] : 1.f;
  const float srow = (KIND == GEMM_W8A8 || KIND == GEMM_W4A8) ? sa[m] : 1.f;
  typedef typename std::conditional<KIND == GEMM_W8A8, i32x4_t, f32x4_t>::type vec_t;
  const vec_t* p = reinterpret_cast<const vec_t*>(reinterpret_cast<const typename std::conditional<
      KIND == GEMM_W8A8, int32_t, float>::type*>(part) + off);
  vec_t s = p[0];
  for (int sp0 = 1; sp0 < splits; sp0 += RUN) {
    vec_t v[RUN];
#pragma unroll
    for (int u = 0; u < RUN; ++u) v[u] = sp0 + u < splits ? p[(sp0 + u) * (plane / 4)] : vec_t{};
#pragma unroll
    for (int u = 0; u < RUN; ++u)
      if (sp0 + u < splits) s += v[u];
  }
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (KIND == GEMM_W8A8)
      y[e] = ((float)s[e] * srow) * scol[e];
    else
      y[e] = KIND == GEMM_W8 ? s[e] * scol[e] : (KIND == GEMM_W4A8 ? s[e] * srow : s[e]);
  }
  if constexpr (KIND == GEMM_W8A8 && ACC_OUT) *reinterpret_cast<i32x4_t*>(acc_out + (int64_t)m * ld_acc + n) = s;
  if constexpr (OUT_BF16) {
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)y[e]);
    const uint2 w = {(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(C) + (int64_t)m * ldc + n) = w;
  } else {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(C) + (int64_t)m * ldc + n) = f32x4_t{y[0], y[1], y[2], y[3]};
  }
}

// Launch plan of the small-M path for one product shape (splits == 1: no
// partial sums in the workspace).
struct SkPlan {
  bool gemv;   // M <= GV_MAX_M: k_qgemv (one launch, no partial sums)
  int fm;      // 16-row activation fragments per block (1, 2 or 4)
  int mb;      // blocks along M
  int nb;      // blocks along N
  int splits;  // blocks along K
  int gps;     // 256-groups per split (the last split may hold fewer)
  int lds;     // dynamic LDS bytes per block
};

constexpr int SK_MAX_M = 64;           // rows up to which the small-M path is used
constexpr int SK_MAX_LDS = 64 * 1024;  // activation stage per block (the default dynamic-LDS limit)
constexpr int SK_CUS = 256;            // compute units of the device the plan is tuned for

// Blocks (one wave per SIMD each) that one CU holds at once as far as the
// register use of the built kernels goes, by kind and fm (1, 2, 4); only the
// plan's speed depends on these.
inline int sk_reg_blocks(int kind, int fm) {
  const int i = fm == 1 ? 0 : (fm == 2 ? 1 : 2);
  static const int w8[3] = {4, 3, 2}, w4[3] = {5, 4, 3}, w8a8[3] = {4, 4, 2};
  return kind == GEMM_W8 ? w8[i] : (kind == GEMM_W4 ? w4[i] : w8a8[i]);
}

// Estimated time (us) of one small-M plan, fitted to measurements of the
// split-K kernel on MI355X (cold weights, 16 to 64 rows, K 3072 and 12288,
// N 3072 to 24576). The kernel takes the largest of three floors: the weights
// at 7 TB/s; the busiest CU streaming its blocks' codes at about 40 GB/s (a
// block's loads are latency-bound); and, per round of resident blocks, about
// 1 us of load latency per two groups plus the products (0.25 us per group
// and 16 rows for W8 and W4, 0.075 for W8A8). Splits add their partial sums
// (written and read once) and the reduction launch.
inline double sk_plan_cost_us(int kind, int64_t m, int64_t n, int64_t k, int fm, int64_t mb, int64_t nb,
                              int64_t gps, int64_t splits, int lds) {
  const double wbytes = (double)n * (double)k * (kind == GEMM_W4 ? 0.5 : 1.0);
  const double blocks = (double)(nb * mb * splits);
  const int per_cu = std::min(std::min(163840 / lds, sk_reg_blocks(kind, fm)), 8);
  const double rounds = std::ceil(blocks / (SK_CUS * per_cu));
  const double busiest = std::ceil(blocks / SK_CUS) * (wbytes * (double)mb / blocks);
  const double mma = (kind == GEMM_W8A8 ? 0.075 : 0.25) * fm * (double)gps;
  const double tblock = 1.0 * (double)((gps + 1) / 2) + mma;
  const double part = splits > 1 ? (double)splits * (double)m * (double)n * 4.0 : 0.0;
  return std::max(std::max(wbytes / 7.0e6, busiest / 4.0e4), rounds * tblock) + 2.0 * part / 7.0e6 +
         (splits > 1 ? 1.0 : 0.0);
}

// The plan with the lowest estimate over fm (up to the fragments M needs) and
// every balanced split of the 256-groups whose activation stage fits in LDS;
// ties go to fewer splits. A pure function of the shape, so the workspace size
// query and the launch agree.
inline bool skinny_plan(int kind, int64_t m, int64_t n, int64_t k, SkPlan* p) {
  if (kind == GEMM_W4A8 || m < 1 || m > SK_MAX_M || n < 1 || k < 256) return false;
  if (m <= GV_MAX_M) {
    *p = SkPlan{true, 1, 1, (int)((n + 15) / 16), 1, (int)(k / 256), 0};
    return (n + 15) / 16 <= INT32_MAX;
  }
  const int ab = kind == GEMM_W8A8 ? 1 : 2;
  const int64_t G = k / 256;
  const int64_t nb = (n + SK_BN - 1) / SK_BN;
  const int fm_need = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  bool found = false;
  double best = 0.0;
  for (int fm = 1; fm <= fm_need; fm *= 2) {
    const int mr = 16 * fm;
    const int64_t mb = (m + mr - 1) / mr;
    for (int64_t sp = 1; sp <= G; ++sp) {
      const int64_t gps = (G + sp - 1) / sp;
      const int64_t splits = (G + gps - 1) / gps;
      if (splits != sp) continue;  // the same split as a smaller count
      const int64_t lds64 = (int64_t)mr * gps * 256 * ab + (kind == GEMM_W4 ? (int64_t)SK_BN * gps * 4 : 0);
      if (lds64 > SK_MAX_LDS) continue;
      if (nb * mb * splits > INT32_MAX) continue;
      const int lds = (int)lds64;
      const double c = sk_plan_cost_us(kind, m, n, k, fm, mb, nb, gps, splits, lds);
      if (!found || c < best) {
        found = true;
        best = c;
        *p = SkPlan{false, fm, (int)mb, (int)nb, (int)splits, (int)gps, lds};
      }
    }
  }
  return found;
}

template <int KIND, int FM>
static hipError_t launch_skinny_fm(const GemmArgs& g, const SkPlan& p, hipStream_t stream) {
  const int64_t lda_bytes = g.lda * (KIND == GEMM_W8A8 ? 1 : 2);
  const uint8_t* a = (const uint8_t*)g.a;
  const uint8_t* b = (const uint8_t*)g.b;
  const dim3 grid((unsigned)(p.nb * p.splits * p.mb)), block(SK_NW * 64);
  const bool split = p.splits > 1;
#define TP_LAUNCH_SK(OB, AO, PA)                                                                                 \
  hipLaunchKernelGGL((k_qgemm_skinny<KIND, FM, OB, AO, PA>), grid, block, p.lds, stream, a, lda_bytes, b, g.ldb, \
                     g.w_scales, g.a_scales, (int)g.m, (int)g.n, (int)g.k, g.c, g.ldc, g.acc_out, g.ld_acc, g.part, \
                     p.nb, p.splits, p.gps)
  if (split) {
    TP_LAUNCH_SK(false, false, true);
  } else if (KIND == GEMM_W8A8 && g.acc_out) {
    if (g.c_bf16) TP_LAUNCH_SK(true, true, false); else TP_LAUNCH_SK(false, true, false);
  } else {
    if (g.c_bf16) TP_LAUNCH_SK(true, false, false); else TP_LAUNCH_SK(false, false, false);
  }
#undef TP_LAUNCH_SK
  if (!split) return hipGetLastError();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce<KIND>(g, p.splits, stream);
}

template <int KIND>
static hipError_t launch_reduce(const GemmArgs& g, int splits, hipStream_t stream) {
  const auto al = [](const void* q, uintptr_t b) { return ((uintptr_t)q & (b - 1)) == 0; };
  const bool four = g.n % 4 == 0 && g.ldc % 4 == 0 && al(g.c, g.c_bf16 ? 8 : 16) && al(g.part, 16) &&
                    (!g.acc_out || (g.ld_acc % 4 == 0 && al(g.acc_out, 16)));
  const dim3 rgrid((unsigned)((four ? g.n / 4 + 255 : g.n + 255) / 256), (unsigned)g.m), rblock(256);
#define TP_LAUNCH_RED(OB, AO)                                                                                     \
  do {                                                                                                            \
    if (four)                                                                                                     \
      hipLaunchKernelGGL((k_qgemm_reduce4<KIND, OB, AO>), rgrid, rblock, 0, stream, g.part, splits, (int)g.m,     \
                         (int)g.n, g.w_scales, g.a_scales, g.c, g.ldc, g.acc_out, g.ld_acc);                     \
    else                                                                                                          \
      hipLaunchKernelGGL((k_qgemm_reduce<KIND, OB, AO>), rgrid, rblock, 0, stream, g.part, splits, (int)g.m,      \
                         (int)g.n, g.w_scales, g.a_scales, g.c, g.ldc, g.acc_out, g.ld_acc);                     \
  } while (0)
  if (KIND == GEMM_W8A8 && g.acc_out) {
    if (g.c_bf16) TP_LAUNCH_RED(true, true); else TP_LAUNCH_RED(false, true);
  } else {
    if (g.c_bf16) TP_LAUNCH_RED(true, false); else TP_LAUNCH_RED(false, false);
  }
#undef TP_LAUNCH_RED
  return hipGetLastError();
}

template <int KIND>
static hipError_t launch_skinny(const GemmArgs& g, const SkPlan& p, hipStream_t stream) {
  if (p.gemv) return launch_gemv<KIND>(g, stream);
  switch (p.fm) {
    case 1: return launch_skinny_fm<KIND, 1>(g, p, stream);
    case 2: return launch_skinny_fm<KIND, 2>(g, p, stream);
    default: return launch_skinny_fm<KIND, 4>(g, p, stream);
  }
}

}  // namespace tp
