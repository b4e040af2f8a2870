// Quantized products on the gfx950 matrix cores.
//
//   W8    C = (bf16(A') . q^T) * s[n]            bf16 MFMA 16x16x32, fp32 sums
//   W4    C = sum_g s[n,g] * (bf16(A'_g) . q_g^T) bf16 MFMA, per-group fp32 fold
//   W8A8  acc = qa . q^T (int32, exact); C = (float(acc) * sa[m]) * sw[n]
//                                                 i8 MFMA 16x16x64, int32 sums
//
// (tensai docs, "画像生成", section "幅とメモリ": int8 weights with one scale
// per row, the 4-bit "-q4" width; section "GPU": activations quantized on the
// device. TensorFold pull request #948: bf16 activations with fp32 sums in
// every projection.)
//
// Both operands are K-contiguous ("NT": A is [m, k], weights are [n, k]).
// A block computes a BM x BN tile of C with (BM/WM) x (BN/WN) waves; each wave
// owns a WM x WN sub-tile built from 16x16 MFMA tiles. Every stage moves 128
// bytes of K per row of A and, after conversion to the MFMA operand type, 128
// bytes per row of B into LDS (double buffered, rows padded to 144 bytes so
// that the 16-byte fragment reads of 8 consecutive lanes hit distinct banks).
// Weight codes are widened to bf16 once per block on their way into LDS (W8,
// W4), so the waves that share them do not repeat the conversion. Rows past M
// or N are clamped on load and masked on store; K needs no tail (k % 256 == 0).
#include <type_traits>

#include "device_common.hpp"
#include "gemm_pp.hpp"
#include "gemm_skinny.hpp"
#include "kernels.hpp"

namespace tp {

constexpr int LDS_ROW = 144;  // bytes per LDS tile row: 128 data + 16 pad

// Logical tile of a block. Blocks are dealt to the 8 XCDs round-robin by the
// hardware (block i runs on XCD i % 8); remap so that each XCD owns one
// contiguous range of logical tiles, then walk tiles in groups of GM tile-rows
// so that blocks running together on one XCD share A rows and B columns in
// that XCD's L2.
__device__ __forceinline__ void map_tile(int pid, int nblk, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = pid & 7, idx = pid >> 3;
  const int logical = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  constexpr int GM = 8;
  const int width = GM * tiles_n;
  const int group = logical / width;
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int within = logical - group * width;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

// 16 int8 codes -> 16 bf16 (exact), natural order, as 8 dwords.
__device__ __forceinline__ void widen_i8x16(const u32x4_t w, uint32_t (&o)[8]) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = d[i];
    o[2 * i] = pack_bf16x2((float)(int8_t)(v), (float)(int8_t)(v >> 8));
    o[2 * i + 1] = pack_bf16x2((float)(int8_t)(v >> 16), (float)(int8_t)(v >> 24));
  }
}

// 32 int4 codes (two's complement nibbles, even column low) -> 32 bf16 (exact),
// natural order, as 16 dwords.
__device__ __forceinline__ void widen_i4x32(const u32x4_t w, uint32_t (&o)[16]) {
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t v = (int32_t)d[i];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float lo = (float)((v << (28 - 8 * b)) >> 28);
      const float hi = (float)((v << (24 - 8 * b)) >> 28);
      o[4 * i + b] = pack_bf16x2(lo, hi);
    }
  }
}

template <int KIND, int BM, int BN, int WM, int WN, bool OUT_BF16, bool ACC_OUT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_qgemm(
    const uint8_t* __restrict__ A, int64_t lda_bytes, const uint8_t* __restrict__ B, int64_t ldb_bytes,
    const float* __restrict__ sw, const float* __restrict__ sa, int M, int N, int K, void* __restrict__ Cv,
    int64_t ldc, int32_t* __restrict__ acc_out, int64_t ld_acc, int tiles_m, int tiles_n) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr bool I8 = (KIND == GEMM_W8A8);
  // bytes of one B row that one stage reads from global memory
  constexpr int BG = (KIND == GEMM_W8A8) ? 128 : (KIND == GEMM_W8) ? 64 : 32;
  constexpr int B_CPR = BG / 16;  // 16-byte chunks per B row per stage
  // 16-byte chunks per thread and stage; when a tile has fewer chunks than
  // threads, the surplus threads load nothing.
  constexpr int A_CHUNKS = BM * 8, B_CHUNKS = BN * B_CPR;
  constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  constexpr bool A_EVEN = A_CHUNKS % NT == 0, B_EVEN = B_CHUNKS % NT == 0;
  constexpr int A_BUF = BM * LDS_ROW, B_BUF = BN * LDS_ROW;

  __shared__ __align__(16) uint8_t smem[2 * (A_BUF + B_BUF)];
  uint8_t* const As = smem;
  uint8_t* const Bs = smem + 2 * A_BUF;

  int tm, tn;
  map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;

  // Global source rows of this thread's chunks (clamped into range).
  const uint8_t* a_src[A_PER_T];
  int a_lds[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int c = A_EVEN ? tid + i * NT : min(tid + i * NT, A_CHUNKS - 1), row = c >> 3, col = c & 7;
    a_src[i] = A + (int64_t)min(m0 + row, M - 1) * lda_bytes + col * 16;
    a_lds[i] = row * LDS_ROW + col * 16;
  }
  const uint8_t* b_src[B_PER_T];
  int b_lds[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int c = B_EVEN ? tid + i * NT : min(tid + i * NT, B_CHUNKS - 1), row = c / B_CPR, col = c % B_CPR;
    b_src[i] = B + (int64_t)min(n0 + row, N - 1) * ldb_bytes + col * 16;
    b_lds[i] = row * LDS_ROW + col * (128 / B_CPR);
  }

  u32x4_t ra[A_PER_T], rb[B_PER_T];
  auto load_stage = [&](int ks) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + (int64_t)ks * 128);
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + (int64_t)ks * BG);
  };
  auto store_stage = [&](int buf) {
    uint8_t* as = As + buf * A_BUF;
    uint8_t* bs = Bs + buf * B_BUF;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i)
      if (A_EVEN || tid + i * NT < A_CHUNKS) *reinterpret_cast<u32x4_t*>(as + a_lds[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      if (!B_EVEN && tid + i * NT >= B_CHUNKS) continue;
      if constexpr (KIND == GEMM_W8A8) {
        *reinterpret_cast<u32x4_t*>(bs + b_lds[i]) = rb[i];
      } else if constexpr (KIND == GEMM_W8) {
        uint32_t o[8];
        widen_i8x16(rb[i], o);
        u32x4_t lo = {o[0], o[1], o[2], o[3]}, hi = {o[4], o[5], o[6], o[7]};
        *reinterpret_cast<u32x4_t*>(bs + b_lds[i]) = lo;
        *reinterpret_cast<u32x4_t*>(bs + b_lds[i] + 16) = hi;
      } else {
        uint32_t o[16];
        widen_i4x32(rb[i], o);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          u32x4_t v = {o[4 * t], o[4 * t + 1], o[4 * t + 2], o[4 * t + 3]};
          *reinterpret_cast<u32x4_t*>(bs + b_lds[i] + 16 * t) = v;
        }
      }
    }
  };

  typedef typename std::conditional<I8, i32x4_t, f32x4_t>::type acc_t;
  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  // W4 only: running sum over groups (acc holds the current group's partial).
  f32x4_t tot[KIND == GEMM_W4 ? FM : 1][KIND == GEMM_W4 ? FN : 1];
  if constexpr (KIND == GEMM_W4) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) tot[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int frag_off = (lane & 15) * LDS_ROW + (lane >> 4) * 16;
  auto compute = [&](int buf) {
    const uint8_t* as = As + buf * A_BUF + wm0 * LDS_ROW + frag_off;
    const uint8_t* bs = Bs + buf * B_BUF + wn0 * LDS_ROW + frag_off;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(as + i * 16 * LDS_ROW + kk * 64);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4_t*>(bs + j * 16 * LDS_ROW + kk * 64);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (I8) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, af[i]),
                                                               __builtin_bit_cast(i32x4_t, bfr[j]), acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[i]),
                                                                 __builtin_bit_cast(bf16x8_t, bfr[j]), acc[i][j], 0, 0, 0);
          }
        }
    }
  };

  const int KSTAGE = I8 ? 128 : 64;  // K elements per stage
  const int KS = K / KSTAGE;
  constexpr int STAGES_PER_GROUP = 256 / 64;
  const int groups = K >> 8;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) load_stage(ks + 1);
    compute(ks & 1);
    if constexpr (KIND == GEMM_W4) {
      if ((ks + 1) % STAGES_PER_GROUP == 0) {
        const int g = ks / STAGES_PER_GROUP;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = min(n0 + wn0 + j * 16 + (lane & 15), N - 1);
          const float s = sw[(int64_t)col * groups + g];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            tot[i][j] += s * acc[i][j];
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    if (ks + 1 < KS) store_stage((ks + 1) & 1);
    __syncthreads();
  }

  // Epilogue: lane l of a 16x16 tile holds rows 4*(l/16)+r, column l%16.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn0 + j * 16 + (lane & 15);
    if (col >= N) continue;
    float wsc = 1.0f;
    if constexpr (KIND != GEMM_W4) wsc = sw[col];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm0 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= M) continue;
        float v;
        if constexpr (KIND == GEMM_W8A8) {
          const int32_t a = acc[i][j][r];
          v = ((float)a * sa[row]) * wsc;
          if constexpr (ACC_OUT) acc_out[(int64_t)row * ld_acc + col] = a;
        } else if constexpr (KIND == GEMM_W8) {
          v = acc[i][j][r] * wsc;
        } else {
          v = tot[i][j][r];
        }
        if constexpr (OUT_BF16) {
          reinterpret_cast<__bf16*>(Cv)[(int64_t)row * ldc + col] = (__bf16)v;
        } else {
          reinterpret_cast<float*>(Cv)[(int64_t)row * ldc + col] = v;
        }
      }
    }
  }
}

template <int KIND, int BM, int BN, int WM, int WN>
static hipError_t launch_tile(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (int)((g.m + BM - 1) / BM), tiles_n = (int)((g.n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block((BM / WM) * (BN / WN) * 64);
  const int64_t lda_bytes = g.lda * (KIND == GEMM_W8A8 ? 1 : 2);
  const uint8_t* a = (const uint8_t*)g.a;
  const uint8_t* b = (const uint8_t*)g.b;
#define TP_LAUNCH(OB, AO)                                                                                  \
  hipLaunchKernelGGL((k_qgemm<KIND, BM, BN, WM, WN, OB, AO>), grid, block, 0, stream, a, lda_bytes, b, g.ldb, \
                     g.w_scales, g.a_scales, (int)g.m, (int)g.n, (int)g.k, g.c, g.ldc, g.acc_out, g.ld_acc,   \
                     tiles_m, tiles_n)
  if (KIND == GEMM_W8A8 && g.acc_out) {
    if (g.c_bf16) TP_LAUNCH(true, true); else TP_LAUNCH(false, true);
  } else {
    if (g.c_bf16) TP_LAUNCH(true, false); else TP_LAUNCH(false, false);
  }
#undef TP_LAUNCH
  return hipGetLastError();
}

// Kernel table (from measured sweeps on MI355X). Outputs with at least 128
// tiles of 256x256 run the two-group multi-stage kernel of gemm_pp.hpp:
//   W8     256x256 tiles of 8 waves (128x64 each), 3 stages;
//   W8A8   256x256 (128x64 waves), 4 stages; 256x192 (64x96 waves) when the
//          256x256 grid would leave CUs idle and the 192-wide one does not
//          (e.g. N = 3072 at M = 4096: 192 -> 256 tiles for 256 CUs);
//   W4     128x192 tiles (64x48 waves), 5 stages: the per-group fold keeps a
//          second set of accumulators, which bounds the wave tile, and the
//          4032x3072 product splits into 512 tiles (two full rounds) instead
//          of 384 (1.5 rounds) for 256x128.
// The last launch argument is the number of tile-rows an XCD walks together
// (pp_map_tile): 4 for W8, W4 and wide W8A8 outputs, 8 otherwise (measured:
// W8 4096x3072x12288 307 -> 257 us from 8 to 4).
// Smaller outputs use the single-stage kernels above with 128x128 tiles, so
// that the 256 CUs still get several tiles each.
enum KernelCfg { CFG_SMALL_128 = 0, CFG_PP_256x256 = 1, CFG_PP_128x192 = 2, CFG_PP_256x192 = 3 };
constexpr int64_t NUM_CUS = 256;

static int pick_cfg(int kind, int64_t m, int64_t n, int64_t k) {
  (void)k;
  const int64_t big = ((m + 255) / 256) * ((n + 255) / 256);
  if (big < 128) return CFG_SMALL_128;
  if (kind == GEMM_W4) return CFG_PP_128x192;
  if (kind == GEMM_W8A8 && big < NUM_CUS && ((m + 255) / 256) * ((n + 191) / 192) <= NUM_CUS) return CFG_PP_256x192;
  return CFG_PP_256x256;
}

void qgemm_tile_for(int kind, int64_t m, int64_t n, int64_t k, int* bm, int* bn) {
  SkPlan sp;
  if (skinny_plan(kind, m, n, k, &sp)) {
    *bm = 16 * sp.fm;
    *bn = SK_BN;
    return;
  }
  switch (pick_cfg(kind, m, n, k)) {
    case CFG_PP_256x256: *bm = 256; *bn = 256; return;
    case CFG_PP_128x192: *bm = 128; *bn = 192; return;
    case CFG_PP_256x192: *bm = 256; *bn = 192; return;
    default: *bm = 128; *bn = 128; return;
  }
}

int64_t qgemm_partial_bytes(int kind, int64_t m, int64_t n, int64_t k) {
  SkPlan p;
  if (!skinny_plan(kind, m, n, k, &p) || p.splits == 1) return 0;
  const int64_t mn = m * n;  // m <= SK_MAX_M, n < 2^31
  if (mn > INT64_MAX / 4 / p.splits) return -1;
  return mn * 4 * p.splits;
}

template <int KIND>
static hipError_t launch_kind(const GemmArgs& g, hipStream_t stream) {
  SkPlan sp;
  if (skinny_plan(KIND, g.m, g.n, g.k, &sp)) {
    if (sp.splits > 1 && !g.part) return hipErrorInvalidValue;
    return launch_skinny<KIND>(g, sp, stream);
  }
  switch (pick_cfg(KIND, g.m, g.n, g.k)) {
    case CFG_PP_256x256:
      if constexpr (KIND == GEMM_W8A8)
        return launch_pp<KIND, 256, 256, 128, 64, 4>(g, stream, (g.n + 255) / 256 >= 64 ? 4 : 8);
      if constexpr (KIND == GEMM_W8) return launch_pp<KIND, 256, 256, 128, 64, 3>(g, stream, 4);
      break;
    case CFG_PP_128x192:
      if constexpr (KIND == GEMM_W4) return launch_pp<KIND, 128, 192, 64, 48, 5>(g, stream, 4);
      break;
    case CFG_PP_256x192:
      if constexpr (KIND == GEMM_W8A8) return launch_pp<KIND, 256, 192, 64, 96, 4>(g, stream);
      break;
    default: break;
  }
  return launch_tile<KIND, 128, 128, 32, 64>(g, stream);
}

hipError_t launch_qgemm(const GemmArgs& g, hipStream_t stream) {
  switch (g.kind) {
    case GEMM_W8: return launch_kind<GEMM_W8>(g, stream);
    case GEMM_W4: return launch_kind<GEMM_W4>(g, stream);
    case GEMM_W8A8: return launch_kind<GEMM_W8A8>(g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tp
