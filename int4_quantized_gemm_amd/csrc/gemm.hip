// Quantized products on the gfx950 matrix cores: the tile table and the
// dispatch over the kernels of gemm_pp.hpp (multi-stage two-group kernel) and
// gemm_skinny.hpp (few activation rows).
//
//   W8    C = (bf16(A') . q^T) * s[n]            bf16 MFMA 16x16x32, fp32 sums
//   W4    C = sum_g s[n,g] * (bf16(A'_g) . q_g^T) bf16 MFMA, per-group fp32 rescale
//   W8A8  acc = qa . q^T (int32, exact); C = (float(acc) * sa[m]) * sw[n]
//                                                 i8 MFMA 16x16x64, int32 sums
//   W4A8  C = (sum_g s[n,g] * float(qa_g . q_g^T)) * sa[m]
//                                                 i8 MFMA, exact int32 per group
//
// (tensai docs, "画像生成", section "幅とメモリ": int8 weights with one scale
// per row, the 4-bit "-q4" width; section "GPU": activations quantized on the
// device. TensorFold pull request #948: bf16 activations with fp32 sums in
// every projection.)
//
// Both operands are K-contiguous ("NT": A is [m, k], weights are [n, k]).
// Rows past M or N are clamped on load and masked on store; K needs no tail
// (k % 256 == 0).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "gemm_pp.hpp"
#include "gemm_skinny.hpp"
#include "kernels.hpp"

namespace tp {

// Kernel table (from measured sweeps on MI355X). Outputs with at least 128
// tiles of 256x256 run the two-group multi-stage kernel of gemm_pp.hpp:
//   W8     256x256 tiles of 8 waves (128x64 each), 3 stages, three of the
//          four code fragments widened in the memory phase (5-7% faster than
//          all in the compute phase, where a wave's VALU work serializes with
//          its own MFMAs; 1.7% faster than all four early);
//   W8A8   256x256 (128x64 waves), 4 stages, or 256x192 (64x96 waves) or
//          256x288 (64x144 waves) when their rounds of tiles, at 0.825 and
//          1.125 of a 256x256 tile's time each, take less (N = 3072 at
//          M = 4096: one full round of 256x192 tiles instead of 192 tiles of
//          256x256; N = 9216: 2 full rounds of 256x288 tiles instead of 2.25
//          of 256x256);
//   W4     256x192 (128x48 waves), 3 stages, when that grid has at least 192
//          tiles (4032x3072 splits into exactly 256): 128-row waves spread
//          the widening of each code over 8 MFMAs (measured 4032x3072x12288:
//          391 us with 64x48 waves and a second accumulator set, 277 us),
//          two of the three code fragments widened in the memory phase and
//          one in the compute phase (6% faster than none or all early: the
//          phases balance, measured with per-phase timestamps);
//          below that, 128x192 (64x48 waves, 5 stages);
//   W4A8   256x128 (128x32 waves, 5 stages) when that grid fills the CUs at
//          least twice (the per-group fold keeps a second accumulator set,
//          and 128-row waves halve the widening per MFMA: 4096x12288x3072
//          286 -> 235 us), else as W4 below 256x192; in both, two code
//          fragments per stage are widened in the memory phase and the
//          group fold runs there too (4096x3072x12288: 278 -> 248 us).
// The last launch argument is the number of tile-rows an XCD walks together
// (pp_map_tile): 4 for W8, W4 and wide W8A8 outputs, 8 otherwise (measured:
// W8 4096x3072x12288 307 -> 257 us from 8 to 4).
// Smaller outputs: see pick_plan.
enum KernelCfg { CFG_PP_256x256 = 1, CFG_PP_128x192 = 2, CFG_PP_256x192 = 3, CFG_PP_256x128 = 4, CFG_PP_256x288 = 5 };
constexpr int64_t W4_MIN_WIDE_TILES = 192;
constexpr int64_t NUM_CUS = 256;

struct PpPlan {
  int cfg;
  int splits;  // blocks along K (1: no partial sums)
  int sps;     // 64-K stages per split, a multiple of 4
};

// Outputs with fewer than 128 tiles of 256x256 run 128x192 tiles with K split
// so that about one block runs per CU (at least 8 stages per split); the
// splits' partial sums go to the workspace and k_qgemm_reduce adds them.
static PpPlan pick_plan(int kind, int64_t m, int64_t n, int64_t k) {
  const int64_t big = ((m + 255) / 256) * ((n + 255) / 256);
  if (kind == GEMM_W4 && ((m + 255) / 256) * ((n + 191) / 192) >= W4_MIN_WIDE_TILES)
    return PpPlan{CFG_PP_256x192, 1, 0};
  if (kind == GEMM_W4A8 && big >= 128 && ((m + 255) / 256) * ((n + 127) / 128) >= 2 * NUM_CUS)
    return PpPlan{CFG_PP_256x128, 1, 0};
  if (big >= 128) {
    if (kind == GEMM_W4 || kind == GEMM_W4A8) return PpPlan{CFG_PP_128x192, 1, 0};
    if (kind == GEMM_W8A8) {
      // Rounds of tiles on the CUs, weighted by a tile's time: a 256x192 tile
      // (64x96 waves) takes about 0.825 of a 256x256 one (0.75 of the area at
      // a lower rate), a 256x288 tile (64x144 waves) about 1.125 (its area).
      // 4096x9216: 2.25 rounds of 256x256 (3, the last a quarter full), 3 of
      // 256x192 (2.475) or 2 of 256x288 (2.25): 138 -> 123.5 us from 256x192
      // to 256x288 (same box).
      const int64_t r256 = (big + NUM_CUS - 1) / NUM_CUS;
      const int64_t r192 = (((m + 255) / 256) * ((n + 191) / 192) + NUM_CUS - 1) / NUM_CUS;
      const int64_t r288 = (((m + 255) / 256) * ((n + 287) / 288) + NUM_CUS - 1) / NUM_CUS;
      const int64_t c256 = r256 * 320, c192 = r192 * 264, c288 = r288 * 360;  // rounds x 320 x relative tile time
      if (c288 < c256 && c288 < c192) return PpPlan{CFG_PP_256x288, 1, 0};
      if (c192 < c256) return PpPlan{CFG_PP_256x192, 1, 0};
    }
    return PpPlan{CFG_PP_256x256, 1, 0};
  }
  const int64_t tiles = ((m + 127) / 128) * ((n + 191) / 192);
  const int64_t stages = k / 64;
  int64_t splits = 1;
  if (tiles > 0 && tiles < NUM_CUS) splits = std::min<int64_t>(NUM_CUS / tiles, stages / 8);
  if (splits <= 1) return PpPlan{CFG_PP_128x192, 1, 0};
  int64_t sps = (stages + splits - 1) / splits;
  sps = (sps + 3) / 4 * 4;
  splits = (stages + sps - 1) / sps;
  return PpPlan{CFG_PP_128x192, (int)splits, (int)sps};
}

static int pick_cfg(int kind, int64_t m, int64_t n, int64_t k) { return pick_plan(kind, m, n, k).cfg; }

void qgemm_tile_for(int kind, int64_t m, int64_t n, int64_t k, int* bm, int* bn) {
  SkPlan sp;
  if (skinny_plan(kind, m, n, k, &sp)) {
    *bm = 16 * sp.fm;
    *bn = SK_BN;
    return;
  }
  switch (pick_cfg(kind, m, n, k)) {
    case CFG_PP_256x256: *bm = 256; *bn = 256; return;
    case CFG_PP_256x192: *bm = 256; *bn = 192; return;
    case CFG_PP_256x288: *bm = 256; *bn = 288; return;
    case CFG_PP_256x128: *bm = 256; *bn = 128; return;
    default: *bm = 128; *bn = 192; return;
  }
}

int64_t qgemm_partial_bytes(int kind, int64_t m, int64_t n, int64_t k) {
  int splits;
  SkPlan p;
  if (skinny_plan(kind, m, n, k, &p))
    splits = p.splits;
  else
    splits = pick_plan(kind, m, n, k).splits;
  if (splits == 1) return 0;
  int64_t mn;
  if (__builtin_mul_overflow(m, n, &mn) || mn > INT64_MAX / 4 / splits) return -1;
  return mn * 4 * splits;
}

template <int KIND>
static hipError_t launch_kind(const GemmArgs& g, hipStream_t stream) {
  SkPlan sp;
  if (g.lora.t) {
    // The side path rides in the store of the single-pass W8A8 kernel; other
    // plans (few rows, split K) store the product and then add the side path
    // with the standalone up-projection, whose arithmetic is the same (fp32 C:
    // the same two roundings, the same MFMA sequence).
    const bool fused = KIND == GEMM_W8A8 && !g.c_bf16 && !g.acc_out && !skinny_plan(KIND, g.m, g.n, g.k, &sp) &&
                       pick_plan(KIND, g.m, g.n, g.k).splits == 1;
    if (!fused) {
      GemmArgs g2 = g;
      g2.lora.t = nullptr;
      const hipError_t e = launch_kind<KIND>(g2, stream);
      if (e != hipSuccess) return e;
      return launch_lora_up(g.lora.t, g.lora.b, true, g.lora.ldb, g.lora.alpha, g.m, g.n, g.lora.r, g.c, g.c_bf16,
                            g.ldc, stream);
    }
  }
  if (skinny_plan(KIND, g.m, g.n, g.k, &sp)) {
    if (sp.splits > 1 && !g.part) return hipErrorInvalidValue;
    return launch_skinny<KIND>(g, sp, stream);
  }
  const PpPlan pl = pick_plan(KIND, g.m, g.n, g.k);
  if (pl.splits > 1 && !g.part) return hipErrorInvalidValue;
  switch (pl.cfg) {
    case CFG_PP_256x256:
      if constexpr (KIND == GEMM_W8A8)
        return launch_pp<KIND, 256, 256, 128, 64, 4>(g, stream, (g.n + 255) / 256 >= 64 ? 4 : 8);
      if constexpr (KIND == GEMM_W8) return launch_pp<KIND, 256, 256, 128, 64, 3, 3>(g, stream, 4);
      break;
    case CFG_PP_256x192:
      if constexpr (KIND == GEMM_W8A8) return launch_pp<KIND, 256, 192, 64, 96, 4>(g, stream);
      // W4: four 38 KB stages (three measured 261 us at 4032x12288 -> 3072, four 254 us, same box and bytes).
      if constexpr (KIND == GEMM_W4) return launch_pp<KIND, 256, 192, 128, 48, 4, 2>(g, stream, 4);
      break;
    case CFG_PP_256x288:
      // The side path in the store needs registers this tile does not leave
      // (its instance spills): such calls take 256x192 tiles.
      if constexpr (KIND == GEMM_W8A8) {
        if (g.lora.t) return launch_pp<KIND, 256, 192, 64, 96, 4>(g, stream);
        return launch_pp<KIND, 256, 288, 64, 144, 4>(g, stream);
      }
      break;
    case CFG_PP_256x128:
      if constexpr (KIND == GEMM_W4A8) return launch_pp<KIND, 256, 128, 128, 32, 5, 2>(g, stream, 4);
      break;
    default:
      if constexpr (KIND == GEMM_W4A8) return launch_pp<KIND, 128, 192, 64, 48, 5, 2>(g, stream, 4, pl.splits, pl.sps);
      return launch_pp<KIND, 128, 192, 64, 48, 5>(g, stream, 4, pl.splits, pl.sps);
  }
  return hipErrorInvalidValue;
}

// The no-allocation entry point's split-K partial sums. In host code the
// array's name stands for a host-side shadow, not a device address: the
// address each device holds it at comes from hipGetSymbolAddress, called once
// per device with that device current, and only that address is passed on.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_qgemm(const GemmArgs& g, hipStream_t stream) {
  switch (g.kind) {
    case GEMM_W8: return launch_kind<GEMM_W8>(g, stream);
    case GEMM_W4: return launch_kind<GEMM_W4>(g, stream);
    case GEMM_W8A8: return launch_kind<GEMM_W8A8>(g, stream);
    case GEMM_W4A8: return launch_kind<GEMM_W4A8>(g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tp
