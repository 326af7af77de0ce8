// Host-only launch planner for the sparse MLA forward. No HIP calls, so it is
// unit-testable on a machine without a GPU.
//
// Choices, after the launcher rules described in "[Triton/Gluon] GFX950
// sparse mla optimizations" (aiter PR 6159) commit notes (program size by
// head count and rounds of programs; split count sized so small launches fill
// the CUs; XCD remap only for rows of two or more head blocks), re-derived for
// this kernel:
//  * head block: 16 heads for H <= 16, 32 for H <= 32, else 64, so one
//    workgroup gathers and stages each KV tile once for as many heads as fit;
//    except that fp8 pools with H <= 32 take 16-head blocks: the 16-head
//    decode kernel twice (its two head blocks of a row side by side on one
//    XCD) measured 260 us against 340 us for the 32-head staged kernel on
//    the 768-row, top-k 2048 decode at 32 heads.
//  * kernel: over bf16 pools the 64-head staged-tile kernel (variant 1);
//    it measured 3-14 % faster than the 8-wave kernel of prefill.hip on
//    every 64-head bf16 shape tried (96..2048 rows, top-k 512 and 2048;
//    55.3 against 63.2 us on the 192-row decode), which stays as variant 2.
//    Over fp8 pools 64-head blocks take the fp8-dot kernel (variant 3)
//    where its structured buffer can address the pool, else the 4-wave
//    kernel (variant 0; variant 4 forces it).
//  * splits: when rows x head blocks leave the CUs' workgroup slots
//    underfilled, each row's slots are split if a makespan model (rounds of
//    workgroups x (tiles per split + a fixed per-workgroup cost) + the
//    combine pass) says it pays; the combine kernel merges the partials.
//  * remap: XCD-aware order when a row has >= 2 head blocks or >= 2 splits,
//    so the workgroups that read the same KV rows share an L2.
#include <stdint.h>

#include <algorithm>

#include "launch.h"

namespace smla {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Cost-model constants, in slots walked (measured on MI355X: a 192-row,
// 64-head, 512-slot launch ran 1.5x slower with 2 splits and 1.7x with 4 than
// unsplit, which a per-workgroup cost of about 256 slots reproduces).
constexpr int64_t kWgFixedSlots = 256;
constexpr int64_t kCombineSlots = 128;

int make_plan(const Problem& pb, const smla_options* opt, int num_cus, smla_plan* plan,
              const char** err) {
  static const char* kBadHb = "head_block override must be 0, 16, 32 or 64";
  static const char* kBadSplit = "splits override must be in [0, 64]";
  static const char* kBadRemap = "remap override must be 0, 1 or 2";
  static const char* kBadGrid = "launch grid exceeds 2^31 - 1 workgroups";
  static const char* kBadVariant =
      "variant override must be 0..4 (2: 64 heads only; 3, 4: 64 heads, fp8 pools only)";
  static const char* kBadWgs = "workgroups must be >= 0";
  if (num_cus <= 0) num_cus = 256;
  *plan = smla_plan{};
  if (opt && opt->workgroups < 0) {
    *err = kBadWgs;
    return SMLA_ERR_INVALID_ARG;
  }

  int hb = 0;
  if (opt && opt->head_block) {
    if (opt->head_block != 16 && opt->head_block != 32 && opt->head_block != 64) {
      *err = kBadHb;
      return SMLA_ERR_INVALID_ARG;
    }
    hb = opt->head_block;
  } else {
    hb = pb.heads <= 16 ? 16 : (pb.heads <= 32 ? (pb.kv_fp8 ? 16 : 32) : 64);
  }
  int variant = 0;
  if (opt && opt->variant) {
    if (opt->variant < 1 || opt->variant > 4 || (opt->variant == 2 && hb != 64) ||
        (opt->variant >= 3 && !(hb == 64 && pb.kv_fp8))) {
      *err = kBadVariant;
      return SMLA_ERR_INVALID_ARG;
    }
    // 4 asks for the 4-wave fp8 kernel, which the plan reports as variant 0.
    variant = opt->variant == 4 ? 0 : opt->variant;
  } else if (hb == 64 && !pb.kv_fp8) {
    variant = 1;
  } else if (hb == 64) {
    // 64-head blocks over fp8 pools: the fp8-dot kernel, measured faster
    // than the 4-wave kernel on both prefill shapes in same-box runs (6 %
    // on the 16384-row 512-wide one, 1.2 % on the 8192-row 576-wide one).
    variant = 3;
  }
  // The decode (16 heads, fp8) and 64-head kernels read the pool through a
  // 32-bit buffer range; a larger pool takes the staged-tile kernel.
  if (uses_buffer_range(hb, pb.kv_fp8 != 0, variant) && pb.pool_bytes > kMaxBufferBytes)
    variant = 1;
  // The fp8-dot kernel addresses rows through a structured buffer; other pool
  // layouts take the 4-wave kernel.
  if (variant == 3 && !mx_pool_ok(pb.pool_rs_bytes, pb.page_bytes)) variant = 0;
  const KernelShape ks = kernel_shape(hb, pb.dqk, pb.kv_fp8 != 0, variant);
  const int waves = ks.waves;
  const int lds = ks.lds_bytes;
  const int64_t head_blocks = ceil_div(pb.heads, hb);
  const int64_t tiles = ceil_div(pb.topk, ks.tile);

  // Workgroups a CU holds at once: 160 KB of LDS and 8 waves (the kernels
  // need up to 256 VGPRs, i.e. 2 waves per SIMD).
  const int64_t by_lds = std::max<int64_t>(1, (160 * 1024) / lds);
  const int64_t by_waves = std::max<int64_t>(1, 8 / waves);
  const int64_t wg_per_cu = std::min(by_lds, by_waves);
  const int64_t slots = int64_t(num_cus) * wg_per_cu;
  const int64_t base = pb.rows * head_blocks;

  int64_t splits = 1;
  if (opt && opt->splits) {
    if (opt->splits < 0 || opt->splits > kMaxSplits) {
      *err = kBadSplit;
      return SMLA_ERR_INVALID_ARG;
    }
    splits = std::min<int64_t>(opt->splits, tiles);
  } else if (base > 0 && base < 2 * slots) {
    // Makespan in tile-walk units: the workgroups one CU runs times the tiles
    // each walks plus a fixed per-workgroup cost (Q load, first gather,
    // epilogue), plus the combine pass when splitting. Smallest cost wins;
    // ties keep fewer splits. Workgroups are counted per CU, not per
    // workgroup slot: the kernels are bound by the CU's memory traffic, so two
    // resident workgroups share it rather than doubling it (measured on the
    // 768-row, 16-head decode: 176 us unsplit against 193 us with 2 splits).
    auto cost = [&](int64_t s) {
      const int64_t tps_s = ceil_div(tiles, s);
      const int64_t rounds = ceil_div(base * s, int64_t(num_cus));
      return rounds * (tps_s * ks.tile + kWgFixedSlots) + (s > 1 ? kCombineSlots : 0);
    };
    int64_t best = cost(1);
    for (int64_t s = 2; s <= std::min<int64_t>(tiles, kMaxSplits); ++s) {
      const int64_t c = cost(s);
      if (c < best) {
        best = c;
        splits = s;
      }
    }
  }
  // No empty splits: every split walks at least one tile.
  const int64_t tps = ceil_div(tiles, splits);
  splits = ceil_div(tiles, tps);

  int remap;
  if (opt && opt->remap) {
    if (opt->remap != 1 && opt->remap != 2) {
      *err = kBadRemap;
      return SMLA_ERR_INVALID_ARG;
    }
    remap = opt->remap == 1 ? 1 : 0;
  } else {
    remap = (head_blocks >= 2 || splits >= 2) ? 1 : 0;
  }

  const int64_t grid = base * splits;
  if (grid > int64_t(0x7fffffff) || pb.rows * pb.heads > int64_t(0x7fffffff)) {
    *err = kBadGrid;
    return SMLA_ERR_UNSUPPORTED;
  }

  plan->head_block = hb;
  plan->head_blocks = int32_t(head_blocks);
  plan->splits = int32_t(splits);
  plan->remap = remap;
  plan->waves = waves;
  plan->lds_bytes = lds;
  plan->tiles_per_split = int32_t(tps);
  plan->tile_slots = ks.tile;
  plan->variant = variant;
  plan->grid = grid;
  if (splits > 1) {
    const int64_t o_bytes = splits * pb.rows * pb.heads * kDv * 4;
    const int64_t l_bytes = splits * pb.rows * pb.heads * 4;
    plan->workspace_bytes = ceil_div(o_bytes, 256) * 256 + ceil_div(l_bytes, 256) * 256;
  }
  return SMLA_OK;
}

}  // namespace smla
