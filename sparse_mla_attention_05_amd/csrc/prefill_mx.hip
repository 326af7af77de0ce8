// gfx950 64-head kernel of the sparse MLA forward over an fp8 e4m3fn pool,
// 576- or 512-wide rows, with both products on the fp8 matrix cores.
//
// The method (per row r, head h, over the row's valid slots j):
//   s_j = sm_scale * q[r,h] . K[idx_j] (D_qk columns), out = softmax(s) V
//   (V = first 512 columns), lse = ln sum_j exp(s_j)
// after "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159):
// Technical Details and the commit notes on the 64-head program (each key
// tile gathered once for all 64 heads, rope dotted after the latent part,
// per-tensor fp8 scale taken off in the epilogue).
//
// The pages widen the fp8 keys to bf16 for their dots and reject fp8 dots on
// accuracy grounds (a single fp8 P). This kernel keeps the dots on
// v_mfma_scale_f32_16x16x128_f8f6f4, which on gfx950 does four times the
// work of a bf16 16x16x32 dot in about twice its time, and keeps bf16-class
// accuracy by splitting the bf16/fp32 operands into two e4m3 terms:
//  * q (bf16, 8 significant bits) times a power of two 2^e that puts the
//    wave's largest |q| in [128, 256) is q' = hi + lo/16 with hi = e4m3(q')
//    and lo = e4m3((q' - hi) * 16). The residual q' - hi is a multiple of
//    q's last bit no larger than half of hi's, so it has at most 4
//    significant bits and lo holds it exactly: the split is exact except for
//    elements below 2^-14 of the largest, where it errs by 2^-22 of it.
//    The MFMA's E8M0 block scales apply 2^-e and 2^-(e+4), so S = K.q comes
//    out exactly as with bf16 dots, up to fp32 accumulation order.
//  * P = 2^(s - m) <= 2^8 (see below) splits the same way into two e4m3
//    terms, 8 significant bits in all, the precision of the pages' bf16 P.
//  * The fp8 keys and values are used as stored (exact), so tiles stay fp8
//    in LDS: half the bytes of a bf16 tile, and no widening anywhere.
//
// Layout of the work (gfx950 specific, not from the pages):
//  * One workgroup = (row, 64 heads, split), 4 wavefronts, one per SIMD, one
//    workgroup per CU. Wave w owns heads 16w..16w+15 for the whole walk: it
//    scores all 128 slots of a tile for its heads, keeps its own softmax
//    state and accumulates O for all 512 columns. The waves share only the
//    LDS tile, so nothing is exchanged between them.
//  * Tiles of 128 slots are gathered by LDS DMA (buffer_load ... lds)
//    straight from the pool into LDS, double buffered: a structured buffer
//    of stride = the pool's row pitch turns each slot index into a row, and
//    a negative index falls outside its records and reads zeros. One
//    barrier per tile publishes the next tile and frees the last one.
//  * Tile row p of LDS holds slot 32(p/32) + 16(p%2) + (p%32)/2, chosen so
//    that a wave's DMA reads 16 consecutive indices per lane and the eight
//    rows of each transposed byte read (ds_read_b64_tr_b8) are adjacent. The
//    16-byte chunk c of row p sits at c ^ (p & 15), which keeps the key reads
//    (16 rows, stride 2) and the value reads (16 adjacent rows) free of bank
//    conflicts on gfx950, where a ds_read_b128 serves in one cycle the 16
//    lanes with equal lane bit 5 and equal parity of lane bits 2..4
//    (measured). The 64 rope bytes of a 576-wide row go to a separate region,
//    row = slot, chunk c at c ^ ((row >> 2) & 2).
//  * S^T = K Q^T leaves lane (head l16, group g) slots 16j + 4g + i of
//    block j; P^T is packed in exactly that lane (byte 8m + t of the PV B
//    operand = slot 32m + 16(t & 1) + 4g + t/2), and the value fragment's
//    transposed reads deliver the matching slot order, so P never moves.
//  * The rope columns run as one MFMA per block whose 128-deep k holds the
//    64 rope columns twice: once against q's hi term, once against its lo
//    term, the two halves scaled by their own E8M0 block scales.
//  * Online softmax in the exp2 domain with a lazy reference: a wave keeps
//    its head's reference m while every weight stays below 2^8; when a tile
//    would exceed it (or at the first tile with a valid slot) the wave takes
//    the tile's maximum, rescales O and its sums, and recomputes the tile's
//    weights. Exact in real arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kMWaves = 4;
constexpr int kMTile = 128;       // slots per tile
constexpr int kMRow = 512;        // LDS bytes per tile row of the first 512 columns
constexpr int kMRope = 64;        // LDS bytes per tile row of the rope columns
constexpr int kMWord3 = 0x00020000;
constexpr int kE8One = 127;       // E8M0 code of 1
constexpr float kMLimit = 8.0f;   // weights stay below 2^kMLimit
// Largest gap (log2) between the weights' reference and O's: P enters O
// scaled by 2^gap, and 2^20 slots x 2^8 x 448 x 2^64 stays far below fp32's
// range.
constexpr float kMMaxDrift = 64.0f;

template <int DQK>
struct MCfg {
  static constexpr bool ROPE = DQK == 576;
  static constexpr int NOPE = kMTile * kMRow;  // 64 KB
  static constexpr int BUF = NOPE + (ROPE ? kMTile * kMRope : 0);
  static constexpr int LDS = 2 * BUF + 2 * kMTile * 4 + 64 * 4;
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Chunk permutation of tile row p (nope region).
__device__ __forceinline__ int row_perm(int p) { return p & 15; }

// Two fp32 values to two e4m3fn codes in half HI of `old` (round to
// nearest even; callers keep |v| <= 256, so nothing saturates).
// The conversion divides by its scale operand (a power of two here, so
// exactly): cvt2<HI>(old, a, b, 1/16) codes 16a and 16b.
template <bool HI>
__device__ __forceinline__ s16x2 cvt2(s16x2 old, float a, float b, float scale = 1.0f) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, scale, HI);
}

// Four fp32 values (a0, a1, b0, b1 -> bytes 0..3) to their hi and lo e4m3
// terms: v = hi + lo / 16 up to lo's rounding.
__device__ __forceinline__ void split4(float a0, float a1, float b0, float b1, uint32_t& hi,
                                       uint32_t& lo) {
  s16x2 h = cvt2<false>(s16x2{0, 0}, a0, a1);
  h = cvt2<true>(h, b0, b1);
  const uint32_t hw = __builtin_bit_cast(uint32_t, h);
  const auto ha = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, false);
  const auto hb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, true);
  s16x2 l = cvt2<false>(s16x2{0, 0}, a0 - ha[0], a1 - ha[1], 0.0625f);
  l = cvt2<true>(l, b0 - hb[0], b1 - hb[1], 0.0625f);
  hi = hw;
  lo = __builtin_bit_cast(uint32_t, l);
}

// D += A B on the fp8 matrix cores; A's block scale 1, B's 2^(sb - 127).
__device__ __forceinline__ floatx4 mx(const i32x8& a, const i32x8& b, floatx4 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kE8One, 0, sb);
}

__device__ __forceinline__ i32x8 cat(const u32x4& a, const u32x4& b) {
  return i32x8{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
}

// Every wave's LDS DMA and LDS writes are complete and visible, and every
// wave is past its reads of the buffer being refilled next. The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void sync_tile() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 scaled values to 16 hi codes (dwords 0..3) and 16 lo codes.
__device__ __forceinline__ void split16(const float (&v)[16], float sc, uint32_t (&hi)[4],
                                        uint32_t (&lo)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    split4(v[4 * k] * sc, v[4 * k + 1] * sc, v[4 * k + 2] * sc, v[4 * k + 3] * sc, hi[k], lo[k]);
}

// PAGED: slot indices of a paged pool are mapped to rows (a separate
// instance, so the plain pool's walk carries none of it).
template <int DQK, bool EPI, bool PAGED>
__global__ void __launch_bounds__(kMWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_mx_kernel(const FwdParams p) {
  using C = MCfg<DQK>;
  constexpr bool ROPE = C::ROPE;
  constexpr int BUF = C::BUF, NOPE = C::NOPE;

  __shared__ __attribute__((aligned(1024))) uint8_t tiles[2 * BUF];
  __shared__ __attribute__((aligned(16))) float kbias[2 * kMTile];  // 0 (valid slot) or -inf
  __shared__ float epi_cs[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar offsets
  const int l16 = lane & 15, g = lane >> 4, hh = lane >> 5;

  int64_t work = p.remap ? smla_xcd_work(blockIdx.x, p.grid) : int64_t(blockIdx.x);
  const int hblk = int(work % p.head_blocks);
  work /= p.head_blocks;
  const int split = int(work % p.splits);
  const int64_t r = work / p.splits;
  float cs_pre = 0.f;
  if constexpr (EPI) {
    if (p.epi.pos != nullptr && tid < 64) cs_pre = epi_cs_row(p.epi, r)[tid];
  }

  const int head = hblk * 64 + 16 * wave + l16;
  const bool head_ok = head < p.heads;
  const int ntiles = (p.topk + kMTile - 1) / kMTile;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);
  const int slot_end = min(p.topk, t_end * kMTile);

  // ---- index rows and the tile DMA
  const __amdgpu_buffer_rsrc_t idx_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(p.idx + r * p.idx_rs), 0, 4 * slot_end, kMWord3);
  const uint32_t rs = uint32_t(p.pool_rs_bytes);
  const uint32_t records = p.pool_bytes >= uint32_t(DQK) ? (p.pool_bytes - DQK) / rs + 1 : 0u;
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.pool), int16_t(rs), int(records), kMWord3);
  const uint32_t page_rows = PAGED ? uint32_t(p.page_bytes / p.pool_rs_bytes) : 0u;

  // This lane's slots of a tile (relative to t * 128 + 32 * wave): the DMA
  // rows 16 hh + k (k < 16), the rope rows 16 k' + lane / 4, the bias slot
  // lane % 32.
  int idn[16], idr[2], idb;
  // The whole offset goes in the vector operand, which the range check
  // covers (reads past slot_end return 0).
  auto load_idx = [&](int t) {
    const uint32_t base = uint32_t(4 * (t * kMTile + 32 * wave));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(idx_rsrc, base + uint32_t(4 * (16 * hh + 4 * q)), 0, 0));
#pragma unroll
      for (int k = 0; k < 4; ++k) idn[4 * q + k] = int(v[k]);
    }
    if constexpr (ROPE) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        idr[k] = __builtin_amdgcn_raw_buffer_load_b32(idx_rsrc, base + uint32_t(4 * (16 * k + (lane >> 2))), 0, 0);
    }
    idb = __builtin_amdgcn_raw_buffer_load_b32(idx_rsrc, base + uint32_t(4 * (lane & 31)), 0, 0);
  };
  // Slots past the split's end read 0 through the index range: mark them
  // invalid; then map slot indices of a paged pool to rows of page_rows.
  auto fix_idx = [&](int t) {
    const int base = t * kMTile + 32 * wave;
    if (base + 32 > slot_end) {
      asm volatile("" ::: "memory");  // a branch, not selects on every tile
#pragma unroll
      for (int k = 0; k < 16; ++k) idn[k] = base + 16 * hh + k < slot_end ? idn[k] : -1;
      if constexpr (ROPE) {
#pragma unroll
        for (int k = 0; k < 2; ++k) idr[k] = base + 16 * k + (lane >> 2) < slot_end ? idr[k] : -1;
      }
      idb = base + (lane & 31) < slot_end ? idb : -1;
    }
    if constexpr (PAGED) {
      auto map = [&](int i) -> int {
        return i < 0 ? -1
                     : int((uint32_t(i) >> p.page_shift) * page_rows + (uint32_t(i) & p.page_mask));
      };
#pragma unroll
      for (int k = 0; k < 16; ++k) idn[k] = map(idn[k]);
      if constexpr (ROPE) {
#pragma unroll
        for (int k = 0; k < 2; ++k) idr[k] = map(idr[k]);
      }
    }
  };
  // DMA of tile t into buffer b (indices loaded and fixed), and its slot
  // validity into kbias.
  const uint32_t dma_vb = (16u * uint32_t(lane & 31)) ^ (16u * uint32_t(hh));
  const uint32_t dma_rope = 512u + 16u * uint32_t((lane & 3) ^ ((lane >> 4) & 2));
  auto issue_dma = [&](int b) {
    uint8_t* buf = tiles + b * BUF;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t voff = dma_vb ^ uint32_t(32 * (k & 7));
      __builtin_amdgcn_struct_ptr_buffer_load_lds(
          pool_rsrc, (lds_void*)(buf + (32 * wave + 2 * k) * kMRow), 16, idn[k], int(voff), 0, 0, 0);
    }
    if constexpr (ROPE) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        __builtin_amdgcn_struct_ptr_buffer_load_lds(
            pool_rsrc, (lds_void*)(buf + NOPE + (32 * wave + 16 * k) * kMRope), 16, idr[k],
            int(dma_rope), 0, 0, 0);
    }
    if (lane < 32) kbias[b * kMTile + 32 * wave + lane] = idb >= 0 ? 0.f : kNegInf;
  };

  // q of this lane's head (computed once, while the first tile's DMA runs):
  // k-step s takes columns 128s + 16g and 128s + 64 + 16g (16 each); the
  // rope part columns 512 + 16g.
  i32x8 qhi[4], qlo[4], qrope;
  int sb_hi = 0, sb_lo = 0, sb_rope = 0;
  auto make_q = [&]() {
    // Every load is issued before any is used (one dtype branch, the
    // address of a masked head clamped into q): a branch per load would make
    // the compiler wait for each in turn.
    constexpr int NCH = ROPE ? 9 : 8;  // 16-column chunks: (s, h) = chunk 2s + h, then rope
    const int hq = head_ok ? head : p.heads - 1;
    const int64_t qp = r * p.q_rs + int64_t(hq) * p.q_hs;
    auto col_of = [&](int c) { return c < 8 ? 128 * (c >> 1) + 64 * (c & 1) + 16 * g : 512 + 16 * g; };
    float v[NCH][16];
    if (p.q_fp8) {
      u32x4 raw[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        raw[c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.q) + qp + col_of(c));
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x2 w = widen_fp8x4(raw[c][k]);
          v[c][4 * k] = __uint_as_float(w.x << 16);
          v[c][4 * k + 1] = __uint_as_float(w.x & 0xFFFF0000u);
          v[c][4 * k + 2] = __uint_as_float(w.y << 16);
          v[c][4 * k + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
    } else {
      u32x4 raw[NCH][2];
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          raw[c][h] = *reinterpret_cast<const u32x4*>(p.q + qp + col_of(c) + 8 * h);
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[c][8 * h + 2 * k] = __uint_as_float(raw[c][h][k] << 16);
            v[c][8 * h + 2 * k + 1] = __uint_as_float(raw[c][h][k] & 0xFFFF0000u);
          }
    }
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[c][k] = head_ok ? v[c][k] : 0.f;
        amax = fmaxf(amax, fabsf(v[c][k]));
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    // 2^e puts the wave's largest |q| in [128, 256)
    int e = 8 - __builtin_amdgcn_frexp_expf(amax);
    e = amax > 0.f ? min(max(e, -100), 100) : 0;
    const float sc = __builtin_ldexpf(1.0f, e);
    sb_hi = kE8One - e;
    sb_lo = kE8One - e - 4;
    sb_rope = hh == 0 ? sb_hi : sb_lo;  // k blocks 0,1: hi term; 2,3: lo term
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t ha[4], la[4], hb[4], lb[4];
      split16(v[2 * s], sc, ha, la);
      split16(v[2 * s + 1], sc, hb, lb);
      qhi[s] = i32x8{int(ha[0]), int(ha[1]), int(ha[2]), int(ha[3]),
                     int(hb[0]), int(hb[1]), int(hb[2]), int(hb[3])};
      qlo[s] = i32x8{int(la[0]), int(la[1]), int(la[2]), int(la[3]),
                     int(lb[0]), int(lb[1]), int(lb[2]), int(lb[3])};
    }
    if constexpr (ROPE) {
      uint32_t h4[4], l4[4];
      split16(v[8], sc, h4, l4);
      qrope = i32x8{int(h4[0]), int(h4[1]), int(h4[2]), int(h4[3]),
                    int(l4[0]), int(l4[1]), int(l4[2]), int(l4[3])};
    } else {
      qrope = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  const float kv_scale = *p.kv_scale;
  const float cscale = p.sm_log2 * q_scale_of(p.q_scale) * kv_scale;

  // ---- per-lane LDS addresses (without the buffer base)
  // keys: block j reads tile row 32(j/2) + 2 l16 + (j & 1); its chunks are
  // permuted by row_perm of that row, which depends on l16 and j & 1 only.
  int kro[2], kperm[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    kro[par] = (2 * l16 + par) * kMRow;
    kperm[par] = row_perm(2 * l16 + par);
  }
  // values: read m of a 16-column block covers tile rows 32m + 8g .. +7; the
  // lane pair (2t, 2t+1) of a group points at row 32m + 8g + t.
  const int vrow = 8 * g + (l16 >> 1);
  const int vro = vrow * kMRow + 8 * (l16 & 1);
  const int vperm16 = 16 * row_perm(vrow);
  // rope: block j reads rope row 16j + l16, chunk g permuted by its row.
  const int rro = NOPE + l16 * kMRope + 16 * (g ^ ((l16 >> 2) & 2));

  floatx4 o[32];
  float m_o = kNegInf;  // reference (log2 domain, an integer) of O and the row sums
  float m_w = kNegInf;  // reference of the weights, m_w >= m_o
  float l_run = 0.f;    // this lane's share of the head's row sum (reference m_o)
  int redo = 0;

  // One walk over the split's tiles. The first walk fixes the references as
  // it goes; a second one (only when a score jumped by more than
  // kMMaxDrift above the first valid tile's maximum) starts from the first
  // walk's last weight reference, which no later score exceeds by 2^kMLimit.
  auto walk = [&](bool first) {
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    if (!first) m_o = m_w;
    float nm = m_o == kNegInf ? 0.f : -m_w;
    const int t0 = t_begin;
    if (t0 < t_end) {
      load_idx(t0);
      fix_idx(t0);
      issue_dma(0);
    }
    if (t0 + 1 < t_end) load_idx(t0 + 1);
    if (first) make_q();
    sync_tile();  // tile t0 and its flags visible
    if (t0 + 1 < t_end) {
      fix_idx(t0 + 1);
      issue_dma(1);
    }
    if (t0 + 2 < t_end) load_idx(t0 + 2);
    for (int t = t0; t < t_end; ++t) {
      const int b = (t - t0) & 1;
      const uint8_t* B = tiles + b * BUF;
      const float* kb = kbias + b * kMTile + 4 * g;

      // ---- S^T = K Q^T over pairs of blocks (2m, 2m + 1): per pair, one
      // unit per k-step (unit 4: the rope) of four dots (two for the rope),
      // the two blocks' dots alternating. With one wavefront per SIMD the
      // wave issues in order and an MFMA only runs alongside what the wave
      // issues before the next one, so every dot is followed by its share of
      // the other work: a quarter of the key fragment reads for two units
      // ahead, and one of the previous pair's ten softmax jobs (eight
      // weights, two splits into P^T bytes) spread over the pair's dots. The
      // scheduling fences keep exactly that order.
      constexpr int UPP = ROPE ? 5 : 4;  // units per pair of blocks
      constexpr int NU = 4 * UPP;
      constexpr int MPP = ROPE ? 18 : 16;  // dots per pair
      constexpr int KR = 3;                // units of key fragments in the ring
      floatx4 sacc[8];
      float pprev[4], pcur[4];
      float xmax = kNegInf, lt = 0.f;
      uint32_t phi[8], plo[8];
      // key fragment f (0, 1: block 2pm, 2pm + 1) of unit u, half hf (the
      // 16 bytes at columns 128s + 16g, then 128s + 64 + 16g; the rope unit
      // reads its chunk twice)
      auto kread = [&](int u, int f, int hf) -> u32x4 {
        const int j = 2 * (u / UPP) + f, sj = u % UPP, par = j & 1;
        if (ROPE && sj == 4) return *reinterpret_cast<const u32x4*>(B + rro + 16 * j * kMRope);
        const uint8_t* krow = B + kro[par] + 32 * (j >> 1) * kMRow;
        return *reinterpret_cast<const u32x4*>(krow + 16 * ((8 * sj + 4 * hf + g) ^ kperm[par]));
      };
      // Slot validity (0 or -inf) of block j's four slots of this lane, read
      // a pair of blocks ahead of its use: a read issued just before its use
      // would make the wait drain every key fragment read in flight.
      floatx4 bias_v[8];
      // weight i of block j
      auto weight = [&](int j, int i) {
        const float x = __builtin_fmaf(sacc[j][i], cscale, bias_v[j][i] + nm);
        xmax = fmaxf(xmax, x);
        pcur[i] = __builtin_amdgcn_exp2f(x);
        lt += pcur[i];
        if (i == 3 && !(j & 1)) {
#pragma unroll
          for (int k = 0; k < 4; ++k) pprev[k] = pcur[k];
        }
      };
      // half h of the P^T bytes 8m .. 8m + 7 from the weights of blocks 2m
      // (pprev) and 2m + 1 (pcur)
      auto split_half = [&](int m, int h) {
        split4(pprev[2 * h], pcur[2 * h], pprev[2 * h + 1], pcur[2 * h + 1], phi[2 * m + h],
               plo[2 * m + h]);
      };
      // softmax job k (0..9) of pair pm: weights of block 2pm (k < 4), of
      // block 2pm + 1 (k = 4, 5, 7, 8), splits (k = 6, 9)
      auto job = [&](int pm, int k) {
        if (k < 4) weight(2 * pm, k);
        else if (k == 4 || k == 5) weight(2 * pm + 1, k - 4);
        else if (k == 6) split_half(pm, 0);
        else if (k == 7 || k == 8) weight(2 * pm + 1, k - 5);
        else split_half(pm, 1);
        // computed here, between the dots: left alone the compiler sinks the
        // weights below the rare-path branch, after all the dots
        asm volatile("" : "+v"(pcur[0]), "+v"(pcur[1]), "+v"(pcur[2]), "+v"(pcur[3]), "+v"(lt));
      };
      {
        u32x4 kring[KR][2][2];
#pragma unroll
        for (int u = 0; u < KR - 1; ++u)
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) kring[u][f][hf] = kread(u, f, hf);
        bias_v[0] = *reinterpret_cast<const floatx4*>(kb);
        bias_v[1] = *reinterpret_cast<const floatx4*>(kb + 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int pm = u / UPP, sj = u % UPP, j0 = 2 * pm, j1 = 2 * pm + 1;
          const bool rope_u = ROPE && sj == 4;
          const int nmf = rope_u ? 2 : 4;  // dots of this unit
          const int un = u + KR - 1;       // unit whose fragments this one reads
          const i32x8 f0 = cat(kring[u % KR][0][0], kring[u % KR][0][1]);
          const i32x8 f1 = cat(kring[u % KR][1][0], kring[u % KR][1][1]);
          if (sj == 0) sacc[j0] = sacc[j1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int mi = 0; mi < nmf; ++mi) {
            if (rope_u) {
              if (mi == 0) sacc[j0] = mx(f0, qrope, sacc[j0], sb_rope);
              else sacc[j1] = mx(f1, qrope, sacc[j1], sb_rope);
            } else {
              const int f = mi & 1;
              const i32x8& kf = f ? f1 : f0;
              floatx4& acc = f ? sacc[j1] : sacc[j0];
              acc = mx(kf, mi < 2 ? qhi[sj] : qlo[sj], acc, mi < 2 ? sb_hi : sb_lo);
            }
            __builtin_amdgcn_sched_barrier(0);
            // this dot's share of the key reads of unit un (4 reads per unit)
            if (un < NU) {
#pragma unroll
              for (int r = 0; r < 4 / nmf; ++r) {
                const int q = mi * (4 / nmf) + r;  // read q: fragment q / 2, half q % 2
                kring[un % KR][q >> 1][q & 1] = kread(un, q >> 1, q & 1);
              }
            }
            // the next pair's slot validity, at this pair's first dot
            if (sj == 0 && mi == 0 && pm < 3) {
              bias_v[2 * pm + 2] = *reinterpret_cast<const floatx4*>(kb + 32 * pm + 32);
              bias_v[2 * pm + 3] = *reinterpret_cast<const floatx4*>(kb + 32 * pm + 48);
            }
            // the previous pair's softmax jobs assigned to this dot
            if (pm > 0) {
              const int oi = (rope_u ? 16 : 4 * sj) + mi;  // dot index within the pair
#pragma unroll
              for (int k = 0; k < 10; ++k)
                if ((k * MPP) / 10 == oi) job(pm - 1, k);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 10; ++k) job(3, k);

      // ---- reference moves (rare): the first tile with a valid slot sets
      // both references to its maximum (rounded up to an integer); a tile
      // whose weights would pass 2^kMLimit moves the weights' reference m up
      // to its maximum, and the tile's weights are taken again. O and the row
      // sums keep the reference m_o: P enters them through the E8M0 block
      // scale 2^(m - m_o) of the P^T operand, so O is never rescaled.
      const bool move = xmax > kMLimit || (m_o == kNegInf && xmax != kNegInf);
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            tmax = fmaxf(tmax, __builtin_fmaf(sacc[j][i], cscale, kb[16 * j + i]));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (tmax != kNegInf) {
          if (m_o == kNegInf) {
            m_o = m_w = __builtin_ceilf(tmax);
          } else if (tmax > m_w + kMLimit) {
            m_w = __builtin_ceilf(tmax);
          }
        }
        if (m_w - m_o > kMMaxDrift) redo = 1;  // past what O can absorb: walk again
        nm = m_o == kNegInf ? 0.f : -m_w;
        xmax = kNegInf;
        lt = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) bias_v[j] = *reinterpret_cast<const floatx4*>(kb + 16 * j);
#pragma unroll
        for (int pm = 0; pm < 4; ++pm)
#pragma unroll
          for (int k = 0; k < 10; ++k) job(pm, k);
      }
      const int drift = m_o == kNegInf ? 0 : int(fminf(m_w - m_o, kMMaxDrift));
      l_run += __builtin_ldexpf(lt, drift);
      const int sb_ph = kE8One + drift, sb_pl = kE8One - 4 + drift;

      // ---- O^T += V^T P^T for the 32 column blocks; each value fragment
      // feeds both terms of P and is read VR - 1 blocks ahead.
      {
        const i32x8 ph = i32x8{int(phi[0]), int(phi[1]), int(phi[2]), int(phi[3]),
                               int(phi[4]), int(phi[5]), int(phi[6]), int(phi[7])};
        const i32x8 pl = i32x8{int(plo[0]), int(plo[1]), int(plo[2]), int(plo[3]),
                               int(plo[4]), int(plo[5]), int(plo[6]), int(plo[7])};
        const uint8_t* vb = B + vro;
        // read m (0..3) of column block c: 8 bytes, slots of tile rows
        // 32m + 8g .. 32m + 8g + 7
        auto vread = [&](int c, int m) -> u32x2 {
          return lds_read_tr8(vb + ((16 * c) ^ vperm16) + 32 * m * kMRow);
        };
        // two column blocks per unit, their dots alternating; each dot is
        // followed by two of the eight value reads of the unit two ahead
        constexpr int VR = 3;
        u32x2 vring[VR][2][4];
#pragma unroll
        for (int u = 0; u < VR - 1; ++u)
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int m = 0; m < 4; ++m) vring[u][f][m] = vread(2 * u + f, m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int c = 2 * u, un = u + VR - 1;
          i32x8 vf[2];
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const u32x2* w = vring[u % VR][f];
            vf[f] = i32x8{int(w[0].x), int(w[0].y), int(w[1].x), int(w[1].y),
                          int(w[2].x), int(w[2].y), int(w[3].x), int(w[3].y)};
          }
#pragma unroll
          for (int mi = 0; mi < 4; ++mi) {
            const int f = mi & 1;
            o[c + f] = mx(vf[f], mi < 2 ? ph : pl, o[c + f], mi < 2 ? sb_ph : sb_pl);
            __builtin_amdgcn_sched_barrier(0);
            if (un < 16) {
#pragma unroll
              for (int r = 0; r < 2; ++r) {
                const int q = 2 * mi + r;  // read q: block q / 4, read q % 4
                vring[un % VR][q >> 2][q & 3] = vread(2 * un + (q >> 2), q & 3);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }

      // O and q stay in the accumulator registers, which MFMA operands may
      // come from, leaving the vector registers to the operand rings (left
      // alone, the allocator copies them between the two files).
#pragma unroll
      for (int c = 0; c < 32; ++c) asm volatile("" : "+a"(o[c]));
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" : "+a"(qhi[s]), "+a"(qlo[s]));
      asm volatile("" : "+a"(qrope));

      sync_tile();  // buffer b free; tile t+1 and its flags visible
      if (t + 2 < t_end) {
        fix_idx(t + 2);
        issue_dma(b);
      }
      if (t + 3 < t_end) load_idx(t + 3);
    }
  };
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
    walk(pass == 0);
    if (pass == 1 || __syncthreads_or(redo) == 0) break;
  }

  // ---- epilogue: the head's row sum over the four lane groups; normalise;
  // store.
  float lt_tot = l_run + __shfl_xor(l_run, 16);
  lt_tot += __shfl_xor(lt_tot, 32);
  if constexpr (EPI) {
    if (tid < 64) epi_cs[tid] = cs_pre;
    __syncthreads();
  }
  if (!head_ok) return;
  const float inv = lt_tot > 0.f ? kv_scale / lt_tot : 0.f;
  const bool split_mode = p.part_o != nullptr;
  if (EPI && !split_mode) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const floatx4 ra = o[2 * m] * inv, rb = o[2 * m + 1] * inv;
      float va[4] = {ra[0], ra[1], ra[2], ra[3]}, vb2[4] = {rb[0], rb[1], rb[2], rb[3]};
      epi_store_c16x2(p.epi, p.epi.pos != nullptr ? epi_cs : nullptr, r, head, 32 * m + 4 * g, va,
                      vb2);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const floatx4 res = o[c] * inv;
      const int col = 16 * c + 4 * g;
      if (!split_mode) {
        *reinterpret_cast<u32x2*>(p.out + r * p.out_rs + int64_t(head) * p.out_hs + col) =
            u32x2{pack_bf16(res[0], res[1]), pack_bf16(res[2], res[3])};
      } else {
        *reinterpret_cast<floatx4*>(
            p.part_o + ((int64_t(split) * p.rows + r) * p.heads + head) * kDv + col) = res;
      }
    }
  }
  if (g == 0) {
    const float lse = lt_tot > 0.f ? (m_o + __log2f(lt_tot)) * kLn2 : kNegInf;
    if (!split_mode)
      p.lse[r * p.lse_rs + int64_t(head) * p.lse_hs] = lse;
    else
      p.part_lse[(int64_t(split) * p.rows + r) * p.heads + head] = lse;
  }
}

}  // namespace

KernelShape prefill_mx_shape(int dqk) {
  KernelShape k;
  k.waves = kMWaves;
  k.tile = kMTile;
  if (dqk == 576)
    k.lds_bytes = MCfg<576>::LDS;
  else if (dqk == 512)
    k.lds_bytes = MCfg<512>::LDS;
  else
    k = KernelShape{};
  return k;
}

template <int DQK, bool PAGED>
void launch_mx(const FwdParams& p, bool epi, dim3 grid, dim3 block, hipStream_t st) {
  if (epi)
    hipLaunchKernelGGL((prefill_mx_kernel<DQK, true, PAGED>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((prefill_mx_kernel<DQK, false, PAGED>), grid, block, 0, st, p);
}

int launch_prefill_mx(const FwdParams& p, int dqk, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool epi = epi_active(p.epi) && p.part_o == nullptr;
  const bool paged = p.page_shift != 31;
  const dim3 grid(uint32_t(p.grid)), block(kMWaves * 64);
  if (dqk == 576)
    paged ? launch_mx<576, true>(p, epi, grid, block, st) : launch_mx<576, false>(p, epi, grid, block, st);
  else if (dqk == 512)
    paged ? launch_mx<512, true>(p, epi, grid, block, st) : launch_mx<512, false>(p, epi, grid, block, st);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace smla
