// gfx950 64-head kernel of the sparse MLA forward over an fp8 e4m3fn pool,
// 576- or 512-wide rows, with both products on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4).
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
// accuracy grounds (a single fp8 P). This kernel keeps the dots on the fp8
// matrix cores and keeps bf16-class accuracy by splitting the bf16/fp32
// operands into two e4m3 terms:
//  * q (bf16, 8 significant bits) times a power of two 2^e that puts the
//    largest |q| of its 32-column block (one k-block of a dot) in [128, 256)
//    is q' = hi + lo/16 with hi = e4m3(q') and lo = e4m3((q' - hi) * 16).
//    The residual q' - hi is a multiple of q's last bit no larger than half
//    of hi's, so it has at most 4 significant bits and lo holds it exactly:
//    the split is exact except for elements below 2^-14 of their block's
//    largest, where it errs by 2^-22 of it. The MFMA's E8M0 block scales
//    (one per column and 32-deep k-block) apply 2^-e and 2^-(e+4), so
//    S = K.q comes out as with bf16 dots up to the fp8 matrix core's
//    accumulation, which is coarser than fp32 (measured: products summed in
//    groups of 8 aligned to each group's largest with a window under 17
//    bits, so a dot errs by about 2^-16 of its largest product; the LSE of a
//    sharply peaked row shows it). A block's scale depends on its own 32
//    values only, so each k-step of q is split as soon as it has landed.
//  * P = 2^(s - m) <= 2^8 (see below) splits the same way into two e4m3
//    terms, 8 significant bits in all, the precision of the pages' bf16 P.
//  * The fp8 keys and values are used as stored (exact), so tiles stay fp8
//    in LDS: half the bytes of a bf16 tile, and no widening anywhere.
//
// Layout of the work (gfx950 specific, not from the pages; the rates below
// were measured with probe kernels):
//  * One workgroup = (row, 64 heads, split), 4 wavefronts, one per SIMD, one
//    workgroup per CU. Wave (hp, kh) holds q of heads 32hp..32hp+31: it
//    scores slot half kh of each 64-slot tile (S^T = K Q^T, one 32x32 block)
//    and accumulates O^T for column half kh over all 64 slots; the two waves
//    of a head half swap their P through LDS (2 KB each way per tile).
//  * The 32x32x64 dot is chosen over the 16x16x128 one because a wave's own
//    vector work only issues in the part of a dot that follows its operand
//    reads (about 16 cycles): a 64-cycle 32x32x64 dot leaves room for about
//    eight vector instructions, a 32-cycle 16x16x128 dot for about three,
//    and the softmax and the P split need about six per dot.
//  * Tiles of 64 slots are gathered by LDS DMA (buffer_load ... lds)
//    straight from the pool into LDS: a structured buffer of stride = the
//    pool's row pitch turns each slot index into a row, and a negative index
//    falls outside its records and reads zeros. The indices come the same
//    way, a tile's 64 in one instruction. The DMA is issued as inline
//    assembly: the compiler, which cannot tell which LDS bytes a DMA writes,
//    would otherwise wait for every DMA in flight before the next LDS access
//    of any kind; every wait on them is the explicit one at the tile
//    barrier. A ring of four tiles: while
//    a wave scores tile t + 1 and weighs tile t (one phase), then multiplies
//    tile t's values (the next), tile t + 2 is landing and tile t + 3 is
//    being requested. One barrier per tile publishes P and the next tile.
//  * Within each 16-row group, tile row 2k + e holds slot 8e + k, so that a
//    wave's DMA reads 8 consecutive indices per lane and each transposed
//    byte read of the values (ds_read_b64_tr_b8) covers 8 adjacent rows. The
//    16-byte chunk c of row p sits at c ^ (2 (p & 7) + ((p >> 3) & 1)), which
//    keeps the key reads (ds_read_b128: one cycle serves the 16 lanes with
//    equal lane bit 5 and equal parity of lane bits 2..4) and the value reads
//    (a 32-lane half per cycle) free of bank conflicts. The 64 rope bytes of
//    a 576-wide row go to a separate three-tile ring, chunk c at
//    c ^ ((p >> 2) & 3).
//  * S^T leaves lane (head c, half h) the 16 slots 8(i/4) + 4h + i%4 of its
//    block; byte i of the P^T operand's half b is exactly S^T register i of
//    wave (hp, b), and the transposed value reads deliver the same slot
//    order, so P is never permuted, only copied to the partner.
//  * Online softmax in the exp2 domain with two integer references per
//    head: m_o for O and the row sums (shared by the wave pair, fixed at the
//    pair's first tile with a valid slot), and m_w for each wave's weights,
//    raised when a weight would pass 2^8. Each half's P enters the PV dot
//    through its own E8M0 block scale 2^(m_w - m_o), so O is never rescaled;
//    if a gap passes 2^64, the workgroup walks again from the final
//    references. Exact in real arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXWaves = 4;
constexpr int kXTile = 64;     // slots per tile
constexpr int kXRing = 4;      // tiles held in LDS (first 512 columns)
constexpr int kXRopeRing = 3;  // tiles held in LDS (rope columns)
constexpr int kXRow = 512;     // LDS bytes per tile row of the first 512 columns
constexpr int kXRope = 64;     // LDS bytes per tile row of the rope columns
constexpr int kXWord3 = 0x00020000;
constexpr int kE8One = 127;      // E8M0 code of 1
constexpr float kXLimit = 8.0f;  // weights stay below 2^kXLimit
// Largest gap (log2) between a weights' reference and O's: P enters O scaled
// by 2^gap, and 2^20 slots x 2^8 x 448 x 2^64 stays far below fp32's range.
constexpr float kXMaxDrift = 64.0f;
// Smallest gap applied (weights further below O's reference are below fp32's
// resolution of the sums); keeps the lo term's scale code 123 + gap >= 0.
constexpr float kXMinDrift = -123.0f;

template <int DQK>
struct XCfg {
  static constexpr bool ROPE = DQK == 576;
  static constexpr int NSTEP = ROPE ? 9 : 8;  // 64-deep k-steps of a score block
  static constexpr int NOPE = kXTile * kXRow;
  static constexpr int ROPEB = kXTile * kXRope;
  static constexpr int XPB = kXWaves * 64 * 32;  // P exchange of one tile
  static constexpr int OFF_ROPE = kXRing * NOPE;
  static constexpr int OFF_XP = OFF_ROPE + (ROPE ? kXRopeRing * ROPEB : 0);  // [2][XPB]
  static constexpr int OFF_XM = OFF_XP + 2 * XPB;                   // [2][4 waves][32] f32
  static constexpr int OFF_BIAS = OFF_XM + 2 * kXWaves * 32 * 4;    // [ring][64] f32
  static constexpr int OFF_XL = OFF_BIAS + kXRing * kXTile * 4;     // [4 waves][32] f32
  static constexpr int OFF_IDX = OFF_XL + kXWaves * 32 * 4;         // [ring][64] i32
  static constexpr int OFF_EPI = OFF_IDX + kXRing * kXTile * 4;     // 64 f32
  static constexpr int LDS = OFF_EPI + 64 * 4;
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Ring places of stream position t >= 0 (unsigned: one mask for the
// power-of-two ring, no sign fix-up).
// One of two buffer descriptors by value (a select of the values, not of
// their addresses, which would keep them in memory).
__device__ __forceinline__ i32x4 sel4(bool c, i32x4 a, i32x4 b) { return c ? a : b; }
__device__ __forceinline__ int ring(int t) { return int(uint32_t(t) % uint32_t(kXRing)); }
__device__ __forceinline__ int rope_ring(int t) { return int(uint32_t(t) % uint32_t(kXRopeRing)); }

// Tile row of slot s (within each group of 16 rows, row 2k + e holds slot
// 8e + k).
__device__ __forceinline__ int row_of_slot(int s) {
  return (s & ~15) | ((s & 7) << 1) | ((s >> 3) & 1);
}
// Chunk permutations: chunk c of tile row p sits at c ^ perm(p).
__device__ __forceinline__ int nope_perm(int p) { return ((p & 7) << 1) | ((p >> 3) & 1); }
__device__ __forceinline__ int rope_perm(int p) { return (p >> 2) & 3; }

// Two fp32 values to two e4m3fn codes in half HI of `old` (round to
// nearest even; callers keep |v| <= 256, so nothing saturates).
// The conversion divides by its scale operand (a power of two here, so
// exactly): cvt2<HI>(old, a, b, 1/16) codes 16a and 16b.
template <bool HI>
__device__ __forceinline__ s16x2 cvt2(s16x2 old, float a, float b, float scale = 1.0f) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, scale, HI);
}

// Four fp32 values (bytes 0..3 in order) to their hi and lo e4m3 terms:
// v = hi + lo / 16 up to lo's rounding.
__device__ __forceinline__ void split4(float a0, float a1, float a2, float a3, uint32_t& hi,
                                       uint32_t& lo) {
  s16x2 h = cvt2<false>(s16x2{0, 0}, a0, a1);
  h = cvt2<true>(h, a2, a3);
  const uint32_t hw = __builtin_bit_cast(uint32_t, h);
  const auto ha = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, false);
  const auto hb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, true);
  s16x2 l = cvt2<false>(s16x2{0, 0}, a0 - ha[0], a1 - ha[1], 0.0625f);
  l = cvt2<true>(l, a2 - hb[0], a3 - hb[1], 0.0625f);
  hi = hw;
  lo = __builtin_bit_cast(uint32_t, l);
}

// Buffer resource of `records` records of `stride` bytes at base (stride 0:
// a raw buffer of `records` bytes); word 3 as the loads here need it.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t stride, uint32_t records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(a)), int((uint32_t(a >> 32) & 0xFFFFu) | (stride << 16)), int(records),
               kXWord3};
}

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_void*)p));
}

// LDS DMA, 16 bytes per lane: record `index` (out of range: zeros), byte
// `voff`, to LDS at lds + 16 lane. lds must be wave-uniform. No vector
// register is written, so nothing in flight can be overwritten; completion
// is waited for explicitly (sync_tile).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and read by the same statement
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds, int index, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 idxen offen lds"
               :: "s"(lds), "v"(i32x2{index, int(voff)}), "s"(rsrc) : "memory", "m0");
}

// LDS DMA, 4 bytes per lane from byte voff of a raw buffer (out of range:
// zero) to LDS at lds + 4 lane.
__device__ __forceinline__ void dma4(const i32x4& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// D += A B on the fp8 matrix cores; A's block scale 1, B's 2^(code - 127)
// with code byte SEL of sb (lane j gives the scale of column j % 32,
// k-block j / 32).
template <int SEL = 0>
__device__ __forceinline__ floatx16 mx32(const i32x8& a, const i32x8& b, floatx16 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kE8One, SEL, sb);
}
__device__ __forceinline__ floatx16 mx32_byte(const i32x8& a, const i32x8& b, floatx16 c, int sb,
                                              int sel) {
  switch (sel & 3) {
    case 0: return mx32<0>(a, b, c, sb);
    case 1: return mx32<1>(a, b, c, sb);
    case 2: return mx32<2>(a, b, c, sb);
    default: return mx32<3>(a, b, c, sb);
  }
}

// Exponent e that puts a bf16 magnitude pattern m (|x| as 15 bits) in
// [128, 256) once scaled by 2^e; 0 for m = 0 (an all-zero block).
__device__ __forceinline__ int block_exp(uint32_t m) {
  const int e = 134 - int(m >> 7);  // m = 1.f x 2^(E - 127): e = 7 - (E - 127)
  return m == 0u ? 0 : min(max(e, -100), 100);
}

__device__ __forceinline__ i32x8 cat(const u32x4& a, const u32x4& b) {
  return i32x8{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
}

__device__ __forceinline__ i32x8 pack8(const uint32_t (&w)[8]) {
  return i32x8{int(w[0]), int(w[1]), int(w[2]), int(w[3]), int(w[4]), int(w[5]), int(w[6]), int(w[7])};
}

// Every wave's LDS DMA and LDS writes are complete and visible, and every
// wave is past its reads before the barrier. The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void sync_tile() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // the same wait, visible to the compiler (no cost: the counters are zero),
  // so that it adds none of its own for loads issued before this point
  __builtin_amdgcn_s_waitcnt(0);
}

// PAGED: slot indices of a paged pool are mapped to rows (a separate
// instance, so the plain pool's walk carries none of it). TWO: the walk
// continues over a second segment (its own 2-D pool, scale and index rows)
// after the main top-k, as one list of tiles (a separate instance too).
template <int DQK, bool EPI, bool PAGED, bool TWO>
__global__ void __launch_bounds__(kXWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_mx_kernel(const FwdParams p) {
  using C = XCfg<DQK>;
  constexpr bool ROPE = C::ROPE;
  constexpr int NSTEP = C::NSTEP;
  constexpr int NNOPE = 8;  // k-steps over the first 512 columns

  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
  float* const kbias = reinterpret_cast<float*>(smem + C::OFF_BIAS);  // 0 (valid) or -inf
  float* const xm = reinterpret_cast<float*>(smem + C::OFF_XM);
  float* const xl = reinterpret_cast<float*>(smem + C::OFF_XL);
  float* const epi_cs = reinterpret_cast<float*>(smem + C::OFF_EPI);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar offsets
  const int hp = wave >> 1, kh = wave & 1;
  const int c32 = lane & 31, h = lane >> 5;

  // This workgroup's work items j = blockIdx.x + k G (k < n_items), each a
  // (row, head block, split). A workgroup walks several items only when the
  // rows are not split (the launch then has fewer workgroups than items), so
  // all its items cover the same tiles.
  const int64_t total = p.grid;
  const int64_t G = gridDim.x;
  const int n_items =
      __builtin_amdgcn_readfirstlane(int((total - int64_t(blockIdx.x) + G - 1) / G));
  int hblk, split;
  // Row of item k (and its head block and split); uniform, in scalar
  // registers. Item numbers are below 2^32 (a grid size).
  auto item_of = [&](int k, int& hb_o, int& sp_o) -> int64_t {
    const int64_t j = int64_t(blockIdx.x) + int64_t(k) * G;
    const uint32_t wk = uint32_t(p.remap ? smla_xcd_work(j, total) : j);
    const uint32_t hb = uint32_t(p.head_blocks), sp = uint32_t(p.splits);
    hb_o = __builtin_amdgcn_readfirstlane(int(wk % hb));
    sp_o = __builtin_amdgcn_readfirstlane(int(wk / hb % sp));
    return int64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(wk / hb / sp))));
  };
  int64_t r = item_of(0, hblk, split);
  float cs_pre = 0.f;
  auto load_cs = [&]() {
    if constexpr (EPI) {
      if (p.epi.pos != nullptr && tid < 64) cs_pre = epi_cs_row(p.epi, r)[tid];
    }
  };
  load_cs();

  int head = hblk * 64 + 32 * hp + c32;
  bool head_ok = head < p.heads;
  // Tiles [0, T1) hold the main top-k (its last one padded with invalid
  // slots), tiles [T1, ntiles) the second segment when one is walked; the
  // splits partition that list.
  const int T1 = (p.topk + kXTile - 1) / kXTile;
  const int ntiles = TWO ? T1 + (p.topk2 + kXTile - 1) / kXTile : T1;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);
  const int slot_end = min(p.topk, t_end * kXTile);
  const int slot_end2 = TWO ? max(0, min(p.topk2, (t_end - T1) * kXTile)) : 0;
  auto in_second = [&](int t) { return TWO && t >= T1; };  // tile t of the second segment

  // ---- index rows and the tile DMA
  auto idx_rsrc_of = [&](int64_t row) { return make_rsrc(p.idx + row * p.idx_rs, 0, 4u * uint32_t(slot_end)); };
  auto idx2_rsrc_of = [&](int64_t row) {
    return TWO ? make_rsrc(p.idx2 + row * p.idx2_rs, 0, 4u * uint32_t(slot_end2)) : make_rsrc(p.idx, 0, 0u);
  };
  i32x4 idx_rsrc = idx_rsrc_of(r), idx2_rsrc = idx2_rsrc_of(r);
  // the next item's, while the walk streams into it
  i32x4 idx_rsrc_next = idx_rsrc, idx2_rsrc_next = idx2_rsrc;
  // The next item's q rows (64 heads of a row, contiguous when the heads
  // are), fetched into the L2 during the walk's last steps: one dword per
  // 64 bytes. A zero-record resource fetches nothing.
  const i32x4 null_rsrc = make_rsrc(p.q, 0, 0u);
  i32x4 q_pf_rsrc = null_rsrc;
  const uint32_t rs = uint32_t(p.pool_rs_bytes);
  const uint32_t records = p.pool_bytes >= uint32_t(DQK) ? (p.pool_bytes - DQK) / rs + 1 : 0u;
  const i32x4 pool_rsrc = make_rsrc(p.pool, rs, records);
  const uint32_t rs2 = TWO ? uint32_t(p.pool2_rs_bytes) : rs;
  const uint32_t records2 =
      TWO ? (p.pool2_bytes >= uint32_t(DQK) ? (p.pool2_bytes - DQK) / rs2 + 1 : 0u) : records;
  const i32x4 pool2_rsrc = TWO ? make_rsrc(p.pool2, rs2, records2) : pool_rsrc;
  const uint32_t page_rows = PAGED ? uint32_t(p.page_bytes / p.pool_rs_bytes) : 0u;
  const uint32_t lds0 = lds_addr(smem);
  const int32_t* const idx_ring = reinterpret_cast<const int32_t*>(smem + C::OFF_IDX);

  // The indices of tile t of the row of `rm` (main segment) or `rx` (second
  // segment) (64 of them; past the segment's slot end the range check reads
  // 0) to the index ring at stream position tt; one instruction. Every wave
  // issues it (the same bytes to the same place), so that no branch splits
  // the code around it.
  auto idx_dma = [&](int tt, int t, i32x4 rm, i32x4 rx) {
    const bool x = in_second(t);
    const i32x4 rsrc = sel4(x, rx, rm);
    dma4(rsrc, lds0 + C::OFF_IDX + ring(tt) * kXTile * 4, uint32_t(4 * ((x ? t - T1 : t) * kXTile + lane)));
  };
  // This lane's slots of a tile (relative to 16 * wave): the DMA slots
  // 8h + k (k < 8; rows 2k + h), the rope slot of rope row lane / 4, the
  // flag slot lane % 16.
  const int rope_slot = 8 * ((lane >> 2) & 1) + ((lane >> 3) & 7);
  int idn[8], idr = -1, idb;
  bool idn_x = false;  // the indices in idn are the second segment's
  // The lane's indices of tile t (ring place tt) from the ring; slots past
  // the split's end (all of them for a tile past the walk's end) are marked
  // invalid, with selects rather than a branch; then slot indices of a
  // paged pool are mapped to rows of page_rows.
  auto read_idx = [&](int tt, int t) {
    const int32_t* ir = idx_ring + ring(tt) * kXTile + 16 * wave;
    const u32x4 a = *reinterpret_cast<const u32x4*>(ir + 8 * h);
    const u32x4 b = *reinterpret_cast<const u32x4*>(ir + 8 * h + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      idn[k] = int(a[k]);
      idn[4 + k] = int(b[k]);
    }
    if constexpr (ROPE) idr = ir[rope_slot];
    idb = ir[lane & 15];
    const bool x = in_second(t);
    if constexpr (TWO) idn_x = x;
    const int base = (x ? t - T1 : t) * kXTile + 16 * wave;
    const int se = x ? slot_end2 : slot_end;
    if (base + 16 > se) {
#pragma unroll
      for (int k = 0; k < 8; ++k) idn[k] = base + 8 * h + k < se ? idn[k] : -1;
      if constexpr (ROPE) idr = base + rope_slot < se ? idr : -1;
      idb = base + (lane & 15) < se ? idb : -1;
    }
    if constexpr (PAGED) {
      if (x) return;  // the second segment's pool is 2-D
      auto map = [&](int i) -> int {
        return i < 0 ? -1
                     : int((uint32_t(i) >> p.page_shift) * page_rows + (uint32_t(i) & p.page_mask));
      };
#pragma unroll
      for (int k = 0; k < 8; ++k) idn[k] = map(idn[k]);
      if constexpr (ROPE) idr = map(idr);
    }
  };
  // DMA of the walk's tile tt (indices read) into its ring places, and its
  // slot flags, in pieces: k < 8 the rows 2k + h of the first 512 columns,
  // k = 8 the rope columns, k = 9 the flags (every lane writes; lanes
  // l and l + 16 write the same value to the same place).
  const uint32_t dma_rope = 512u + 16u * uint32_t((lane & 3) ^ ((lane >> 4) & 3));
  constexpr int kPieces = 10;
  auto dma_piece = [&](int tt, int k) {
    const i32x4 prs = sel4(TWO && idn_x, pool2_rsrc, pool_rsrc);
    if (k < 8) {
      dma16(prs, lds0 + ring(tt) * C::NOPE + 16 * wave * kXRow + 2 * k * kXRow, idn[k],
            16u * uint32_t((lane & 31) ^ nope_perm(2 * k + h)));
    } else if (k == 8) {
      if constexpr (ROPE)
        dma16(prs, lds0 + C::OFF_ROPE + rope_ring(tt) * C::ROPEB + 16 * wave * kXRope,
              idr, dma_rope);
    } else {
      kbias[ring(tt) * kXTile + 16 * wave + (lane & 15)] = idb >= 0 ? 0.f : kNegInf;
    }
  };
  auto issue_dma = [&](int tt) {
#pragma unroll
    for (int k = 0; k < kPieces; ++k) dma_piece(tt, k);
  };
  // A walk's start: the indices of its first four tiles, then (indices
  // landed) the DMAs of the first three.
  // A walk whose first tiles are already requested (`fresh` false: the
  // previous item's walk streamed into them) only waits for them.
  auto start_walk = [&](int nt, bool fresh) __attribute__((always_inline)) {
    if (fresh) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (tt < nt) idx_dma(tt, t_begin + tt, idx_rsrc, idx2_rsrc);
    }
    sync_tile();
    if (fresh) {
#pragma unroll
      for (int tt = 0; tt < 3; ++tt) {
        if (tt < nt) {
          read_idx(tt, t_begin + tt);
          issue_dma(tt);  // waits for the read: ring place tt may be refilled after this
        }
      }
      if (nt > 4) idx_dma(4, t_begin + 4, idx_rsrc, idx2_rsrc);
    }
  };

  // q of this lane's head: k-step st takes columns 64 st + 16h and
  // 64 st + 32 + 16h (16 each, one in each k-block), split into hi and lo
  // e4m3 terms under each k-block's power of two (2^e puts the block's
  // largest |q| in [128, 256)). The loads are issued before the walk's
  // first barrier, whose wait covers them, so the split after it waits for
  // nothing (in particular not for the tile DMAs issued in between).
  i32x8 qhi[NSTEP], qlo[NSTEP];
  // Walks carry one stream of tiles through the rings: gbase is the stream
  // position of a walk's first tile.
  int gbase = 0;
  // E8M0 codes of the q terms' block scales, byte st % 4 of word st / 4:
  // this lane gives k-block h's (hi: 127 - e, lo: 127 - e - 4).
  constexpr int NSB = (NSTEP + 3) / 4;
  int sbh[NSB], sbl[NSB];
#pragma unroll
  for (int i = 0; i < NSB; ++i) sbh[i] = sbl[i] = 0x7F7F7F7F;
  auto q_col = [&](int st, int d) { return 64 * st + 32 * d + 16 * h; };
  // q of one k-step given as 8 bf16 bit patterns per u32x4 ([block d][half]):
  // each k-block's largest magnitude (this lane's 16 values and the partner
  // lane's, l ^ 32), its exponent, and the (hi, lo) terms under 2^e. Returns
  // the E8M0 code of this lane's k-block h (hi term: 127 - e).
  auto split_terms = [&](const u32x4 (&raw)[2][2], uint32_t (&hw)[8], uint32_t (&lw)[8])
      __attribute__((always_inline)) -> int {
    uint32_t mb[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t m = 0u;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t w = raw[d][hf][k] & 0x7FFF7FFFu;
          m = max(m, max(w & 0xFFFFu, w >> 16));
        }
      mb[d] = m;
    }
    const uint32_t both = mb[0] | (mb[1] << 16);
    const uint32_t other = uint32_t(__shfl_xor(int(both), 32));
    const int e0 = block_exp(max(mb[0], other & 0xFFFFu));
    const int e1 = block_exp(max(mb[1], other >> 16));
    const float sc0 = head_ok ? __builtin_ldexpf(1.0f, e0) : 0.f;
    const float sc1 = head_ok ? __builtin_ldexpf(1.0f, e1) : 0.f;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float sc = d ? sc1 : sc0;
          const uint32_t w0 = raw[d][hf][2 * k], w1 = raw[d][hf][2 * k + 1];
          split4(__uint_as_float(w0 << 16) * sc, __uint_as_float(w0 & 0xFFFF0000u) * sc,
                 __uint_as_float(w1 << 16) * sc, __uint_as_float(w1 & 0xFFFF0000u) * sc,
                 hw[4 * d + 2 * hf + k], lw[4 * d + 2 * hf + k]);
        }
    return kE8One - (h ? e1 : e0);
  };
  // k-step st's terms and block scale codes into place
  auto set_q = [&](int st, const u32x4 (&t)[4], int code) __attribute__((always_inline)) {
    qhi[st] = cat(t[0], t[1]);
    qlo[st] = cat(t[2], t[3]);
    const int sh = 8 * (st & 3);
    sbh[st / 4] = (sbh[st / 4] & ~(0xFF << sh)) | (code << sh);
    sbl[st / 4] = (sbl[st / 4] & ~(0xFF << sh)) | ((code - 4) << sh);
  };
  // The two waves of a pair need the same q terms: wave kh loads and splits
  // the k-steps st = 2i + kh, and the pair swaps them through LDS that is
  // free while a walk starts: the ring place of the walk's fourth tile
  // (k-steps 0..7, 4 KB each as four 1 KB quarters [quarter][lane] of 16
  // bytes, so that every access is contiguous and free of bank conflicts)
  // and the P-exchange area (the scale codes). The area holds one pair's
  // terms, so the pairs take turns. A wave reads back all swapped k-steps
  // (its own too), which keeps every register index compile-time. An odd
  // last k-step (the rope columns of a 576-wide row) is loaded and split by
  // both waves and set from registers, outside the swap.
  constexpr int NH = (NSTEP + 1) / 2;  // k-steps a wave loads and splits
  constexpr int NX = NSTEP / 2;        // of them, swapped
  auto xq_terms = [&](int st) -> u32x4* {
    return reinterpret_cast<u32x4*>(smem + ring(gbase + 3) * C::NOPE + st * 4096) + lane;  // quarter k at [64 k]
  };
  auto xq_code = [&](int st) -> int* {
    return reinterpret_cast<int*>(smem + C::OFF_XP + (st * 64 + lane) * 4);
  };
  auto swap_q = [&](const uint32_t (&hw)[NH][8], const uint32_t (&lw)[NH][8], const int (&code)[NH])
      __attribute__((always_inline)) {
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      if (hp == rp) {
#pragma unroll
        for (int i = 0; i < NX; ++i) {
          u32x4* const t = xq_terms(2 * i + kh);
          t[0] = u32x4{hw[i][0], hw[i][1], hw[i][2], hw[i][3]};
          t[64] = u32x4{hw[i][4], hw[i][5], hw[i][6], hw[i][7]};
          t[128] = u32x4{lw[i][0], lw[i][1], lw[i][2], lw[i][3]};
          t[192] = u32x4{lw[i][4], lw[i][5], lw[i][6], lw[i][7]};
          *xq_code(2 * i + kh) = code[i];
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (hp == rp) {
#pragma unroll
        for (int st = 0; st < 2 * NX; ++st) {
          const u32x4* const t = xq_terms(st);
          const u32x4 tt[4] = {t[0], t[64], t[128], t[192]};
          set_q(st, tt, *xq_code(st));
        }
      }
      // the other pair overwrites the area next; after the second turn the
      // walk's first barrier follows
      if (rp == 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  auto start_first_walk = [&](int nt, bool fresh) __attribute__((always_inline)) {
    const int hq = head_ok ? head : p.heads - 1;  // a masked head reads a real one, scaled by 0
    const int64_t qp = r * p.q_rs + int64_t(hq) * p.q_hs;
    uint32_t hw[NH][8], lw[NH][8];
    int code[NH];
    if (p.q_fp8) {
      u32x4 raw[NH][2];
#pragma unroll
      for (int i = 0; i < NH; ++i)
#pragma unroll
        for (int d = 0; d < 2; ++d)
          raw[i][d] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.q) + qp +
                                                      q_col(min(2 * i + kh, NSTEP - 1), d));
      start_walk(nt, fresh);
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        u32x4 bf[2][2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const u32x2 a = widen_fp8x4(raw[i][d][0]), b = widen_fp8x4(raw[i][d][1]);
          const u32x2 c = widen_fp8x4(raw[i][d][2]), e = widen_fp8x4(raw[i][d][3]);
          bf[d][0] = u32x4{a.x, a.y, b.x, b.y};
          bf[d][1] = u32x4{c.x, c.y, e.x, e.y};
        }
        code[i] = split_terms(bf, hw[i], lw[i]);
      }
    } else {
      u32x4 raw[NH][2][2];
#pragma unroll
      for (int i = 0; i < NH; ++i)
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            raw[i][d][hf] = *reinterpret_cast<const u32x4*>(
                p.q + qp + q_col(min(2 * i + kh, NSTEP - 1), d) + 8 * hf);
      start_walk(nt, fresh);
#pragma unroll
      for (int i = 0; i < NH; ++i) code[i] = split_terms(raw[i], hw[i], lw[i]);
    }
    swap_q(hw, lw, code);
    if constexpr (NH > NX) {
      const u32x4 t[4] = {u32x4{hw[NX][0], hw[NX][1], hw[NX][2], hw[NX][3]},
                          u32x4{hw[NX][4], hw[NX][5], hw[NX][6], hw[NX][7]},
                          u32x4{lw[NX][0], lw[NX][1], lw[NX][2], lw[NX][3]},
                          u32x4{lw[NX][4], lw[NX][5], lw[NX][6], lw[NX][7]}};
      set_q(NSTEP - 1, t, code[NX]);
    }
  };
  const float kv_scale = *p.kv_scale;
  const float cscale = p.sm_log2 * q_scale_of(p.q_scale) * kv_scale;
  // The second segment's scale (its own, else the main one). With two
  // segments O is kept in units of the larger scale s_ref: a tile's weights
  // (the numerator's P) are taken times its segment's scale / s_ref, as
  // 2^(x + lr) with lr = log2 of that ratio (at least -100, so that a zero
  // scale gives weights of 2^-100 rather than 0), and its row sum times
  // 2^-lr, so that the denominator and the LSE see the plain weights.
  // Scales are dequantisation scales: nonnegative.
  const float kv_scale2 = TWO && p.kv_scale2 != nullptr ? *p.kv_scale2 : kv_scale;
  const float cscale2 = p.sm_log2 * q_scale_of(p.q_scale) * kv_scale2;
  const float s_ref = TWO ? fmaxf(kv_scale, kv_scale2) : kv_scale;
  auto lr_of = [&](float sc) { return s_ref > 0.f ? fmaxf(__log2f(sc / s_ref), -100.f) : 0.f; };
  const float lr1 = TWO ? lr_of(kv_scale) : 0.f, lr2 = TWO ? lr_of(kv_scale2) : 0.f;
  const float lq1 = TWO ? __builtin_amdgcn_exp2f(-lr1) : 1.f, lq2 = TWO ? __builtin_amdgcn_exp2f(-lr2) : 1.f;

  // ---- per-lane LDS offsets (without the tile's base)
  // keys: this lane's score row is slot 32kh + c32; k-step st, half d reads
  // chunk 4st + 2d + h of its tile row (the rope k-step: rope chunk 2d + h).
  const int krow = row_of_slot(32 * kh + c32);
  const int kperm = nope_perm(krow);
  const int kro = krow * kXRow;
  const int rro = krow * kXRope;
  const int rperm = rope_perm(krow);
  // values: read v (0..3) of column block m covers tile rows
  // 32((v/2) ^ kh) + 16(v%2) + 8h .. +7 (the wave's own key half first, as
  // its P^T bytes are); the lane pair (2t, 2t+1) of a 16-lane group
  // points at row 8h + 2(t & 3) + t/2 of that group of 16, bytes 8(lane & 1)
  // of chunk 16kh + 2m + (lane bit 4).
  const int vt = (lane & 15) >> 1;
  const int vplow = 8 * h + 2 * (vt & 3) + (vt >> 2);
  const int vperm = nope_perm(vplow);
  const int vro = vplow * kXRow + 256 * kh + 8 * (lane & 1);
  const int vro_own = vro + 32 * kh * kXRow, vro_oth = vro + 32 * (kh ^ 1) * kXRow;
  const int ve = (lane >> 4) & 1;

  floatx16 o[8];
  float m_o = kNegInf;  // reference (log2 domain, an integer) of O and the row sums
  float m_w = kNegInf;  // reference of this wave's weights
  float l_run = 0.f;    // this lane's share of its slots' row sum (reference m_o)
  int redo = 0;

  // Key fragment (k-step st, half d) of the walk's tile tt: chunk 4st + 2d + h
  // of this lane's tile row (the rope k-step: rope chunk 2d + h).
  int kro_i = kro, kperm_i = kperm, rro_i = rro, rperm_i = rperm;  // refreshed per tile
  auto kread = [&](int tt, int st, int d) -> u32x4 {
    if (ROPE && st == NNOPE)
      return *reinterpret_cast<const u32x4*>(smem + C::OFF_ROPE + rope_ring(tt) * C::ROPEB +
                                             rro_i + 16 * ((2 * d + h) ^ rperm_i));
    return *reinterpret_cast<const u32x4*>(smem + ring(tt) * C::NOPE + kro_i +
                                           16 * ((4 * st + 2 * d + h) ^ kperm_i));
  };
  // One k-step of S^T: both terms of q against one key fragment.
  auto kstep = [&](floatx16& s, int st, const u32x4 (&kf)[2]) {
    const i32x8 a = cat(kf[0], kf[1]);
    s = mx32_byte(a, qhi[st], s, sbh[st / 4], st);
    s = mx32_byte(a, qlo[st], s, sbl[st / 4], st);
  };
  // Slot flags (0 or -inf) of this lane's 16 slots of the walk's tile tt.
  auto read_bias = [&](int tt, floatx4 (&b)[4]) {
    const float* kb = kbias + ring(tt) * kXTile + 32 * kh + 4 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const floatx4*>(kb + 8 * j);
  };
  // Per-iteration copies of the lane's LDS offsets: recomputing what is
  // derived from them is cheaper than holding it across the iteration.
  auto fresh = [](int v) {
    asm volatile("" : "+v"(v));
    return v;
  };

  // One walk over the split's tiles. The first walk fixes the references as
  // it goes; a second one (only when a score jumped by more than
  // kXMaxDrift above the pair's first valid tile's maximum) starts from the
  // first walk's final references, which no later score exceeds by
  // 2^kXLimit.
  // A streaming walk (`stream`) requests, in its last steps, the indices and
  // first tiles of the next item's walk instead of tiles past its end.
  const int nt = t_end - t_begin;
  auto walk = [&](bool first, bool fresh, bool stream) {
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = floatx16{};
    l_run = 0.f;
    if (nt <= 0) return;
    // start: the first tiles requested (and, on the first walk, q split
    // while they land)
    if (fresh) gbase = 0;
    if (first)
      start_first_walk(nt, fresh);
    else
      start_walk(nt, true);
    sync_tile();

    floatx16 s_cur = floatx16{}, s_next;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      u32x4 kf[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) kf[d] = kread(gbase, st, d);
      kstep(s_cur, st, kf);
    }
    float nm = m_w == kNegInf ? 0.f : -m_w;
    // carried from one step to the next: slot flag - m_w of the next tile's
    // 16 slots of this lane
    float bn[4][4];
    // (tt: the tile's ring position, t: its tile number)
    auto make_bn = [&](int tt, int t) {
      floatx4 b[4];
      read_bias(tt, b);
      float a = nm;
      if constexpr (TWO) a += in_second(t) ? lr2 : lr1;
#pragma unroll
      for (int i = 0; i < 16; ++i) bn[i / 4][i % 4] = b[i / 4][i % 4] + a;
    };
    make_bn(gbase, t_begin);
    for (int tt = 0; tt < nt; ++tt) {
      const int g = gbase + tt;  // stream position: ring places
      const int par = g & 1;
      // The indices of tile tt + 3 (their ring place landed a step ago), or
      // past the walk's end the next item's first tiles when streaming (else
      // all invalid: the DMAs write zeros to ring places that are free);
      // tile tt + 5's indices the same way. Read here, off the stretch after
      // the barrier.
      const int t3 = tt + 3 < nt ? t_begin + tt + 3 : (stream ? t_begin + tt + 3 - nt : t_end);
      const bool x5 = tt + 5 >= nt;
      const int t5 = !x5 ? t_begin + tt + 5 : (stream ? t_begin + tt + 5 - nt : t_end);
      read_idx(g + 3, t3);
      const bool has_next = tt + 1 < nt;
      float xmax, lt;
      uint32_t phi[4], plo[4];
      // The tile's weights (exp2 domain) and their split into P^T bytes
      // (byte i of this half's 16 is weight i), as 20 stages over groups g
      // of 4 weights: stage 0 the exponents, 1 the powers and the group
      // maximum, 2 the group sum and the hi codes, 3 the residuals, 4 the lo
      // codes. A stage depends only on earlier stages of its group.
      float x[16], w[16], m4[4], l4[4], ra[4][4];
      uint32_t hw[4];
      const bool second = in_second(t_begin + tt);
      const float cs_t = second ? cscale2 : cscale;
      auto stage = [&](int st, int g) {
        if (st == 0) {
#pragma unroll
          for (int u = 0; u < 4; ++u) x[4 * g + u] = __builtin_fmaf(s_cur[4 * g + u], cs_t, bn[g][u]);
        } else if (st == 1) {
#pragma unroll
          for (int u = 0; u < 4; ++u) w[4 * g + u] = __builtin_amdgcn_exp2f(x[4 * g + u]);
          m4[g] = fmaxf(fmaxf(x[4 * g], x[4 * g + 1]), fmaxf(x[4 * g + 2], x[4 * g + 3]));
        } else if (st == 2) {
          l4[g] = (w[4 * g] + w[4 * g + 1]) + (w[4 * g + 2] + w[4 * g + 3]);
          s16x2 hc = cvt2<false>(s16x2{0, 0}, w[4 * g], w[4 * g + 1]);
          hw[g] = __builtin_bit_cast(uint32_t, cvt2<true>(hc, w[4 * g + 2], w[4 * g + 3]));
        } else if (st == 3) {
          const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[g], 1.0f, false);
          const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw[g], 1.0f, true);
          ra[g][0] = w[4 * g] - a[0];
          ra[g][1] = w[4 * g + 1] - a[1];
          ra[g][2] = w[4 * g + 2] - b[0];
          ra[g][3] = w[4 * g + 3] - b[1];
        } else {
          s16x2 lc = cvt2<false>(s16x2{0, 0}, ra[g][0], ra[g][1], 0.0625f);
          plo[g] = __builtin_bit_cast(uint32_t, cvt2<true>(lc, ra[g][2], ra[g][3], 0.0625f));
          phi[g] = hw[g];
        }
      };
      auto finish = [&]() {
        xmax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        lt = (l4[0] + l4[1]) + (l4[2] + l4[3]);
      };
      // stage instance j (0..19) in dependency order with a gap between
      // the stages of a group
      auto stage_of = [](int j, int& st, int& g) {
        constexpr int kSt[20] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 2, 3, 4, 2, 3, 4, 3, 4, 4};
        constexpr int kG[20] = {0, 1, 0, 2, 1, 0, 3, 2, 1, 0, 3, 2, 1, 0, 3, 2, 1, 3, 2, 3};
        st = kSt[j];
        g = kG[j];
      };
      auto softmax = [&]() {
#pragma unroll
        for (int j = 0; j < 20; ++j) {
          int st, g;
          stage_of(j, st, g);
          stage(st, g);
        }
        finish();
      };

      // ---- S^T of the next tile over all but its last k-step, with this
      // tile's softmax stages between the dots
      u32x4 kr[3][2];
      if (has_next) {
        s_next = floatx16{};
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int d = 0; d < 2; ++d) kr[st][d] = kread(g + 1, st, d);
        // the first two stages while the fragments arrive
        {
          int sst, g;
          stage_of(0, sst, g);
          stage(sst, g);
          stage_of(1, sst, g);
          stage(sst, g);
        }
        constexpr int ND = 2 * (NSTEP - 1);  // dots before the barrier
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < NSTEP - 1; ++st) {
          const i32x8 a = cat(kr[st % 3][0], kr[st % 3][1]);
#pragma unroll
          for (int term = 0; term < 2; ++term) {
            s_next = mx32_byte(a, term ? qlo[st] : qhi[st], s_next, term ? sbl[st / 4] : sbh[st / 4], st);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 2 < NSTEP) kr[(st + 2) % 3][term] = kread(g + 1, st + 2, term);
            const int di = 2 * st + term;
#pragma unroll
            for (int j = 2; j < 20; ++j)
              if (((j - 2) * ND) / 18 == di) {
                int sst, g;
                stage_of(j, sst, g);
                stage(sst, g);
              }
            if (di == ND - 1) finish();
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        softmax();
        // the next tile's last k-step below runs on zeros (its result is
        // not used)
        kr[(NSTEP - 1) % 3][0] = kr[(NSTEP - 1) % 3][1] = u32x4{};
      }
      // computed here, before the rare-path branch
      asm volatile("" :: "v"(phi[0]), "v"(phi[1]), "v"(phi[2]), "v"(phi[3]), "v"(plo[0]),
                   "v"(plo[1]), "v"(plo[2]), "v"(plo[3]), "v"(lt), "v"(xmax));

      // ---- reference moves (rare): the first tile with a valid slot sets
      // the weights' reference to its maximum (rounded up to an integer); a
      // tile whose weights would pass 2^kXLimit raises it to its maximum;
      // the tile's weights are then taken again.
      const bool move = xmax > kXLimit || (m_w == kNegInf && xmax != kNegInf);
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
        // the tile's largest score (this lane's, then the head's): its
        // exponents less the reference they were taken against
        float tmax = xmax - nm;
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        if (tmax != kNegInf && (m_w == kNegInf || tmax > m_w + kXLimit))
          m_w = __builtin_ceilf(tmax);
        const float dn = (m_w == kNegInf ? 0.f : -m_w) - nm;
        nm += dn;
#pragma unroll
        for (int i = 0; i < 16; ++i) bn[i / 4][i % 4] += dn;
        softmax();
      }

      // ---- publish this half's P^T bytes and weight reference
      {
        uint8_t* xp = smem + C::OFF_XP + par * C::XPB + (wave * 64 + lane) * 32;
        *reinterpret_cast<u32x4*>(xp) = u32x4{phi[0], phi[1], phi[2], phi[3]};
        *reinterpret_cast<u32x4*>(xp + 16) = u32x4{plo[0], plo[1], plo[2], plo[3]};
        xm[(par * kXWaves + wave) * 32 + c32] = m_w;
      }
      // The values of the first two column blocks (tile tt has been in the
      // ring since the last barrier): read before this one, so that only
      // the partner's P is read after it.
      const uint8_t* const vb = smem + ring(g) * C::NOPE;
      // Value fragment (block m, read v): keys of this wave's own half for
      // v < 2, the partner's for v >= 2, the order of the P^T bytes below.
      auto vread = [&](int m, int v) -> u32x2 {
        return lds_read_tr8(vb + (v < 2 ? vro_own : vro_oth) + 16 * ((2 * m + ve) ^ vperm) +
                            16 * (v & 1) * kXRow);
      };
      constexpr int VR = 3;
      u32x2 vr[VR][4];
#pragma unroll
      for (int m = 0; m < VR - 1; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) vr[m][v] = vread(m, v);
      sync_tile();  // P and references visible; tile tt + 2 landed; tile tt - 1 free

      // ---- the partner's P^T and reference (the own half stays in
      // registers: the dots take the own keys first). The scale of k-block
      // h is the reference of its half: own for h = 0, the partner's for 1.
      u32x4 xho, xlo;
      float m_other;
      {
        const uint8_t* xp = smem + C::OFF_XP + par * C::XPB + ((wave ^ 1) * 64 + lane) * 32;
        xho = *reinterpret_cast<const u32x4*>(xp);
        xlo = *reinterpret_cast<const u32x4*>(xp + 16);
        m_other = xm[(par * kXWaves + (wave ^ 1)) * 32 + c32];
      }
      const float m_blk = h ? m_other : m_w;
      // the next item's q into the L2: 256 64-byte lines a step over the
      // five steps before the last. The dwords land in the slot flags of
      // tile tt's ring place, which were read a step ago and are written
      // next after the following barrier (tile tt + 4's).
      const int pf = tt - (nt - 6);
      const bool pf_on = stream && pf >= 0 && pf < 5;
      const i32x4 pf_rsrc = pf_on ? q_pf_rsrc : null_rsrc;
      const uint32_t pf_off = 64u * uint32_t((pf_on ? pf : 0) * 256 + 64 * wave + lane);

      const float m_first = fmaxf(m_w, m_other);
      m_o = m_o == kNegInf ? m_first : m_o;  // the pair's first valid tile
      const bool ref = m_o != kNegInf;
      redo |= int(ref && ((m_blk - m_o > kXMaxDrift) || (m_w - m_o > kXMaxDrift)));
      const float d_blk = ref ? fminf(fmaxf(m_blk - m_o, kXMinDrift), kXMaxDrift) : 0.f;
      const float d_own = ref ? fminf(fmaxf(m_w - m_o, kXMinDrift), kXMaxDrift) : 0.f;
      l_run += __builtin_ldexpf(TWO ? lt * (second ? lq2 : lq1) : lt, int(d_own));
      const int sb_ph = kE8One + int(d_blk), sb_pl = kE8One - 4 + int(d_blk);
      const i32x8 ph = cat(u32x4{phi[0], phi[1], phi[2], phi[3]}, xho);
      const i32x8 pl = cat(u32x4{plo[0], plo[1], plo[2], plo[3]}, xlo);

      // ---- the next tile's last k-step, then O^T += V^T P^T over this
      // wave's 8 column blocks; each value fragment feeds both terms of P
      // and is read two blocks ahead. One piece of tile tt + 3's DMA (then
      // tile tt + 5's indices) goes out after each of the first dots, so
      // that the address unit never holds the wave; the next step's slot
      // flags are read before the last two blocks. No branch in this
      // stretch: the order below is the order issued.
      {
        __builtin_amdgcn_sched_barrier(0);
        kstep(s_next, NSTEP - 1, kr[(NSTEP - 1) % 3]);
        asm volatile("" : "+a"(s_next));  // issued here, ahead of the DMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const u32x2* q = vr[m % VR];
          const i32x8 vf = i32x8{int(q[0].x), int(q[0].y), int(q[1].x), int(q[1].y),
                                 int(q[2].x), int(q[2].y), int(q[3].x), int(q[3].y)};
          const int mn = m + VR - 1;
#pragma unroll
          for (int term = 0; term < 2; ++term) {
            o[m] = mx32(vf, term ? pl : ph, o[m], term ? sb_pl : sb_ph);
            __builtin_amdgcn_sched_barrier(0);
            if (mn < 8) {
              vr[mn % VR][2 * term] = vread(mn, 2 * term);
              vr[mn % VR][2 * term + 1] = vread(mn, 2 * term + 1);
            }
            const int j = 2 * m + term;
            if (j < kPieces) dma_piece(g + 3, j);
            if (j == kPieces)
              idx_dma(g + 5, t5, sel4(x5, idx_rsrc_next, idx_rsrc), sel4(x5, idx2_rsrc_next, idx2_rsrc));
            if (j == 11) dma4(pf_rsrc, lds0 + C::OFF_BIAS + ring(g) * kXTile * 4, pf_off);
            if (j == 12) make_bn(g + 1, t_begin + tt + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // O and the first seven k-steps of q stay in the accumulator
      // registers, which MFMA operands may come from (the other 16 hold the
      // score accumulator), leaving the vector registers to the operand
      // rings.
#pragma unroll
      for (int c = 0; c < 8; ++c) asm volatile("" : "+a"(o[c]));
#pragma unroll
      for (int st = 0; st < 7; ++st) asm volatile("" : "+a"(qhi[st]), "+a"(qlo[st]));
      s_cur = s_next;
    }
    gbase += nt;
    // a walk that does not stream: the DMAs past its end have landed before
    // the ring is reused or the workgroup ends
    if (!stream) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // Streaming needs the next item's indices within the walk's last five
  // steps, so a walk of fewer tiles starts every item afresh.
  const bool can_stream = nt >= 5;
  bool prefetched = false;  // this item's first tiles are in the ring
  for (int k = 0; k < n_items; ++k) {
    if (k > 0) {
      r = item_of(k, hblk, split);
      head = hblk * 64 + 32 * hp + c32;
      head_ok = head < p.heads;
      idx_rsrc = idx_rsrc_of(r);
      idx2_rsrc = idx2_rsrc_of(r);
      load_cs();
    }
    const bool more = can_stream && k + 1 < n_items;
    if (more) {
      int hb1, sp1;
      const int64_t r1 = item_of(k + 1, hb1, sp1);
      idx_rsrc_next = idx_rsrc_of(r1);
      idx2_rsrc_next = idx2_rsrc_of(r1);
      const int64_t es = p.q_fp8 ? 1 : 2;
      const int64_t nh1 = min(64, p.heads - 64 * hb1);
      const int64_t span = min(nh1 * p.q_hs * es, int64_t(2 * 64 * DQK) * es);
      q_pf_rsrc = make_rsrc(reinterpret_cast<const uint8_t*>(p.q) + (r1 * p.q_rs + 64 * hb1 * p.q_hs) * es,
                            0, uint32_t(span));
    }
    m_o = kNegInf;
    m_w = kNegInf;
    redo = 0;
    bool streamed = false;
#pragma clang loop unroll(disable)
    for (int pass = 0; pass < 2; ++pass) {
      walk(pass == 0, pass == 1 || !prefetched, pass == 0 && more);
      streamed = pass == 0 && more;
      if (pass == 1 || __syncthreads_or(redo) == 0) break;
      // the second walk starts from the pair's final weight references,
      // after the stream into the next item has drained (its tiles are
      // requested again)
      const int par = (gbase - 1) & 1;
      m_o = fmaxf(m_w, xm[(par * kXWaves + (wave ^ 1)) * 32 + c32]);
      sync_tile();  // every wave has read them before the walk reuses the area
    }
    prefetched = streamed;

    // ---- the item's end: the head's row sum over both lane halves and
    // both waves of the pair; normalise; store.
    const float l_lane = l_run + __shfl_xor(l_run, 32);
    xl[wave * 32 + c32] = l_lane;
    if constexpr (EPI) {
      if (tid < 64) epi_cs[tid] = cs_pre;
    }
    // the LDS traffic only: the stream's DMAs stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float lt_tot = l_lane + xl[(wave ^ 1) * 32 + c32];
    const int64_t r_st = r;
    const int head_st = head, split_st = split;
    if (head_ok) {
      const float inv = lt_tot > 0.f ? s_ref / lt_tot : 0.f;
      const bool split_mode = p.part_o != nullptr;
      const int colh = 256 * kh + 4 * h;  // column of register 0 of block 0
      if (EPI && !split_mode) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float v[4][4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) v[j][u] = o[m][4 * j + u] * inv;
          epi_store_c32x4(p.epi, p.epi.pos != nullptr ? epi_cs : nullptr, r_st, head_st, colh + 32 * m,
                          v);
        }
      } else if (!split_mode) {
        // bf16 rows, 16 contiguous columns per store: lane h and its
        // partner lane (h flipped) trade half of each 32-column block, so
        // that h = 0 holds columns 0..15 of the block and h = 1 columns
        // 16..31.
        uint16_t* const orow = p.out + r_st * p.out_rs + int64_t(head_st) * p.out_hs + 256 * kh + 16 * h;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          uint32_t w[8];  // columns 8j + 4h + (0..3) of the block, as bf16 pairs
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = pack_bf16(o[m][2 * i] * inv, o[m][2 * i + 1] * inv);
          uint32_t x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = __shfl_xor(h ? w[i] : w[4 + i], 32);
          const u32x4 lo = h ? u32x4{x[0], x[1], w[4], w[5]} : u32x4{w[0], w[1], x[0], x[1]};
          const u32x4 hi = h ? u32x4{x[2], x[3], w[6], w[7]} : u32x4{w[2], w[3], x[2], x[3]};
          *reinterpret_cast<u32x4*>(orow + 32 * m) = lo;
          *reinterpret_cast<u32x4*>(orow + 32 * m + 8) = hi;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = colh + 32 * m + 8 * j;
            *reinterpret_cast<floatx4*>(
                p.part_o + ((int64_t(split_st) * p.rows + r_st) * p.heads + head_st) * kDv + col) =
                floatx4{o[m][4 * j] * inv, o[m][4 * j + 1] * inv, o[m][4 * j + 2] * inv,
                        o[m][4 * j + 3] * inv};
          }
      }
      if (kh == 0 && h == 0) {
        const float lse = lt_tot > 0.f ? (m_o + __log2f(lt_tot)) * kLn2 : kNegInf;
        if (!split_mode)
          p.lse[r_st * p.lse_rs + int64_t(head_st) * p.lse_hs] = lse;
        else
          p.part_lse[(int64_t(split_st) * p.rows + r_st) * p.heads + head_st] = lse;
      }
    }
  }
}

}  // namespace

KernelShape prefill_mx_shape(int dqk) {
  KernelShape k;
  k.waves = kXWaves;
  k.tile = kXTile;
  if (dqk == 576)
    k.lds_bytes = XCfg<576>::LDS;
  else if (dqk == 512)
    k.lds_bytes = XCfg<512>::LDS;
  else
    k = KernelShape{};
  return k;
}

template <int DQK, bool PAGED, bool TWO>
void launch_mx(const FwdParams& p, bool epi, dim3 grid, dim3 block, hipStream_t st) {
  if (epi)
    hipLaunchKernelGGL((prefill_mx_kernel<DQK, true, PAGED, TWO>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((prefill_mx_kernel<DQK, false, PAGED, TWO>), grid, block, 0, st, p);
}

int launch_prefill_mx(const FwdParams& p, int dqk, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool epi = epi_active(p.epi) && p.part_o == nullptr;
  const bool paged = p.page_shift != 31;
  // Rows not split: one workgroup per CU (rounded down to whole rounds of
  // the 8 XCDs, so a workgroup's items stay on its XCD) walks its share of
  // the work items as one stream of tiles. Split rows: one workgroup per
  // item.
  int64_t wgs = p.grid;
  if (p.splits == 1 && p.persist_cap > 0 && p.grid > p.persist_cap)
    wgs = p.persist_cap >= 8 ? p.persist_cap / 8 * 8 : p.persist_cap;
  const dim3 grid{uint32_t(wgs)}, block{uint32_t(kXWaves * 64)};
  // A second segment's pool is 2-D, with a row pitch the structured buffer
  // addresses (the planner composes the other cases from two launches).
  const bool two = p.idx2 != nullptr;
  if (two && !mx_pool_ok(p.pool2_rs_bytes, 0)) return int(hipErrorInvalidValue);
  if (dqk == 576) {
    if (two)
      paged ? launch_mx<576, true, true>(p, epi, grid, block, st)
            : launch_mx<576, false, true>(p, epi, grid, block, st);
    else
      paged ? launch_mx<576, true, false>(p, epi, grid, block, st)
            : launch_mx<576, false, false>(p, epi, grid, block, st);
  } else if (dqk == 512) {
    if (two)
      paged ? launch_mx<512, true, true>(p, epi, grid, block, st)
            : launch_mx<512, false, true>(p, epi, grid, block, st);
    else
      paged ? launch_mx<512, true, false>(p, epi, grid, block, st)
            : launch_mx<512, false, false>(p, epi, grid, block, st);
  } else {
    return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

}  // namespace smla
