// gfx950 64-head kernel of the sparse MLA forward over an fp8 e4m3fn pool,
// 576- or 512-wide rows.
//
// The method (per row r, head h, over the row's valid slots j):
//   s_j = sm_scale * q[r,h] . K[idx_j] (D_qk columns), out = softmax(s) V
//   (V = first 512 columns), lse = ln sum_j exp(s_j)
// after "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159):
// Technical Details and the commit notes on the 64-head program (each key
// tile gathered once for all 64 heads, fp8 keys widened to bf16 for the
// 16x16x32 bf16 dots, online softmax in the exp2 domain).
//
// Layout of the work, chosen for gfx950 rather than taken from the pages:
//  * One workgroup = (row, 64 heads, split), 4 wavefronts, one workgroup per
//    CU, one wavefront per SIMD. The kernel is bound by LDS traffic, so each
//    operand fragment read from LDS feeds two dots: wave (hp, kh) holds Q^T
//    of heads 32hp..32hp+31 and computes S^T = K Q^T for slot half kh of
//    each 64-slot tile (one K fragment, two head blocks); for O^T += V^T P^T
//    it owns output columns 256kh..256kh+255 of the same 32 heads over all
//    64 slots (one V fragment, two head blocks). S^T leaves each lane 4
//    consecutive slots of one head, the B operand layout of the PV dot, so a
//    wave's own P never leaves its registers; the two waves of a pair swap
//    the other half's P through LDS (2 KB each way per tile).
//  * K/V tiles are staged once per workgroup as bf16 rows in LDS, double
//    buffered. Rows are unpadded; the 16-byte chunk index of row r is
//    XOR-permuted by a function of r chosen so that the K operand reads
//    (ds_read_b128), the transposed V reads (ds_read_b64_tr_b16) and the
//    staging writes (ds_write_b128) are all free of bank conflicts on gfx950.
//  * QK runs slot block 0 (16 slots) over all k-steps, then block 1. Tile
//    t+1 is widened and written into the other buffer between the QK dots
//    of tile t, a quarter chunk per k-step; as each of a thread's chunks is
//    written, its registers are refilled with the gather for tile t+2
//    (unconditional raw buffer loads: invalid slots read past the buffer
//    range and get zeros), so each gather has a whole tile to land. Block
//    0's softmax weights are computed between block 1's dots. Two barriers
//    per tile: P swap, buffer reuse.
//  * Fixed reference: a head's reference max is the max over the first tile
//    that has a valid slot, taken by the walk's first step from that tile's
//    scores before any weight (the pair agrees on it through LDS), so O is
//    never rescaled and stays in the MFMA accumulators. P = exp2(s - ref) is exact in real arithmetic whatever the
//    reference; the bf16 P and fp32 sums stay in range while every weight is
//    at most 2^64. Every weight a lane adds is at most the lane's partial
//    row sum, so if no partial sum passes 2^64 none did; otherwise the
//    workgroup scores all its tiles for the exact row max and walks its
//    slots a second time with that as the reference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

constexpr int kXWaves = 4;
constexpr int kXTile = 64;
constexpr float kXSumLimit = 0x1p64f;  // bound on the weights against the reference
constexpr uint32_t kXOutOfRange = 0xFFFFF000u;
constexpr int kXBufferWord3 = 0x00020000;

template <int DQK>
struct XCfg {
  static constexpr int HB = 64;
  static constexpr int NT = kXWaves * 64;
  static constexpr int TK = kXTile;
  static constexpr int KSTEPS = DQK / 32;
  static constexpr int ROW = DQK * 2;              // bytes per bf16 tile row
  static constexpr int SRC_CH = DQK / 16;          // 16-byte fp8 chunks per pool row
  static constexpr int TPR = NT / TK;              // staging threads per slot
  static constexpr int LPT = SRC_CH / TPR;         // fp8 chunks per staging thread
  static constexpr int TILE = TK * ROW;            // bytes per bf16 tile
  static constexpr int NDW = kDv / 16 / 2;         // 16-column output blocks per wave
  static constexpr int SWB = DQK == 576 ? 8 : 16;  // chunk span the row permutation touches
  static constexpr int NQB = SWB / 4;              // K-operand address bases
  static constexpr int NVB = SWB / 2;              // V-operand address bases
  static constexpr int NSB = SWB / 8;              // staging address bases per half
  static constexpr int LDS_BYTES = 2 * TILE + 2 * TK * 4 + kXWaves * 2 * 64 * 16 + 64 +
                                    kXWaves * 2 * 64 * 4;
  static_assert(SRC_CH % TPR == 0, "staging split");
  static_assert(LPT % NSB == 0, "staging bases");
  static_assert(4 * LPT <= 2 * KSTEPS, "staging spread over the k-steps");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Physical chunk of logical 16-byte chunk c in tile row r is c ^ tile_perm(r).
// The permutation only touches the low 3 (576) or 4 (512) bits of the chunk
// index, so it stays inside the row.
template <int DQK>
__device__ __forceinline__ int tile_perm(int r) {
  if constexpr (DQK == 576) return (r & 3) | (((r ^ (r >> 2)) & 1) << 2);
  return ((r & 1) * 3) | (((r ^ (r >> 1)) & 1) << 2) | (((r >> 2) & 1) << 3);
}

// EPI: the final store goes through the output epilogue (epilogue.h).
template <int DQK, bool EPI>
__global__ void __launch_bounds__(kXWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_fp8_kernel(const FwdParams p) {
  using C = XCfg<DQK>;
  constexpr int TK = C::TK, ROW = C::ROW, TILE = C::TILE, KSTEPS = C::KSTEPS;
  constexpr int LPT = C::LPT, NDW = C::NDW, SWB = C::SWB;
  constexpr int NQB = C::NQB, NVB = C::NVB, NSB = C::NSB;

  // Two bf16 tile buffers as separate arrays, so the compiler can tell the
  // staging writes into one from the operand reads of the other.
  __shared__ __attribute__((aligned(16))) uint8_t tile0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[TILE];
  __shared__ __attribute__((aligned(16))) float kbias[2 * TK];   // 0 (valid slot) or -inf
  // P swap (and, outside the tile loop, the pair's max / sum exchange):
  // [wave][head block][lane] 16 bytes.
  __shared__ __attribute__((aligned(16))) u32x4 xch[kXWaves * 2 * 64];
  __shared__ uint32_t redo[1];
  // The pair's head maxima of the first tile, when the walk fixes the
  // reference itself: [wave][head block][lane].
  __shared__ float mxch[kXWaves * 2 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int hp = wave >> 1, kh = wave & 1;
  const int partner = wave ^ 1;

  int64_t work = p.remap ? smla_xcd_work(blockIdx.x, p.grid) : int64_t(blockIdx.x);
  const int hblk = int(work % p.head_blocks);
  work /= p.head_blocks;
  const int split = int(work % p.splits);
  const int64_t r = work / p.splits;
  // Output epilogue: this row's cos/sin row, read now so that the two
  // dependent reads (position, then cache) overlap the walk; one wave keeps
  // it in a register until the epilogue copies it to LDS.
  __shared__ float epi_cs[64];
  float cs_pre = 0.f;
  if constexpr (EPI) {
    if (p.epi.pos != nullptr && tid < 64) cs_pre = epi_cs_row(p.epi, r)[tid];
  }

  const int h0 = hblk * C::HB + 32 * hp;  // heads h0 + 16hb + l16 of this lane

  const int ntiles = (p.topk + TK - 1) / TK;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

  // Q^T operands: head h0 + 16hb + l16, columns 8g + 32s .. +7 (zero for a
  // head past the last). Loaded by each walk right after the gathers of its
  // first tile, so the two loads' latencies overlap.
  bf16x8 qf[2][KSTEPS];
  // The two waves of a pair hold the same Q^T: each loads the k-steps
  // s = kh (mod 2), puts them in the pair's region of the second tile
  // buffer (free until the walk's first step stages into it), and reads all
  // k-steps back from there, which halves the workgroup's Q requests.
  // Region of pair hp: [hb][s][lane], 16 bytes. (Register indices stay
  // compile-time: the parity only moves addresses. An array indexed by a
  // run-time value, or written differently on the two sides of a branch on
  // the parity, would live in scratch memory.)
  bf16x8 qh[2][KSTEPS / 2];
  auto load_q_half = [&]() {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i) qh[hb][i] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      const int h = h0 + 16 * hb + l16;
      if (h < p.heads) {
        const int64_t qp = r * p.q_rs + int64_t(h) * p.q_hs + 8 * g + 32 * kh;
        if (p.q_fp8) {
          u32x2 c[KSTEPS / 2];
#pragma unroll
          for (int i = 0; i < KSTEPS / 2; ++i)
            c[i] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(p.q) + qp + 64 * i);
#pragma unroll
          for (int i = 0; i < KSTEPS / 2; ++i) qh[hb][i] = widen_fp8x8(c[i].x, c[i].y);
        } else {
#pragma unroll
          for (int i = 0; i < KSTEPS / 2; ++i)
            qh[hb][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p.q + qp + 64 * i));
        }
      }
    }
  };
  auto q_slot = [&](uint8_t* buf, int hb, int s) -> u32x4* {
    return reinterpret_cast<u32x4*>(buf + (((hp * 2 + hb) * KSTEPS + s) * 64 + lane) * 16);
  };
  auto put_q_half = [&](uint8_t* buf) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i)
        *q_slot(buf, hb, 2 * i + kh) = __builtin_bit_cast(u32x4, qh[hb][i]);
  };
  auto get_q = [&](uint8_t* buf) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[hb][s] = __builtin_bit_cast(bf16x8, *q_slot(buf, hb, s));
    // Keep Q^T in VGPRs: left to itself the allocator parks it in AGPRs (the
    // dots can read it there) and then has no AGPRs left for O^T and S^T.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(qf[hb][s]));
  };
  const float kv_scale = *p.kv_scale;
  const float score_scale = p.sm_log2 * q_scale_of(p.q_scale) * kv_scale;

  // ---- staging role: slot gk of a tile, fp8 chunks gq, gq + 4, ...
  const int gk = tid / C::TPR, gq = tid % C::TPR;
  const int32_t* idx_row = p.idx + r * p.idx_rs;
  const int last_slot = min(p.topk, t_end * TK) - 1;
  // The index load and its validity mask are split so that a load can be
  // issued a tile before it is used: applying the mask right after the load
  // would make the wave wait for every gather issued before it.
  // The row's indices up to last_slot through a buffer resource: a load past
  // it reads 0, which the mask then marks invalid. The loads run up to three
  // tiles past the row's end (past the tensor's end on its last row) and the
  // hardware range check covers the vector and immediate offsets but not the
  // scalar one, so the whole byte offset goes in the vector offset.
  const __amdgpu_buffer_rsrc_t idx_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(idx_row), 0, 4 * (last_slot + 1), kXBufferWord3);
  auto idx_raw = [&](int t) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(idx_rsrc, uint32_t(4 * (gk + t * TK)), 0, 0);
  };
  auto idx_mask = [&](int t) -> int { return -int(!(t < t_end && gk <= last_slot - t * TK)); };
  auto load_idx = [&](int t) -> int { return idx_raw(t) | idx_mask(t); };
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.pool), 0, p.pool_bytes, kXBufferWord3);
  u32x4 pre[LPT];
  const PoolMap pm{uint32_t(p.pool_rs_bytes), uint32_t(p.page_bytes), uint32_t(p.page_shift),
                   p.page_mask};
  auto row_off = [&](int id) -> uint32_t { return id >= 0 ? slot_offset(pm, id) : kXOutOfRange; };
  auto gather_one = [&](int i, uint32_t off) {
    pre[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           pool_rsrc, off + 16u * uint32_t(gq + 4 * i), 0, 0));
  };
  auto gather = [&](int id) {
    const uint32_t off = row_off(id);
#pragma unroll
    for (int i = 0; i < LPT; ++i) gather_one(i, off);
  };
  // Destination of widened chunk i (low or high 8 columns) in a tile:
  // logical chunk 8i + 2gq + half of row gk.
  const int gperm = tile_perm<DQK>(gk);
  int sbase[2][NSB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int b = 0; b < NSB; ++b)
      sbase[half][b] = gk * ROW + 16 * ((8 * b + 2 * gq + half) ^ gperm);
  auto stage_chunk = [&](int i, uint8_t* tile) {
    const u32x2 w0 = widen_fp8x4(pre[i].x), w1 = widen_fp8x4(pre[i].y);
    const u32x2 w2 = widen_fp8x4(pre[i].z), w3 = widen_fp8x4(pre[i].w);
    const int hi_off = 16 * SWB * (i / NSB);
    *reinterpret_cast<u32x4*>(tile + sbase[0][i % NSB] + hi_off) = u32x4{w0.x, w0.y, w1.x, w1.y};
    *reinterpret_cast<u32x4*>(tile + sbase[1][i % NSB] + hi_off) = u32x4{w2.x, w2.y, w3.x, w3.y};
  };

  // ---- K operand addresses: row 32kh + 16j + l16, logical chunk g + 4s.
  const int qperm = tile_perm<DQK>(l16);
  int kbase[NQB];
#pragma unroll
  for (int b = 0; b < NQB; ++b) kbase[b] = (32 * kh + l16) * ROW + 16 * ((4 * b + g) ^ qperm);
  // ---- V^T operand addresses: rows 32x + 4g + l16/4 (+16) of slot half x,
  // columns 256kh + 16d + 4(l16 % 4) .. +3, i.e. logical chunk
  // 32kh + 2d + (l16/2)%2, byte 8(l16%2).
  const int vrow = 4 * g + (l16 >> 2);
  const int vperm = tile_perm<DQK>(vrow);
  int vbase[NVB];
#pragma unroll
  for (int b = 0; b < NVB; ++b)
    vbase[b] = vrow * ROW + 16 * 32 * kh + 16 * ((2 * b + ((l16 >> 1) & 1)) ^ vperm) + 8 * (l16 & 1);

  floatx4 o[NDW][2];
  float m_ref[2] = {kNegInf, kNegInf};  // reference max (log2) of head 16hb + l16, shared by the pair
  float nmu[2];      // -m_ref, or 0 when the split has no valid slot
  float l_part[2];   // this lane's share of the head's row sum over the wave's slots

  // Scores of this wave's 32 slots of a tile: S^T blocks j = 0 (slots
  // 32kh..32kh+15) and j = 1 (the next 16), head blocks hb.
  floatx4 sacc[2][2];
  // Softmax weights of slots 4g..4g+3 of block j = i / 4 (i % 4 within them)
  // for head block hb, and the bf16 pairs of block 0.
  float ew[2][8];
  u32x2 p0[2];
  // Weight of slot i of head block hb: 2^(s * score_scale + bias - m_ref);
  // bias = 0 for a valid slot, -inf for an invalid one. Summed into l_part.
  auto weight = [&](int hb, int i, const float (&bias)[8]) {
    const float v = __builtin_fmaf(sacc[i / 4][hb][i % 4], score_scale, bias[i] + nmu[hb]);
    ew[hb][i] = __builtin_amdgcn_exp2f(v);
    l_part[hb] += ew[hb][i];
    // Pure arithmetic would otherwise be sunk to its uses after the dots.
    asm volatile("" : "+v"(ew[hb][i]), "+v"(l_part[hb]));
  };
  auto pack_block0 = [&]() {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      p0[hb] = u32x2{pack2_bf16(ew[hb][0], ew[hb][1]), pack2_bf16(ew[hb][2], ew[hb][3])};
    asm volatile("" : "+v"(p0[0]), "+v"(p0[1]));
  };
  // QK of this wave's 32 slots of the tile in `cur`, block j = 0 over all
  // k-steps first, then j = 1, each K fragment feeding both head blocks.
  // With `stage`, the next tile's chunks are widened from `pre` into `nxt`
  // between the dots, one chunk per 4 k-steps (each chunk's registers then
  // refilled with the gather of the tile after, which so gets a whole tile to
  // land); with `soft`, the block-0 weights are computed between the dots of
  // block 1.
  constexpr int NU = 2 * KSTEPS;
  constexpr int KRING = 4;  // K fragments read KRING-1 steps ahead of their dots
  auto load_k = [&](const uint8_t* cur, int u) -> bf16x8 {
    const int j = u / KSTEPS, s = u % KSTEPS;
    return *reinterpret_cast<const bf16x8*>(cur + kbase[s % NQB] + 16 * SWB * (s / NQB) + 16 * ROW * j);
  };
  auto qk = [&](const uint8_t* cur, uint8_t* nxt, uint32_t next_off, bool stage, bool soft,
                const float (&bias)[8]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) sacc[j][0] = sacc[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ka[KRING];
    u32x2 wz[4];  // widened quarters of the chunk being staged
#pragma unroll
    for (int u = 0; u < KRING - 1; ++u) ka[u] = load_k(cur, u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      // The fences keep the scheduler from sinking the reads to their uses.
      if (u + KRING - 1 < NU) ka[(u + KRING - 1) % KRING] = load_k(cur, u + KRING - 1);
      __builtin_amdgcn_sched_barrier(0);
      const int j = u / KSTEPS, s = u % KSTEPS;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        sacc[j][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u % KRING], qf[hb][s], sacc[j][hb], 0, 0, 0);
      if (stage && u / 4 < LPT) {
        // Chunk u/4 of the next tile is widened a quarter per k-step and
        // written a half every other step (a burst of widenings or writes
        // between two dots stalls them); its registers are then refilled
        // with the gather of the tile after.
        const int c = u / 4, ph = u % 4;
        wz[ph] = widen_fp8x4(pre[c][ph]);
        const int hi_off = 16 * SWB * (c / NSB);
        if (ph == 1)
          *reinterpret_cast<u32x4*>(nxt + sbase[0][c % NSB] + hi_off) = u32x4{wz[0].x, wz[0].y, wz[1].x, wz[1].y};
        if (ph == 3) {
          *reinterpret_cast<u32x4*>(nxt + sbase[1][c % NSB] + hi_off) = u32x4{wz[2].x, wz[2].y, wz[3].x, wz[3].y};
          gather_one(c, next_off);
        }
      }
      // Block 0's last dots went out at u = KSTEPS - 1; one step later their
      // results are in.
      const int k = u - (KSTEPS + 1);
      if (soft && k >= 0 && k < 8) weight(k / 4, k % 4, bias);
      if (soft && k == 8) pack_block0();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // This lane's bias terms of the tile whose flags are kbias[kb..]: slots
  // 32kh + 4g + i (i < 4) and 32kh + 16 + 4g + i - 4.
  auto load_bias = [&](int kb, float (&bias)[8]) {
    const floatx4 b0 = *reinterpret_cast<const floatx4*>(kbias + kb + 32 * kh + 4 * g);
    const floatx4 b1 = *reinterpret_cast<const floatx4*>(kbias + kb + 32 * kh + 16 + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bias[i] = b0[i];
      bias[4 + i] = b1[i];
    }
  };
  // V^T fragments of slot half x (0: the wave's own, 1: the partner's) for
  // the wave's output blocks d, in a ring of VRING; the first VRING-1 of a
  // pass are read ahead of the work that precedes it.
  constexpr int VRING = 3;
  bf16x8 vf[VRING];
  const int vhalf[2] = {32 * kh * ROW, 32 * (kh ^ 1) * ROW};
  auto load_v = [&](const uint8_t* cur, int x, int d) -> bf16x8 {
    const uint16_t* va = reinterpret_cast<const uint16_t*>(
        cur + vbase[d % NVB] + 16 * SWB * (d / NVB) + vhalf[x]);
    const u32x2 v0 = lds_read_tr16(va);
    const u32x2 v1 = lds_read_tr16(va + 8 * ROW);  // 16 rows further
    return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
  };
  auto pv_prefetch = [&](const uint8_t* cur, int x) {
#pragma unroll
    for (int d = 0; d < VRING - 1; ++d) vf[d] = load_v(cur, x, d);
    __builtin_amdgcn_sched_barrier(0);
  };
  // O^T += V^T P^T over slot half x of the tile in `cur` for this wave's
  // output columns; pk is that half's P^T operand.
  auto pv_half = [&](const uint8_t* cur, int x, const bf16x8 (&pk)[2]) {
#pragma unroll
    for (int d = 0; d < NDW; ++d) {
      if (d + VRING - 1 < NDW) vf[(d + VRING - 1) % VRING] = load_v(cur, x, d + VRING - 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        o[d][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d % VRING], pk[hb], o[d][hb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float* const xf = reinterpret_cast<float*>(xch);
  // Reference: per head, the max score (log2 domain, valid slots only) over
  // tiles [t_from, t_to), agreed by the pair; -inf if there is none. Each
  // tile is staged and scored on its own (no overlap): this runs over one
  // tile per walk, and over all of them only before a second walk.
  auto max_pass = [&](int t_from, int t_to) {
    float mx[2] = {kNegInf, kNegInf};
#pragma clang loop unroll(disable)
    for (int t = t_from; t < t_to; ++t) {
      const int id = load_idx(t);
      gather(id);
#pragma unroll
      for (int i = 0; i < LPT; ++i) stage_chunk(i, tile0);
      if (gq == 0) kbias[gk] = id >= 0 ? 0.f : kNegInf;
      __syncthreads();
      float bias[8];
      load_bias(0, bias);
      qk(tile0, tile1, 0u, false, false, bias);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          mx[hb] = fmaxf(mx[hb], __builtin_fmaf(sacc[i / 4][hb][i % 4], score_scale, bias[i]));
      __syncthreads();  // tile0 and the flags are free for the next tile
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float t = fmaxf(mx[hb], __shfl_xor(mx[hb], 16));
      t = fmaxf(t, __shfl_xor(t, 32));
      xf[(wave * 2 + hb) * 64 + lane] = t;
      mx[hb] = t;
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) m_ref[hb] = fmaxf(mx[hb], xf[(partner * 2 + hb) * 64 + lane]);
    __syncthreads();  // the exchange area is free again
  };

  // One walk over tiles [t0, t_end) with the references in m_ref, or, with
  // fix_ref, with the references fixed by the walk's first tile.
  // The first walk gets the indices of its first three tiles already
  // loaded (ids[0..1] masked, ids[2] raw), so its start waits for one
  // gather after the other and no index load between them.
  auto walk = [&](int t0, bool fix_ref, const int (&ids)[3]) {
#pragma unroll
    for (int d = 0; d < NDW; ++d) o[d][0] = o[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) nmu[hb] = m_ref[hb] == kNegInf ? 0.f : -m_ref[hb];
    l_part[0] = l_part[1] = 0.f;
    if (t0 >= t_end) return;
    const int id_a = fix_ref ? ids[0] : load_idx(t0);
    int id_b = fix_ref ? ids[1] : load_idx(t0 + 1);
    int raw_n = fix_ref ? ids[2] : idx_raw(t0 + 2);  // masked where it is used
    gather(id_a);
    load_q_half();  // (a second walk loads it again: Q^T is then not live across walks)
#pragma unroll
    for (int i = 0; i < LPT; ++i) stage_chunk(i, tile0);
    if (gq == 0) kbias[gk] = id_a >= 0 ? 0.f : kNegInf;
    gather(id_b);
    put_q_half(tile1);
    __syncthreads();
    get_q(tile1);
    __syncthreads();  // every wave has its Q^T before the first step stages into tile1
    // One tile: QK of tile t from `cur` with tile t+1 (zeros past the end:
    // harmless, never read) staged into `nxt`, the buffer tile t-1 used,
    // which every wave finished before the last barrier; softmax; P swap;
    // PV. The index of tile t+3 is loaded before the gathers of tile t+2, so
    // waiting for it never waits for them.
    auto step = [&](auto first, int t, const uint8_t* cur, uint8_t* nxt, int buf) {
      constexpr bool FIRST = decltype(first)::value;
      const int raw_f = idx_raw(t + 3);
      __builtin_amdgcn_sched_barrier(0);
      const int id_n = raw_n | idx_mask(t + 2);
      float bias[8];
      load_bias(buf * TK, bias);
      qk(cur, nxt, row_off(id_n), true, !FIRST, bias);
      if constexpr (FIRST) {
        // The walk's first tile fixes the reference: each head's max score
        // over the tile (valid slots), agreed by the pair; then block 0's
        // weights, which the other steps compute between the QK dots.
        float mx[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          mx[hb] = kNegInf;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            mx[hb] = fmaxf(mx[hb], __builtin_fmaf(sacc[i / 4][hb][i % 4], score_scale, bias[i]));
          mx[hb] = fmaxf(mx[hb], __shfl_xor(mx[hb], 16));
          mx[hb] = fmaxf(mx[hb], __shfl_xor(mx[hb], 32));
          mxch[(wave * 2 + hb) * 64 + lane] = mx[hb];
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          m_ref[hb] = fmaxf(mx[hb], mxch[(partner * 2 + hb) * 64 + lane]);
          nmu[hb] = m_ref[hb] == kNegInf ? 0.f : -m_ref[hb];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) weight(k / 4, k % 4, bias);
        pack_block0();
      }
      if (gq == 0) kbias[(buf ^ 1) * TK + gk] = id_b >= 0 ? 0.f : kNegInf;
      id_b = id_n;
      raw_n = raw_f;
      pv_prefetch(cur, 0);
      // Block 1's weights; P^T operands in k-slot order: slots 4g..4g+3 of
      // block 0, then of block 1.
#pragma unroll
      for (int k = 0; k < 8; ++k) weight(k / 4, 4 + k % 4, bias);
      bf16x8 pown[2], ppart[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        pown[hb] = __builtin_bit_cast(
            bf16x8, u32x4{p0[hb].x, p0[hb].y, pack2_bf16(ew[hb][4], ew[hb][5]), pack2_bf16(ew[hb][6], ew[hb][7])});
        xch[(wave * 2 + hb) * 64 + lane] = __builtin_bit_cast(u32x4, pown[hb]);
      }
      // The wave's own half first: its P is in registers, and the work
      // covers the partner's softmax before the swap.
      pv_half(cur, 0, pown);
      pv_prefetch(cur, 1);
      __syncthreads();  // P of both halves visible; tile t+1 staged
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        ppart[hb] = __builtin_bit_cast(bf16x8, xch[(partner * 2 + hb) * 64 + lane]);
      pv_half(cur, 1, ppart);
      __syncthreads();  // every wave is done with `cur` and with the P swap
    };
    // Tiles go in pairs (static buffer roles); an odd count ends with one
    // tile past the end, all slots invalid, which adds exactly nothing.
    const std::integral_constant<bool, true> first_tile{};
    const std::integral_constant<bool, false> later_tile{};
    int t = t0;
    if (fix_ref) {
      step(first_tile, t, tile0, tile1, 0);
      step(later_tile, t + 1, tile1, tile0, 1);
      t += 2;
    }
    for (; t < t_end; t += 2) {
      step(later_tile, t, tile0, tile1, 0);
      step(later_tile, t + 1, tile1, tile0, 1);
    }
  };

  // The first tile with a valid slot (uniform over the workgroup); tiles
  // before it add nothing.
  int t0 = t_begin;
  int ids[3];  // the first walk's indices of tiles t0, t0 + 1 (masked) and t0 + 2 (raw)
  ids[0] = -1;
  while (t0 < t_end) {
    ids[0] = load_idx(t0);
    ids[1] = load_idx(t0 + 1);  // in flight with the test
    ids[2] = idx_raw(t0 + 2);
    if (__syncthreads_or(ids[0] >= 0) != 0) break;
    ++t0;
  }
  // Walk once with the first valid tile's max as the reference. Every
  // weight of a lane is at most its partial row sum, so if no lane's sum
  // passed kXSumLimit no weight did, and the bf16 weights and fp32 sums
  // stayed in range. Otherwise walk again from the exact max of the split
  // (the loop body is emitted once).
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) max_pass(t0, t_end);
    walk(t0, pass == 0, ids);
    if (pass == 1) break;
    if (tid == 0) redo[0] = 0u;
    __syncthreads();
    const bool over = l_part[0] > kXSumLimit || l_part[1] > kXSumLimit;
    if (__ballot(over) != 0 && lane == 0) redo[0] = 1u;
    __syncthreads();
    const bool again = redo[0] != 0u;
    __syncthreads();  // every wave has read the flag before it is reset
    if (!again) break;
  }

  // ---- epilogue: row sums over both slot halves; normalise; store.
  float lt[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float t = l_part[hb] + __shfl_xor(l_part[hb], 16);
    t += __shfl_xor(t, 32);
    xf[(wave * 2 + hb) * 64 + lane] = t;
    lt[hb] = t;
  }
  if constexpr (EPI) {
    if (tid < 64) epi_cs[tid] = cs_pre;
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) lt[hb] += xf[(partner * 2 + hb) * 64 + lane];
  const bool split_mode = p.part_o != nullptr;  // partials for the combine kernel
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = h0 + 16 * hb + l16;
    if (h >= p.heads) continue;
    const float inv = lt[hb] > 0.f ? kv_scale / lt[hb] : 0.f;
    if (EPI && !split_mode) {
      // 32-column blocks: d = 2m and 2m + 1 of the four lanes g of a head
#pragma unroll
      for (int m = 0; m < NDW / 2; ++m) {
        const floatx4 ra = o[2 * m][hb] * inv, rb = o[2 * m + 1][hb] * inv;
        float va[4] = {ra[0], ra[1], ra[2], ra[3]}, vb[4] = {rb[0], rb[1], rb[2], rb[3]};
        epi_store_c16x2(p.epi, p.epi.pos != nullptr ? epi_cs : nullptr, r, h,
                        256 * kh + 32 * m + 4 * g, va, vb);
      }
    } else {
#pragma unroll
      for (int d = 0; d < NDW; ++d) {
        const floatx4 res = o[d][hb] * inv;
        const int col = 256 * kh + 16 * d + 4 * g;
        if (!split_mode) {
          *reinterpret_cast<u32x2*>(p.out + r * p.out_rs + int64_t(h) * p.out_hs + col) =
              u32x2{pack_bf16(res[0], res[1]), pack_bf16(res[2], res[3])};
        } else {
          *reinterpret_cast<floatx4*>(
              p.part_o + ((int64_t(split) * p.rows + r) * p.heads + h) * kDv + col) = res;
        }
      }
    }
    if (kh == 0 && g == 0) {
      const float lse = lt[hb] > 0.f ? (m_ref[hb] + __log2f(lt[hb])) * kLn2 : kNegInf;
      if (!split_mode)
        p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = lse;
      else
        p.part_lse[(int64_t(split) * p.rows + r) * p.heads + h] = lse;
    }
  }
}

}  // namespace

KernelShape prefill_fp8_shape(int dqk) {
  KernelShape k;
  k.waves = kXWaves;
  k.tile = kXTile;
  if (dqk == 576)
    k.lds_bytes = XCfg<576>::LDS_BYTES;
  else if (dqk == 512)
    k.lds_bytes = XCfg<512>::LDS_BYTES;
  else
    k = KernelShape{};
  return k;
}

int launch_prefill_fp8(const FwdParams& p, int dqk, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool epi = epi_active(p.epi) && p.part_o == nullptr;
  const dim3 grid(uint32_t(p.grid)), block(kXWaves * 64);
  if (dqk == 576 && epi)
    hipLaunchKernelGGL((prefill_fp8_kernel<576, true>), grid, block, 0, st, p);
  else if (dqk == 576)
    hipLaunchKernelGGL((prefill_fp8_kernel<576, false>), grid, block, 0, st, p);
  else if (dqk == 512 && epi)
    hipLaunchKernelGGL((prefill_fp8_kernel<512, true>), grid, block, 0, st, p);
  else if (dqk == 512)
    hipLaunchKernelGGL((prefill_fp8_kernel<512, false>), grid, block, 0, st, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace smla
