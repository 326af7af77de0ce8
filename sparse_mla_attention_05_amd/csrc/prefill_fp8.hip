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
//    CU, one wavefront per SIMD. Wave w owns heads 16w..16w+15 over every
//    slot: Q^T in VGPRs, S^T and O^T accumulators in AGPRs. S^T = K Q^T
//    leaves each lane 4 consecutive slots of one head, which is the B operand
//    layout of O^T += V^T P^T, so P never leaves the registers and the
//    softmax needs no exchange between waves.
//  * K/V tiles of 64 slots are staged once per workgroup as bf16 rows in
//    LDS, double buffered. Rows are unpadded; the 16-byte chunk index of
//    row r is XOR-permuted by a function of r chosen so that the K operand
//    reads (ds_read_b128), the transposed V reads (ds_read_b64_tr_b16) and
//    the staging writes (ds_write_b128) are all free of bank conflicts on
//    gfx950.
//  * The gather for tile t+2 (unconditional raw buffer loads: invalid slots
//    read past the buffer range and get zeros) is in flight while tile t is
//    computed; tile t+1 is widened and written into the other buffer between
//    the QK dots of tile t. One barrier per tile.
//  * Fixed reference: a head's reference max is the max of its first tile
//    with a valid slot (O is still zero then), so O is never rescaled and
//    stays in the MFMA accumulators. P = exp2(s - ref) is exact in real
//    arithmetic whatever the reference; the bf16 P and fp32 sums stay in
//    range while every later score is below ref + 64 (log2 domain). If any
//    head exceeds that, the workgroup walks its slots a second time with the
//    exact row max, tracked during the first walk, as the reference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

constexpr int kXWaves = 4;
constexpr int kXTile = 64;
constexpr float kXRefSlack = 64.0f;  // P <= 2^64 against the reference
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
  static constexpr int NDB = kDv / 16;             // 16-column output blocks
  static constexpr int SWB = DQK == 576 ? 8 : 16;  // chunk span the row permutation touches
  static constexpr int NQB = SWB / 4;              // K-operand address bases
  static constexpr int NVB = SWB / 2;              // V-operand address bases
  static constexpr int NSB = SWB / 8;              // staging address bases per half
  static constexpr int NSLOTB = TK / 16;           // 16-slot blocks per tile
  static constexpr int LDS_BYTES = 2 * TILE + 2 * TK * 4 + 16;
  static_assert(SRC_CH % TPR == 0, "staging split");
  static_assert(LPT % NSB == 0, "staging bases");
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

template <int DQK>
__global__ void __launch_bounds__(kXWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_fp8_kernel(const FwdParams p) {
  using C = XCfg<DQK>;
  constexpr int TK = C::TK, ROW = C::ROW, TILE = C::TILE, KSTEPS = C::KSTEPS;
  constexpr int LPT = C::LPT, NDB = C::NDB, SWB = C::SWB;
  constexpr int NQB = C::NQB, NVB = C::NVB, NSB = C::NSB;

  // Two bf16 tile buffers as separate arrays, so the compiler can tell the
  // staging writes into one from the operand reads of the other.
  __shared__ __attribute__((aligned(16))) uint8_t tile0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[TILE];
  __shared__ __attribute__((aligned(16))) float kbias[2 * TK];  // 0 (valid slot) or -inf
  __shared__ uint32_t redo[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  int64_t work = p.remap ? smla_xcd_work(blockIdx.x, p.grid) : int64_t(blockIdx.x);
  const int hblk = int(work % p.head_blocks);
  work /= p.head_blocks;
  const int split = int(work % p.splits);
  const int64_t r = work / p.splits;
  const int head = hblk * C::HB + 16 * wave + l16;  // this lane's head (S^T / O^T column)
  const bool head_ok = head < p.heads;

  const int ntiles = (p.topk + TK - 1) / TK;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

  // Q^T operands: columns 8g + 32s .. +7 of this lane's head.
  bf16x8 qf[KSTEPS];
  if (head_ok) {
    const uint16_t* qp = p.q + r * p.q_rs + int64_t(head) * p.q_hs + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const float kv_scale = *p.kv_scale;
  const float score_scale = p.sm_log2 * kv_scale;

  // ---- staging role: slot gk of a tile, fp8 chunks gq, gq + 4, ...
  const int gk = tid / C::TPR, gq = tid % C::TPR;
  const int32_t* idx_row = p.idx + r * p.idx_rs;
  const int last_slot = min(p.topk, t_end * TK) - 1;
  auto load_idx = [&](int t) -> int {
    const int j = t * TK + gk;
    const int v = idx_row[min(j, last_slot)];
    return v | -int(!(t < t_end && j <= last_slot));
  };
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.pool), 0, p.pool_bytes, kXBufferWord3);
  u32x4 pre[LPT];
  auto gather = [&](int id) {
    const uint32_t off = id >= 0 ? uint32_t(id) * uint32_t(p.pool_rs_bytes) : kXOutOfRange;
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      pre[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             pool_rsrc, off + 16u * uint32_t(gq + 4 * i), 0, 0));
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

  // ---- K operand addresses: row 16j + l16, logical chunk g + 4s.
  const int qperm = tile_perm<DQK>(l16);
  int kbase[NQB];
#pragma unroll
  for (int b = 0; b < NQB; ++b) kbase[b] = l16 * ROW + 16 * ((4 * b + g) ^ qperm);
  // ---- V^T operand addresses: rows 32ks + 4g + l16/4 (+16), columns
  // 16d + 4(l16 % 4) .. +3, i.e. logical chunk 2d + (l16/2)%2, byte 8(l16%2).
  const int vrow = 4 * g + (l16 >> 2);
  const int vperm = tile_perm<DQK>(vrow);
  int vbase[NVB];
#pragma unroll
  for (int b = 0; b < NVB; ++b)
    vbase[b] = vrow * ROW + 16 * ((2 * b + ((l16 >> 1) & 1)) ^ vperm) + 8 * (l16 & 1);

  floatx4 o[NDB];
  float m_ref;       // reference max (log2 domain) of this lane's head
  float m_run;       // running max of this lane's scores
  float l_part;      // this lane's share of the head's row sum
  bool over;         // some score of this lane exceeded m_ref + kXRefSlack

  // QK of the tile in `cur`, with the staging of the next tile from `pre`
  // into `nxt` spread between the k-steps.
  floatx4 sacc[C::NSLOTB];
  auto qk_and_stage = [&](const uint8_t* cur, uint8_t* nxt) {
#pragma unroll
    for (int j = 0; j < C::NSLOTB; ++j) sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    // K fragments in a ring of KRING k-steps: the reads run KRING-1 k-steps
    // ahead of the dots that use them.
    constexpr int KRING = 3;
    bf16x8 ka[KRING][C::NSLOTB];
    auto load_k = [&](int s, bf16x8 (&dst)[C::NSLOTB]) {
      const uint8_t* kp = cur + kbase[s % NQB] + 16 * SWB * (s / NQB);
#pragma unroll
      for (int j = 0; j < C::NSLOTB; ++j)
        dst[j] = *reinterpret_cast<const bf16x8*>(kp + j * 16 * ROW);
    };
#pragma unroll
    for (int s = 0; s < KRING - 1; ++s) load_k(s, ka[s]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      // The fences keep the scheduler from sinking the reads to their uses.
      if (s + KRING - 1 < KSTEPS) load_k(s + KRING - 1, ka[(s + KRING - 1) % KRING]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < C::NSLOTB; ++j)
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s % KRING][j], qf[s], sacc[j], 0, 0, 0);
      if (s % 2 == 1 && s / 2 < LPT) stage_chunk(s / 2, nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Softmax weights of the tile in buffer `buf`; returns the P^T operands of
  // the two 32-slot k-steps (k-slot order: slots 4g..4g+3 of block 2ks, then
  // of block 2ks+1).
  auto softmax = [&](int buf, bf16x8 (&pf)[2]) {
    const float* kb = kbias + buf * TK + 4 * g;
    float v[C::NSLOTB][4];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < C::NSLOTB; ++j) {
      const floatx4 b = *reinterpret_cast<const floatx4*>(kb + 16 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][i] = __builtin_fmaf(sacc[j][i], score_scale, b[i]);
        mx = fmaxf(mx, v[j][i]);
      }
    }
    m_run = fmaxf(m_run, mx);
    // Slot validity is shared by all heads, so the reference is unset either
    // for every lane of the wave or for none.
    if (m_ref == kNegInf) {
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      m_ref = fmaxf(mx, __shfl_xor(mx, 32));
    }
    over = over || mx > m_ref + kXRefSlack;
    const float mu = m_ref == kNegInf ? 0.f : m_ref;
    float e[C::NSLOTB][4];
#pragma unroll
    for (int j = 0; j < C::NSLOTB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[j][i] = __builtin_amdgcn_exp2f(v[j][i] - mu);
        l_part += e[j][i];
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pf[ks] = __builtin_bit_cast(
          bf16x8, u32x4{pack2_bf16(e[2 * ks][0], e[2 * ks][1]), pack2_bf16(e[2 * ks][2], e[2 * ks][3]),
                        pack2_bf16(e[2 * ks + 1][0], e[2 * ks + 1][1]),
                        pack2_bf16(e[2 * ks + 1][2], e[2 * ks + 1][3])});
  };
  // O^T += V^T P^T over the tile in `cur`.
  // V^T fragments in a ring of VRING output blocks; the first VRING-1 are
  // read before the softmax (they do not depend on P).
  constexpr int VRING = 3;
  bf16x8 vf[VRING][2];
  auto load_v = [&](const uint8_t* cur, int d, bf16x8 (&dst)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint16_t* va = reinterpret_cast<const uint16_t*>(
          cur + vbase[d % NVB] + 16 * SWB * (d / NVB) + 32 * ks * ROW);
      const u32x2 v0 = lds_read_tr16(va);
      const u32x2 v1 = lds_read_tr16(va + 8 * ROW);  // 16 rows further
      dst[ks] = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
    }
  };
  auto pv_prefetch = [&](const uint8_t* cur) {
#pragma unroll
    for (int d = 0; d < VRING - 1; ++d) load_v(cur, d, vf[d]);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pv = [&](const uint8_t* cur, const bf16x8 (&pf)[2]) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      if (d + VRING - 1 < NDB) load_v(cur, d + VRING - 1, vf[(d + VRING - 1) % VRING]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d % VRING][ks], pf[ks], o[d], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One walk over this split's tiles with the given starting reference.
  auto walk = [&](float m_init) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_ref = m_init;
    m_run = kNegInf;
    l_part = 0.f;
    over = false;
    if (t_begin >= t_end) return;
    int id_a = load_idx(t_begin);
    gather(id_a);
#pragma unroll
    for (int i = 0; i < LPT; ++i) stage_chunk(i, tile0);
    if (gq == 0) kbias[gk] = id_a >= 0 ? 0.f : kNegInf;
    int id_b = load_idx(t_begin + 1);
    gather(id_b);
    int id_n = load_idx(t_begin + 2);
    __syncthreads();
    // One tile: QK of tile t from `cur` with tile t+1 (zeros past the end:
    // harmless, never read) staged into `nxt`, the buffer tile t-1 used,
    // which every wave finished before the last barrier; then softmax, PV.
    auto step = [&](int t, const uint8_t* cur, uint8_t* nxt, int buf) {
      qk_and_stage(cur, nxt);
      if (gq == 0) kbias[(buf ^ 1) * TK + gk] = id_b >= 0 ? 0.f : kNegInf;
      id_b = id_n;
      gather(id_b);
      id_n = load_idx(t + 3);
      pv_prefetch(cur);
      bf16x8 pf[2];
      softmax(buf, pf);
      pv(cur, pf);
      __syncthreads();
    };
    // Tiles go in pairs (static buffer roles); an odd count ends with one
    // tile past the end, all slots invalid, which adds exactly nothing.
    for (int t = t_begin; t < t_end; t += 2) {
      step(t, tile0, tile1, 0);
      step(t + 1, tile1, tile0, 1);
    }
  };
  // Walk once; if any lane of the workgroup went over the slack, walk again
  // from the row max (the loop body is emitted once).
  float m_init = kNegInf;
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
    walk(m_init);
    if (pass == 1) break;
    if (tid == 0) redo[0] = 0u;
    __syncthreads();
    if (__ballot(over) != 0 && lane == 0) redo[0] = 1u;
    __syncthreads();
    const bool again = redo[0] != 0u;
    __syncthreads();  // every wave has read the flag before a walk reuses LDS
    if (!again) break;
    m_init = fmaxf(m_run, __shfl_xor(m_run, 16));
    m_init = fmaxf(m_init, __shfl_xor(m_init, 32));
  }

  // ---- epilogue: the four lanes of a head hold parts of its row sum.
  float lt = l_part;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (head_ok) {
    const float inv = lt > 0.f ? kv_scale / lt : 0.f;
    const bool split_mode = p.splits > 1;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const floatx4 res = o[d] * inv;
      const int col = 16 * d + 4 * g;
      if (!split_mode) {
        *reinterpret_cast<u32x2*>(p.out + r * p.out_rs + int64_t(head) * p.out_hs + col) =
            u32x2{pack_bf16(res[0], res[1]), pack_bf16(res[2], res[3])};
      } else {
        *reinterpret_cast<floatx4*>(
            p.part_o + ((int64_t(split) * p.rows + r) * p.heads + head) * kDv + col) = res;
      }
    }
    if (g == 0) {
      const float lse = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : kNegInf;
      if (!split_mode)
        p.lse[r * p.lse_rs + int64_t(head) * p.lse_hs] = lse;
      else
        p.part_lse[(int64_t(split) * p.rows + r) * p.heads + head] = lse;
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
  const dim3 grid(uint32_t(p.grid)), block(kXWaves * 64);
  if (dqk == 576)
    hipLaunchKernelGGL((prefill_fp8_kernel<576>), grid, block, 0, st, p);
  else if (dqk == 512)
    hipLaunchKernelGGL((prefill_fp8_kernel<512>), grid, block, 0, st, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace smla
