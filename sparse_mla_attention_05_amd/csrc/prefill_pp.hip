// gfx950 64-head kernel of the sparse MLA forward over an fp8 e4m3fn pool,
// 576- or 512-wide rows, with the QK and PV work on different wavefronts.
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
//  * One workgroup = (row, 64 heads, split), 8 wavefronts, two per SIMD, one
//    workgroup per CU. Waves 0-3 are QK waves, waves 4-7 PV waves; a SIMD
//    runs one of each, so the MFMA work of one overlaps the staging, softmax
//    and LDS waits of the other. QK wave (hp, kh) holds Q^T of heads
//    32hp..32hp+31 and computes S^T = K Q^T for slots 16kh..16kh+15 of each
//    32-slot tile (one K fragment feeds two head blocks), then the weights
//    P = 2^(s - ref) of those slots; PV wave (hp, ch) holds O^T for output
//    columns 256ch..256ch+255 of the same 32 heads and runs O^T += V^T P^T
//    over all 32 slots (one V fragment feeds two head blocks), taking P from
//    LDS. Q (144 registers) and O (128) never share a wave, so both fit the
//    256 registers a wave has at two waves per SIMD.
//  * Tiles are staged as bf16 rows in LDS, three buffers: while the QK waves
//    score tile t+1 the PV waves multiply tile t. One barrier per tile: QK
//    waves arrive after writing P(t), PV waves wait on it before PV(t).
//    Staging is 8 threads per slot and 8-byte fp8 chunks, each widened to
//    one 16-byte bf16 chunk and written once, and is split between the
//    roles by cost: the QK waves write the first chunks of tile t+1 between
//    their dots (their LDS has room), the PV waves the rest of tile t+2
//    between theirs (their transposed reads leave less). Each chunk's
//    registers are then refilled with the next gather (unconditional raw
//    buffer loads: invalid slots read past the buffer range and get zeros).
//    Rows are unpadded, the 16-byte chunk index XOR-permuted per row so that
//    the K reads, the transposed V reads and the staging writes are free of
//    bank conflicts.
//  * Fixed reference: a head's reference max is the max over the first tile
//    with a valid slot, from a scoring pre-pass over that tile, so O is
//    never rescaled. The bf16 P and fp32 sums stay in range while every
//    weight is at most 2^64; every weight a lane adds is at most its partial
//    row sum, so if no partial sum passes 2^64 none did. Otherwise the
//    workgroup scores all its tiles for the exact max and walks again.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

constexpr int kPWaves = 8;
constexpr int kPTile = 32;
constexpr float kPSumLimit = 0x1p64f;  // bound on the weights against the reference
constexpr uint32_t kPOutOfRange = 0xFFFFF000u;
constexpr int kPBufferWord3 = 0x00020000;

template <int DQK>
struct PCfg {
  static constexpr int TK = kPTile;
  static constexpr int KSTEPS = DQK / 32;
  static constexpr int ROW = DQK * 2;              // bytes per bf16 tile row
  static constexpr int TILE = TK * ROW;            // bytes per bf16 tile
  static constexpr int TPR = 256 / TK;             // staging threads per slot (per role)
  static constexpr int CH8 = DQK / 8;              // 8-byte fp8 chunks per pool row
  static constexpr int LPT = CH8 / TPR;            // chunks per staging thread
  static constexpr int NDW = kDv / 16 / 2;         // 16-column output blocks per PV wave
  static constexpr int SWB = DQK == 576 ? 8 : 16;  // chunk span the row permutation touches
  static constexpr int NQB = SWB / 4;              // K-operand address bases
  static constexpr int NVB = SWB / 2;              // V-operand address bases
  static constexpr int QKC = DQK == 576 ? 6 : 4;    // chunks per thread staged by the QK waves
  static constexpr int PBUF = 2 * 4 * 2 * 64 * 8;  // P of a tile: [qk wave][head block][lane] 8 B, x2
  static constexpr int LDS_BYTES = 3 * TILE + 3 * TK * 4 + PBUF + 4 * 2 * 64 * 4 + 16;
  static_assert(CH8 % TPR == 0, "staging split");
  static_assert(2 * QKC <= KSTEPS && LPT - QKC <= NDW, "staging spread over the dots");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int DQK>
__device__ __forceinline__ int pp_perm(int r) {
  if constexpr (DQK == 576) return (r & 3) | (((r ^ (r >> 2)) & 1) << 2);
  return ((r & 1) * 3) | (((r ^ (r >> 1)) & 1) << 2) | (((r >> 2) & 1) << 3);
}

// EPI: the final store goes through the output epilogue (epilogue.h).
template <int DQK, bool EPI>
__global__ void __launch_bounds__(kPWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_pp_kernel(const FwdParams p) {
  using C = PCfg<DQK>;
  constexpr int TK = C::TK, ROW = C::ROW, TILE = C::TILE, KSTEPS = C::KSTEPS;
  constexpr int LPT = C::LPT, NDW = C::NDW, SWB = C::SWB, NQB = C::NQB, NVB = C::NVB;
  constexpr int QKC = C::QKC;

  __shared__ __attribute__((aligned(16))) uint8_t tiles[3 * TILE];
  __shared__ __attribute__((aligned(16))) float kbias[3 * TK];  // 0 (valid slot) or -inf
  // P of tile parity x: [x][qk wave][head block][lane], 4 bf16 each.
  __shared__ __attribute__((aligned(16))) u32x2 pbuf[2 * 4 * 2 * 64];
  // Max / row-sum exchange: [qk wave][head block][lane].
  __shared__ __attribute__((aligned(16))) float xq[4 * 2 * 64];
  __shared__ uint32_t redo[1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const bool qk_role = wave < 4;
  const int w4 = wave & 3;
  const int hp = w4 >> 1, kh = w4 & 1;  // kh: slot block (QK) or column half (PV)

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
    if (p.epi.pos != nullptr && wave == 4) cs_pre = epi_cs_row(p.epi, r)[lane];
  }

  const int h0 = hblk * 64 + 32 * hp;  // heads h0 + 16hb + l16 of this lane

  const int ntiles = (p.topk + TK - 1) / TK;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);
  const float kv_scale = *p.kv_scale;
  const float score_scale = p.sm_log2 * q_scale_of(p.q_scale) * kv_scale;
  const bool split_mode = p.part_o != nullptr;  // partials for the combine kernel

  // ---- staging (both roles, same mapping): slot gk of a tile, 8-byte chunks gq + 8i.
  const int qtid = tid & 255;
  const int gk = qtid / C::TPR, gq = qtid % C::TPR;
  const int32_t* idx_row = p.idx + r * p.idx_rs;
  const int last_slot = min(p.topk, t_end * TK) - 1;
  const __amdgpu_buffer_rsrc_t idx_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(idx_row), 0, 4 * (last_slot + 1), kPBufferWord3);
  auto idx_raw = [&](int t) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(idx_rsrc, uint32_t(4 * gk), 4 * t * TK, 0);
  };
  auto idx_mask = [&](int t) -> int { return -int(!(t < t_end && gk <= last_slot - t * TK)); };
  auto load_idx = [&](int t) -> int { return idx_raw(t) | idx_mask(t); };
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.pool), 0, p.pool_bytes, kPBufferWord3);
  const PoolMap pm{uint32_t(p.pool_rs_bytes), uint32_t(p.page_bytes), uint32_t(p.page_shift),
                   p.page_mask};
  auto row_off = [&](int id) -> uint32_t { return id >= 0 ? slot_offset(pm, id) : kPOutOfRange; };
  const int gperm = pp_perm<DQK>(gk);
  auto chunk_addr = [&](int i) -> int {  // bf16 16-byte chunk gq + 8i of row gk
    const int c = gq + 8 * i;
    return gk * ROW + 16 * ((c & ~(SWB - 1)) | ((c & (SWB - 1)) ^ gperm));
  };
  u32x2 pre[LPT];
  auto gather_one = [&](int i, uint32_t off) {
    pre[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                           pool_rsrc, off + 8u * uint32_t(gq + 8 * i), 0, 0));
  };
  auto gather = [&](int id, int lo, int hi) {
    const uint32_t off = row_off(id);
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      if (i >= lo && i < hi) gather_one(i, off);
  };
  auto stage_chunk = [&](int i, uint8_t* tile) {
    *reinterpret_cast<bf16x8*>(tile + chunk_addr(i)) = widen_fp8x8(pre[i].x, pre[i].y);
  };
  auto buf_of = [&](int k) -> uint8_t* { return tiles + k * TILE; };

  float* const xf = xq;
  int t0 = t_begin;
  while (t0 < t_end && __syncthreads_or(qk_role && gq == 0 ? (load_idx(t0) >= 0) : 0) == 0) ++t0;

  if (qk_role) {
    // ================================================================ QK waves
    bf16x8 qf[2][KSTEPS];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = h0 + 16 * hb + l16;
      if (h < p.heads) {
        const int64_t qp = r * p.q_rs + int64_t(h) * p.q_hs + 8 * g;
        load_q_frags(p.q, p.q_fp8, qp, 32, qf[hb]);
      } else {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[hb][s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      }
    }
    const int qperm = pp_perm<DQK>(l16);
    int kbase[NQB];
#pragma unroll
    for (int b = 0; b < NQB; ++b) kbase[b] = (16 * kh + l16) * ROW + 16 * ((4 * b + g) ^ qperm);

    floatx4 sacc[2];
    // S^T of this wave's 16 slots of the tile in `cur`; with `stage`, chunks
    // 0..QKC-1 of the next tile are widened from `pre` into `nxt` between the
    // dots and their registers refilled from next_off.
    auto qk = [&](const uint8_t* cur, uint8_t* nxt, uint32_t next_off, bool stage) {
      sacc[0] = sacc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
      constexpr int KRING = 4;
      bf16x8 ka[KRING];
      auto load_k = [&](int s) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(cur + kbase[s % NQB] + 16 * SWB * (s / NQB));
      };
#pragma unroll
      for (int s = 0; s < KRING - 1; ++s) ka[s] = load_k(s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        if (s + KRING - 1 < KSTEPS) ka[(s + KRING - 1) % KRING] = load_k(s + KRING - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s % KRING], qf[hb][s], sacc[hb], 0, 0, 0);
        if (stage && s % 2 == 1 && s / 2 < QKC) {
          stage_chunk(s / 2, nxt);
          gather_one(s / 2, next_off);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto load_bias = [&](int buf, float (&b)[4]) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(kbias + buf * TK + 16 * kh + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = v[i];
    };

    float m_ref[2], nmu[2], l_part[2];
    auto max_pass = [&](int t_from, int t_to) {
      float mx[2] = {kNegInf, kNegInf};
#pragma clang loop unroll(disable)
      for (int t = t_from; t < t_to; ++t) {
        __syncthreads();  // tile t staged in buffer 0 by the PV waves
        float b[4];
        load_bias(0, b);
        qk(buf_of(0), buf_of(1), 0u, false);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx[hb] = fmaxf(mx[hb], __builtin_fmaf(sacc[hb][i], score_scale, b[i]));
        __syncthreads();  // buffer 0 and the flags are free for the next tile
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float t = fmaxf(mx[hb], __shfl_xor(mx[hb], 16));
        t = fmaxf(t, __shfl_xor(t, 32));
        xf[(w4 * 2 + hb) * 64 + lane] = t;
        mx[hb] = t;
      }
      __syncthreads();
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) m_ref[hb] = fmaxf(mx[hb], xf[((w4 ^ 1) * 2 + hb) * 64 + lane]);
      __syncthreads();
    };

    auto walk = [&](int tw) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) nmu[hb] = m_ref[hb] == kNegInf ? 0.f : -m_ref[hb];
      l_part[0] = l_part[1] = 0.f;
      if (tw >= t_end) return;
      // Chunks 0..QKC-1 of tile tw staged, those of tile tw+1 in flight.
      int id_a = load_idx(tw);
      gather(id_a, 0, QKC);
#pragma unroll
      for (int i = 0; i < QKC; ++i) stage_chunk(i, buf_of(0));
      if (gq == 0) kbias[gk] = id_a >= 0 ? 0.f : kNegInf;
      int id_b = load_idx(tw + 1);
      int raw_n = idx_raw(tw + 2);  // masked where it is used
      gather(id_b, 0, QKC);
      __syncthreads();  // tile tw staged; the other chunks of tile tw+1 too
#pragma clang loop unroll(disable)
      for (int t = tw; t < t_end; ++t) {
        const int k = (t - tw) % 3;
        const int kn = k == 2 ? 0 : k + 1;
        const int raw_f = idx_raw(t + 3);
        __builtin_amdgcn_sched_barrier(0);
        const int id_n = raw_n | idx_mask(t + 2);
        qk(buf_of(k), buf_of(kn), row_off(id_n), true);
        if (gq == 0) kbias[kn * TK + gk] = id_b >= 0 ? 0.f : kNegInf;
        id_b = id_n;
        raw_n = raw_f;
        float b[4];
        load_bias(k, b);
        u32x2* const pw = pbuf + (((t - tw) & 1) * 4 + w4) * 2 * 64 + lane;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[hb][i], score_scale, b[i] + nmu[hb]));
            l_part[hb] += e[i];
          }
          pw[hb * 64] = u32x2{pack2_bf16(e[0], e[1]), pack2_bf16(e[2], e[3])};
        }
        __syncthreads();  // P(t) visible; tile t+2 staged while the PV waves multiply tile t
      }
      __syncthreads();  // the PV waves are done with the last tile
    };

#pragma clang loop unroll(disable)
    for (int pass = 0; pass < 2; ++pass) {
      max_pass(t0, pass == 0 ? min(t0 + 1, t_end) : t_end);
      walk(t0);
      if (pass == 1) break;
      if (tid == 0) redo[0] = 0u;
      __syncthreads();
      const bool over = l_part[0] > kPSumLimit || l_part[1] > kPSumLimit;
      if (__ballot(over) != 0 && lane == 0) redo[0] = 1u;
      __syncthreads();
      const bool again = redo[0] != 0u;
      __syncthreads();
      if (!again) break;
    }
    // Row sums: this wave's share for its 16-slot blocks; the pair adds up.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float t = l_part[hb] + __shfl_xor(l_part[hb], 16);
      t += __shfl_xor(t, 32);
      xf[(w4 * 2 + hb) * 64 + lane] = t;
    }
    __syncthreads();
    if (kh == 0 && g == 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int h = h0 + 16 * hb + l16;
        if (h >= p.heads) continue;
        const float lt = xf[(w4 * 2 + hb) * 64 + lane] + xf[((w4 ^ 1) * 2 + hb) * 64 + lane];
        const float lse = lt > 0.f ? (m_ref[hb] + __log2f(lt)) * kLn2 : kNegInf;
        if (!split_mode)
          p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = lse;
        else
          p.part_lse[(int64_t(split) * p.rows + r) * p.heads + h] = lse;
      }
    }
  } else {
    // ================================================================ PV waves
    const int vrow = 4 * g + (l16 >> 2);
    const int vperm = pp_perm<DQK>(vrow);
    int vbase[NVB];
#pragma unroll
    for (int b = 0; b < NVB; ++b)
      vbase[b] = vrow * ROW + 16 * 32 * kh + 16 * ((2 * b + ((l16 >> 1) & 1)) ^ vperm) + 8 * (l16 & 1);
    constexpr int VRING = 3;
    bf16x8 vf[VRING];
    auto load_v = [&](const uint8_t* cur, int d) -> bf16x8 {
      const uint16_t* va = reinterpret_cast<const uint16_t*>(cur + vbase[d % NVB] + 16 * SWB * (d / NVB));
      const u32x2 v0 = lds_read_tr16(va);
      const u32x2 v1 = lds_read_tr16(va + 8 * ROW);  // 16 rows further
      return __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
    };
    floatx4 o[NDW][2];
#pragma unroll
    for (int d = 0; d < NDW; ++d) o[d][0] = o[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The PV waves also stage every tile. Their barriers mirror the QK
    // waves': the reference pre-pass (2 per tile plus 2), the walk (1 + 1
    // per tile + 1), the redo check (3).
    auto max_pass_stage = [&](int t_from, int t_to) {
#pragma clang loop unroll(disable)
      for (int t = t_from; t < t_to; ++t) {
        const int id = load_idx(t);
        gather(id, 0, LPT);
#pragma unroll
        for (int i = 0; i < LPT; ++i) stage_chunk(i, buf_of(0));
        if (gq == 0) kbias[gk] = id >= 0 ? 0.f : kNegInf;
        __syncthreads();
        __syncthreads();  // the QK waves are done with buffer 0
      }
      __syncthreads();
      __syncthreads();
    };
    auto walk = [&](int tw) {
#pragma unroll
      for (int d = 0; d < NDW; ++d) o[d][0] = o[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (tw >= t_end) return;
      // Chunks QKC..LPT-1 of tiles tw and tw+1 staged, those of tile tw+2 in
      // flight (the QK waves stage chunks 0..QKC-1, one tile ahead).
      int id_c = load_idx(tw);
      gather(id_c, QKC, LPT);
#pragma unroll
      for (int i = QKC; i < LPT; ++i) stage_chunk(i, buf_of(0));
      id_c = load_idx(tw + 1);
      gather(id_c, QKC, LPT);
#pragma unroll
      for (int i = QKC; i < LPT; ++i) stage_chunk(i, buf_of(1));
      id_c = load_idx(tw + 2);
      int raw_n = idx_raw(tw + 3);  // masked where it is used
      gather(id_c, QKC, LPT);
      __syncthreads();  // tiles tw and tw+1 staged
#pragma clang loop unroll(disable)
      for (int t = tw; t < t_end; ++t) {
        const int k = (t - tw) % 3;
        const int ks = k == 0 ? 2 : k - 1;  // buffer of tile t+2 (last used by tile t-1)
        const uint8_t* cur = buf_of(k);
        uint8_t* const stg = buf_of(ks);
        // The index of tile t+4 is loaded before the gathers of tile t+3, so
        // waiting for it never waits for them.
        const int raw_f = idx_raw(t + 4);
        __builtin_amdgcn_sched_barrier(0);
        const int id_n = raw_n | idx_mask(t + 3);
        const uint32_t next_off = row_off(id_n);
        __syncthreads();  // P(t) visible; every wave is done with tile t-1
        const u32x2* const pr = pbuf + (((t - tw) & 1) * 4 + 2 * hp) * 2 * 64 + lane;
        bf16x8 pk[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const u32x2 a = pr[hb * 64], b = pr[2 * 64 + hb * 64];
          pk[hb] = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
        }
#pragma unroll
        for (int d = 0; d < VRING - 1; ++d) vf[d] = load_v(cur, d);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < NDW; ++d) {
          if (d + VRING - 1 < NDW) vf[(d + VRING - 1) % VRING] = load_v(cur, d + VRING - 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            o[d][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d % VRING], pk[hb], o[d][hb], 0, 0, 0);
          if (d < LPT - QKC) {
            // Tile t+2, chunk QKC+d: widened into its buffer, then the
            // registers refilled with the gather of tile t+3.
            stage_chunk(QKC + d, stg);
            gather_one(QKC + d, next_off);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        id_c = id_n;
        raw_n = raw_f;
      }
      __syncthreads();  // done with the last tile
    };
#pragma clang loop unroll(disable)
    for (int pass = 0; pass < 2; ++pass) {
      max_pass_stage(t0, pass == 0 ? min(t0 + 1, t_end) : t_end);
      walk(t0);
      if (pass == 1) break;
      __syncthreads();
      __syncthreads();
      const bool again = redo[0] != 0u;
      __syncthreads();
      if (!again) break;
    }
    if constexpr (EPI) {
      if (wave == 4) epi_cs[lane] = cs_pre;
    }
    __syncthreads();  // row sums of the QK waves in xq
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = h0 + 16 * hb + l16;
      if (h >= p.heads) continue;
      const float lt = xf[((2 * hp) * 2 + hb) * 64 + lane] + xf[((2 * hp + 1) * 2 + hb) * 64 + lane];
      const float inv = lt > 0.f ? kv_scale / lt : 0.f;
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
    }
  }
}

}  // namespace

KernelShape prefill_pp_shape(int dqk) {
  KernelShape k;
  k.waves = kPWaves;
  k.tile = kPTile;
  if (dqk == 576)
    k.lds_bytes = PCfg<576>::LDS_BYTES;
  else if (dqk == 512)
    k.lds_bytes = PCfg<512>::LDS_BYTES;
  else
    k = KernelShape{};
  return k;
}

int launch_prefill_pp(const FwdParams& p, int dqk, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool epi = epi_active(p.epi) && p.part_o == nullptr;
  const dim3 grid(uint32_t(p.grid)), block(kPWaves * 64);
  if (dqk == 576 && epi)
    hipLaunchKernelGGL((prefill_pp_kernel<576, true>), grid, block, 0, st, p);
  else if (dqk == 576)
    hipLaunchKernelGGL((prefill_pp_kernel<576, false>), grid, block, 0, st, p);
  else if (dqk == 512 && epi)
    hipLaunchKernelGGL((prefill_pp_kernel<512, true>), grid, block, 0, st, p);
  else if (dqk == 512)
    hipLaunchKernelGGL((prefill_pp_kernel<512, false>), grid, block, 0, st, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace smla
