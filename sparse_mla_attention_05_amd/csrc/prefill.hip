// gfx950 prefill kernel of the sparse MLA forward: 64 heads per workgroup,
// 576- or 512-wide rows, bf16 or fp8 e4m3fn pool.
//
// The method (per row r, head h, over the row's valid slots j):
//   s_j = sm_scale * q[r,h] . K[idx_j] (D_qk columns), out = softmax(s) V
//   (V = first 512 columns), lse = ln sum_j exp(s_j)
// after "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159):
// Technical Details and the commit notes on the 64-head program (one program
// gathers each key tile once for all 64 heads, 8 warps split 64 heads x 64
// keys as 4 x 2), the softmax row exchange through LDS, the padded LDS tile
// and the 16x16x32 bf16 dots.
//
// One workgroup = (row, 64 heads, split), 8 wavefronts, one workgroup per CU.
//  * Tiles of 64 slots, double-buffered in LDS as bf16 rows padded to an odd
//    multiple of 16 bytes modulo 256 (conflict-free MFMA operand reads). The
//    gather for tile t+2 runs into VGPRs (unconditional raw buffer loads:
//    invalid slots read past the buffer range and get zeros) while tile t is
//    computed; tile t+1 is widened and staged into the other buffer.
//  * Wave (hg, kg) owns head group hg (16 heads, Q^T in VGPRs) and slot half
//    kg for S^T = K Q^T; the two halves of a head group exchange their tile
//    row max through LDS, so both use the same running max.
//  * P (bf16, in the PV k-slot order S^T leaves in the lanes) goes through
//    LDS; for O += P V each wave owns 64 output columns of all 64 heads and
//    reads V with the transposed 16-bit read.
//  * Per tile the waves run PV(t) and QK(t+1) back to back (one MFMA phase),
//    then the softmax of t+1 and the staging of t+2 (one VALU/LDS phase):
//    two barriers per tile.
//  * Lazy max: the reference max of a head moves only when a tile max exceeds
//    it by more than 8 in the log2 domain (P <= 2^8); a workgroup-wide flag
//    lets the PV waves skip the O rescale on the (usual) tiles where nothing
//    moved. Exact in real arithmetic: the final normalisation uses the same
//    reference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

constexpr int kPreWaves = 8;
constexpr int kPreTile = 64;
constexpr float kPreLazyMax = 8.0f;
constexpr uint32_t kPreOutOfRange = 0xFFFFF000u;
constexpr int kPreBufferWord3 = 0x00020000;

template <int DQK, bool FP8>
struct PreCfg {
  static constexpr int HB = 64, NHG = 4, NKG = 2, BPW = 2;
  static constexpr int NT = kPreWaves * 64;
  static constexpr int TK = kPreTile;
  static constexpr int KSTEPS = DQK / 32;
  static constexpr int PITCH = DQK + 8;        // bf16 elements per LDS row
  static constexpr int PP = TK + 8;            // P row pitch (elements)
  static constexpr int DW = kDv / kPreWaves;   // output columns per wave (64)
  static constexpr int NB = DW / 16;
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int CH = DQK * EB / 16;     // 16-byte chunks per pool row
  static constexpr int TPK = NT / TK;          // gather threads per slot (8)
  static constexpr int LPT = (CH + TPK - 1) / TPK;
  static constexpr int TILE_BYTES = TK * PITCH * 2;
  static constexpr int LDS_BYTES = 2 * TILE_BYTES + HB * PP * 2 + NKG * HB * 4 + 2 * HB * 4 +
                                   2 * TK + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// EPI: the final store goes through the output epilogue (epilogue.h).
template <int DQK, bool FP8, bool EPI>
__global__ void __launch_bounds__(kPreWaves * 64, 1) prefill_kernel(const FwdParams p) {
  using C = PreCfg<DQK, FP8>;
  constexpr int HB = C::HB, NHG = C::NHG, NKG = C::NKG, BPW = C::BPW, TK = C::TK;
  constexpr int PITCH = C::PITCH, PP = C::PP, NB = C::NB, TPK = C::TPK, LPT = C::LPT;
  constexpr int CH = C::CH, KSTEPS = C::KSTEPS;

  __shared__ __attribute__((aligned(16))) uint16_t kt[2][TK * PITCH];  // bf16 tiles
  __shared__ __attribute__((aligned(16))) uint16_t pt[HB * PP];        // bf16 P
  __shared__ __attribute__((aligned(16))) float red[NKG * HB];         // row max / sum exchange
  __shared__ __attribute__((aligned(16))) float alpha_s[HB];           // rescale factors
  __shared__ __attribute__((aligned(16))) float mfin_s[HB];            // final reference max
  __shared__ __attribute__((aligned(4))) uint8_t kvalid[2][TK];        // slot validity per buffer
  __shared__ __attribute__((aligned(16))) uint32_t upd_flag[4];        // any rescale, per head group

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  int64_t work = p.remap ? smla_xcd_work(blockIdx.x, p.grid) : int64_t(blockIdx.x);
  const int hb = int(work % p.head_blocks);
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

  const int h0 = hb * HB;

  // Tiles [0, T1) hold the main top-k, tiles [T1, ntiles) a second segment
  // when one is given (bf16 pools: its rows need no scale of their own); the
  // main segment is padded to whole tiles with invalid slots.
  const bool two = p.idx2 != nullptr;
  const int T1 = (p.topk + TK - 1) / TK;
  const int ntiles = two ? T1 + (p.topk2 + TK - 1) / TK : T1;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

  const int hg = wave / NKG, kg = wave % NKG;  // QK role

  bf16x8 qf[KSTEPS];
  {
    const int h = h0 + hg * 16 + l16;
    if (h < p.heads) {
      const int64_t qp = r * p.q_rs + int64_t(h) * p.q_hs + 8 * g;
      load_q_frags(p.q, p.q_fp8, qp, 32, qf);
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  float score_scale = p.sm_log2 * q_scale_of(p.q_scale);
  float out_scale = 1.0f;
  if constexpr (FP8) {
    const float ks = *p.kv_scale;
    score_scale *= ks;
    out_scale = ks;
  }

  // Gather role: slot gk of a tile, 16-byte chunks gp, gp + 8, ...
  const int gk = tid / TPK, gp = tid % TPK;
  const int32_t* idx_row = p.idx + r * p.idx_rs;
  const int32_t* idx2_row = two ? p.idx2 + r * p.idx2_rs : idx_row;
  // Index of slot gk of tile t (-1: invalid, padding or past the split).
  auto load_idx = [&](int t) -> int {
    const bool seg2 = two && t >= T1;
    const int j = (seg2 ? t - T1 : t) * TK + gk;
    const int kseg = seg2 ? p.topk2 : p.topk;
    const int v = (seg2 ? idx2_row : idx_row)[min(j, kseg - 1)];
    return v | -int(!(t < t_end && j < kseg));
  };
  const __amdgpu_buffer_rsrc_t pool_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.pool), 0, p.pool_bytes, kPreBufferWord3);
  const __amdgpu_buffer_rsrc_t pool2_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(two ? p.pool2 : p.pool), 0, two ? p.pool2_bytes : p.pool_bytes,
      kPreBufferWord3);
  // Rows of tile t, whose slot gk holds index `id`.
  auto gather = [&](u32x4 (&pre)[LPT], int id, int t) {
    const bool seg2 = two && t >= T1;
    const __amdgpu_buffer_rsrc_t rsrc = seg2 ? pool2_rsrc : pool_rsrc;
    const PoolMap pm = seg2 ? PoolMap{uint32_t(p.pool2_rs_bytes), 0u, 31u, 0x7fffffffu}
                            : PoolMap{uint32_t(p.pool_rs_bytes), uint32_t(p.page_bytes),
                                      uint32_t(p.page_shift), p.page_mask};
    const uint32_t off = id >= 0 ? slot_offset(pm, id) : kPreOutOfRange;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = min(gp + TPK * i, CH - 1);
      pre[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16u * uint32_t(c), 0, 0));
    }
  };
  auto stage = [&](const u32x4 (&pre)[LPT], int id, int buf) {
    uint16_t* rowp = kt[buf] + gk * PITCH;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = gp + TPK * i;
      if (c < CH) {
        if constexpr (FP8) {
          const u32x2 w0 = widen_fp8x4(pre[i].x), w1 = widen_fp8x4(pre[i].y);
          const u32x2 w2 = widen_fp8x4(pre[i].z), w3 = widen_fp8x4(pre[i].w);
          *reinterpret_cast<u32x4*>(rowp + 16 * c) = u32x4{w0.x, w0.y, w1.x, w1.y};
          *reinterpret_cast<u32x4*>(rowp + 16 * c + 8) = u32x4{w2.x, w2.y, w3.x, w3.y};
        } else {
          *reinterpret_cast<u32x4*>(rowp + 8 * c) = pre[i];
        }
      }
    }
    if (gp == 0) kvalid[buf][gk] = id >= 0 ? 1 : 0;
  };

  floatx4 o[NHG][NB];
#pragma unroll
  for (int a = 0; a < NHG; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) o[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // reference max (log2 domain) of head hg*16 + l16
  float l_part = 0.f;     // this lane's share of that head's row sum

  floatx4 sacc[BPW][2];
  // S^T for this wave's two 16-slot blocks of the tile in buffer buf; leaves
  // the partial row max in red.
  auto qk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < BPW; ++j) sacc[j][0] = sacc[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* kb0 = kt[buf] + (kg * BPW * 16 + l16) * PITCH + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb0 + j * 16 * PITCH + 32 * s);
        sacc[j][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[j][s & 1], 0, 0, 0);
      }
    }
  };
  float sv[BPW][4];
  auto scores_max = [&](int buf) {
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const uint32_t vf =
          *reinterpret_cast<const uint32_t*>(kvalid[buf] + (kg * BPW + j) * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = ((vf >> (8 * i)) & 0xffu) ? (sacc[j][0][i] + sacc[j][1][i]) * score_scale
                                                   : kNegInf;
        sv[j][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) red[kg * HB + hg * 16 + l16] = mx;
  };
  // After the max exchange: reference update, P, row sums.
  auto softmax = [&]() {
    float mt = red[hg * 16 + l16];
#pragma unroll
    for (int k2 = 1; k2 < NKG; ++k2) mt = fmaxf(mt, red[k2 * HB + hg * 16 + l16]);
    const bool upd = mt > m_ref + kPreLazyMax;
    const float m_new = upd ? mt : m_ref;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
    l_part *= alpha;
    m_ref = m_new;
    const float mu = m_ref == kNegInf ? 0.f : m_ref;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(sv[j][i] - mu);
        l_part += e[i];
      }
      // PV k-slot order: in each 32-slot step, k-slots 8g..8g+3 hold slots
      // 4g..4g+3 and k-slots 8g+4..8g+7 hold slots 16+4g..16+4g+3.
      const int kb = kg * BPW + j;
      *reinterpret_cast<u32x2*>(pt + (hg * 16 + l16) * PP + (kb >> 1) * 32 + 8 * g + 4 * (kb & 1)) =
          u32x2{pack2_bf16(e[0], e[1]), pack2_bf16(e[2], e[3])};
    }
    if (kg == 0) {
      if (g == 0) alpha_s[hg * 16 + l16] = alpha;
      const uint64_t any = __ballot(upd);
      if (lane == 0) upd_flag[hg] = any != 0 ? 1u : 0u;
    }
  };
  // O = alpha O + P V for this wave's 64 columns, all 64 heads.
  auto pv = [&](int buf) {
    const u32x4 fl = *reinterpret_cast<const u32x4*>(upd_flag);
    if ((fl.x | fl.y | fl.z | fl.w) != 0) {
#pragma unroll
      for (int a = 0; a < NHG; ++a) {
        const floatx4 a4 = *reinterpret_cast<const floatx4*>(alpha_s + a * 16 + 4 * g);
#pragma unroll
        for (int b = 0; b < NB; ++b) o[a][b] *= a4;
      }
    }
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      bf16x8 pa[NHG];
#pragma unroll
      for (int a = 0; a < NHG; ++a)
        pa[a] = *reinterpret_cast<const bf16x8*>(pt + (a * 16 + l16) * PP + 32 * ks + 8 * g);
      const uint16_t* vrow =
          kt[buf] + (32 * ks + 4 * g + (l16 >> 2)) * PITCH + wave * C::DW + 4 * (l16 & 3);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x2 v0 = lds_read_tr16(vrow + b * 16);
        const u32x2 v1 = lds_read_tr16(vrow + 16 * PITCH + b * 16);
        const bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
        for (int a = 0; a < NHG; ++a)
          o[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[a], vb, o[a][b], 0, 0, 0);
      }
    }
  };

  if (t_begin < t_end) {
    u32x4 pre[LPT];
    int id_a = load_idx(t_begin);
    gather(pre, id_a, t_begin);
    int id_b = load_idx(t_begin + 1);
    stage(pre, id_a, 0);
    gather(pre, id_b, t_begin + 1);
    int id_n = load_idx(t_begin + 2);
    __syncthreads();  // tile t_begin visible
    qk(0);
    scores_max(0);
    __syncthreads();  // A
    softmax();
    if (t_begin + 1 < t_end) {
      stage(pre, id_b, 1);
      id_b = id_n;
      gather(pre, id_b, t_begin + 2);
      id_n = load_idx(t_begin + 3);
    }
    __syncthreads();  // B: P(t_begin), tile t_begin+1 visible
    for (int t = t_begin; t < t_end; ++t) {
      const int buf = (t - t_begin) & 1;
      pv(buf);
      const bool more = t + 1 < t_end;
      if (more) {
        qk(buf ^ 1);
        scores_max(buf ^ 1);
      }
      __syncthreads();  // A
      if (more) {
        softmax();
        if (t + 2 < t_end) {
          stage(pre, id_b, buf);
          id_b = id_n;
          gather(pre, id_b, t + 3);
          id_n = load_idx(t + 4);
        }
      }
      __syncthreads();  // B
    }
  }

  // ---- epilogue: combine the two slot halves' row sums, normalise, store.
  // The four lanes of a head hold parts of its sum (same reference max).
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16);
  l_head += __shfl_xor(l_head, 32);
  if (g == 0) red[kg * HB + hg * 16 + l16] = l_head;
  if (kg == 0 && g == 0) mfin_s[hg * 16 + l16] = m_ref;
  if constexpr (EPI) {
    if (tid < 64) epi_cs[tid] = cs_pre;
  }
  __syncthreads();
  const bool split_mode = p.part_o != nullptr;  // partials for the combine kernel
  const bool epi = EPI && !split_mode;
  uint16_t* const eblk = &kt[0][0];  // every wave is past its last tile read
#pragma unroll
  for (int a = 0; a < NHG; ++a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = a * 16 + 4 * g + i;
      const int h = h0 + head;
      float lt = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < NKG; ++k2) lt += red[k2 * HB + head];
      const float inv = lt > 0.f ? out_scale / lt : 0.f;
      if (h < p.heads) {
        if (epi) {  // bf16 row block in LDS, stored through the epilogue below
          uint16_t* op = eblk + head * kEpiPitch + wave * C::DW + l16;
#pragma unroll
          for (int b = 0; b < NB; ++b) op[b * 16] = uint16_t(bf16_rne(o[a][b][i] * inv));
        } else if (!split_mode) {
          uint16_t* op = p.out + r * p.out_rs + int64_t(h) * p.out_hs + wave * C::DW + l16;
#pragma unroll
          for (int b = 0; b < NB; ++b) op[b * 16] = uint16_t(bf16_rne(o[a][b][i] * inv));
        } else {
          float* op = p.part_o + ((int64_t(split) * p.rows + r) * p.heads + h) * kDv +
                      wave * C::DW + l16;
#pragma unroll
          for (int b = 0; b < NB; ++b) op[b * 16] = o[a][b][i] * inv;
        }
      }
    }
  }
  if (epi) {
    static_assert(HB * kEpiPitch <= TK * PITCH, "epilogue block fits the tile");
    __syncthreads();
    epi_store_lds_block(p.epi, p.epi.pos != nullptr ? epi_cs : nullptr, eblk,
                        eblk + 32 * kEpiPitch, 32, HB, r, h0, p.heads, tid, C::NT);
  }
  if (tid < HB) {
    const int h = h0 + tid;
    if (h < p.heads) {
      float lt = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < NKG; ++k2) lt += red[k2 * HB + tid];
      const float lse = lt > 0.f ? (mfin_s[tid] + __log2f(lt)) * kLn2 : kNegInf;
      if (!split_mode)
        p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = lse;
      else
        p.part_lse[(int64_t(split) * p.rows + r) * p.heads + h] = lse;
    }
  }
}

}  // namespace

KernelShape prefill_shape(int dqk, bool fp8) {
  KernelShape k;
  k.waves = kPreWaves;
  k.tile = kPreTile;
  if (dqk == 576)
    k.lds_bytes = fp8 ? PreCfg<576, true>::LDS_BYTES : PreCfg<576, false>::LDS_BYTES;
  else if (dqk == 512)
    k.lds_bytes = fp8 ? PreCfg<512, true>::LDS_BYTES : PreCfg<512, false>::LDS_BYTES;
  else
    k = KernelShape{};
  return k;
}

template <bool EPI>
static int launch_prefill_inst(const FwdParams& p, int dqk, bool fp8, hipStream_t st) {
  const dim3 grid(uint32_t(p.grid)), block(kPreWaves * 64);
  if (dqk == 576) {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<576, true, EPI>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_kernel<576, false, EPI>), grid, block, 0, st, p);
  } else if (dqk == 512) {
    if (fp8) hipLaunchKernelGGL((prefill_kernel<512, true, EPI>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((prefill_kernel<512, false, EPI>), grid, block, 0, st, p);
  } else {
    return int(hipErrorInvalidValue);
  }
  return int(hipGetLastError());
}

int launch_prefill(const FwdParams& p, int dqk, bool fp8, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (epi_active(p.epi) && p.part_o == nullptr) return launch_prefill_inst<true>(p, dqk, fp8, st);
  return launch_prefill_inst<false>(p, dqk, fp8, st);
}

}  // namespace smla
