// gfx950 kernels of the sparse MLA forward: the attention kernel and the
// split combine kernel.
//
// What is computed, per query row r and head h over the row's valid slots j
// (a negative index is an invalid slot):
//   s_j = sm_scale * q[r,h] . K[idx_j]      (all D_qk = 576 or 512 columns)
//   out = sum_j softmax(s)_j V[idx_j]       (V = first 512 columns)
//   lse = ln sum_j exp(s_j)
// after "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159):
// Technical Details (576 = 512 latent + 64 rope, or 512 rope-free; bf16 or
// per-tensor fp8 rows) and its commit notes on the staged walk, the softmax
// row exchange through LDS, the LDS pad, the 16x16x32 bf16 dots and the
// split-K reduce.
//
// Attention kernel, one workgroup per (row, block of HB heads, split):
//  * The split's slots are walked in tiles of 64. Each thread owns one slot
//    of the tile (threads-per-slot = block size / 64) and loads its 16-byte
//    chunks of that pool row straight into registers one tile ahead, so the
//    next tile's gathers are in flight while this tile computes.
//  * The tile is widened to bf16 on the way into LDS (fp8 e4m3fn codes are
//    exact in bf16; the per-tensor scale is folded into the score scale and
//    the output) and stored row-major with a 16-byte pad per row, which keeps
//    128-bit accesses aligned and puts the 16 rows an MFMA operand reads on
//    distinct banks.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: K (16 slots x 32 columns) is
//    the A operand read from LDS, Q^T the B operand, held in VGPRs for the
//    whole walk (one 16-head group per wave). The transposed product leaves
//    each lane with four consecutive slots of one head, which is exactly the
//    row layout P needs.
//  * Online softmax in the exp2 domain. Waves that share a head group but own
//    different slots exchange their tile row max through a small LDS buffer
//    (one barrier), so every wave uses the same running max and the row sums
//    can stay per wave until the end.
//  * P (bf16) goes to LDS; each wave then owns 512/waves output columns for
//    all HB heads and runs O += P V on 16x16x32 MFMAs, V being the first 512
//    columns of the same staged tile (no second gather).
//  * Epilogue: O / l (times the fp8 scale) rounded to bf16 and LSE = ln 2 *
//    (m + log2 l); a head with no valid slot gets O = 0 and LSE = -inf. Given
//    a workspace (splits > 1, or a segment of a two-segment call), the
//    normalised fp32 O and the LSE go there and the combine kernel merges
//    them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

template <int NHG, int NW, int TK_, int DQK, bool FP8>
struct Cfg {
  static constexpr int HB = 16 * NHG;          // heads per workgroup
  static constexpr int NT = NW * 64;           // threads per workgroup
  static constexpr int TK = TK_;               // slots per tile
  static constexpr int KSTEPS = DQK / 32;      // k-steps of the QK dot
  static constexpr int PITCH = DQK + 8;        // LDS tile row pitch (elements)
  static constexpr int PP = TK + 8;            // LDS P row pitch (elements)
  static constexpr int NKG = NW / NHG;         // waves sharing one head group
  static constexpr int BPW = (TK / 16) / NKG;  // 16-slot blocks per wave in QK
  static constexpr int DW = kDv / NW;          // output columns per wave in PV
  static constexpr int NB = DW / 16;           // 16-column blocks per wave
  static constexpr int EB = FP8 ? 1 : 2;       // pool bytes per element
  static constexpr int CH = DQK * EB / 16;     // 16-byte chunks per pool row
  static constexpr int TPK = NT / TK;          // gather threads per slot
  static constexpr int LPT = (CH + TPK - 1) / TPK;  // chunks per gather thread
  static constexpr int LDS_BYTES =
      TK * PITCH * 2 + HB * PP * 2 + NKG * HB * 4 + 2 * HB * 4 + TK;
  static_assert(NKG * NHG == NW && BPW >= 1 && BPW * NKG * 16 == TK, "wave split");
  static_assert(NT % TK == 0 && DW % 16 == 0 && DQK % 32 == 0 && TK % 32 == 0, "shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// One workgroup: (row, block of HB = 16*NHG heads, split). NW waves, TK-slot
// tiles, one tile of gathers in flight.
template <int NHG, int NW, int TK_, int DQK, bool FP8, bool EPI>
__global__ void __launch_bounds__(NW * 64, 2) fwd_kernel(const FwdParams p) {
  using C = Cfg<NHG, NW, TK_, DQK, FP8>;
  constexpr int HB = C::HB, TK = C::TK, PITCH = C::PITCH, PP = C::PP;
  constexpr int NKG = C::NKG, BPW = C::BPW, NB = C::NB, TPK = C::TPK, LPT = C::LPT;
  constexpr int CH = C::CH, KSTEPS = C::KSTEPS;

  __shared__ __attribute__((aligned(16))) uint16_t kt[TK * PITCH];  // bf16 tile
  __shared__ __attribute__((aligned(16))) uint16_t pt[HB * PP];     // bf16 P
  __shared__ __attribute__((aligned(16))) float red[NKG * HB];      // row max / sum exchange
  __shared__ __attribute__((aligned(16))) float alpha_s[HB];        // rescale factors
  __shared__ __attribute__((aligned(16))) float mfin_s[HB];         // final row max
  __shared__ __attribute__((aligned(4))) uint8_t kvalid[TK];        // slot validity

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

  const int ntiles = (p.topk + TK - 1) / TK;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

  // QK role: head group hg, slot group kg.
  const int hg = wave / NKG, kg = wave % NKG;

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

  // Gather role: slot gk of the tile, chunks gp, gp + TPK, ...
  const int gk = tid / TPK, gp = tid % TPK;
  const int32_t* idx_row = p.idx + r * p.idx_rs;
  auto load_idx = [&](int t) -> int {
    const int j = t * TK + gk;
    return (t < t_end && j < p.topk) ? idx_row[j] : -1;
  };

  auto gather = [&](u32x4 (&pre)[LPT], int id) {
    if (id >= 0) {
      const uint8_t* rp = p.pool + int64_t(uint32_t(id) >> p.page_shift) * p.page_bytes +
                          int64_t(uint32_t(id) & p.page_mask) * p.pool_rs_bytes;
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int c = gp + TPK * i;
        if (c < CH) pre[i] = *reinterpret_cast<const u32x4*>(rp + 16 * c);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) pre[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto stage = [&](const u32x4 (&pre)[LPT], int id) {
    uint16_t* rowp = kt + gk * PITCH;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = gp + TPK * i;
      if (c < CH) {
        if constexpr (FP8) {
          const u32x2 w0 = widen_fp8x4(pre[i].x), w1 = widen_fp8x4(pre[i].y);
          const u32x2 w2 = widen_fp8x4(pre[i].z), w3 = widen_fp8x4(pre[i].w);
          const u32x4 a = {w0.x, w0.y, w1.x, w1.y};
          const u32x4 b = {w2.x, w2.y, w3.x, w3.y};
          *reinterpret_cast<u32x4*>(rowp + 16 * c) = a;
          *reinterpret_cast<u32x4*>(rowp + 16 * c + 8) = b;
        } else {
          *reinterpret_cast<u32x4*>(rowp + 8 * c) = pre[i];
        }
      }
    }
    if (gp == 0) kvalid[gk] = id >= 0 ? 1 : 0;
  };

  floatx4 o[NHG][NB];
#pragma unroll
  for (int a = 0; a < NHG; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) o[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // Everything after the tile is staged and visible: QK, softmax, PV.
  auto compute = [&]() {
    // ---- S^T = K Q^T for this wave's 16-slot blocks and 16-head group; two
    // accumulators per block halve the dependent MFMA chain.
    floatx4 sacc[BPW][2];
#pragma unroll
    for (int j = 0; j < BPW; ++j)
      sacc[j][0] = sacc[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int key = (kg * BPW + j) * 16 + l16;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + key * PITCH + 32 * s + 8 * g);
        sacc[j][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[j][s & 1], 0, 0, 0);
      }
    }

    // ---- scale, mask, tile row max (lane: head l16, slots blk*16 + 4g + i)
    float sv[BPW][4];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const uint32_t vf = *reinterpret_cast<const uint32_t*>(kvalid + (kg * BPW + j) * 16 + 4 * g);
      const floatx4 sj = sacc[j][0] + sacc[j][1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = ((vf >> (8 * i)) & 0xffu) ? sj[i] * score_scale : kNegInf;
        sv[j][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) red[kg * HB + hg * 16 + l16] = mx;
    __syncthreads();
    float mt = red[hg * 16 + l16];
#pragma unroll
    for (int k2 = 1; k2 < NKG; ++k2) mt = fmaxf(mt, red[k2 * HB + hg * 16 + l16]);
    const float m_new = fmaxf(m_run, mt);
    const float m_ref = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(sv[j][i] - m_ref);
        psum += e[i];
      }
      // P is stored in the PV MFMA's k-slot order: within each 32-slot step,
      // k-slots 8g..8g+3 hold slots 4g..4g+3 and k-slots 8g+4..8g+7 hold slots
      // 16+4g..16+4g+3, which is the order S^T leaves in the lanes.
      const int kb = kg * BPW + j;
      *reinterpret_cast<u32x2*>(pt + (hg * 16 + l16) * PP + (kb >> 1) * 32 + 8 * g + 4 * (kb & 1)) =
          u32x2{pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3])};
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = alpha * l_run + psum;
    m_run = m_new;
    if (kg == 0 && g == 0) alpha_s[hg * 16 + l16] = alpha;
    __syncthreads();  // P and alpha visible

    // ---- O = alpha O + P V for this wave's output columns, all HB heads
#pragma unroll
    for (int a = 0; a < NHG; ++a) {
      const floatx4 a4 = *reinterpret_cast<const floatx4*>(alpha_s + a * 16 + 4 * g);
#pragma unroll
      for (int b = 0; b < NB; ++b) o[a][b] *= a4;
    }
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      bf16x8 pa[NHG];
#pragma unroll
      for (int a = 0; a < NHG; ++a)
        pa[a] = *reinterpret_cast<const bf16x8*>(pt + (a * 16 + l16) * PP + 32 * ks + 8 * g);
      // V operand: k-slots 8g..8g+3 = slots 32ks+4g+(0..3), k-slots 8g+4..8g+7
      // = slots 32ks+16+4g+(0..3), two transposed reads of 4 rows each. The 16
      // rows one read touches are consecutive, so with the tile pitch an odd
      // multiple of 16 bytes modulo 256 they fall on distinct banks.
      const uint16_t* vrow = kt + (32 * ks + 4 * g + (l16 >> 2)) * PITCH + wave * C::DW + 4 * (l16 & 3);
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

  u32x4 pre0[LPT];
  int id0 = load_idx(t_begin);
  gather(pre0, id0);
  int id_next = load_idx(t_begin + 1);
  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();  // every wave is done with the previous tile, P and alpha
    stage(pre0, id0);
    id0 = id_next;
    if (t + 1 < t_end) gather(pre0, id0);
    id_next = load_idx(t + 2);
    __syncthreads();  // tile visible
    compute();
  }

  // ---- epilogue: combine the per-wave row sums, normalise, store
  if (g == 0) red[kg * HB + hg * 16 + l16] = l_run;
  if (kg == 0 && g == 0) mfin_s[hg * 16 + l16] = m_run;
  if constexpr (EPI) {
    if (tid < 64) epi_cs[tid] = cs_pre;
  }
  __syncthreads();

  const bool split_mode = p.part_o != nullptr;  // partials for the combine kernel
  const bool epi = EPI && !split_mode;
  uint16_t* const eblk = kt;  // every wave is past its last tile read
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

// Split combine: one 128-thread workgroup per (row, head), 4 columns per
// thread. lse = M + ln sum_s e^(lse_s - M), out = sum_s e^(lse_s - lse) O_s,
// splits with lse_s = -inf weigh 0, all -inf gives out = 0 and lse = -inf.
// EPI: the final store goes through the output epilogue (epilogue.h); each
// thread holds 4 columns and 8 consecutive threads one 32-column block.
template <bool EPI>
__global__ void __launch_bounds__(128) combine_kernel(const FwdParams p) {
  const int64_t rh = blockIdx.x;
  const int64_t r = rh / p.heads;
  const int h = int(rh % p.heads);
  const int tid = threadIdx.x;
  const int64_t stride_s = p.rows * p.heads;
  const float* pl = p.part_lse + r * p.heads + h;
  float m = kNegInf;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, pl[s * stride_s]);
  uint16_t* op = p.out + r * p.out_rs + int64_t(h) * p.out_hs + 4 * tid;
  const float* cs_row = EPI ? epi_cs_row(p.epi, r) : nullptr;
  if (m == kNegInf) {
    if constexpr (EPI) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      epi_store<4>(p.epi, cs_row, r, h, 4 * tid, v);
    } else {
      *reinterpret_cast<u32x2*>(op) = u32x2{0u, 0u};
    }
    if (tid == 0) p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = kNegInf;
    return;
  }
  float tot = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = p.part_o + (r * p.heads + h) * kDv + 4 * tid;
  for (int s = 0; s < p.splits; ++s) {
    const float ls = pl[s * stride_s];
    if (ls == kNegInf) continue;
    const float w = __expf(ls - m);
    tot += w;
    acc += w * *reinterpret_cast<const floatx4*>(po + s * stride_s * kDv);
  }
  const float inv = 1.0f / tot;
  if constexpr (EPI) {
    float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    epi_store<4>(p.epi, cs_row, r, h, 4 * tid, v);
  } else {
    *reinterpret_cast<u32x2*>(op) =
        u32x2{pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv)};
  }
  if (tid == 0) p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = m + __logf(tot);
}

// Kernel instances per (head block, pool dtype, variant): waves and tile size. For 16 heads over an fp8
// pool, variant 0 is the decode kernel (decode.hip) and variant 1 the
// 4-wave, 64-slot instance below. For 64 heads, variant 0 is the 4-wave
// kernel of prefill_fp8.hip over fp8 pools and the 8-wave kernel of
// prefill.hip over bf16 pools, variant 1 the 8-wave staged-tile instance
// below, variant 2 the 8-wave kernel of prefill.hip and variant 3 (fp8 pools)
// the fp8-dot kernel of prefill_mx.hip. Elsewhere every variant is variant 0.
template <int NHG, int NW, int TK>
struct Inst {
  static constexpr int kNHG = NHG, kNW = NW, kTK = TK;
};
template <int HB, bool FP8, int V> struct InstFor;
template <int V> struct InstFor<16, true, V> : Inst<1, 4, 64> {};
template <int V> struct InstFor<16, false, V> : Inst<1, 4, 64> {};
template <bool FP8, int V> struct InstFor<32, FP8, V> : Inst<2, 8, 64> {};
template <bool FP8, int V> struct InstFor<64, FP8, V> : Inst<4, 8, 64> {};

template <int HB, int V, int DQK, bool FP8>
hipError_t launch_inst(const FwdParams& p, hipStream_t st) {
  using I = InstFor<HB, FP8, V>;
  const dim3 grid(uint32_t(p.grid)), block(I::kNW * 64);
  if (epi_active(p.epi) && p.part_o == nullptr)
    hipLaunchKernelGGL((fwd_kernel<I::kNHG, I::kNW, I::kTK, DQK, FP8, true>), grid,
                       block, 0, st, p);
  else
    hipLaunchKernelGGL((fwd_kernel<I::kNHG, I::kNW, I::kTK, DQK, FP8, false>), grid,
                       block, 0, st, p);
  return hipGetLastError();
}

template <int HB, bool FP8, int V>
KernelShape shape_of(int dqk) {
  using I = InstFor<HB, FP8, V>;
  KernelShape k;
  k.waves = I::kNW;
  k.tile = I::kTK;
  k.lds_bytes = dqk == 576 ? Cfg<I::kNHG, I::kNW, I::kTK, 576, FP8>::LDS_BYTES
                           : Cfg<I::kNHG, I::kNW, I::kTK, 512, FP8>::LDS_BYTES;
  return k;
}

template <int DQK, bool FP8>
hipError_t launch_by_head_block(int head_block, int variant, const FwdParams& p, hipStream_t st) {
  switch (head_block) {
    case 16:
      if (FP8 && variant == 0) return static_cast<hipError_t>(launch_decode(p, DQK, st));
      return launch_inst<16, 0, DQK, FP8>(p, st);
    case 32: return launch_inst<32, 0, DQK, FP8>(p, st);
    case 64:
      if (variant == 1) return launch_inst<64, 0, DQK, FP8>(p, st);
      if (FP8 && variant == 0) return static_cast<hipError_t>(launch_prefill_fp8(p, DQK, st));
      if (FP8 && variant == 3) return static_cast<hipError_t>(launch_prefill_mx(p, DQK, st));
      return static_cast<hipError_t>(launch_prefill(p, DQK, FP8, st));
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

KernelShape kernel_shape(int head_block, int dqk, bool fp8, int variant) {
  if (dqk != 576 && dqk != 512) return KernelShape{};
  switch (head_block) {
    case 16:
      if (fp8 && variant == 0) return decode_shape(dqk);
      return fp8 ? shape_of<16, true, 0>(dqk) : shape_of<16, false, 0>(dqk);
    case 32: return fp8 ? shape_of<32, true, 0>(dqk) : shape_of<32, false, 0>(dqk);
    case 64:
      if (variant == 1) return fp8 ? shape_of<64, true, 0>(dqk) : shape_of<64, false, 0>(dqk);
      if (fp8 && variant == 0) return prefill_fp8_shape(dqk);
      if (fp8 && variant == 3) return prefill_mx_shape(dqk);
      return prefill_shape(dqk, fp8);
    default: return KernelShape{};
  }
}

int launch_attention(const FwdParams& p, const smla_plan& plan, int dqk, bool fp8, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dqk == 576)
    e = fp8 ? launch_by_head_block<576, true>(plan.head_block, plan.variant, p, st)
            : launch_by_head_block<576, false>(plan.head_block, plan.variant, p, st);
  else
    e = fp8 ? launch_by_head_block<512, true>(plan.head_block, plan.variant, p, st)
            : launch_by_head_block<512, false>(plan.head_block, plan.variant, p, st);
  return int(e);
}

int launch_combine(const FwdParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(uint32_t(p.rows * p.heads)), block(128);
  if (epi_active(p.epi))
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, st, p);
  return int(hipGetLastError());
}

int launch_forward(const FwdParams& p, const smla_plan& plan, int dqk, bool fp8, void* stream) {
  const int e = launch_attention(p, plan, dqk, fp8, stream);
  if (e != 0 || plan.splits <= 1) return e;
  return launch_combine(p, stream);
}

}  // namespace smla
