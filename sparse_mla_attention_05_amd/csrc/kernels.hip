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
//    (m + log2 l); a head with no valid slot gets O = 0 and LSE = -inf. With
//    splits > 1 the normalised fp32 O and the LSE go to a workspace and the
//    combine kernel merges them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Four e4m3fn codes (one dword, code 0 in the low byte) to four bf16 values
// (two dwords, value 0 in the low half). Exact: every finite e4m3fn value is
// a bf16 value, and the scale operand is 1.
__device__ __forceinline__ u32x2 widen_fp8x4(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

template <int NHG, int NW, int DQK, bool FP8>
struct Cfg {
  static constexpr int HB = 16 * NHG;          // heads per workgroup
  static constexpr int NT = NW * 64;           // threads per workgroup
  static constexpr int TK = kTileKeys;         // slots per tile
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
  static_assert(NKG * NHG == NW && NKG >= 1 && NKG <= 4, "wave split");
  static_assert(DW % 16 == 0 && DQK % 32 == 0, "shape");
};

template <int NHG, int NW, int DQK, bool FP8>
__global__ void __launch_bounds__(NW * 64, 2) fwd_kernel(const FwdParams p) {
  using C = Cfg<NHG, NW, DQK, FP8>;
  constexpr int HB = C::HB, TK = C::TK, PITCH = C::PITCH, PP = C::PP;
  constexpr int NKG = C::NKG, BPW = C::BPW, NB = C::NB, TPK = C::TPK, LPT = C::LPT;
  constexpr int CH = C::CH;

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
  const int h0 = hb * HB;

  const int ntiles = (p.topk + TK - 1) / TK;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

  // QK role: head group hg, slot group kg.
  const int hg = wave / NKG, kg = wave % NKG;

  bf16x8 qf[C::KSTEPS];
  {
    const int h = h0 + hg * 16 + l16;
    if (h < p.heads) {
      const uint16_t* qp = p.q + r * p.q_rs + int64_t(h) * p.q_hs + 8 * g;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * s));
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }

  float score_scale = p.sm_log2;
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

  u32x4 pre[LPT];
  auto gather = [&](int id) {
    if (id >= 0) {
      const uint8_t* rp = p.pool + int64_t(id) * p.pool_rs_bytes;
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
  auto stage = [&](int id) {
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

  int id_cur = load_idx(t_begin);
  int id_next = load_idx(t_begin + 1);
  gather(id_cur);

  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();  // every wave is done with the previous tile, P and alpha
    stage(id_cur);
    id_cur = id_next;
    if (t + 1 < t_end) gather(id_cur);
    id_next = load_idx(t + 2);
    __syncthreads();  // tile visible

    // ---- S^T = K Q^T for this wave's 16-slot blocks and 16-head group
    floatx4 sacc[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int key = (kg * BPW + j) * 16 + l16;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + key * PITCH + 32 * s + 8 * g);
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[j], 0, 0, 0);
      }
    }

    // ---- scale, mask, tile row max (lane: head l16, slots blk*16 + 4g + i)
    float sv[BPW][4];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const uint32_t vf = *reinterpret_cast<const uint32_t*>(kvalid + (kg * BPW + j) * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = ((vf >> (8 * i)) & 0xffu) ? sacc[j][i] * score_scale : kNegInf;
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
      *reinterpret_cast<u32x2*>(pt + (hg * 16 + l16) * PP + (kg * BPW + j) * 16 + 4 * g) =
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
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint16_t* vp = kt + (32 * ks + 8 * g) * PITCH + wave * C::DW + b * 16 + l16;
        u32x4 vv;
        vv.x = uint32_t(vp[0]) | (uint32_t(vp[PITCH]) << 16);
        vv.y = uint32_t(vp[2 * PITCH]) | (uint32_t(vp[3 * PITCH]) << 16);
        vv.z = uint32_t(vp[4 * PITCH]) | (uint32_t(vp[5 * PITCH]) << 16);
        vv.w = uint32_t(vp[6 * PITCH]) | (uint32_t(vp[7 * PITCH]) << 16);
        const bf16x8 vb = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int a = 0; a < NHG; ++a)
          o[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[a], vb, o[a][b], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: combine the per-wave row sums, normalise, store
  if (g == 0) red[kg * HB + hg * 16 + l16] = l_run;
  if (kg == 0 && g == 0) mfin_s[hg * 16 + l16] = m_run;
  __syncthreads();

  const bool split_mode = p.splits > 1;
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
        if (!split_mode) {
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
  if (m == kNegInf) {
    *reinterpret_cast<u32x2*>(op) = u32x2{0u, 0u};
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
  *reinterpret_cast<u32x2*>(op) =
      u32x2{pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv)};
  if (tid == 0) p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = m + __logf(tot);
}

template <int NHG, int NW, int DQK, bool FP8>
hipError_t launch_fwd(const FwdParams& p, hipStream_t st) {
  hipLaunchKernelGGL((fwd_kernel<NHG, NW, DQK, FP8>), dim3(uint32_t(p.grid)), dim3(NW * 64), 0,
                     st, p);
  return hipGetLastError();
}

template <int DQK, bool FP8>
hipError_t launch_by_head_block(int head_block, const FwdParams& p, hipStream_t st) {
  switch (head_block) {
    case 16: return launch_fwd<1, 4, DQK, FP8>(p, st);
    case 32: return launch_fwd<2, 8, DQK, FP8>(p, st);
    case 64: return launch_fwd<4, 8, DQK, FP8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int kernel_waves(int head_block) { return head_block == 16 ? 4 : 8; }

int kernel_lds_bytes(int head_block, int dqk) {
  // Cfg<...>::LDS_BYTES does not depend on the pool dtype.
  if (dqk == 576) {
    switch (head_block) {
      case 16: return Cfg<1, 4, 576, false>::LDS_BYTES;
      case 32: return Cfg<2, 8, 576, false>::LDS_BYTES;
      case 64: return Cfg<4, 8, 576, false>::LDS_BYTES;
    }
  } else if (dqk == 512) {
    switch (head_block) {
      case 16: return Cfg<1, 4, 512, false>::LDS_BYTES;
      case 32: return Cfg<2, 8, 512, false>::LDS_BYTES;
      case 64: return Cfg<4, 8, 512, false>::LDS_BYTES;
    }
  }
  return -1;
}

int launch_forward(const FwdParams& p, const smla_plan& plan, int dqk, bool fp8, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dqk == 576)
    e = fp8 ? launch_by_head_block<576, true>(plan.head_block, p, st)
            : launch_by_head_block<576, false>(plan.head_block, p, st);
  else
    e = fp8 ? launch_by_head_block<512, true>(plan.head_block, p, st)
            : launch_by_head_block<512, false>(plan.head_block, p, st);
  if (e != hipSuccess) return int(e);
  if (plan.splits > 1) {
    hipLaunchKernelGGL(combine_kernel, dim3(uint32_t(p.rows * p.heads)), dim3(128), 0, st, p);
    e = hipGetLastError();
  }
  return int(e);
}

}  // namespace smla
