// gfx950 decode kernel of the sparse MLA forward: up to 16 heads per
// workgroup, fp8 e4m3fn pool, 576- or 512-wide rows.
//
// The method (per row r, head h, over the row's valid slots j):
//   s_j = sm_scale * q[r,h] . K[idx_j] (D_qk columns), out = softmax(s) V
//   (V = first 512 columns), lse = ln sum_j exp(s_j)
// after "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159),
// Technical Details and the commit notes on the per-tensor fp8 route and the
// split-K reduce. With 16 heads the work per gathered byte is small, so the
// kernel is built to keep gathers in flight and spend few cycles per slot:
//
//  * One workgroup = (row, 16-head block, split), 4 wavefronts; two
//    workgroups per CU (256 VGPRs and 61 KB of LDS each), so one
//    workgroup's start (index staging, first gathers) and end (merge, store)
//    overlap the other's walk. Each wave walks its own quarter of the split's
//    slots in 16-slot steps (steps w, w+4, ...) with its own running max, row
//    sum and O, like an independent split; the four are merged once at the
//    end, through LDS, a quarter of the columns at a time. No barrier inside
//    the walk.
//  * Q^T is kept in LDS and each k-step's fragment is read one k-step ahead
//    of its dot, which is what leaves the registers to two workgroups.
//  * Gathers go straight into VGPRs, two steps in flight per wave. Lane
//    (l16, g) loads 16-byte chunks 4i+g (i = 0..8) of the step's slot l16, so
//    every load instruction reads 64 contiguous bytes of 16 rows. Those
//    chunks are exactly the A operand of S^T = K Q^T on
//    v_mfma_f32_16x16x32_bf16 once widened to bf16 in registers, provided
//    Q^T uses the same column order (k-step 2i+h takes columns
//    64i + 16g + 8h .. +8), which it does: K never goes through LDS.
//  * S^T leaves each lane with slots 4g..4g+3 of head l16, which is the A
//    operand of P on v_mfma_f32_16x16x16_bf16 (k-slots 4g..4g+3): P stays in
//    registers.
//  * V (the first 512 columns, still fp8) is written to a wave-private LDS
//    area and read back with the transposed byte read: pointing rows 0..3 of
//    the 8 x 16 byte block at slots 4g..4g+3 of one 16-column block and rows
//    4..7 at the same slots of the next one hands each lane the B operands of
//    two column blocks in one read. The 32-byte row pitch offset puts the
//    rows one half-wave reads on distinct banks.
//  * Online softmax in the exp2 domain with a lazy reference: the reference
//    max moves only when a tile max exceeds it by more than 8 (so P <= 2^8),
//    which skips most O rescales and is exact in real arithmetic (the final
//    normalisation uses the same reference).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecStep = 16;        // slots per wave step
constexpr int kDecBufs = 2;         // steps of gathers in flight per wave
constexpr int kVPitch = 544;        // V staging row pitch (bytes): 512 + 32
constexpr int kVWave = 16 * kVPitch;  // V staging bytes per wave
constexpr int kIdxChunk = 2048;     // slot indices staged in LDS at a time
constexpr int kIdxOffset = kDecWaves * kVWave;  // their LDS offset (bytes)
constexpr int kQOffset = kIdxOffset + 4 * kIdxChunk;  // Q^T fragments (bytes)
constexpr int kDecSmem = kQOffset + (576 / 32) * 64 * 16;
// The four waves' O are merged through LDS a quarter of the columns at a
// time, in the V staging area: [wave][head][128 columns], row pitch 132
// floats (4 * 132 = 16 mod 64 banks, so a wave's 64 lanes hit 64 banks).
constexpr int kMCols = kDv / 4;
constexpr int kMPitch = kMCols + 4;
constexpr int kMWave = 16 * kMPitch * 4;
static_assert(kDecWaves * kMWave <= kIdxOffset, "merge area");
constexpr float kLazyMax = 8.0f;    // log2-domain slack before the reference max moves
constexpr uint32_t kOutOfRange = 0xFFFFF000u;  // buffer offset of an invalid slot's row
constexpr int kBufferWord3 = 0x00020000;       // raw buffer descriptor word 3 (gfx9 family)

// EPI: the final store goes through the output epilogue (epilogue.h).
template <int DQK, bool EPI>
__global__ void __launch_bounds__(kDecWaves * 64, 2) decode_kernel(const FwdParams p) {
  constexpr int NCH = DQK / 16;  // 16-byte fp8 chunks per row
  constexpr int NI = NCH / 4;    // chunks per lane per step
  constexpr int KS = DQK / 32;   // k-steps of the QK dot
  constexpr int VI = kDv / 64;   // chunk rounds holding V columns (8)
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  static_assert(NCH % 4 == 0 && 2 * NI == KS, "row width");

  __shared__ __attribute__((aligned(16))) uint8_t smem[kDecSmem];
  __shared__ float red_m[kDecWaves * 16];
  __shared__ float red_l[kDecWaves * 16];

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

  const int h0 = hb * 16;

  // Q^T fragments in the gather's column order, kept in LDS (fragment s of
  // lane l at kQOffset + (64 s + l) 16 bytes) and read back a k-step ahead of
  // their dots, which leaves the registers to two workgroups per CU.
  bf16x8 qf[KS];
  if (wave == 0) {
    const int h = h0 + l16;
    if (h < p.heads) {
      const int64_t qp = r * p.q_rs + int64_t(h) * p.q_hs + 16 * g;
      // Fragment s holds columns 64 (s / 2) + 8 (s % 2) + 16g .. +8.
      bf16x8 qe[KS / 2], qo[KS / 2];
      load_q_frags(p.q, p.q_fp8, qp, 64, qe);
      load_q_frags(p.q, p.q_fp8, qp + 8, 64, qo);
#pragma unroll
      for (int s = 0; s < KS / 2; ++s) {
        qf[2 * s] = qe[s];
        qf[2 * s + 1] = qo[s];
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
      reinterpret_cast<u32x4*>(smem + kQOffset)[64 * s + lane] = __builtin_bit_cast(u32x4, qf[s]);
  }
  const u32x4* q_lds = reinterpret_cast<const u32x4*>(smem + kQOffset) + lane;
  const float kv_scale = *p.kv_scale;
  const float qs = q_scale_of(p.q_scale);
  float c = p.sm_log2 * qs * kv_scale;  // raw dot -> log2-domain score (per segment)
  float vs = kv_scale;             // scale of the V codes O is accumulated in

  // This split's slots of the virtual list [main top-k | second segment],
  // walked segment by segment in chunks whose indices are staged in LDS.
  const int ktot = p.topk + (p.idx2 ? p.topk2 : 0);
  const int kbeg = split * p.tiles_per_split * kDecStep;
  const int kend = min(ktot, kbeg + p.tiles_per_split * kDecStep);
  int32_t* idx_s = reinterpret_cast<int32_t*>(smem + kIdxOffset);

  // Every global load in the walk is unconditional and its result is only
  // read where it is consumed: loads in divergent branches, or loaded values
  // copied between iterations, make the compiler wait for all outstanding
  // loads. An invalid slot's row is read at an offset past the end of the
  // pool's buffer range, which returns zeros without touching memory.
  auto gather = [&](const __amdgpu_buffer_rsrc_t& rsrc, const PoolMap& pm, u32x4 (&kr)[NI], int id) {
    const uint32_t off = id >= 0 ? slot_offset(pm, id) + 16u * g : kOutOfRange;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 64u * i, 0, 0));
  };

  uint8_t* vst = smem + wave * kVWave;
  // Transposed-read address of this lane: byte row t = l16/2 of the read is
  // slot 4g + (t & 3) in column block nb + (t >> 2); column half l16 & 1.
  const int t8 = l16 >> 1;
  const uint8_t* vrd = vst + (4 * g + (t8 & 3)) * kVPitch + 16 * (t8 >> 2) + 8 * (l16 & 1);

  floatx4 o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;  // log2-domain reference max of head l16
  float l_part = 0.f;     // this lane's share of the row sum of head l16

  auto step = [&](const u32x4 (&kr)[NI], int id) {
    // V columns into the wave's staging area (fp8 as is).
#pragma unroll
    for (int i = 0; i < VI; ++i)
      *reinterpret_cast<u32x4*>(vst + l16 * kVPitch + 16 * (4 * i + g)) = kr[i];

    // S^T = K Q^T, two accumulators.
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 qa = __builtin_bit_cast(bf16x8, q_lds[0]), qb = __builtin_bit_cast(bf16x8, q_lds[64]);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      bf16x8 na = qa, nb = qb;
      if (i + 1 < NI) {
        na = __builtin_bit_cast(bf16x8, q_lds[64 * (2 * i + 2)]);
        nb = __builtin_bit_cast(bf16x8, q_lds[64 * (2 * i + 3)]);
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen_fp8x8(kr[i].x, kr[i].y), qa, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen_fp8x8(kr[i].z, kr[i].w), qb, s1, 0, 0, 0);
      qa = na;
      qb = nb;
      // Keep each k-step's widening next to its MFMAs: hoisting all of them
      // would hold 18 widened operands (72 VGPRs) at once.
      __builtin_amdgcn_sched_barrier(0);
    }

    // Scores of head l16 for slots 4g + i; invalid slots -> -inf.
    const uint32_t bits = uint32_t(__ballot(id >= 0) >> (4 * g));
    float sv[4];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((bits >> i) & 1u) ? (s0[i] + s1[i]) * c : kNegInf;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    const bool upd = mx > m_ref + kLazyMax;
    if (__ballot(upd) != 0) {
      const float m_new = upd ? mx : m_ref;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      l_part *= alpha;
      floatx4 a4;
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) o[nb] *= a4;
      m_ref = m_new;
    }
    const float mu = m_ref == kNegInf ? 0.f : m_ref;
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
      l_part += e[i];
    }
    const s16x4 pa = __builtin_bit_cast(s16x4, u32x2{pack2_bf16(e[0], e[1]), pack2_bf16(e[2], e[3])});

    // O += P V, two column blocks per transposed read.
#pragma unroll
    for (int nb = 0; nb < 32; nb += 2) {
      const u32x2 v = lds_read_tr8(vrd + 16 * nb);
      const u32x2 w0 = widen_fp8x4(v.x), w1 = widen_fp8x4(v.y);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, w0), o[nb], 0, 0, 0);
      o[nb + 1] =
          __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, w1), o[nb + 1], 0, 0, 0);
      if ((nb & 6) == 6) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Slots [lo, hi) of the virtual list, all in the segment that starts at
  // virtual slot sb, whose rows come from `rsrc` (slot offsets from pm) and
  // whose indices are idx_seg[0..).
  auto walk_range = [&](const __amdgpu_buffer_rsrc_t& rsrc, const PoolMap& pm,
                        const int32_t* idx_seg, int lo, int hi, int sb) {
    for (int c0 = lo; c0 < hi; c0 += kIdxChunk) {
      const int c1 = min(hi, c0 + kIdxChunk);
      __syncthreads();  // every wave is done with the previous chunk's indices
      {
        // All of a thread's index loads are issued before the first is
        // waited on (a plain strided copy loop waits on each load in turn:
        // that many memory round trips before the walk's first gather).
        // Loads past the chunk's end read 0 through the buffer range.
        constexpr int PER = kIdxChunk / (kDecWaves * 64);
        const __amdgpu_buffer_rsrc_t ir = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(idx_seg + (c0 - sb)), 0, 4 * (c1 - c0), kBufferWord3);
        int v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k)
          v[k] = __builtin_amdgcn_raw_buffer_load_b32(
              ir, 4u * uint32_t(tid + kDecWaves * 64 * k), 0, 0);
#pragma unroll
        for (int k = 0; k < PER; ++k) idx_s[tid + kDecWaves * 64 * k] = v[k];
      }
      __syncthreads();
      const int nst = (c1 - c0 + kDecStep - 1) / kDecStep;
      const int nj = nst > wave ? (nst - wave + kDecWaves - 1) / kDecWaves : 0;
      // Index of this lane's slot in the wave's step j, -1 when out of range.
      auto slot_idx = [&](int j) -> int {
        const int t = kDecStep * (wave + kDecWaves * j) + l16;
        return (j < nj && t < c1 - c0) ? idx_s[t] : -1;
      };
      if (nj > 0) {
        // kDecBufs steps of gathers in flight; the walk is unrolled by
        // kDecBufs so each buffer keeps its registers, and runs a multiple of
        // kDecBufs steps with no condition inside (steps past nj have no
        // valid slot: their loads return zeros and their scores are -inf).
        u32x4 kr[kDecBufs][NI];
        int idb[kDecBufs];
#pragma unroll
        for (int u = 0; u < kDecBufs; ++u) {
          idb[u] = slot_idx(u);
          gather(rsrc, pm, kr[u], idb[u]);
        }
        const int nj_pad = (nj + kDecBufs - 1) / kDecBufs * kDecBufs;
        for (int j = 0; j < nj_pad; j += kDecBufs) {
#pragma unroll
          for (int u = 0; u < kDecBufs; ++u) {
            step(kr[u], idb[u]);
            idb[u] = slot_idx(j + u + kDecBufs);
            gather(rsrc, pm, kr[u], idb[u]);
          }
        }
      }
    }
  };
  // Segment 0 is the main top-k; segment 1, when given, the second one with
  // its own rows and scale. Before segment 1, O (so far in units of the main
  // scale) is rebased onto the second scale so one O serves both (exact in
  // real arithmetic, like any rescale of the online softmax). The walk code
  // is emitted once.
  const int nseg = (p.idx2 && kend > p.topk) ? 2 : 1;
#pragma clang loop unroll(disable)
  for (int seg = 0; seg < nseg; ++seg) {
    const bool second = seg == 1;
    if (second) {
      const float s2 = *p.kv_scale2;
      const float rebase = vs / s2;
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) o[nb] *= rebase;
      vs = s2;
      c = p.sm_log2 * qs * s2;
    }
    const int sb = second ? p.topk : 0;
    const int lo = max(kbeg, sb), hi = min(kend, second ? ktot : p.topk);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(second ? p.pool2 : p.pool), 0, second ? p.pool2_bytes : p.pool_bytes,
        kBufferWord3);
    const PoolMap pm = second ? PoolMap{uint32_t(p.pool2_rs_bytes), 0u, 31u, 0x7fffffffu}
                              : PoolMap{uint32_t(p.pool_rs_bytes), uint32_t(p.page_bytes),
                                        uint32_t(p.page_shift), p.page_mask};
    const int32_t* idx_seg = second ? p.idx2 + r * p.idx2_rs : p.idx + r * p.idx_rs;
    walk_range(rsrc, pm, idx_seg, lo, hi, sb);
  }

  // ---- merge the four waves: M = max_w m_w, L = sum_w 2^(m_w - M) l_w,
  // out = sum_w 2^(m_w - M) O_w * vs / L, summed in wave order.
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16);
  l_head += __shfl_xor(l_head, 32);
  if (g == 0) {
    red_m[wave * 16 + l16] = m_ref;
    red_l[wave * 16 + l16] = l_head;
  }
  if constexpr (EPI) {
    if (tid < 64) epi_cs[tid] = cs_pre;
  }
  __syncthreads();  // also: every wave is done with its V staging area

  // Per-head weight of this wave's O: 2^(m_w - M) * vs / L.
  float fw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * g + i;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_m[w * 16 + head]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = red_m[w * 16 + head];
      L += mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M) * red_l[w * 16 + head];
    }
    const float mine = red_m[wave * 16 + head];
    fw[i] = (L > 0.f && mine != kNegInf) ? __builtin_amdgcn_exp2f(mine - M) * vs / L : 0.f;
  }

  // Four passes of 128 columns: each wave writes its weighted O, then thread
  // t sums the waves for head t / 16, columns 8 (t % 16) .. +7 of the pass,
  // so consecutive threads store consecutive 16-byte pieces of one head.
  const bool split_mode = p.part_o != nullptr;  // partials for the combine kernel
  float* part = reinterpret_cast<float*>(smem) + wave * (kMWave / 4);
  const float* parts = reinterpret_cast<const float*>(smem);
#pragma unroll
  for (int pass = 0; pass < kDv / kMCols; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's sums are read
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* prow = part + (4 * g + i) * kMPitch + l16;
#pragma unroll
      for (int nb = 0; nb < kMCols / 16; ++nb) prow[16 * nb] = o[pass * (kMCols / 16) + nb][i] * fw[i];
    }
    __syncthreads();
    const int head = tid >> 4;
    const int cl = 8 * (tid & 15);
    const int col = pass * kMCols + cl;
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* src = parts + w * (kMWave / 4) + head * kMPitch + cl;
      s0 += *reinterpret_cast<const floatx4*>(src);
      s1 += *reinterpret_cast<const floatx4*>(src + 4);
    }
    const int h = h0 + head;
    if (h < p.heads) {  // uniform over each group of 16 lanes
      if (EPI && !split_mode) {
        float v[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        epi_store<8>(p.epi, p.epi.pos != nullptr ? epi_cs : nullptr, r, h, col, v);
      } else if (!split_mode) {
        *reinterpret_cast<u32x4*>(p.out + r * p.out_rs + int64_t(h) * p.out_hs + col) =
            u32x4{pack2_bf16(s0.x, s0.y), pack2_bf16(s0.z, s0.w), pack2_bf16(s1.x, s1.y),
                  pack2_bf16(s1.z, s1.w)};
      } else {
        float* dst = p.part_o + ((int64_t(split) * p.rows + r) * p.heads + h) * kDv + col;
        *reinterpret_cast<floatx4*>(dst) = s0;
        *reinterpret_cast<floatx4*>(dst + 4) = s1;
      }
    }
  }
  if (tid < 16) {
    const int h = h0 + tid;
    if (h < p.heads) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_m[w * 16 + tid]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = red_m[w * 16 + tid];
        L += mw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mw - M) * red_l[w * 16 + tid];
      }
      const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
      if (!split_mode)
        p.lse[r * p.lse_rs + int64_t(h) * p.lse_hs] = lse;
      else
        p.part_lse[(int64_t(split) * p.rows + r) * p.heads + h] = lse;
    }
  }
}

}  // namespace

KernelShape decode_shape(int dqk) {
  KernelShape k;
  if (dqk != 576 && dqk != 512) return k;
  k.waves = kDecWaves;
  k.tile = kDecStep;
  k.lds_bytes = kDecSmem + 2 * kDecWaves * 16 * 4;
  return k;
}

int launch_decode(const FwdParams& p, int dqk, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(uint32_t(p.grid)), block(kDecWaves * 64);
  const bool epi = epi_active(p.epi) && p.part_o == nullptr;
  if (dqk == 576 && !epi)
    hipLaunchKernelGGL((decode_kernel<576, false>), grid, block, 0, st, p);
  else if (dqk == 576)
    hipLaunchKernelGGL((decode_kernel<576, true>), grid, block, 0, st, p);
  else if (dqk == 512 && !epi)
    hipLaunchKernelGGL((decode_kernel<512, false>), grid, block, 0, st, p);
  else if (dqk == 512)
    hipLaunchKernelGGL((decode_kernel<512, true>), grid, block, 0, st, p);
  else
    return int(hipErrorInvalidValue);
  return int(hipGetLastError());
}

}  // namespace smla
