// The indexer that produces the sparse attention's index rows: fp8 MQA
// logits and a per-row top-k, after "[HIP] [JIT] fp8_mqa_logits: v35w gfx950
// prefill indexer logits kernel" (aiter PR 7183), Motivation and Design:
//
//   logits[m, n] = sum_h relu(Q[m,h,:] . K[n,:]) * w[m,h] * kv_scale[n]
//                  for n in [ks[m], ke[m]), -inf elsewhere
//
// Logits kernel. A workgroup takes 16 query rows (4 waves x 4 rows) and one
// 4096-key column of the output; Q (4 rows x 32 heads x 128 fp8 = 64 VGPRs)
// and w stay in registers, and all waves walk the same K sequence through
// LDS (64-key stages, double-buffered, chunk-XOR swizzled rows), so K is read
// once per 16 rows; three workgroups share a CU (168 VGPRs, no spills), so
// one wave's relu and head sums run under the others' MFMAs. One v_mfma_f32_16x16x128_f8f6f4 computes
// 16 heads x 16 keys over all 128 dims (A = Q rows, B = K rows, the same
// lane->k mapping on both sides). A lane's accumulator holds heads 4g..4g+3 of one key; relu
// and the head weight are applied there, the four lanes g of a key are summed
// by lane-row swaps arranged as a transpose over the wave's four rows
// (afterwards lane g owns row g), and the key's scale is applied after the
// head sum. Tiles outside every row's window are not computed; with `clean`
// the kernel writes -inf there itself.
//
// Top-k kernel. One workgroup per row: a radix select (12, 10 and 10 bits)
// on the order-preserving integer image of the fp32 logits finds the k-th
// largest value T, and the output holds, in ascending index order, every
// key above T and the lowest-index keys equal to T. The first level reads
// the window; the keys in and above its chosen bin are then compacted into
// LDS by a second read when they fit, and the other levels and the output
// work there. Only the window is read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace smla {
namespace {

constexpr int kIxWaves = 4;
constexpr int kIxRowsPerWave = 4;
constexpr int kIxRows = kIxWaves * kIxRowsPerWave;
constexpr int kIxTile = 64;                    // keys per LDS stage
constexpr int kIxTileBytes = kIxTile * kIxDim;  // 8 KB
constexpr uint32_t kIxOutOfRange = 0xFFFFF000u;  // buffer offset past every range
constexpr int kIxBufferWord3 = 0x00020000;      // raw buffer descriptor word 3 (gfx9 family)

typedef int v8i __attribute__((ext_vector_type(8)));

// max(x, 0) as one integer max: a negative float is a negative int32 and
// -0.0 becomes +0.0 (fmaxf would first quiet NaNs, a second instruction).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ v8i cat(u32x4 a, u32x4 b) {
  return v8i{int(a.x), int(a.y), int(a.z), int(a.w), int(b.x), int(b.y), int(b.z), int(b.w)};
}

__global__ void __launch_bounds__(kIxWaves * 64) __attribute__((amdgpu_waves_per_eu(3, 3)))
ix_logits_kernel(const IxParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][kIxTileBytes];
  __shared__ float ksc[2][kIxTile];
  __shared__ int wlo[kIxWaves], whi[kIxWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar row base
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t m0 = int64_t(blockIdx.x) * kIxRows + kIxRowsPerWave * wave;
  const int n_begin = int(blockIdx.y) * kIxChunk;
  const int n_end = min(p.n, n_begin + kIxChunk);

  // ---- this wave's rows: windows, Q and w in registers.
  int lo[kIxRowsPerWave], hi[kIxRowsPerWave];
  v8i qa[kIxRowsPerWave][2];
  floatx4 wv[kIxRowsPerWave][2];
  int my_lo = 0, my_hi = 0;  // the window of row g (the row this lane stores)
#pragma unroll
  for (int j = 0; j < kIxRowsPerWave; ++j) {
    const int64_t m = m0 + j;
    const int64_t mc = m < p.m ? m : p.m - 1;
    int a = m < p.m ? p.ks[m] : 0, b = m < p.m ? p.ke[m] : 0;
    a = a < 0 ? 0 : (a > p.n ? p.n : a);
    b = b < a ? a : (b > p.n ? p.n : b);
    lo[j] = a;
    hi[j] = b;
    if (g == j) {
      my_lo = a;
      my_hi = b;
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.q + mc * p.q_rs +
                                                        int64_t(16 * ht + l16) * p.q_hs + 32 * g);
      qa[j][ht] = cat(src[0], src[1]);
      wv[j][ht] = *reinterpret_cast<const floatx4*>(p.w + mc * p.w_rs + 16 * ht + 4 * g);
    }
  }

  // ---- keys any of the workgroup's rows sees inside this column: whole tiles.
  int ulo = p.n, uhi = 0;
#pragma unroll
  for (int j = 0; j < kIxRowsPerWave; ++j)
    if (hi[j] > lo[j]) {
      ulo = min(ulo, lo[j]);
      uhi = max(uhi, hi[j]);
    }
  if (lane == 0) {
    wlo[wave] = ulo;
    whi[wave] = uhi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kIxWaves; ++w) {
    ulo = min(ulo, wlo[w]);
    uhi = max(uhi, whi[w]);
  }
  ulo = max(ulo, n_begin);
  uhi = min(uhi, n_end);
  const int t_first = ulo < uhi ? (ulo / kIxTile) * kIxTile : n_begin;
  const int ntiles = ulo < uhi ? (uhi - t_first + kIxTile - 1) / kIxTile : 0;
  const int t_stop = min(n_end, t_first + ntiles * kIxTile);

  // ---- -inf outside the computed tiles (clean mode): rows of this wave.
  if (p.clean) {
#pragma unroll
    for (int j = 0; j < kIxRowsPerWave; ++j) {
      const int64_t m = m0 + j;
      if (m >= p.m) continue;
      float* row = p.logits + m * p.l_rs;
      for (int n = n_begin + lane; n < t_first; n += 64) row[n] = kNegInf;
      for (int n = t_stop + lane; n < n_end; n += 64) row[n] = kNegInf;
    }
  }
  if (ntiles == 0) return;

  // ---- K staging: thread t moves 16-byte pieces (key, chunk) = (t/8 + 32i,
  // t%8) of a tile; physical chunk = chunk ^ (key & 7). K and the key scales
  // are read through buffer resources whose ranges end at key N, so a piece
  // past the last key reads 0 without a branch; two tiles are in flight.
  constexpr int NT = kIxWaves * 64;
  constexpr int SPT = kIxTileBytes / 16 / NT;  // pieces per thread
  const int skey = tid >> 3, schunk = tid & 7;
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.k), 0, uint32_t(int64_t(p.n) * p.k_rs), kIxBufferWord3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.kv_scale), 0, uint32_t(4 * p.n), kIxBufferWord3);
  // Offsets go in the per-lane operand (the range check covers it; the
  // scalar offset is not checked).
  auto load_tile = [&](int n0, u32x4 (&v)[SPT], float& sc) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const uint32_t key = uint32_t(n0 + skey + (NT / 8) * i);
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           k_rsrc, key * uint32_t(p.k_rs) + 16u * uint32_t(schunk), 0, 0));
    }
    sc = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, tid < kIxTile ? 4u * uint32_t(n0 + tid) : 0u, 0, 0));
  };
  auto store_tile = [&](int b, const u32x4 (&v)[SPT], float sc) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int key = skey + (NT / 8) * i;
      *reinterpret_cast<u32x4*>(&kt[b][key * kIxDim + 16 * (schunk ^ (key & 7))]) = v[i];
    }
    if (tid < kIxTile) ksc[b][tid] = sc;
  };

  // ---- logits: this wave's 4 rows through one buffer resource (rows past M
  // and dropped positions get an offset past its range, so stores need no
  // branch); lane group g stores row g.
  const int rv = int(min<int64_t>(kIxRowsPerWave, p.m - m0));  // valid rows of the wave (>= 0)
  const __amdgpu_buffer_rsrc_t l_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      p.logits + (m0 < p.m ? m0 : 0) * p.l_rs, 0,
      rv > 0 ? uint32_t(4 * (int64_t(rv - 1) * p.l_rs + p.n)) : 0u, kIxBufferWord3);
  const uint32_t row_off = 4u * uint32_t(g) * uint32_t(p.l_rs);

  auto compute = [&](int buf, int n0) {
    const uint8_t* tile = kt[buf];
#pragma unroll
    for (int kb = 0; kb < kIxTile / 16; ++kb) {
      const int key = 16 * kb + l16;
      const uint8_t* krow = tile + key * kIxDim;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * g) ^ (key & 7)));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(krow + 16 * ((2 * g + 1) ^ (key & 7)));
      const v8i kb8 = cat(b0, b1);
      float sc = ksc[buf][key];
      asm volatile("" : "+v"(sc));  // read unconditionally: no branch around the LDS read
      float part[kIxRowsPerWave];
#pragma unroll
      for (int j = 0; j < kIxRowsPerWave; ++j) {
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        const floatx4 s0 =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[j][0], kb8, zero, 0, 0, 0, 0, 0, 0);
        const floatx4 s1 =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[j][1], kb8, zero, 0, 0, 0, 0, 0, 0);
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a = __builtin_fmaf(relu(s0[i]), wv[j][0][i], a);
          b = __builtin_fmaf(relu(s1[i]), wv[j][1][i], b);
        }
        part[j] = a + b;
      }
      // Transposing sums over the lane groups g (bits 4, 5), by row swaps
      // between register pairs: the 16-lane swap leaves group g rows
      // (g & 1) and 2 + (g & 1) summed over the group pair {g & 2, (g & 2) + 1},
      // the 32-lane swap then adds the other pair, so that lane g holds row
      // g's sum over all 32 heads for key `key`.
      const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]),
                                                        __float_as_uint(part[1]), false, false);
      const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[2]),
                                                        __float_as_uint(part[3]), false, false);
      const float q01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
      const float q23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
      const auto s4 = __builtin_amdgcn_permlane32_swap(__float_as_uint(q01), __float_as_uint(q23),
                                                       false, false);
      const float tot = __uint_as_float(s4[0]) + __uint_as_float(s4[1]);
      const int n = n0 + key;
      const bool inside = n >= my_lo && n < my_hi;
      const bool write = n < t_stop && (inside || p.clean != 0);
      const float val = inside ? tot * sc : kNegInf;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), l_rsrc,
                                            write ? row_off + 4u * uint32_t(n) : kIxOutOfRange, 0, 0);
    }
  };

  u32x4 pa[SPT], pb[SPT];
  float sa, sb;
  load_tile(t_first, pa, sa);
  if (ntiles > 1) load_tile(t_first + kIxTile, pb, sb);
  store_tile(0, pa, sa);
  __syncthreads();
  // Tile t's staging registers: pa for even t, pb for odd t. Iteration t
  // loads tile t + 2 into the set tile t left, computes tile t, then moves
  // tile t + 1 into the other LDS buffer.
  for (int it = 0; it < ntiles; it += 2) {
    const int n0 = t_first + it * kIxTile;
    if (it + 2 < ntiles) load_tile(n0 + 2 * kIxTile, pa, sa);
    compute(0, n0);
    if (it + 1 < ntiles) store_tile(1, pb, sb);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    if (it + 3 < ntiles) load_tile(n0 + 3 * kIxTile, pb, sb);
    compute(1, n0 + kIxTile);
    if (it + 2 < ntiles) store_tile(0, pa, sa);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ top-k

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkPer = 8;                       // contiguous keys per thread in a round
constexpr int kTkRound = kTkThreads * kTkPer;   // keys per round
constexpr int kTkBits0 = 12;                    // bits of the first radix level
constexpr int kTkShift0 = 32 - kTkBits0;
constexpr int kTkCap = 8192;                    // candidates kept in LDS

// Order-preserving integer image of an fp32 value (-0 taken as +0, so the two
// zeros tie as they do as numbers).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the block in thread order, and the block's
// total; sh holds kTkWaves words. Every thread of the block calls it.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;  // inclusive prefix within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t t = sh[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();
  return x - v + before;
}

// Bin of a radix level holding the `need`-th largest key: `h` are this
// thread's `per` consecutive bins starting at per * tid (of `bins`); writes
// (bin, count in the bins above it) to pick.
__device__ __forceinline__ void pick_bin(const uint32_t* h, int per, uint32_t need, uint32_t* sh,
                                         uint32_t* pick) {
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += h[i];
  uint32_t total;
  const uint32_t before = block_excl_scan(mine, sh, total);
  // keys in bins above this thread's: total - before - mine
  uint32_t above = total - before - mine;
  for (int i = per - 1; i >= 0; --i) {
    if (above < need && above + h[i] >= need) {
      pick[0] = uint32_t(per * threadIdx.x + i);
      pick[1] = above;
    }
    above += h[i];
  }
  __syncthreads();
}

// One workgroup per row. A 12-bit histogram of the order keys over the
// window (one read) fixes the bin of the k-th largest key; when that bin and
// the ones above hold at most kTkCap keys (the usual case: logits are
// continuous), a second read compacts them into LDS in index order and the
// rest (two 10-bit levels and the output) runs on those. Otherwise two more
// full-window levels and an output read finish the select. Keys above the
// k-th largest value T are written, then the lowest-index keys equal to T,
// in ascending index order. Only the window is read.
__global__ void __launch_bounds__(kTkThreads) topk_kernel(const TopkParams p) {
  __shared__ uint32_t cand_u[kTkCap];  // the first level's histogram, then candidate keys
  __shared__ int32_t cand_n[kTkCap];   // candidate indices
  __shared__ uint32_t hist[1024];      // the 10-bit levels
  __shared__ uint32_t scan[kTkWaves];
  __shared__ uint32_t pick[2];         // bin, count above it

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const float* row = p.logits + r * p.l_rs;
  int32_t* out = p.out + r * p.o_rs;
  int lo = p.ks[r], hi = p.ke[r];
  lo = lo < 0 ? 0 : (lo > p.n ? p.n : lo);
  hi = hi < lo ? lo : (hi > p.n ? p.n : hi);
  const int len = hi - lo;
  if (len <= p.k) {
    for (int i = tid; i < p.k; i += kTkThreads) out[i] = i < len ? lo + i : -1;
    return;
  }
  // Keys n0 .. n0 + 7 of a round (n0 a multiple of 8: two 16-byte loads),
  // through a buffer resource that ends at the window's end (keys past it
  // read 0); keys outside [lo, hi) are masked where they are used.
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, uint32_t(4 * hi), kIxBufferWord3);
  auto load8 = [&](int n0, uint32_t (&u)[kTkPer]) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, 4u * uint32_t(n0), 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, 4u * uint32_t(n0) + 16u, 0, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u[j] = order_key(__uint_as_float(a[j]));
      u[4 + j] = order_key(__uint_as_float(b[j]));
    }
  };
  const int lo8 = lo & ~(kTkPer - 1);  // rounds start 32-byte aligned
  auto in = [&](int n) { return n >= lo && n < hi; };

  // ---- level 0: 12-bit histogram over the window
  uint32_t* const hist0 = cand_u;
  for (int i = tid; i < (1 << kTkBits0); i += kTkThreads) hist0[i] = 0u;
  __syncthreads();
  for (int base = lo8; base < hi; base += kTkRound) {
    const int n0 = base + kTkPer * tid;
    uint32_t u[kTkPer];
    load8(n0, u);
#pragma unroll
    for (int j = 0; j < kTkPer; ++j)
      if (in(n0 + j)) atomicAdd(&hist0[u[j] >> kTkShift0], 1u);
  }
  __syncthreads();
  constexpr int kPer0 = (1 << kTkBits0) / kTkThreads;
  uint32_t h0[kPer0];
#pragma unroll
  for (int i = 0; i < kPer0; ++i) h0[i] = hist0[kPer0 * tid + i];
  pick_bin(h0, kPer0, uint32_t(p.k), scan, pick);
  const uint32_t b0 = pick[0];
  uint32_t need = uint32_t(p.k) - pick[1];        // keys of bin b0 still to take
  const uint32_t ncand = pick[1] + hist0[b0];     // keys in bins >= b0
  __syncthreads();

  uint32_t prefix = b0;
  if (ncand <= uint32_t(kTkCap)) {
    // ---- candidates: the keys in bins >= b0, compacted in index order
    uint32_t pos = 0;
    for (int base = lo8; base < hi; base += kTkRound) {
      const int n0 = base + kTkPer * tid;
      uint32_t u[kTkPer];
      load8(n0, u);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kTkPer; ++j) c += (in(n0 + j) && (u[j] >> kTkShift0) >= b0) ? 1u : 0u;
      uint32_t total;
      uint32_t at = pos + block_excl_scan(c, scan, total);
#pragma unroll
      for (int j = 0; j < kTkPer; ++j)
        if (in(n0 + j) && (u[j] >> kTkShift0) >= b0) {
          cand_u[at] = u[j];
          cand_n[at] = n0 + j;
          ++at;
        }
      pos += total;
    }
    __syncthreads();
    // ---- two 10-bit levels over the candidates of bin b0
#pragma unroll
    for (int lv = 0; lv < 2; ++lv) {
      const int sh = lv == 0 ? 10 : 0;
      hist[tid] = 0u;
      __syncthreads();
      for (int i = tid; i < int(ncand); i += kTkThreads) {
        const uint32_t u = cand_u[i];
        if ((u >> (sh + 10)) == prefix) atomicAdd(&hist[(u >> sh) & 1023u], 1u);
      }
      __syncthreads();
      uint32_t h1[1] = {hist[tid]};
      pick_bin(h1, 1, need, scan, pick);
      prefix = (prefix << 10) | pick[0];
      need -= pick[1];
      __syncthreads();
    }
    const uint32_t T = prefix;
    // ---- output: candidates above T, then the first `need` equal to it,
    // in index order (thread t takes candidates 8t .. 8t + 7)
    uint32_t u[kTkPer];
    int32_t nn[kTkPer];
    uint32_t ce = 0;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
      const int i = kTkPer * tid + j;
      u[j] = i < int(ncand) ? cand_u[i] : 0u;
      nn[j] = i < int(ncand) ? cand_n[i] : 0;
      ce += (i < int(ncand) && u[j] == T) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t eq_before = block_excl_scan(ce, scan, tot);
    bool sel[kTkPer];
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
      const int i = kTkPer * tid + j;
      const bool eq = i < int(ncand) && u[j] == T;
      sel[j] = i < int(ncand) && (u[j] > T || (eq && eq_before < need));
      eq_before += eq ? 1u : 0u;
      cs += sel[j] ? 1u : 0u;
    }
    uint32_t at = block_excl_scan(cs, scan, tot);
#pragma unroll
    for (int j = 0; j < kTkPer; ++j)
      if (sel[j]) out[at++] = nn[j];
    return;
  }

  // ---- many keys in and above the k-th key's bin: two more levels over the
  // whole window, then the output read
#pragma unroll
  for (int lv = 0; lv < 2; ++lv) {
    const int sh = lv == 0 ? 10 : 0;
    hist[tid] = 0u;
    __syncthreads();
    for (int base = lo8; base < hi; base += kTkRound) {
      const int n0 = base + kTkPer * tid;
      uint32_t u[kTkPer];
      load8(n0, u);
#pragma unroll
      for (int j = 0; j < kTkPer; ++j)
        if (in(n0 + j) && (u[j] >> (sh + 10)) == prefix) atomicAdd(&hist[(u[j] >> sh) & 1023u], 1u);
    }
    __syncthreads();
    uint32_t h1[1] = {hist[tid]};
    pick_bin(h1, 1, need, scan, pick);
    prefix = (prefix << 10) | pick[0];
    need -= pick[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  uint32_t eq_base = 0, sel_base = 0;
  for (int base = lo8; base < hi; base += kTkRound) {
    const int n0 = base + kTkPer * tid;
    uint32_t u[kTkPer];
    load8(n0, u);
    uint32_t ce = 0;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) ce += (in(n0 + j) && u[j] == T) ? 1u : 0u;
    uint32_t tot_e;
    uint32_t eq_before = eq_base + block_excl_scan(ce, scan, tot_e);
    bool sel[kTkPer];
    uint32_t cs = 0;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
      const bool inw = in(n0 + j);
      const bool eq = inw && u[j] == T;
      sel[j] = inw && (u[j] > T || (eq && eq_before < need));
      eq_before += eq ? 1u : 0u;
      cs += sel[j] ? 1u : 0u;
    }
    uint32_t tot_s;
    uint32_t at = sel_base + block_excl_scan(cs, scan, tot_s);
#pragma unroll
    for (int j = 0; j < kTkPer; ++j)
      if (sel[j]) out[at++] = n0 + j;
    eq_base += tot_e;
    sel_base += tot_s;
  }
}

}  // namespace

int launch_ix_logits(const IxParams& p, void* stream) {
  if (p.m == 0 || p.n == 0) return 0;
  const dim3 grid(uint32_t((p.m + kIxRows - 1) / kIxRows), uint32_t((p.n + kIxChunk - 1) / kIxChunk));
  hipLaunchKernelGGL(ix_logits_kernel, grid, dim3(kIxWaves * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

int launch_topk(const TopkParams& p, void* stream) {
  if (p.rows == 0) return 0;
  hipLaunchKernelGGL(topk_kernel, dim3(uint32_t(p.rows)), dim3(kTkThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

}  // namespace smla
