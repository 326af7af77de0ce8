// Output epilogue of the forward: the inverse RoPE of columns 448..511 and
// the MXFP8 store (float8_e4m3fn codes, one E8M0 power-of-two scale per 32
// columns), applied by whichever kernel stores a row's final values. After
// "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159), the
// commit notes on the fused epilogue: the row is rounded to bf16 first and
// every product of the rotation is rounded to fp32 on its own, so a fused
// store equals the separate pass over the bf16 rows bit for bit.
//
// Rotation pairs are adjacent columns (448 + 2j, 449 + 2j); the cos/sin cache
// row of a position holds cos of the 32 pair angles, then their sines. The
// scale of a 32-column block is 2^(floor(log2 amax) - 8) (the OCP MX v1.0
// conversion for e4m3), clamped to 2^-127 for tiny or zero blocks; elements
// are divided by it exactly (a power of two), rounded to nearest even and
// saturated at 448.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace smla {

constexpr int kRopeStart = kDv - 64;  // first rotated column
constexpr int kEpiPitch = kDv + 8;    // bf16 per row of an LDS output block (1040 B)

// Four values, already divided by their block scale, to four float8_e4m3fn
// codes in one dword (the first value in the low byte). The gfx950
// conversion (scale operand 1) rounds to nearest even and keeps the sign of
// a value that rounds to zero; the clamp to +-448 first makes the
// saturation explicit.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const auto sat = [](float x) { return __builtin_amdgcn_fmed3f(x, -448.f, 448.f); };
  const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, sat(a), sat(b), 1.0f, false);
  const s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, sat(c), sat(d), 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Inverse rotation of the pairs among N consecutive columns starting at an
// even column of the rotated range; cs points at the cos of the first pair.
template <int N>
__device__ __forceinline__ void inverse_rope_pairs(float (&v)[N], const float* cs) {
#pragma clang fp contract(off)
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const float c = cs[k >> 1], s = cs[32 + (k >> 1)];
    const float x = v[k], y = v[k + 1];
    v[k] = x * c + y * s;
    v[k + 1] = y * c - x * s;
  }
}

// Row of the cos/sin cache at row r's position (clamped into the cache), or
// nullptr when the epilogue does not rotate. Kernels load it early (the
// position read and the cache read are two dependent round trips) and hand
// the epilogue a copy in LDS.
__device__ __forceinline__ const float* epi_cs_row(const EpiOut& e, int64_t r) {
  if (e.pos == nullptr) return nullptr;
  int pos = e.pos[r];
  pos = pos < 0 ? 0 : (pos >= e.cs_rows ? e.cs_rows - 1 : pos);
  return e.cs + int64_t(pos) * e.cs_rs;
}

// First half of a store through the epilogue: the bf16 rounding of N
// consecutive columns [col0, col0 + N) (col0 even), then the inverse
// rotation where they fall in the rotated range; cs_row is the row's
// cos/sin (global or LDS), nullptr for no rotation.
template <int N>
__device__ __forceinline__ void epi_prepare(const float* cs_row, int col0, float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const uint32_t w = pack2_bf16(v[k], v[k + 1]);  // round to nearest even, two at once
    v[k] = __uint_as_float(w << 16);
    v[k + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
  if (cs_row != nullptr && col0 >= kRopeStart)
    inverse_rope_pairs<N>(v, cs_row + ((col0 - kRopeStart) >> 1));
}

template <int N>
__device__ __forceinline__ float abs_max(const float (&v)[N]) {
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < N; ++k) a = fmaxf(a, fabsf(v[k]));
  return a;
}

// E8M0 code of a 32-column block with largest magnitude amax: max(E - 8, 0),
// E the fp32 exponent field of amax; *inv = 1 / X = 2^(127 - code).
__device__ __forceinline__ uint32_t e8m0_code(float amax, float* inv) {
  const uint32_t ebits = __float_as_uint(amax) >> 23;
  const uint32_t sc = ebits > 8u ? ebits - 8u : 0u;
  *inv = __uint_as_float((254u - sc) << 23);
  return sc;
}

// Second half: stores the N prepared columns, as bf16, or as e4m3fn codes
// with the block's scale code sc (the lane holding the block's first column
// stores sc).
template <int N>
__device__ __forceinline__ void epi_emit(const EpiOut& e, int64_t r, int h, int col0,
                                         const float (&v)[N], uint32_t sc, float inv) {
  const int64_t off = r * e.out_rs + int64_t(h) * e.out_hs + col0;
  if (e.q8 == nullptr) {
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k) w[k] = pack2_bf16(v[2 * k], v[2 * k + 1]);
    if constexpr (N == 4) {
      *reinterpret_cast<u32x2*>(e.out + off) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int k = 0; k < N / 8; ++k)
        *reinterpret_cast<u32x4*>(e.out + off + 8 * k) =
            u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    }
    return;
  }
  uint32_t w[N / 4];
#pragma unroll
  for (int k = 0; k < N / 4; ++k)
    w[k] = e4m3x4(v[4 * k] * inv, v[4 * k + 1] * inv, v[4 * k + 2] * inv, v[4 * k + 3] * inv);
  if constexpr (N == 4) {
    *reinterpret_cast<uint32_t*>(e.q8 + off) = w[0];
  } else if constexpr (N == 8) {
    *reinterpret_cast<u32x2*>(e.q8 + off) = u32x2{w[0], w[1]};
  } else {
#pragma unroll
    for (int k = 0; k < N / 16; ++k)
      *reinterpret_cast<u32x4*>(e.q8 + off + 16 * k) =
          u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
  }
  if ((col0 & 31) == 0) e.sc[r * e.sc_rs + int64_t(h) * e.sc_hs + (col0 >> 5)] = uint8_t(sc);
}

// Stores N consecutive output columns [col0, col0 + N) of row r, head h
// through the epilogue (cs_row as for epi_prepare). The 32-column scale group of an MXFP8 store spans
// 32 / N consecutive lanes, which must all make this call together (N = 32:
// one lane). v holds the values before the bf16 rounding.
template <int N>
__device__ __forceinline__ void epi_store(const EpiOut& e, const float* cs_row, int64_t r, int h,
                                          int col0, float (&v)[N]) {
  static_assert(N == 4 || N == 8 || N == 32, "columns per lane");
  epi_prepare<N>(cs_row, col0, v);
  uint32_t sc = 0u;
  float inv = 1.f;
  if (e.q8 != nullptr) {
    float amax = abs_max<N>(v);
#pragma unroll
    for (int m = 1; m < 32 / N; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    sc = e8m0_code(amax, &inv);
  }
  epi_emit<N>(e, r, h, col0, v, sc, inv);
}

// The store of an MFMA 16x16 accumulator layout in which a lane holds 4
// consecutive columns at col_a = 32m + 4g and 4 more at col_a + 16 (g = lane
// bits 4..5): the 32-column block [32m, 32m + 32) is spread over the four
// lanes with equal bits 0..3, which must all make this call together.
__device__ __forceinline__ void epi_store_c16x2(const EpiOut& e, const float* cs_row, int64_t r,
                                                int h, int col_a, float (&va)[4], float (&vb)[4]) {
  epi_prepare<4>(cs_row, col_a, va);
  epi_prepare<4>(cs_row, col_a + 16, vb);
  uint32_t sc = 0u;
  float inv = 1.f;
  if (e.q8 != nullptr) {
    float amax = fmaxf(abs_max<4>(va), abs_max<4>(vb));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    sc = e8m0_code(amax, &inv);
  }
  epi_emit<4>(e, r, h, col_a, va, sc, inv);
  epi_emit<4>(e, r, h, col_a + 16, vb, sc, inv);
}

// The store of an MFMA 32x32 accumulator layout in which a lane holds four
// groups of 4 consecutive columns at col_a + 8j (j = 0..3, col_a = 32m + 4h,
// h = lane bit 5): the 32-column block [32m, 32m + 32) is spread over the
// two lanes l and l ^ 32, which must make this call together.
__device__ __forceinline__ void epi_store_c32x4(const EpiOut& e, const float* cs_row, int64_t r,
                                                int h, int col_a, float (&v)[4][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) epi_prepare<4>(cs_row, col_a + 8 * j, v[j]);
  uint32_t sc = 0u;
  float inv = 1.f;
  if (e.q8 != nullptr) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, abs_max<4>(v[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    sc = e8m0_code(amax, &inv);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) epi_emit<4>(e, r, h, col_a + 8 * j, v[j], sc, inv);
}

// A workgroup's block of nh heads of row r staged in LDS as bf16 rows of
// kEpiPitch elements: local head i < split at lo + i * kEpiPitch, the others
// at hi + (i - split) * kEpiPitch. Thread tid of nt stores 32-column pieces
// through the epilogue, heads h0 .. h0 + nh - 1 below `heads` only. The
// caller has made the block visible (barrier).
__device__ __forceinline__ void epi_store_lds_block(const EpiOut& e, const float* cs_row,
                                                    const uint16_t* lo,
                                                    const uint16_t* hi, int split, int nh,
                                                    int64_t r, int h0, int heads, int tid,
                                                    int nt) {
  for (int it = tid; it < nh * (kDv / 32); it += nt) {
    const int head = it / (kDv / 32), c = it % (kDv / 32);
    if (h0 + head >= heads) continue;
    const uint16_t* row = head < split ? lo + head * kEpiPitch : hi + (head - split) * kEpiPitch;
    const u32x4* src = reinterpret_cast<const u32x4*>(row + 32 * c);
    float v[32];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 q = src[k];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * k + 2 * j] = __uint_as_float(q[j] << 16);
        v[8 * k + 2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
      }
    }
    epi_store<32>(e, cs_row, r, h0 + head, 32 * c, v);
  }
}

}  // namespace smla
