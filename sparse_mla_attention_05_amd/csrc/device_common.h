// Device helpers shared by the gfx950 sparse MLA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Two floats to two bf16 (round to nearest even) in one dword, low half
// first; gfx950 does this in one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});
}

// Four e4m3fn codes (one dword, code 0 in the low byte) to four bf16 values
// (two dwords, value 0 in the low half). Exact: every finite e4m3fn value is
// a bf16 value, and the scale operand is 1.
__device__ __forceinline__ u32x2 widen_fp8x4(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// Eight e4m3fn codes (two dwords) to an MFMA bf16x8 operand, code order kept.
__device__ __forceinline__ bf16x8 widen_fp8x8(uint32_t lo, uint32_t hi) {
  const u32x2 a = widen_fp8x4(lo), b = widen_fp8x4(hi);
  return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i's 8-byte chunk is taken as row i/4, columns 4(i%4)..4(i%4)+3
// of a 4 x 16 matrix of 16-bit values, and lane j receives column j (rows
// 0..3). Pointing the 16 lanes of a group at 4 rows x 16 columns of a
// row-major tile therefore hands each lane 4 consecutive rows of one column:
// 4 k-values of an MFMA B operand whose k runs down the rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Transposed LDS read of bytes (gfx950 ds_read_b64_tr_b8). Within each group
// of 16 lanes, lane i's 8-byte chunk is taken as row i/2, columns 8(i%2)..
// 8(i%2)+7 of an 8 x 16 byte matrix, and lane j receives column j: byte t of
// the result is row t. Eight rows of one column: 8 k-values of an fp8 B
// operand whose k runs down the rows.
__device__ __forceinline__ u32x2 lds_read_tr8(const uint8_t* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// N MFMA bf16 operands of eight query elements each, starting at element
// offsets base + stride * s: a bf16 q as it is (16 bytes), a float8_e4m3fn
// q (q8 != 0) widened exactly from 8 codes (its per-tensor scale is applied
// to the scores). The dtype branch is taken once, outside the loads, and the
// codes are widened only after all of them are issued: a branch per load
// makes the compiler wait for each load in turn.
template <int N>
__device__ __forceinline__ void load_q_frags(const uint16_t* q, int32_t q8, int64_t base,
                                             int64_t stride, bf16x8 (&dst)[N]) {
  if (q8) {
    u32x2 c[N];
#pragma unroll
    for (int s = 0; s < N; ++s)
      c[s] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(q) + base + stride * s);
#pragma unroll
    for (int s = 0; s < N; ++s) dst[s] = widen_fp8x8(c[s].x, c[s].y);
  } else {
#pragma unroll
    for (int s = 0; s < N; ++s)
      dst[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + base + stride * s));
  }
}

// Byte offset of pool slot `id` in a paged pool: row id & mask of page
// id >> shift, pages `page_bytes` apart. A 2-D pool has shift 31, mask
// 0x7fffffff and page_bytes 0, which leaves id * rs.
struct PoolMap {
  uint32_t rs;          // row stride (bytes)
  uint32_t page_bytes;  // page pitch (bytes)
  uint32_t shift;
  uint32_t mask;
};
__device__ __forceinline__ uint32_t slot_offset(const PoolMap& m, int id) {
  return (uint32_t(id) >> m.shift) * m.page_bytes + (uint32_t(id) & m.mask) * m.rs;
}

// Per-tensor scale of the query (1 for a bf16 q or when none is given).
__device__ __forceinline__ float q_scale_of(const float* qs) { return qs ? *qs : 1.0f; }

}  // namespace smla
