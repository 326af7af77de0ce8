// The output epilogue as a pass of its own over bf16 attention rows: the
// separate pass that the fused stores replace ("[Triton/Gluon] GFX950 sparse
// mla optimizations" (aiter PR 6159), commit notes on the fused epilogue).
// One wave per (row, head): lane i loads columns 8i..8i+7 (16 bytes, so a
// wave reads the 1 KB row in one coalesced sweep), and four lanes form one
// 32-column scale group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "epilogue.h"
#include "launch.h"

namespace smla {
namespace {

constexpr int kEpiPassThreads = 256;

__global__ void __launch_bounds__(kEpiPassThreads) out_epilogue_kernel(const EpiPassParams p) {
  const int64_t item = int64_t(blockIdx.x) * (kEpiPassThreads / 64) + (threadIdx.x >> 6);
  if (item >= p.rows * p.heads) return;  // whole waves leave together
  const int64_t r = item / p.heads;
  const int h = int(item % p.heads);
  const int col = 8 * (threadIdx.x & 63);
  const float* cs_row = epi_cs_row(p.epi, r);
  const u32x4 q = *reinterpret_cast<const u32x4*>(p.in + r * p.in_rs + int64_t(h) * p.in_hs + col);
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(q[j] << 16);
    v[2 * j + 1] = __uint_as_float(q[j] & 0xFFFF0000u);
  }
  epi_store<8>(p.epi, cs_row, r, h, col, v);
}

}  // namespace

int launch_out_epilogue(const EpiPassParams& p, void* stream) {
  const int64_t items = p.rows * p.heads;
  if (items == 0) return 0;
  const int64_t blocks = (items + kEpiPassThreads / 64 - 1) / (kEpiPassThreads / 64);
  hipLaunchKernelGGL(out_epilogue_kernel, dim3(uint32_t(blocks)), dim3(kEpiPassThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return int(hipGetLastError());
}

}  // namespace smla
