// Work order shared by the attention kernel and its host-side mirror.
//
// The hardware deals the workgroups of a launch to the 8 XCDs of an MI355X
// round-robin by linear id, so in grid order neighbouring work items (a row's
// head blocks and splits, a decode request's rows, neighbouring prefill rows)
// land on different L2s. The XCD-aware order gives each XCD one contiguous run
// of work ids instead, so the workgroups that gather the same KV rows run on
// one L2 at the same time ("[Triton/Gluon] GFX950 sparse mla optimizations",
// commit note on the XCD remap of program ids).
//
// Workgroup pid on XCD x = pid mod 8 is the i = pid div 8-th workgroup that
// XCD receives. XCD x owns c_x = floor(G/8) + [x < G mod 8] work ids starting
// at sum_{y<x} c_y = x*floor(G/8) + min(x, G mod 8), so pid maps to that start
// plus i: a bijection of [0, G).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SMLA_HD __host__ __device__
#else
#define SMLA_HD
#endif

SMLA_HD inline int64_t smla_xcd_work(int64_t pid, int64_t grid) {
  const int64_t x = pid & 7;
  const int64_t i = pid >> 3;
  const int64_t per = grid >> 3;
  const int64_t rem = grid & 7;
  return x * per + (x < rem ? x : rem) + i;
}
