// Internal interface between the host API (api.cpp), the planner (plan.cpp)
// and the kernels (kernels.hip). Not part of the public C ABI.
#pragma once
#include <stdint.h>

#include <string>

#include "../../include/sparse_mla.h"

namespace smla {

constexpr int kDv = 512;        // value width: the first 512 columns of a row
constexpr int kMaxSplits = 64;
constexpr int kMaxHeads = 1024;
constexpr int64_t kMaxTopk = int64_t(1) << 20;
constexpr int kMaxDevices = 64;
// Bytes of the fixed device scratch of the no-allocation forward.
constexpr int64_t kScratchBytes = SMLA_NOALLOC_SCRATCH_BYTES;

// The calling thread's current device's copy of that scratch (noalloc.hip):
// its device address, resolved once per device. Returns a status and sets
// *err on failure. Makes no allocation.
int scratch_buffer(int dev, void** out, std::string* err);

// Where and how the output epilogue stores (epilogue.h): the inverse RoPE of
// columns 448..511 when pos is set, and an MXFP8 store (codes in q8, E8M0
// scales in sc) when q8 is set, else a bf16 store to out.
struct EpiOut {
  uint16_t* out;            // bf16 [R, H, 512] (q8 == nullptr)
  uint8_t* q8;              // e4m3fn codes [R, H, 512], or nullptr
  int64_t out_rs, out_hs;   // strides of out or q8
  uint8_t* sc;              // E8M0 codes [R, H, 16]
  int64_t sc_rs, sc_hs;
  const int32_t* pos;       // int32 [R] position of each row, or nullptr
  const float* cs;          // fp32 [cs_rows, 64]: cos of the 32 pair angles, then sin
  int64_t cs_rs;
  int32_t cs_rows;
};

inline bool epi_active(const EpiOut& e) { return e.pos != nullptr || e.q8 != nullptr; }

// Everything the attention kernel reads, with strides in elements except
// where named "_bytes".
struct FwdParams {
  const uint16_t* q;        // bf16 [R, H, Dqk]
  int64_t q_rs, q_hs;
  const uint8_t* pool;      // bf16 or e4m3fn rows
  int64_t pool_rs_bytes;
  uint32_t pool_bytes;      // bytes from pool to the end of its last row read, capped
                            // at kMaxBufferBytes (buffer-load range)
  const float* kv_scale;    // fp32 [1] (fp8 pools) or nullptr
  const int32_t* idx;       // int32 [R, K]
  int64_t idx_rs;
  uint16_t* out;            // bf16 [R, H, 512]
  int64_t out_rs, out_hs;
  float* lse;               // fp32 [R, H]
  int64_t lse_rs, lse_hs;
  float* part_o;            // fp32 [S, R, H, 512]; non-null: write split partials
  float* part_lse;          // fp32 [S, R, H]
  int64_t rows;
  int32_t heads;
  int32_t topk;
  int32_t splits;
  int32_t tiles_per_split;
  int32_t head_blocks;
  int32_t remap;
  int64_t grid;
  float sm_log2;            // sm_scale * log2(e)
  // Second segment of a two-segment call walked inside the kernel (decode
  // kernel only): its slots follow the topk main slots in one virtual list of
  // topk + topk2 slots that the splits partition. idx2 == nullptr: none.
  const uint8_t* pool2;
  int64_t pool2_rs_bytes;
  uint32_t pool2_bytes;
  const float* kv_scale2;
  const int32_t* idx2;
  int64_t idx2_rs;
  int32_t topk2;
  // Output epilogue of the final store (the attention kernel's without
  // splits, the combine kernel's with them); inactive: plain bf16 to out.
  EpiOut epi;
  // q as float8_e4m3fn codes (q then points at bytes, strides in bytes) and
  // its per-tensor scale (nullptr: 1).
  int32_t q_fp8;
  const float* q_scale;
  // Paged main pool ([pages, page rows, W] with its own page pitch): slot i
  // is row i & page_mask of page i >> page_shift. A 2-D pool: shift 31,
  // mask 0x7fffffff, page_bytes 0. The second segment's pool is 2-D.
  int32_t page_shift;
  uint32_t page_mask;
  int64_t page_bytes;
  // CUs of the device: a kernel that keeps one workgroup per CU and streams
  // its share of the work items launches at most this many workgroups.
  int32_t persist_cap;
};

// The output epilogue as a pass of its own over bf16 rows [rows, heads, 512].
struct EpiPassParams {
  const uint16_t* in;
  int64_t in_rs, in_hs;
  int64_t rows;
  int32_t heads;
  EpiOut epi;
};
int launch_out_epilogue(const EpiPassParams& p, void* stream);

// Indexer logits (indexer.hip): 32 heads x 128 dims of fp8, strides in bytes
// for the fp8 tensors and in elements otherwise.
constexpr int kIxHeads = 32;
constexpr int kIxDim = 128;
constexpr int kIxChunk = 4096;  // keys per workgroup column
struct IxParams {
  const uint8_t* q;          // e4m3fn [M, 32, 128]
  int64_t q_rs, q_hs;
  const uint8_t* k;          // e4m3fn [N, 128]
  int64_t k_rs;
  const float* kv_scale;     // fp32 [N]
  const float* w;            // fp32 [M, 32]
  int64_t w_rs;
  const int32_t* ks;         // int32 [M]
  const int32_t* ke;
  float* logits;             // fp32 [M, N]
  int64_t l_rs;
  int64_t m;
  int32_t n;
  int32_t clean;             // 1: write -inf outside each row's window too
};
int launch_ix_logits(const IxParams& p, void* stream);

// Per-row top-k of logits inside each row's window (indexer.hip).
struct TopkParams {
  const float* logits;       // fp32 [R, N]
  int64_t l_rs;
  const int32_t* ks;         // int32 [R]
  const int32_t* ke;
  int32_t* out;              // int32 [R, k]
  int64_t o_rs;
  int64_t rows;
  int32_t n;
  int32_t k;
};
int launch_topk(const TopkParams& p, void* stream);

struct Problem {
  int64_t rows;
  int32_t heads;
  int32_t dqk;
  int32_t topk;
  int32_t kv_fp8;
  int64_t pool_bytes;       // bytes from pool to the end of its last row read
  int64_t pool_rs_bytes;    // row stride (bytes)
  int64_t page_bytes;       // page pitch of a paged pool (bytes), 0 for a 2-D pool
};

// Largest pool (bytes) the decode kernel addresses through a buffer
// descriptor with 32-bit offsets; larger pools use the staged-tile kernel.
constexpr int64_t kMaxBufferBytes = 0xFFFFF000ll - 4096;

// Shape of the attention-kernel instance used for (head_block, dqk, pool
// dtype, variant): wavefronts per workgroup, slots per tile, LDS per
// workgroup.
struct KernelShape {
  int waves = 0;
  int tile = 0;
  int lds_bytes = 0;
};
KernelShape kernel_shape(int head_block, int dqk, bool fp8, int variant);

// The 16-head fp8 decode kernel (decode.hip): its shape and its launch.
KernelShape decode_shape(int dqk);
int launch_decode(const FwdParams& p, int dqk, void* stream);

// The 8-wave 64-head kernel (prefill.hip): its shape and its launch.
KernelShape prefill_shape(int dqk, bool fp8);
int launch_prefill(const FwdParams& p, int dqk, bool fp8, void* stream);

// The 4-wave 64-head kernel for fp8 pools (prefill_fp8.hip).
KernelShape prefill_fp8_shape(int dqk);
int launch_prefill_fp8(const FwdParams& p, int dqk, void* stream);

// The 64-head kernel for fp8 pools with fp8 dots on two-term splits and LDS
// DMA tiles (prefill_mx.hip).
KernelShape prefill_mx_shape(int dqk);
int launch_prefill_mx(const FwdParams& p, int dqk, void* stream);

// The pool layouts prefill_mx.hip can address: rows through a structured
// buffer whose stride field holds at most 14 bits, pages a whole number of
// rows apart.
inline bool mx_pool_ok(int64_t rs_bytes, int64_t page_bytes) {
  return rs_bytes > 0 && rs_bytes < (1 << 14) && (page_bytes == 0 || page_bytes % rs_bytes == 0);
}

// True when the (head block, pool dtype, variant) instance addresses the pool
// through a buffer descriptor with 32-bit offsets (pools up to
// kMaxBufferBytes); the other instances use 64-bit addresses.
// The plan launches the 16-head fp8 decode kernel (decode.hip).
inline bool uses_decode_kernel(int head_block, bool fp8, int variant) {
  return head_block == 16 && fp8 && variant == 0;
}

// The plan launches a kernel that walks a second segment itself: the decode
// kernel (its walk splits at the segment boundary) or the 64-head kernel of
// prefill.hip over bf16 pools (the main segment padded to whole tiles).
inline bool walks_second_segment(int head_block, bool fp8, int variant) {
  return uses_decode_kernel(head_block, fp8, variant) ||
         (head_block == 64 && !fp8 && (variant == 0 || variant == 2)) ||
         (head_block == 64 && fp8 && variant == 3);
}

inline bool uses_buffer_range(int head_block, bool fp8, int variant) {
  return (head_block == 16 && fp8 && variant == 0) || (head_block == 64 && variant != 1);
}

// Pure host planner: no HIP calls. Returns SMLA_OK or an error status and
// fills `err` with the reason.
int make_plan(const Problem& pb, const smla_options* opt, int num_cus, smla_plan* plan,
              const char** err);

// Launches the attention kernel (and the combine kernel when splits > 1) on
// `stream`. Returns 0 or a hipError_t value.
int launch_forward(const FwdParams& p, const smla_plan& plan, int dqk, bool fp8, void* stream);

// The two halves of launch_forward: the attention kernel alone (it writes
// partials iff p.part_o is set), and the combine kernel over p.splits
// partials.
int launch_attention(const FwdParams& p, const smla_plan& plan, int dqk, bool fp8, void* stream);
int launch_combine(const FwdParams& p, void* stream);

}  // namespace smla
