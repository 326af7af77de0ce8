/*
 * sparse_mla.h - C ABI of the gfx950 sparse multi-head latent attention (MLA)
 * forward library (libsparse_mla.so).
 *
 * The operation. For query row r, head h and the row's K int32 slot indices
 * idx[r, 0..K) into a pool of shared latent KV rows (one row serves every
 * head, which is what makes it MLA):
 *
 *   s_j      = sm_scale * q[r,h,:D_qk] . K[idx[r,j], :D_qk]        valid j only
 *   out[r,h] = sum_j softmax(s)_j * V[idx[r,j]]       V = the row's first 512
 *   lse[r,h] = ln sum_j exp(s_j)
 *
 * A slot with a negative index is invalid and masked. A row with no valid
 * slot gives out = 0 and lse = -inf. Pool rows are 576 wide (512 latent + 64
 * rope) or 512 wide (rope-free), stored as bf16 or as float8_e4m3fn codes
 * with one fp32 per-tensor scale (value = code * scale, for K and V alike).
 * Sources: "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159),
 * Technical Details (row widths, cache formats, index counts) and the commit
 * notes on the 64-head program (rope dotted after the latent part), the
 * per-tensor fp8 route (per-tensor scale, V scale taken off in the epilogue),
 * the split-K reduce, and the sentinel slots of the walk.
 *
 * Conventions (after the status-code and dtype-code precedents of "aiter
 * PR 6563" (dense MLA decode planner notes: int status enum, ctypes packers
 * cast it) and "aiter PR 7183" (explicit fp8 dtype checks, is_supported)):
 *   - every entry point returns an int status (smla_status); nothing throws;
 *   - all tensors are caller-owned device memory described by smla_tensor;
 *     the library never frees caller memory;
 *   - arguments are validated on the host before any HIP call;
 *   - work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream); no host synchronisation and no device->host copy on the
 *     call path, except a one-time workspace growth (see sparse_mla_fwd_ex).
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_API __attribute__((visibility("default")))

/* Element type codes. One-byte storage alone does not say which fp8 flavour
 * it is, so the caller names it: only OCP float8_e4m3fn is accepted. */
typedef enum smla_dtype {
  SMLA_BF16 = 0,
  SMLA_FP8_E4M3FN = 1,
  SMLA_FP32 = 2,
  SMLA_INT32 = 3,
  SMLA_E8M0 = 4 /* one byte, a power of two 2^(code - 127); MX block scales */
} smla_dtype;

typedef enum smla_status {
  SMLA_OK = 0,
  SMLA_ERR_INVALID_ARG = 1, /* null pointer, bad rank/dtype/stride/shape mismatch */
  SMLA_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels cover */
  SMLA_ERR_HIP = 3          /* a HIP call or kernel launch failed */
} smla_status;

/* A strided tensor view of caller memory. Strides are in elements. Only the
 * first `ndim` entries of shape/stride are read. */
typedef struct smla_tensor {
  void* data;
  int32_t dtype; /* smla_dtype */
  int32_t ndim;
  int64_t shape[3];
  int64_t stride[3];
} smla_tensor;

/* Optional call parameters (planner overrides for tests and benchmarks, a
 * caller workspace, the scale of an fp8 q); zero-initialise for the defaults. */
typedef struct smla_options {
  int32_t head_block;      /* 0 = planner's choice, else 16, 32 or 64 heads per workgroup */
  int32_t splits;          /* 0 = planner's choice, else 1..64 splits of each row's slots */
  int32_t remap;           /* 0 = planner's choice, 1 = XCD-aware order, 2 = grid order */
  int32_t variant;         /* kernel instance; 0 = the planner's choice: the 16-head
                              decode kernel over fp8 pools (H <= 32), the staged-tile
                              kernel (16 and 32 heads over bf16 pools; 64 heads over
                              bf16 pools), for 64 heads over fp8 pools the fp8-dot
                              kernel (the 4-wave kernel where it cannot address the
                              pool).
                              1 = the staged-tile kernel (any head block; also what
                              pools past the 32-bit buffer range use). 2 = 64 heads
                              only: the 8-wave double-buffered kernel. 3 = 64 heads
                              over fp8 pools only: the fp8-dot kernel (both products
                              on the fp8 matrix cores over two-term e4m3 splits of q
                              and P); falls back to the 4-wave kernel where the pool's
                              row pitch does not fit its structured buffer. 4 = 64
                              heads over fp8 pools only: the 4-wave kernel (bf16 dots
                              on widened tiles), reported by the plan as variant 0 */
  void* workspace;         /* optional caller device buffer for split partials */
  int64_t workspace_bytes; /* its size; must be >= smla_plan.workspace_bytes when given */
  const void* q_scale;     /* fp32 [1] device pointer: per-tensor scale of a float8_e4m3fn q
                              (value = code * q_scale; NULL = 1). Must be NULL for a bf16 q */
  int32_t workgroups;      /* kernels that walk several work items per workgroup (the
                              fp8-dot kernel on rows that are not split): 0 = one
                              workgroup per compute unit of the device, else at most
                              this many (rounded down to a multiple of 8 when >= 8);
                              negative is an error. Results do not depend on it */
} smla_options;

/* What the planner picked for a call (sparse_mla_plan). */
typedef struct smla_plan {
  int32_t head_block;      /* heads per workgroup: 16, 32 or 64 */
  int32_t head_blocks;     /* ceil(H / head_block) */
  int32_t splits;          /* splits of each row's K slots (1 = no combine kernel) */
  int32_t remap;           /* 1 = XCD-aware work order, 0 = grid order */
  int32_t waves;           /* wavefronts per workgroup */
  int32_t lds_bytes;       /* LDS per workgroup */
  int32_t tiles_per_split; /* tiles walked by one workgroup */
  int32_t tile_slots;      /* slots per tile (16, 64 or 128) */
  int64_t grid;            /* workgroups of the attention kernel */
  int64_t workspace_bytes; /* split partials (0 when splits == 1) */
  int32_t variant;         /* kernel instance variant */
  int32_t reserved;
} smla_plan;

/*
 * sparse_mla_fwd - the forward pass.
 *
 *  q        bf16 [R, H, D_qk], or float8_e4m3fn codes with a per-tensor scale
 *           (smla_options.q_scale, through the _ex/2/_epi entry points), widened
 *           exactly to bf16 in the kernels with the scale applied to the scores
 *           (commit notes on the two-loop route: an fp8 q is widened in the
 *           kernel); last dim contiguous; base and strides 16-byte aligned.
 *  kv_pool  bf16 or fp8 e4m3fn [N, W], W >= D_qk (only the first D_qk columns
 *           are read, so a padded row pitch needs no copy); last dim
 *           contiguous; the row stride in bytes must be a multiple of 16 and
 *           the base 16-byte aligned. Or paged, [P, B, W] with B a power of
 *           two: slot index i is row i % B of page i / B, with the page pitch
 *           stride[0] (>= one page, a multiple of 16 bytes) free, so a pool
 *           whose pages are padded needs no copy either (commit notes on the
 *           two-loop route: the launcher keeps a padded [nb, block, R] pool
 *           paged). N = P * B.
 *  kv_scale fp32 [1] device pointer, given iff kv_pool is fp8 (NULL for bf16).
 *  indices  int32 [R, K]; last dim contiguous; any negative value is an
 *           invalid slot. Values >= N are a caller error: not checked on the
 *           device, the result is then undefined.
 *  sm_scale softmax scale applied to q.k.
 *  out      bf16 [R, H, 512]; last dim contiguous; base, row and head strides
 *           16-byte aligned; fully written.
 *  lse      fp32 [R, H]; fully written (natural log; -inf for empty rows).
 *
 * D_qk must be 576 or 512; H in [1, 1024]; K in [1, 2^20]; R >= 0 (R == 0 is
 * a no-op returning SMLA_OK); q, out and pool rows 16-byte aligned.
 * out and lse must not alias any input. The same inputs and the same plan give
 * bitwise-identical outputs.
 */
SMLA_API int sparse_mla_fwd(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
                   const smla_tensor* indices, float sm_scale, smla_tensor* out, smla_tensor* lse,
                   void* stream);

/*
 * sparse_mla_fwd_ex - sparse_mla_fwd with planner overrides and an optional
 * caller workspace (opt may be NULL). With splits > 1 the partial outputs go
 * to opt->workspace when given, else to a library-owned per-device buffer that
 * grows on demand (growth synchronises the device once; the buffer is kept
 * until process exit and is shared by calls on that device, so concurrent
 * split calls on different streams of one device must pass their own
 * workspace).
 */
SMLA_API int sparse_mla_fwd_ex(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
                      const smla_tensor* indices, float sm_scale, smla_tensor* out, smla_tensor* lse,
                      void* stream, const smla_options* opt);

/*
 * sparse_mla_fwd_noalloc - sparse_mla_fwd_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): it calls no hipMalloc, hipFree or allocating
 * library routine. Split partials go to a fixed device array of
 * SMLA_NOALLOC_SCRATCH_BYTES that each GPU holds from the first call on it
 * until the process ends. Every rule of sparse_mla_fwd_ex holds, except:
 *   - opt->workspace must be NULL and opt->workspace_bytes 0 (else
 *     SMLA_ERR_INVALID_ARG);
 *   - a plan whose partials (smla_plan.workspace_bytes) exceed
 *     SMLA_NOALLOC_SCRATCH_BYTES returns SMLA_ERR_UNSUPPORTED before any
 *     launch; force fewer splits (opt->splits) or use sparse_mla_fwd_ex.
 * All calls on one GPU share its array: calls whose work overlaps on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller. Nothing in the array needs to start at zero: each split writes its
 * partial output and LSE in full before the combine kernel reads them.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (32ll * 1024 * 1024)
SMLA_API int sparse_mla_fwd_noalloc(const smla_tensor* q, const smla_tensor* kv_pool,
                           const smla_tensor* kv_scale, const smla_tensor* indices,
                           float sm_scale, smla_tensor* out, smla_tensor* lse, void* stream,
                           const smla_options* opt);

/*
 * sparse_mla_fwd2 - two-segment forward, after "[Triton/Gluon] GFX950 sparse
 * mla optimizations" (aiter PR 6159), the commit notes on the per-tensor fp8
 * two-loop route: a row attends, under one softmax, to the valid slots of its
 * main indices (into kv_pool, scale kv_scale) and of its extra indices (into
 * extra_pool, scale extra_kv_scale), e.g. top-k slots of a compressed cache
 * plus a sliding window of a second cache. For row r and head h, with
 * K1 = kv_scale * codes (or bf16 values) and K2 likewise for the extra pool:
 *   s over { K1[i] : indices[r,j] = i >= 0 } and { K2[i] : extra_indices[r,j]
 *   = i >= 0 }, out = softmax(sm_scale * q . k) V, lse = ln sum exp(...).
 *
 *  extra_pool      same dtype as kv_pool, [N2, W2] with W2 >= D_qk, same
 *                  alignment rules; its own rows and row stride (2-D only).
 *  extra_kv_scale  fp32 [1] device pointer for an fp8 pool; NULL means the
 *                  extra segment uses kv_scale. Must be NULL for bf16 pools.
 *  extra_indices   int32 [R, K2], K2 in [1, 2^20]; negative = invalid slot.
 *                  NULL makes this sparse_mla_fwd_ex.
 *  opt             as for sparse_mla_fwd_ex; head_block, splits, remap and
 *                  variant apply to each segment's launch. The workspace
 *                  holds both segments' partials (sparse_mla_plan2 gives its
 *                  size); without one the library's per-device buffer is used.
 *
 * When the plan of the whole call (both segments' slots) launches the
 * 16-head fp8 decode kernel, that kernel walks the main slots and then the
 * extra ones, rebasing its accumulator from kv_scale onto extra_kv_scale
 * between them (acc *= kv_scale / extra_kv_scale, as the pages do); the
 * 64-head kernel over bf16 pools likewise walks the extra slots after the
 * main ones (no scale to rebase). The 64-head fp8-dot kernel (variant 3)
 * does so too when extra_pool's row pitch is below 16 KB (kv_pool may be
 * paged): it keeps its accumulator in units of the larger scale and weighs
 * each segment's slots by its scale over that one (kv_scale and
 * extra_kv_scale must then be nonnegative, as dequantisation scales are).
 * Otherwise
 * each segment's kernel writes normalised partials with its own scale and the
 * split-combine kernel merges them. All are exact in real arithmetic. Every
 * other rule is sparse_mla_fwd's; out and lse must not alias any input.
 */
SMLA_API int sparse_mla_fwd2(const smla_tensor* q, const smla_tensor* kv_pool,
                    const smla_tensor* kv_scale, const smla_tensor* indices,
                    const smla_tensor* extra_pool, const smla_tensor* extra_kv_scale,
                    const smla_tensor* extra_indices, float sm_scale, smla_tensor* out,
                    smla_tensor* lse, void* stream, const smla_options* opt);

/* The launches sparse_mla_fwd2 would make and the bytes of workspace they
 * need: each segment's plan, or, when one launch walks both segments, that
 * launch's plan in plan_main and grid 0 in plan_extra.
 * Host-only; makes no HIP call. */
SMLA_API int sparse_mla_plan2(const smla_tensor* q, const smla_tensor* kv_pool,
                     const smla_tensor* indices, const smla_tensor* extra_pool,
                     const smla_tensor* extra_indices, const smla_options* opt,
                     int32_t num_cus, smla_plan* plan_main, smla_plan* plan_extra,
                     int64_t* workspace_bytes);

/*
 * Output epilogue, after "[Triton/Gluon] GFX950 sparse mla optimizations"
 * (aiter PR 6159), the commit notes on the fused epilogue: before the output
 * projection a serving stack rotates the last 64 columns of each attention
 * output row back (inverse RoPE) and, for an MXFP8 projection, quantises the
 * row to float8_e4m3fn with one E8M0 scale per 32 columns. The store that
 * writes the output does both (the attention kernel's, or the split-combine
 * kernel's when the plan splits).
 *
 * Arithmetic, for row r and head h: the output row is rounded to bf16 first;
 * with positions, pair j = 0..31 of columns (448 + 2j, 449 + 2j) = (x, y) and
 * c = cos_sin[pos[r], j], s = cos_sin[pos[r], 32 + j] becomes
 * (x*c + y*s, y*c - x*s), every product and sum rounded to fp32 on its own.
 * Then either a bf16 store (round to nearest even) or MXFP8: per 32-column
 * block, scale code e = clamp(floor(log2(max |v|)) - 8 + 127, 0, 254) (code 0
 * for an all-zero block), codes = e4m3fn(v / 2^(e - 127)) rounded to nearest
 * even, saturated at +-448, sign kept. The fused result is bit-identical to
 * running sparse_mla_out_epilogue on the bf16 output of the same call.
 *
 *  rope_positions  int32 [R] or NULL (no rotation). Positions outside
 *                  [0, P) are a caller error: the kernels clamp them into
 *                  range so no read leaves the cache.
 *  rope_cos_sin    fp32 [P, 64], last dim contiguous, 4-byte aligned; given
 *                  iff rope_positions is.
 *  out_scale       E8M0 [R, H, 16] or NULL. Given: `out` holds the
 *                  float8_e4m3fn codes [R, H, 512] (MXFP8); NULL: `out` is
 *                  bf16 [R, H, 512]. Base, row and head strides of an MXFP8
 *                  `out` must be multiples of 16 bytes.
 * Every epilogue tensor is caller-owned device memory; none may alias out,
 * out_scale or lse.
 */
typedef struct smla_epilogue {
  const smla_tensor* rope_positions;
  const smla_tensor* rope_cos_sin;
  smla_tensor* out_scale;
} smla_epilogue;

/*
 * sparse_mla_fwd_epi - the forward with its output epilogue: sparse_mla_fwd2
 * (extra_* may be NULL for one segment) whose final store applies `epi`
 * (NULL or an epilogue with nothing set: a plain bf16 store). Every other
 * rule is sparse_mla_fwd2's.
 */
SMLA_API int sparse_mla_fwd_epi(const smla_tensor* q, const smla_tensor* kv_pool,
                       const smla_tensor* kv_scale, const smla_tensor* indices,
                       const smla_tensor* extra_pool, const smla_tensor* extra_kv_scale,
                       const smla_tensor* extra_indices, float sm_scale,
                       const smla_epilogue* epi, smla_tensor* out, smla_tensor* lse,
                       void* stream, const smla_options* opt);

/*
 * sparse_mla_out_epilogue - the epilogue as a pass of its own over bf16 rows
 * [R, H, 512] (e.g. a forward's output): the separate pass that the fused
 * store replaces. rows: bf16, last dim contiguous, base and strides 16-byte
 * aligned; epi must not be NULL; out as for sparse_mla_fwd_epi and must not
 * alias rows. R * H == 0 is a no-op.
 */
SMLA_API int sparse_mla_out_epilogue(const smla_tensor* rows, const smla_epilogue* epi,
                            smla_tensor* out, void* stream);

/*
 * Indexer (the stage that produces the index rows the forward consumes),
 * after "[HIP] [JIT] fp8_mqa_logits: v35w gfx950 prefill indexer logits
 * kernel" (aiter PR 7183), Motivation:
 *
 *   logits[m, n] = sum_h relu(q[m,h,:] . k[n,:]) * w[m,h] * kv_scale[n]
 *                  for n in [ks[m], ke[m]) (clipped to [0, N)), -inf elsewhere
 *
 * sparse_mla_indexer_logits
 *  q        float8_e4m3fn [M, 32, 128] (the indexer's 32 heads x 128 dims);
 *           last dim contiguous, base and strides multiples of 16 bytes.
 *  k        float8_e4m3fn [N, 128], N <= 2^27; base and row stride multiples
 *           of 16 bytes.
 *  kv_scale fp32 [N], contiguous: each key's dequantisation scale.
 *  w        fp32 [M, 32], last dim contiguous, base 16-byte aligned, row
 *           stride a multiple of 4: the per-(row, head) weights.
 *  ks, ke   int32 [M], contiguous: each row's window [ks, ke).
 *  clean    1: positions outside a row's window are written -inf; 0: only
 *           the window is written (the rest of the row is left as it was).
 *  logits   fp32 [M, N], last dim contiguous; must not alias an input.
 * Products and dots are formed by fp8 MFMA with fp32 accumulation; relu, the
 * head weights and the head sum in fp32, then the key scale.
 *
 * sparse_mla_indexer_topk - per row, the indices of the k largest logits
 * inside [ks, ke) (clipped to [0, N)), ascending, ties at the k-th value to
 * the lower index, -1 after the window's keys when it holds fewer than k
 * (the pages describe no selection; this is the plainest reading). Only the
 * window is read, so the rest of a row may hold anything.
 *  logits   fp32 [R, N], N < 2^31, last dim contiguous.
 *  ks, ke   int32 [R].
 *  k        1 .. 65536.
 *  indices  int32 [R, k], last dim contiguous; must not alias an input. An
 *           index row the forward can take directly (negative = invalid).
 */
SMLA_API int sparse_mla_indexer_logits(const smla_tensor* q, const smla_tensor* k,
                              const smla_tensor* kv_scale, const smla_tensor* w,
                              const smla_tensor* ks, const smla_tensor* ke, int32_t clean,
                              smla_tensor* logits, void* stream);
SMLA_API int sparse_mla_indexer_topk(const smla_tensor* logits, const smla_tensor* ks,
                            const smla_tensor* ke, int32_t k, smla_tensor* indices,
                            void* stream);

/* 1 if the shapes/dtypes/strides are covered by the kernels, else 0 (the
 * reason is left in sparse_mla_last_error). Host-only; makes no HIP call. */
SMLA_API int sparse_mla_is_supported(const smla_tensor* q, const smla_tensor* kv_pool,
                            const smla_tensor* indices);

/* The launch the forward would make for these shapes (opt may be NULL).
 * Host-only; makes no HIP call. Returns a status. `num_cus` is the compute
 * unit count to plan for (0 = 256, an MI355X). */
SMLA_API int sparse_mla_plan(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* indices,
                    const smla_options* opt, int32_t num_cus, smla_plan* plan_out);

/* Work-order map used by the attention kernel: the work item that workgroup
 * `pid` of a `grid`-workgroup launch processes, with the XCD-aware order
 * (remap = 1) or grid order (remap = 0). Host-side copy of the device map,
 * exported so the order can be checked without a GPU. Returns -1 on bad input. */
SMLA_API int64_t sparse_mla_work_of(int64_t pid, int64_t grid, int32_t remap);

/* Bytes of the library-owned split workspace currently held for `device`
 * (0 before the first split call there; -1 for a device id outside
 * [0, 64)). Host-only; makes no HIP call. */
SMLA_API int64_t sparse_mla_workspace_bytes(int32_t device);

/* Thread-local text for the last non-OK status of the calling thread. */
SMLA_API const char* sparse_mla_last_error(void);

/* Library version, "major.minor.patch". */
SMLA_API const char* sparse_mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
