// C ABI of libsparse_mla.so: argument validation (host only, before any HIP
// call), planning, workspace management and launch. See include/sparse_mla.h
// for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.h"
#include "work_order.h"

namespace smla {
namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

const char* dtype_name(int32_t d) {
  switch (d) {
    case SMLA_BF16: return "bf16";
    case SMLA_FP8_E4M3FN: return "fp8_e4m3fn";
    case SMLA_FP32: return "fp32";
    case SMLA_INT32: return "int32";
    case SMLA_E8M0: return "e8m0";
    default: return "unknown";
  }
}

int elem_size(int32_t d) {
  switch (d) {
    case SMLA_BF16: return 2;
    case SMLA_FP8_E4M3FN: return 1;
    case SMLA_FP32: return 4;
    case SMLA_INT32: return 4;
    case SMLA_E8M0: return 1;
    default: return 0;
  }
}

// Structural checks shared by every tensor argument.
int check_tensor(const smla_tensor* t, const char* name, int ndim, int32_t dtype) {
  if (!t) return fail(SMLA_ERR_INVALID_ARG, std::string(name) + ": null descriptor");
  if (t->ndim != ndim)
    return fail(SMLA_ERR_INVALID_ARG, std::string(name) + ": expected " + std::to_string(ndim) +
                                          " dims, got " + std::to_string(t->ndim));
  if (t->dtype != dtype)
    return fail(SMLA_ERR_UNSUPPORTED, std::string(name) + ": dtype " + dtype_name(t->dtype) +
                                          " (code " + std::to_string(t->dtype) +
                                          ") not supported, expected " + dtype_name(dtype));
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0)
      return fail(SMLA_ERR_INVALID_ARG, std::string(name) + ": negative extent");
    if (t->stride[i] < 0)
      return fail(SMLA_ERR_INVALID_ARG, std::string(name) + ": negative stride");
  }
  if (t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1)
    return fail(SMLA_ERR_UNSUPPORTED, std::string(name) + ": last dimension must be contiguous");
  return SMLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) touched by a strided tensor (empty if any extent is 0).
void extent(const smla_tensor* t, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = 0;
  for (int i = 0; i < t->ndim; ++i) {
    if (t->shape[i] == 0) {
      *lo = *hi = 0;
      return;
    }
    last += (t->shape[i] - 1) * t->stride[i];
  }
  *lo = reinterpret_cast<uintptr_t>(t->data);
  *hi = *lo + uintptr_t((last + 1) * elem_size(t->dtype));
}

bool overlap(const smla_tensor* a, const smla_tensor* b) {
  uintptr_t alo, ahi, blo, bhi;
  extent(a, &alo, &ahi);
  extent(b, &blo, &bhi);
  if (alo == ahi || blo == bhi) return false;
  return alo < bhi && blo < ahi;
}

struct Checked {
  Problem pb;
  bool fp8;
  bool q_fp8;
};

// q / kv_pool / indices: shapes, dtypes, strides, alignment.
int validate_inputs(const smla_tensor* q, const smla_tensor* kv, const smla_tensor* idx,
                    Checked* c) {
  int s;
  if (!q) return fail(SMLA_ERR_INVALID_ARG, "q: null descriptor");
  if (q->dtype != SMLA_BF16 && q->dtype != SMLA_FP8_E4M3FN)
    return fail(SMLA_ERR_UNSUPPORTED, std::string("q: dtype ") + dtype_name(q->dtype) +
                                          " (code " + std::to_string(q->dtype) +
                                          ") not supported, expected bf16 or fp8_e4m3fn");
  if ((s = check_tensor(q, "q", 3, q->dtype))) return s;
  if (!kv) return fail(SMLA_ERR_INVALID_ARG, "kv_pool: null descriptor");
  if (kv->dtype != SMLA_BF16 && kv->dtype != SMLA_FP8_E4M3FN)
    return fail(SMLA_ERR_UNSUPPORTED, std::string("kv_pool: dtype ") + dtype_name(kv->dtype) +
                                          " (code " + std::to_string(kv->dtype) +
                                          ") not supported, expected bf16 or fp8_e4m3fn");
  // [N, W], or paged [pages, page rows, W] with its own page pitch
  const bool paged = kv->ndim == 3;
  if ((s = check_tensor(kv, "kv_pool", paged ? 3 : 2, kv->dtype))) return s;
  if ((s = check_tensor(idx, "indices", 2, SMLA_INT32))) return s;
  const int64_t page_rows = paged ? kv->shape[1] : 1;
  const int64_t N = paged ? kv->shape[0] * kv->shape[1] : kv->shape[0];
  const int64_t W = paged ? kv->shape[2] : kv->shape[1];
  const int64_t rs = paged ? kv->stride[1] : kv->stride[0];  // row stride (elements)

  const int64_t R = q->shape[0], H = q->shape[1], D = q->shape[2];
  if (D != 576 && D != 512)
    return fail(SMLA_ERR_UNSUPPORTED, "q: D_qk must be 576 or 512, got " + std::to_string(D));
  if (H < 1 || H > kMaxHeads)
    return fail(SMLA_ERR_UNSUPPORTED, "q: heads must be in [1, 1024], got " + std::to_string(H));
  if (idx->shape[0] != R)
    return fail(SMLA_ERR_INVALID_ARG, "indices: rows " + std::to_string(idx->shape[0]) +
                                          " != q rows " + std::to_string(R));
  const int64_t K = idx->shape[1];
  if (K < 1 || K > kMaxTopk)
    return fail(SMLA_ERR_UNSUPPORTED, "indices: top-k must be in [1, 2^20], got " +
                                          std::to_string(K));
  if (W < D)
    return fail(SMLA_ERR_INVALID_ARG, "kv_pool: row width " + std::to_string(W) +
                                          " < D_qk " + std::to_string(D));
  if (R > 0 && N < 1) return fail(SMLA_ERR_INVALID_ARG, "kv_pool: no rows");
  if (paged && (page_rows < 1 || (page_rows & (page_rows - 1)) != 0))
    return fail(SMLA_ERR_UNSUPPORTED, "kv_pool: rows per page must be a power of two");
  if (R > 0) {
    if (!q->data) return fail(SMLA_ERR_INVALID_ARG, "q: null data");
    if (!kv->data) return fail(SMLA_ERR_INVALID_ARG, "kv_pool: null data");
    if (!idx->data) return fail(SMLA_ERR_INVALID_ARG, "indices: null data");
  }
  const int eb = elem_size(kv->dtype);
  if (page_rows > 1 || !paged) {
    if ((paged ? page_rows : N) > 1 && rs < W)
      return fail(SMLA_ERR_INVALID_ARG, "kv_pool: row stride smaller than row width");
    if ((rs * eb) % 16 != 0)
      return fail(SMLA_ERR_UNSUPPORTED, "kv_pool: base and row stride must be 16-byte aligned");
  }
  if (paged && kv->shape[0] > 1) {
    if (kv->stride[0] < page_rows * (page_rows > 1 ? rs : W))
      return fail(SMLA_ERR_INVALID_ARG, "kv_pool: page pitch smaller than a page");
    if ((kv->stride[0] * eb) % 16 != 0)
      return fail(SMLA_ERR_UNSUPPORTED, "kv_pool: page pitch must be 16-byte aligned");
  }
  if (!aligned16(kv->data))
    return fail(SMLA_ERR_UNSUPPORTED, "kv_pool: base and row stride must be 16-byte aligned");
  const int qb = elem_size(q->dtype);
  if (!aligned16(q->data) || (q->stride[0] * qb) % 16 != 0 || (q->stride[1] * qb) % 16 != 0)
    return fail(SMLA_ERR_UNSUPPORTED, "q: base, row and head strides must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(idx->data) & 3u) != 0)
    return fail(SMLA_ERR_INVALID_ARG, "indices: base must be 4-byte aligned");
  if (N > (int64_t(1) << 31)) return fail(SMLA_ERR_UNSUPPORTED, "kv_pool: more than 2^31 rows");
  c->pb.rows = R;
  c->pb.heads = int32_t(H);
  c->pb.dqk = int32_t(D);
  c->pb.topk = int32_t(K);
  c->pb.kv_fp8 = kv->dtype == SMLA_FP8_E4M3FN;
  c->pb.pool_rs_bytes = rs * eb;
  c->pb.page_bytes = paged ? kv->stride[0] * eb : 0;
  c->fp8 = c->pb.kv_fp8 != 0;
  c->q_fp8 = q->dtype == SMLA_FP8_E4M3FN;
  // bytes from the base to the end of the last row read
  if (N == 0)
    c->pb.pool_bytes = 0;
  else if (paged)
    c->pb.pool_bytes = ((kv->shape[0] - 1) * kv->stride[0] + (page_rows - 1) * rs + D) * eb;
  else
    c->pb.pool_bytes = ((N - 1) * rs + D) * eb;
  return SMLA_OK;
}

// out is bf16, or float8_e4m3fn codes for an MXFP8 epilogue (out_dtype).
int validate_all(const smla_tensor* q, const smla_tensor* kv, const smla_tensor* scale,
                 const smla_tensor* idx, float sm_scale, const smla_tensor* out,
                 const smla_tensor* lse, Checked* c, int32_t out_dtype = SMLA_BF16) {
  int s;
  if ((s = validate_inputs(q, kv, idx, c))) return s;
  const int64_t R = c->pb.rows, H = c->pb.heads;
  if (c->fp8) {
    if (!scale || !scale->data)
      return fail(SMLA_ERR_INVALID_ARG, "kv_scale: required for an fp8 pool");
    if ((s = check_tensor(scale, "kv_scale", 1, SMLA_FP32))) return s;
    if (scale->shape[0] < 1) return fail(SMLA_ERR_INVALID_ARG, "kv_scale: empty");
  } else if (scale && scale->data) {
    return fail(SMLA_ERR_INVALID_ARG, "kv_scale: must be NULL for a bf16 pool");
  }
  if (!std::isfinite(sm_scale)) return fail(SMLA_ERR_INVALID_ARG, "sm_scale: not finite");
  if ((s = check_tensor(out, "out", 3, out_dtype))) return s;
  if ((s = check_tensor(lse, "lse", 2, SMLA_FP32))) return s;
  if (out->shape[0] != R || out->shape[1] != H || out->shape[2] != kDv)
    return fail(SMLA_ERR_INVALID_ARG, "out: shape must be [R, H, 512]");
  if (lse->shape[0] != R || lse->shape[1] != H)
    return fail(SMLA_ERR_INVALID_ARG, "lse: shape must be [R, H]");
  if (R > 0) {
    if (!out->data) return fail(SMLA_ERR_INVALID_ARG, "out: null data");
    if (!lse->data) return fail(SMLA_ERR_INVALID_ARG, "lse: null data");
    const int ob = elem_size(out_dtype);
    if (!aligned16(out->data) || (out->stride[0] * ob) % 16 != 0 || (out->stride[1] * ob) % 16 != 0)
      return fail(SMLA_ERR_UNSUPPORTED, "out: base, row and head strides must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse->data) & 3u) != 0)
      return fail(SMLA_ERR_INVALID_ARG, "lse: base must be 4-byte aligned");
    const smla_tensor* ins[4] = {q, kv, idx, c->fp8 ? scale : nullptr};
    for (const smla_tensor* in : ins) {
      if (!in) continue;
      if (overlap(out, in) || overlap(lse, in))
        return fail(SMLA_ERR_INVALID_ARG, "out/lse must not alias an input");
    }
    if (overlap(out, lse)) return fail(SMLA_ERR_INVALID_ARG, "out and lse overlap");
  }
  return SMLA_OK;
}

// Library-owned split workspace, one per device, grown on demand. Growth
// synchronises the device before releasing the old buffer, so no in-flight
// kernel still reads it.
struct Workspace {
  void* ptr = nullptr;
  int64_t bytes = 0;
};
std::mutex g_ws_mutex;
Workspace g_ws[kMaxDevices];

int device_workspace(int dev, int64_t need, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(SMLA_ERR_UNSUPPORTED, "device id beyond 63");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[dev];
  if (w.bytes < need) {
    hipError_t e;
    // At least double, so a run of growing requests reallocates O(log) times.
    const int64_t grow = std::max<int64_t>(need, 2 * w.bytes);
    if (w.ptr) {
      if ((e = hipDeviceSynchronize()) != hipSuccess)
        return fail(SMLA_ERR_HIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(e));
      if ((e = hipFree(w.ptr)) != hipSuccess)
        return fail(SMLA_ERR_HIP, std::string("hipFree: ") + hipGetErrorString(e));
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if ((e = hipMalloc(&w.ptr, size_t(grow))) != hipSuccess) {
      w.ptr = nullptr;
      return fail(SMLA_ERR_HIP, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
    }
    w.bytes = grow;
  }
  *out = w.ptr;
  return SMLA_OK;
}

int g_cu_count[kMaxDevices] = {0};

int device_cus(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

// The per-tensor scale of an fp8 q (options): NULL means 1; a bf16 q takes
// none.
int check_q_scale(const Checked& c, const smla_options* opt) {
  const void* qs = opt ? opt->q_scale : nullptr;
  if (qs && !c.q_fp8) return fail(SMLA_ERR_INVALID_ARG, "q_scale: must be NULL for a bf16 q");
  if (qs && (reinterpret_cast<uintptr_t>(qs) & 3u))
    return fail(SMLA_ERR_INVALID_ARG, "q_scale: must be 4-byte aligned");
  return SMLA_OK;
}

// dtype of `out` under an epilogue: e4m3fn codes with an MXFP8 scale tensor,
// else bf16.
int32_t epi_out_dtype(const smla_epilogue* epi) {
  return (epi && epi->out_scale) ? SMLA_FP8_E4M3FN : SMLA_BF16;
}

// Checks the epilogue tensors of an R x H output (out already checked) and
// fills the kernels' view of them; `ins` are the call's inputs, which the
// epilogue's outputs must not alias.
int validate_epilogue(const smla_epilogue* epi, int64_t R, int64_t H, smla_tensor* out,
                      const smla_tensor* lse, const smla_tensor* const* ins, int n_ins,
                      EpiOut* e) {
  *e = EpiOut{};
  e->out = static_cast<uint16_t*>(out->data);
  e->out_rs = out->stride[0];
  e->out_hs = out->stride[1];
  if (!epi) return SMLA_OK;
  int s;
  const smla_tensor* pos = epi->rope_positions;
  const smla_tensor* cs = epi->rope_cos_sin;
  smla_tensor* sc = epi->out_scale;
  if (pos) {
    if ((s = check_tensor(pos, "rope_positions", 1, SMLA_INT32))) return s;
    if (pos->shape[0] != R) return fail(SMLA_ERR_INVALID_ARG, "rope_positions: shape must be [R]");
    if (!cs) return fail(SMLA_ERR_INVALID_ARG, "rope_cos_sin: required with rope_positions");
    if ((s = check_tensor(cs, "rope_cos_sin", 2, SMLA_FP32))) return s;
    if (cs->shape[1] != 64) return fail(SMLA_ERR_UNSUPPORTED, "rope_cos_sin: shape must be [P, 64]");
    if (cs->shape[0] < 1 || cs->shape[0] > INT32_MAX)
      return fail(SMLA_ERR_INVALID_ARG, "rope_cos_sin: P must be in [1, 2^31)");
    if (cs->shape[0] > 1 && cs->stride[0] < 64)
      return fail(SMLA_ERR_INVALID_ARG, "rope_cos_sin: row stride smaller than 64");
    if (R > 0) {
      if (!pos->data || !cs->data) return fail(SMLA_ERR_INVALID_ARG, "rope: null data");
      if ((reinterpret_cast<uintptr_t>(pos->data) & 3u) || (reinterpret_cast<uintptr_t>(cs->data) & 3u))
        return fail(SMLA_ERR_INVALID_ARG, "rope: base must be 4-byte aligned");
    }
    e->pos = static_cast<const int32_t*>(pos->data);
    e->cs = static_cast<const float*>(cs->data);
    e->cs_rs = cs->stride[0];
    e->cs_rows = int32_t(cs->shape[0]);
  } else if (cs) {
    return fail(SMLA_ERR_INVALID_ARG, "rope_cos_sin: given without rope_positions");
  }
  if (sc) {
    if ((s = check_tensor(sc, "out_scale", 3, SMLA_E8M0))) return s;
    if (sc->shape[0] != R || sc->shape[1] != H || sc->shape[2] != kDv / 32)
      return fail(SMLA_ERR_INVALID_ARG, "out_scale: shape must be [R, H, 16]");
    if (R > 0 && !sc->data) return fail(SMLA_ERR_INVALID_ARG, "out_scale: null data");
    e->out = nullptr;
    e->q8 = static_cast<uint8_t*>(out->data);
    e->sc = static_cast<uint8_t*>(sc->data);
    e->sc_rs = sc->stride[0];
    e->sc_hs = sc->stride[1];
  }
  if (R > 0 && H > 0) {
    const smla_tensor* outs[3] = {out, sc, lse};
    for (const smla_tensor* o : outs) {
      if (!o) continue;
      for (int i = 0; i < n_ins; ++i)
        if (ins[i] && overlap(o, ins[i]))
          return fail(SMLA_ERR_INVALID_ARG, "outputs must not alias an input");
      if (o != out && overlap(o, out)) return fail(SMLA_ERR_INVALID_ARG, "out_scale/lse overlap out");
      if (pos && (overlap(o, pos) || overlap(o, cs)))
        return fail(SMLA_ERR_INVALID_ARG, "outputs must not alias the rope tensors");
    }
    if (sc && lse && overlap(sc, lse)) return fail(SMLA_ERR_INVALID_ARG, "out_scale and lse overlap");
  }
  return SMLA_OK;
}

// Kernel parameters of one segment: q/out/lse of the call, pool/scale/indices
// of the segment, its plan's launch shape.
FwdParams segment_params(const smla_tensor* q, const smla_tensor* pool, const float* scale,
                         const smla_tensor* idx, const Checked& c, const smla_plan& plan,
                         float sm_scale, smla_tensor* out, smla_tensor* lse,
                         const smla_options* opt) {
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q->data);
  p.q_rs = q->stride[0];
  p.q_hs = q->stride[1];
  p.pool = static_cast<const uint8_t*>(pool->data);
  const int eb = elem_size(pool->dtype);
  if (pool->ndim == 3) {  // paged: slot i is row i % page_rows of page i / page_rows
    int shift = 0;
    while ((int64_t(1) << shift) < pool->shape[1]) ++shift;
    p.pool_rs_bytes = pool->stride[1] * eb;
    p.page_shift = shift;
    p.page_mask = uint32_t(pool->shape[1] - 1);
    p.page_bytes = pool->stride[0] * eb;
  } else {
    p.pool_rs_bytes = pool->stride[0] * eb;
    p.page_shift = 31;
    p.page_mask = 0x7fffffffu;
    p.page_bytes = 0;
  }
  p.pool_bytes = uint32_t(std::min<int64_t>(c.pb.pool_bytes, kMaxBufferBytes));
  p.kv_scale = c.fp8 ? scale : nullptr;
  p.idx = static_cast<const int32_t*>(idx->data);
  p.idx_rs = idx->stride[0];
  p.out = static_cast<uint16_t*>(out->data);
  p.out_rs = out->stride[0];
  p.out_hs = out->stride[1];
  p.lse = static_cast<float*>(lse->data);
  p.lse_rs = lse->stride[0];
  p.lse_hs = lse->stride[1];
  p.rows = c.pb.rows;
  p.heads = c.pb.heads;
  p.topk = c.pb.topk;
  p.splits = plan.splits;
  p.tiles_per_split = plan.tiles_per_split;
  p.head_blocks = plan.head_blocks;
  p.remap = plan.remap;
  p.grid = plan.grid;
  int dev = 0;
  p.persist_cap = opt && opt->workgroups > 0
                      ? opt->workgroups
                      : (hipGetDevice(&dev) == hipSuccess ? device_cus(dev) : 0);
  p.q_scale = opt ? static_cast<const float*>(opt->q_scale) : nullptr;
  p.sm_log2 = sm_scale * 1.4426950408889634f;
  p.q_fp8 = c.q_fp8 ? 1 : 0;
  return p;
}

// Bytes of split partials for `splits` partial results of R x H rows: the
// fp32 outputs, then (256-byte aligned) the fp32 LSEs.
int64_t partial_bytes(int64_t splits, int64_t rows, int64_t heads, int64_t* lse_offset) {
  const int64_t o_bytes = splits * rows * heads * kDv * 4;
  const int64_t off = (o_bytes + 255) / 256 * 256;
  if (lse_offset) *lse_offset = off;
  return off + splits * rows * heads * 4;
}

// The caller's workspace when given (checked), else the device's own.
int get_workspace(int dev, const smla_options* opt, int64_t need, void** ws) {
  if (opt && opt->workspace) {
    if (opt->workspace_bytes < need)
      return fail(SMLA_ERR_INVALID_ARG,
                  "workspace smaller than the plan needs (" + std::to_string(need) + " bytes)");
    if (!aligned16(opt->workspace)) return fail(SMLA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    *ws = opt->workspace;
    return SMLA_OK;
  }
  return device_workspace(dev, need, ws);
}

// Validation of the extra segment of a two-segment call: same q, same pool
// dtype; for fp8 its own scale or, when none is given, the main one.
int validate_extra(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
                   const smla_tensor* extra_pool, const smla_tensor* extra_scale,
                   const smla_tensor* extra_idx, const smla_tensor* out, const smla_tensor* lse,
                   Checked* c2, const float** scale2) {
  int s;
  if ((s = validate_inputs(q, extra_pool, extra_idx, c2)))
    return fail(s, "extra segment: " + g_last_error);
  if (extra_pool->dtype != kv_pool->dtype)
    return fail(SMLA_ERR_UNSUPPORTED, "extra_pool: dtype must match kv_pool");
  if (extra_pool->ndim != 2)
    return fail(SMLA_ERR_UNSUPPORTED, "extra_pool: must be 2-D (only the main pool may be paged)");
  *scale2 = nullptr;
  if (c2->fp8) {
    if (extra_scale && extra_scale->data) {
      if ((s = check_tensor(extra_scale, "extra_kv_scale", 1, SMLA_FP32))) return s;
      if (extra_scale->shape[0] < 1) return fail(SMLA_ERR_INVALID_ARG, "extra_kv_scale: empty");
      *scale2 = static_cast<const float*>(extra_scale->data);
    } else {
      *scale2 = static_cast<const float*>(kv_scale->data);
    }
  } else if (extra_scale && extra_scale->data) {
    return fail(SMLA_ERR_INVALID_ARG, "extra_kv_scale: must be NULL for a bf16 pool");
  }
  if (c2->pb.rows > 0) {
    const smla_tensor* ins[3] = {extra_pool, extra_idx,
                                 (c2->fp8 && extra_scale && extra_scale->data) ? extra_scale : nullptr};
    for (const smla_tensor* in : ins) {
      if (!in) continue;
      if (overlap(out, in) || overlap(lse, in))
        return fail(SMLA_ERR_INVALID_ARG, "out/lse must not alias an input");
    }
  }
  return SMLA_OK;
}

// Plans of a two-segment call and their workspace. When the plan of the
// combined problem (both segments' slots, the larger pool range) launches a
// kernel that walks a second segment (the 16-head fp8 decode kernel, the
// 64-head bf16 kernel, the 64-head fp8-dot kernel when the second pool's
// row pitch fits its structured buffer), that kernel walks both segments
// in one launch: *p1 is that plan and *p2 has grid 0. Otherwise each segment
// gets its own plan and the workspace holds both segments' partials for the
// combine kernel.
int plan_two(const Checked& c1, const Checked& c2, const smla_options* opt, int num_cus,
             smla_plan* p1, smla_plan* p2, int64_t* ws_bytes) {
  const char* perr = nullptr;
  int s;
  Problem tot = c1.pb;
  tot.topk = c1.pb.topk + c2.pb.topk;
  tot.pool_bytes = std::max(c1.pb.pool_bytes, c2.pb.pool_bytes);
  if ((s = make_plan(tot, opt, num_cus, p1, &perr))) return fail(s, perr);
  // 64 heads over bf16 pools: unless the caller chose a kernel, the 8-wave
  // kernel, which walks both segments in one launch (the one-segment
  // default, the staged-tile kernel, would need two launches and a combine).
  smla_options o2 = opt ? *opt : smla_options{};
  if (p1->head_block == 64 && !c1.fp8 && o2.variant == 0) {
    o2.variant = 2;
    opt = &o2;
    if ((s = make_plan(tot, opt, num_cus, p1, &perr))) return fail(s, perr);
  }
  bool one = walks_second_segment(p1->head_block, c1.fp8, p1->variant);
  if (one && p1->variant == 3) one = mx_pool_ok(c2.pb.pool_rs_bytes, 0);
  if (one) {
    if (!uses_decode_kernel(p1->head_block, c1.fp8, p1->variant)) {
      // Tiled walk: the second segment starts at a whole tile.
      const int tile = std::max(1, p1->tile_slots);
      tot.topk = (c1.pb.topk + tile - 1) / tile * tile + c2.pb.topk;
      if ((s = make_plan(tot, opt, num_cus, p1, &perr))) return fail(s, perr);
    }
    *p2 = smla_plan{};
    *ws_bytes = p1->splits > 1 ? partial_bytes(p1->splits, c1.pb.rows, c1.pb.heads, nullptr) : 0;
    return SMLA_OK;
  }
  if ((s = make_plan(c1.pb, opt, num_cus, p1, &perr))) return fail(s, perr);
  if ((s = make_plan(c2.pb, opt, num_cus, p2, &perr))) return fail(s, perr);
  *ws_bytes = partial_bytes(int64_t(p1->splits) + p2->splits, c1.pb.rows, c1.pb.heads, nullptr);
  return SMLA_OK;
}

// One-segment forward with an optional output epilogue. With `noalloc` the
// split partials go to the fixed device scratch (noalloc.hip) and nothing is
// allocated; a plan whose partials do not fit it is rejected.
int fwd_one(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
            const smla_tensor* indices, float sm_scale, const smla_epilogue* epi,
            smla_tensor* out, smla_tensor* lse, void* stream, const smla_options* opt,
            bool noalloc = false) {
  Checked c;
  int s = validate_all(q, kv_pool, kv_scale, indices, sm_scale, out, lse, &c, epi_out_dtype(epi));
  if (s) return s;
  if ((s = check_q_scale(c, opt))) return s;
  EpiOut eo;
  const smla_tensor* ins[4] = {q, kv_pool, indices, c.fp8 ? kv_scale : nullptr};
  if ((s = validate_epilogue(epi, c.pb.rows, c.pb.heads, out, lse, ins, 4, &eo))) return s;
  if (c.pb.rows == 0) return SMLA_OK;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  smla_plan plan;
  const char* perr = nullptr;
  if ((s = make_plan(c.pb, opt, device_cus(dev), &plan, &perr))) return fail(s, perr);

  FwdParams p = segment_params(q, kv_pool, c.fp8 ? static_cast<const float*>(kv_scale->data) : nullptr,
                               indices, c, plan, sm_scale, out, lse, opt);
  p.epi = eo;
  p.q_scale = opt ? static_cast<const float*>(opt->q_scale) : nullptr;
  if (plan.splits > 1) {
    void* ws = nullptr;
    int64_t lse_off = 0;
    const int64_t need = std::max(partial_bytes(plan.splits, c.pb.rows, c.pb.heads, &lse_off),
                                  plan.workspace_bytes);
    if (noalloc) {
      if (need > kScratchBytes)
        return fail(SMLA_ERR_UNSUPPORTED,
                    "split partials need " + std::to_string(need) +
                        " bytes, more than the no-allocation scratch (" +
                        std::to_string(kScratchBytes) +
                        " bytes): force fewer splits or use sparse_mla_fwd_ex");
      std::string err;
      if ((s = scratch_buffer(dev, &ws, &err))) return fail(s, err);
    } else if ((s = get_workspace(dev, opt, need, &ws))) {
      return s;
    }
    p.part_o = static_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_off);
  }
  const int le = launch_forward(p, plan, c.pb.dqk, c.fp8, stream);
  if (le != 0)
    return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                  hipGetErrorString(static_cast<hipError_t>(le)));
  return SMLA_OK;
}

// Two-segment forward (extra_indices NULL: one segment) with an optional
// output epilogue.
int fwd_two(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
            const smla_tensor* indices, const smla_tensor* extra_pool,
            const smla_tensor* extra_kv_scale, const smla_tensor* extra_indices, float sm_scale,
            const smla_epilogue* epi, smla_tensor* out, smla_tensor* lse, void* stream,
            const smla_options* opt) {
  if (!extra_indices)
    return fwd_one(q, kv_pool, kv_scale, indices, sm_scale, epi, out, lse, stream, opt);
  Checked c1, c2;
  int s = validate_all(q, kv_pool, kv_scale, indices, sm_scale, out, lse, &c1, epi_out_dtype(epi));
  if (s) return s;
  if ((s = check_q_scale(c1, opt))) return s;
  const float* scale2 = nullptr;
  if ((s = validate_extra(q, kv_pool, kv_scale, extra_pool, extra_kv_scale, extra_indices, out, lse,
                          &c2, &scale2)))
    return s;
  EpiOut eo;
  const smla_tensor* ins[7] = {q, kv_pool, indices, c1.fp8 ? kv_scale : nullptr, extra_pool,
                               extra_indices, c1.fp8 ? extra_kv_scale : nullptr};
  if ((s = validate_epilogue(epi, c1.pb.rows, c1.pb.heads, out, lse, ins, 7, &eo))) return s;
  if (c1.pb.rows == 0) return SMLA_OK;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SMLA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  smla_plan plan1, plan2;
  int64_t need = 0;
  if ((s = plan_two(c1, c2, opt, device_cus(dev), &plan1, &plan2, &need))) return s;
  if (plan2.grid == 0) {
    // One launch walks both segments (the combine kernel follows only when
    // the plan splits).
    FwdParams p = segment_params(q, kv_pool,
                                 c1.fp8 ? static_cast<const float*>(kv_scale->data) : nullptr,
                                 indices, c1, plan1, sm_scale, out, lse, opt);
    p.epi = eo;
    p.q_scale = opt ? static_cast<const float*>(opt->q_scale) : nullptr;
    p.pool2 = static_cast<const uint8_t*>(extra_pool->data);
    p.pool2_rs_bytes = extra_pool->stride[0] * elem_size(extra_pool->dtype);
    p.pool2_bytes = uint32_t(std::min<int64_t>(c2.pb.pool_bytes, kMaxBufferBytes));
    p.kv_scale2 = scale2;
    p.idx2 = static_cast<const int32_t*>(extra_indices->data);
    p.idx2_rs = extra_indices->stride[0];
    p.topk2 = c2.pb.topk;
    if (plan1.splits > 1) {
      void* ws = nullptr;
      int64_t lse_off = 0;
      partial_bytes(plan1.splits, c1.pb.rows, c1.pb.heads, &lse_off);
      if ((s = get_workspace(dev, opt, need, &ws))) return s;
      p.part_o = static_cast<float*>(ws);
      p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_off);
    }
    const int le = launch_forward(p, plan1, c1.pb.dqk, c1.fp8, stream);
    if (le != 0)
      return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                    hipGetErrorString(static_cast<hipError_t>(le)));
    return SMLA_OK;
  }
  void* ws = nullptr;
  if ((s = get_workspace(dev, opt, need, &ws))) return s;
  const int64_t S = int64_t(plan1.splits) + plan2.splits;
  int64_t lse_off = 0;
  partial_bytes(S, c1.pb.rows, c1.pb.heads, &lse_off);
  float* part_o = static_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_off);
  const int64_t per_split = c1.pb.rows * c1.pb.heads;

  // Each segment writes its normalised partials with its own scale folded in;
  // the combine kernel's LSE-weighted merge is then the softmax over the
  // union of both segments' slots.
  FwdParams p1 = segment_params(q, kv_pool, c1.fp8 ? static_cast<const float*>(kv_scale->data) : nullptr,
                                indices, c1, plan1, sm_scale, out, lse, opt);
  p1.part_o = part_o;
  p1.part_lse = part_lse;
  FwdParams p2 = segment_params(q, extra_pool, scale2, extra_indices, c2, plan2, sm_scale, out, lse,
                                opt);
  p1.q_scale = p2.q_scale = opt ? static_cast<const float*>(opt->q_scale) : nullptr;
  p2.part_o = part_o + int64_t(plan1.splits) * per_split * kDv;
  p2.part_lse = part_lse + int64_t(plan1.splits) * per_split;
  FwdParams pc = p1;
  pc.splits = int32_t(S);
  pc.epi = eo;
  int le = launch_attention(p1, plan1, c1.pb.dqk, c1.fp8, stream);
  if (le == 0) le = launch_attention(p2, plan2, c2.pb.dqk, c2.fp8, stream);
  if (le == 0) le = launch_combine(pc, stream);
  if (le != 0)
    return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                  hipGetErrorString(static_cast<hipError_t>(le)));
  return SMLA_OK;
}

}  // namespace
}  // namespace smla

using namespace smla;

extern "C" {

int sparse_mla_fwd_ex(const smla_tensor* q, const smla_tensor* kv_pool,
                      const smla_tensor* kv_scale, const smla_tensor* indices, float sm_scale,
                      smla_tensor* out, smla_tensor* lse, void* stream,
                      const smla_options* opt) {
  return fwd_one(q, kv_pool, kv_scale, indices, sm_scale, nullptr, out, lse, stream, opt);
}

int sparse_mla_fwd_noalloc(const smla_tensor* q, const smla_tensor* kv_pool,
                           const smla_tensor* kv_scale, const smla_tensor* indices,
                           float sm_scale, smla_tensor* out, smla_tensor* lse, void* stream,
                           const smla_options* opt) {
  if (opt && (opt->workspace || opt->workspace_bytes))
    return fail(SMLA_ERR_INVALID_ARG,
                "workspace: must be NULL/0 (this entry point uses the library's fixed scratch)");
  return fwd_one(q, kv_pool, kv_scale, indices, sm_scale, nullptr, out, lse, stream, opt, true);
}

int sparse_mla_fwd2(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
                    const smla_tensor* indices, const smla_tensor* extra_pool,
                    const smla_tensor* extra_kv_scale, const smla_tensor* extra_indices,
                    float sm_scale, smla_tensor* out, smla_tensor* lse, void* stream,
                    const smla_options* opt) {
  return fwd_two(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices,
                 sm_scale, nullptr, out, lse, stream, opt);
}

int sparse_mla_fwd_epi(const smla_tensor* q, const smla_tensor* kv_pool,
                       const smla_tensor* kv_scale, const smla_tensor* indices,
                       const smla_tensor* extra_pool, const smla_tensor* extra_kv_scale,
                       const smla_tensor* extra_indices, float sm_scale,
                       const smla_epilogue* epi, smla_tensor* out, smla_tensor* lse,
                       void* stream, const smla_options* opt) {
  return fwd_two(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices,
                 sm_scale, epi, out, lse, stream, opt);
}

int sparse_mla_out_epilogue(const smla_tensor* rows, const smla_epilogue* epi, smla_tensor* out,
                            void* stream) {
  int s;
  if (!epi) return fail(SMLA_ERR_INVALID_ARG, "epi: null");
  if ((s = check_tensor(rows, "rows", 3, SMLA_BF16))) return s;
  const int64_t R = rows->shape[0], H = rows->shape[1];
  if (rows->shape[2] != kDv) return fail(SMLA_ERR_INVALID_ARG, "rows: shape must be [R, H, 512]");
  const int32_t od = epi_out_dtype(epi);
  if ((s = check_tensor(out, "out", 3, od))) return s;
  if (out->shape[0] != R || out->shape[1] != H || out->shape[2] != kDv)
    return fail(SMLA_ERR_INVALID_ARG, "out: shape must be [R, H, 512]");
  if (R * H > (int64_t(1) << 31))
    return fail(SMLA_ERR_UNSUPPORTED, "rows: more than 2^31 rows x heads");
  if (R * H > 0) {
    if (!rows->data || !out->data) return fail(SMLA_ERR_INVALID_ARG, "rows/out: null data");
    if (!aligned16(rows->data) || (rows->stride[0] * 2) % 16 != 0 || (rows->stride[1] * 2) % 16 != 0)
      return fail(SMLA_ERR_UNSUPPORTED, "rows: base, row and head strides must be 16-byte aligned");
    const int ob = elem_size(od);
    if (!aligned16(out->data) || (out->stride[0] * ob) % 16 != 0 || (out->stride[1] * ob) % 16 != 0)
      return fail(SMLA_ERR_UNSUPPORTED, "out: base, row and head strides must be 16-byte aligned");
  }
  EpiPassParams p{};
  const smla_tensor* ins[1] = {rows};
  if ((s = validate_epilogue(epi, R, H, out, nullptr, ins, 1, &p.epi))) return s;
  if (R * H == 0) return SMLA_OK;
  p.in = static_cast<const uint16_t*>(rows->data);
  p.in_rs = rows->stride[0];
  p.in_hs = rows->stride[1];
  p.rows = R;
  p.heads = int32_t(H);
  const int le = launch_out_epilogue(p, stream);
  if (le != 0)
    return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                  hipGetErrorString(static_cast<hipError_t>(le)));
  return SMLA_OK;
}

int sparse_mla_indexer_logits(const smla_tensor* q, const smla_tensor* k,
                              const smla_tensor* kv_scale, const smla_tensor* w,
                              const smla_tensor* ks, const smla_tensor* ke, int32_t clean,
                              smla_tensor* logits, void* stream) {
  int s;
  if ((s = check_tensor(q, "q", 3, SMLA_FP8_E4M3FN))) return s;
  if ((s = check_tensor(k, "k", 2, SMLA_FP8_E4M3FN))) return s;
  if ((s = check_tensor(kv_scale, "kv_scale", 1, SMLA_FP32))) return s;
  if ((s = check_tensor(w, "w", 2, SMLA_FP32))) return s;
  if ((s = check_tensor(ks, "ks", 1, SMLA_INT32))) return s;
  if ((s = check_tensor(ke, "ke", 1, SMLA_INT32))) return s;
  if ((s = check_tensor(logits, "logits", 2, SMLA_FP32))) return s;
  const int64_t M = q->shape[0], N = k->shape[0];
  if (q->shape[1] != kIxHeads || q->shape[2] != kIxDim)
    return fail(SMLA_ERR_UNSUPPORTED, "q: the indexer takes 32 heads of 128 dims");
  if (k->shape[1] != kIxDim) return fail(SMLA_ERR_UNSUPPORTED, "k: rows must be 128 wide");
  if (kv_scale->shape[0] != N) return fail(SMLA_ERR_INVALID_ARG, "kv_scale: shape must be [N]");
  if (w->shape[0] != M || w->shape[1] != kIxHeads)
    return fail(SMLA_ERR_INVALID_ARG, "w: shape must be [M, 32]");
  if (ks->shape[0] != M || ke->shape[0] != M)
    return fail(SMLA_ERR_INVALID_ARG, "ks/ke: shape must be [M]");
  if (logits->shape[0] != M || logits->shape[1] != N)
    return fail(SMLA_ERR_INVALID_ARG, "logits: shape must be [M, N]");
  if (N > (int64_t(1) << 27)) return fail(SMLA_ERR_UNSUPPORTED, "k: more than 2^27 keys");
  if (clean != 0 && clean != 1) return fail(SMLA_ERR_INVALID_ARG, "clean must be 0 or 1");
  if (M == 0 || N == 0) return SMLA_OK;
  const smla_tensor* all[7] = {q, k, kv_scale, w, ks, ke, logits};
  for (const smla_tensor* t : all)
    if (!t->data) return fail(SMLA_ERR_INVALID_ARG, "null data");
  if (!aligned16(q->data) || q->stride[0] % 16 != 0 || q->stride[1] % 16 != 0)
    return fail(SMLA_ERR_UNSUPPORTED, "q: base, row and head strides must be 16-byte aligned");
  if (!aligned16(k->data) || (N > 1 && k->stride[0] % 16 != 0))
    return fail(SMLA_ERR_UNSUPPORTED, "k: base and row stride must be 16-byte aligned");
  if (!aligned16(w->data) || (M > 1 && w->stride[0] % 4 != 0))
    return fail(SMLA_ERR_UNSUPPORTED, "w: base 16-byte aligned, row stride a multiple of 4");
  const smla_tensor* vecs[3] = {kv_scale, ks, ke};
  for (const smla_tensor* t : vecs)
    if ((reinterpret_cast<uintptr_t>(t->data) & 3u) != 0)
      return fail(SMLA_ERR_INVALID_ARG, "kv_scale/ks/ke: base must be 4-byte aligned");
  if ((reinterpret_cast<uintptr_t>(logits->data) & 3u) != 0)
    return fail(SMLA_ERR_INVALID_ARG, "logits: base must be 4-byte aligned");
  for (int i = 0; i < 6; ++i)
    if (overlap(logits, all[i])) return fail(SMLA_ERR_INVALID_ARG, "logits must not alias an input");
  IxParams p{};
  p.q = static_cast<const uint8_t*>(q->data);
  p.q_rs = q->stride[0];
  p.q_hs = q->stride[1];
  p.k = static_cast<const uint8_t*>(k->data);
  p.k_rs = k->stride[0];
  p.kv_scale = static_cast<const float*>(kv_scale->data);
  p.w = static_cast<const float*>(w->data);
  p.w_rs = w->stride[0];
  p.ks = static_cast<const int32_t*>(ks->data);
  p.ke = static_cast<const int32_t*>(ke->data);
  p.logits = static_cast<float*>(logits->data);
  p.l_rs = logits->stride[0];
  p.m = M;
  p.n = int32_t(N);
  p.clean = clean;
  const int le = launch_ix_logits(p, stream);
  if (le != 0)
    return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                  hipGetErrorString(static_cast<hipError_t>(le)));
  return SMLA_OK;
}

int sparse_mla_indexer_topk(const smla_tensor* logits, const smla_tensor* ks,
                            const smla_tensor* ke, int32_t k, smla_tensor* indices,
                            void* stream) {
  int s;
  if ((s = check_tensor(logits, "logits", 2, SMLA_FP32))) return s;
  if ((s = check_tensor(ks, "ks", 1, SMLA_INT32))) return s;
  if ((s = check_tensor(ke, "ke", 1, SMLA_INT32))) return s;
  if ((s = check_tensor(indices, "indices", 2, SMLA_INT32))) return s;
  const int64_t R = logits->shape[0], N = logits->shape[1];
  if (k < 1 || k > 65536) return fail(SMLA_ERR_UNSUPPORTED, "k must be in [1, 65536]");
  if (ks->shape[0] != R || ke->shape[0] != R)
    return fail(SMLA_ERR_INVALID_ARG, "ks/ke: shape must be [R]");
  if (indices->shape[0] != R || indices->shape[1] != k)
    return fail(SMLA_ERR_INVALID_ARG, "indices: shape must be [R, k]");
  if (N >= (int64_t(1) << 31)) return fail(SMLA_ERR_UNSUPPORTED, "logits: 2^31 or more keys");
  if (R > (int64_t(1) << 31)) return fail(SMLA_ERR_UNSUPPORTED, "logits: more than 2^31 rows");
  if (R == 0) return SMLA_OK;
  const smla_tensor* all[4] = {logits, ks, ke, indices};
  for (const smla_tensor* t : all) {
    if (!t->data) return fail(SMLA_ERR_INVALID_ARG, "null data");
    if ((reinterpret_cast<uintptr_t>(t->data) & 3u) != 0)
      return fail(SMLA_ERR_INVALID_ARG, "base must be 4-byte aligned");
  }
  for (int i = 0; i < 3; ++i)
    if (overlap(indices, all[i])) return fail(SMLA_ERR_INVALID_ARG, "indices must not alias an input");
  TopkParams p{};
  p.logits = static_cast<const float*>(logits->data);
  p.l_rs = logits->stride[0];
  p.ks = static_cast<const int32_t*>(ks->data);
  p.ke = static_cast<const int32_t*>(ke->data);
  p.out = static_cast<int32_t*>(indices->data);
  p.o_rs = indices->stride[0];
  p.rows = R;
  p.n = int32_t(N);
  p.k = k;
  const int le = launch_topk(p, stream);
  if (le != 0)
    return fail(SMLA_ERR_HIP, std::string("kernel launch: ") +
                                  hipGetErrorString(static_cast<hipError_t>(le)));
  return SMLA_OK;
}

int sparse_mla_plan2(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* indices,
                     const smla_tensor* extra_pool, const smla_tensor* extra_indices,
                     const smla_options* opt, int32_t num_cus, smla_plan* plan_main,
                     smla_plan* plan_extra, int64_t* workspace_bytes) {
  if (!plan_main || !plan_extra || !workspace_bytes)
    return fail(SMLA_ERR_INVALID_ARG, "plan2: null output");
  Checked c1, c2;
  int s = validate_inputs(q, kv_pool, indices, &c1);
  if (s) return s;
  if ((s = validate_inputs(q, extra_pool, extra_indices, &c2))) return s;
  if (extra_pool->dtype != kv_pool->dtype)
    return fail(SMLA_ERR_UNSUPPORTED, "extra_pool: dtype must match kv_pool");
  if (extra_pool->ndim != 2)
    return fail(SMLA_ERR_UNSUPPORTED, "extra_pool: must be 2-D (only the main pool may be paged)");
  return plan_two(c1, c2, opt, num_cus, plan_main, plan_extra, workspace_bytes);
}

int sparse_mla_fwd(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* kv_scale,
                   const smla_tensor* indices, float sm_scale, smla_tensor* out, smla_tensor* lse,
                   void* stream) {
  return sparse_mla_fwd_ex(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream, nullptr);
}

int sparse_mla_is_supported(const smla_tensor* q, const smla_tensor* kv_pool,
                            const smla_tensor* indices) {
  Checked c;
  return validate_inputs(q, kv_pool, indices, &c) == SMLA_OK ? 1 : 0;
}

int sparse_mla_plan(const smla_tensor* q, const smla_tensor* kv_pool, const smla_tensor* indices,
                    const smla_options* opt, int32_t num_cus, smla_plan* plan_out) {
  if (!plan_out) return fail(SMLA_ERR_INVALID_ARG, "plan_out: null");
  Checked c;
  int s = validate_inputs(q, kv_pool, indices, &c);
  if (s) return s;
  const char* perr = nullptr;
  s = make_plan(c.pb, opt, num_cus, plan_out, &perr);
  return s ? fail(s, perr) : SMLA_OK;
}

int64_t sparse_mla_work_of(int64_t pid, int64_t grid, int32_t remap) {
  if (grid <= 0 || pid < 0 || pid >= grid) return -1;
  return remap ? smla_xcd_work(pid, grid) : pid;
}

int64_t sparse_mla_workspace_bytes(int32_t device) {
  if (device < 0 || device >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  return g_ws[device].bytes;
}

const char* sparse_mla_last_error(void) { return g_last_error.c_str(); }

const char* sparse_mla_version(void) { return "0.1.0"; }

}  // extern "C"
