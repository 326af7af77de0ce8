"""ctypes binding of libsparse_mla.so (include/sparse_mla.h).

Argument marshalling only: torch tensors are turned into smla_tensor
descriptors (data pointer, dtype code, shape, strides) and the current torch
stream is passed through. Every step of the forward pass runs in the library's
HIP kernels; there is no fallback. If the library is missing, ``load()``
raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_mla.so")

SMLA_BF16, SMLA_FP8_E4M3FN, SMLA_FP32, SMLA_INT32, SMLA_E8M0 = 0, 1, 2, 3, 4
SMLA_OK, SMLA_ERR_INVALID_ARG, SMLA_ERR_UNSUPPORTED, SMLA_ERR_HIP = 0, 1, 2, 3
STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_INVALID_ARG", 2: "SMLA_ERR_UNSUPPORTED", 3: "SMLA_ERR_HIP"}
UNKNOWN_DTYPE = 1000  # any dtype the library does not know (e.g. float8_e4m3fnuz)

EXPORTED = (
    "sparse_mla_fwd", "sparse_mla_fwd_ex", "sparse_mla_fwd_noalloc", "sparse_mla_fwd2",
    "sparse_mla_fwd_epi", "sparse_mla_workspace_bytes",
    "sparse_mla_out_epilogue", "sparse_mla_is_supported", "sparse_mla_plan", "sparse_mla_plan2",
    "sparse_mla_work_of", "sparse_mla_last_error", "sparse_mla_version",
    "sparse_mla_indexer_logits", "sparse_mla_indexer_topk",
)


class SmlaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


class SmlaOptions(ctypes.Structure):
    _fields_ = [("head_block", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("remap", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("q_scale", ctypes.c_void_p), ("workgroups", ctypes.c_int32)]


class SmlaPlan(ctypes.Structure):
    _fields_ = [("head_block", ctypes.c_int32), ("head_blocks", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("remap", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("tiles_per_split", ctypes.c_int32),
                ("tile_slots", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("variant", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class SmlaEpilogue(ctypes.Structure):
    _fields_ = [("rope_positions", ctypes.POINTER(SmlaTensor)),
                ("rope_cos_sin", ctypes.POINTER(SmlaTensor)),
                ("out_scale", ctypes.POINTER(SmlaTensor))]


class SparseMLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library once and declare its signatures."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m sparse_mla_attention_05_amd.build`")
    lib = ctypes.CDLL(p)
    T = ctypes.POINTER(SmlaTensor)
    lib.sparse_mla_fwd.argtypes = [T, T, T, T, ctypes.c_float, T, T, ctypes.c_void_p]
    lib.sparse_mla_fwd.restype = ctypes.c_int
    lib.sparse_mla_fwd_ex.argtypes = [T, T, T, T, ctypes.c_float, T, T, ctypes.c_void_p,
                                      ctypes.POINTER(SmlaOptions)]
    lib.sparse_mla_fwd_ex.restype = ctypes.c_int
    lib.sparse_mla_fwd_noalloc.argtypes = [T, T, T, T, ctypes.c_float, T, T, ctypes.c_void_p,
                                           ctypes.POINTER(SmlaOptions)]
    lib.sparse_mla_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_mla_workspace_bytes.argtypes = [ctypes.c_int32]
    lib.sparse_mla_workspace_bytes.restype = ctypes.c_int64
    lib.sparse_mla_fwd2.argtypes = [T, T, T, T, T, T, T, ctypes.c_float, T, T, ctypes.c_void_p,
                                    ctypes.POINTER(SmlaOptions)]
    lib.sparse_mla_fwd2.restype = ctypes.c_int
    E = ctypes.POINTER(SmlaEpilogue)
    lib.sparse_mla_fwd_epi.argtypes = [T, T, T, T, T, T, T, ctypes.c_float, E, T, T,
                                       ctypes.c_void_p, ctypes.POINTER(SmlaOptions)]
    lib.sparse_mla_fwd_epi.restype = ctypes.c_int
    lib.sparse_mla_out_epilogue.argtypes = [T, E, T, ctypes.c_void_p]
    lib.sparse_mla_out_epilogue.restype = ctypes.c_int
    lib.sparse_mla_indexer_logits.argtypes = [T, T, T, T, T, T, ctypes.c_int32, T, ctypes.c_void_p]
    lib.sparse_mla_indexer_logits.restype = ctypes.c_int
    lib.sparse_mla_indexer_topk.argtypes = [T, T, T, ctypes.c_int32, T, ctypes.c_void_p]
    lib.sparse_mla_indexer_topk.restype = ctypes.c_int
    lib.sparse_mla_plan2.argtypes = [T, T, T, T, T, ctypes.POINTER(SmlaOptions), ctypes.c_int32,
                                     ctypes.POINTER(SmlaPlan), ctypes.POINTER(SmlaPlan),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.sparse_mla_plan2.restype = ctypes.c_int
    lib.sparse_mla_is_supported.argtypes = [T, T, T]
    lib.sparse_mla_is_supported.restype = ctypes.c_int
    lib.sparse_mla_plan.argtypes = [T, T, T, ctypes.POINTER(SmlaOptions), ctypes.c_int32,
                                    ctypes.POINTER(SmlaPlan)]
    lib.sparse_mla_plan.restype = ctypes.c_int
    lib.sparse_mla_work_of.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    lib.sparse_mla_work_of.restype = ctypes.c_int64
    lib.sparse_mla_last_error.argtypes = []
    lib.sparse_mla_last_error.restype = ctypes.c_char_p
    lib.sparse_mla_version.argtypes = []
    lib.sparse_mla_version.restype = ctypes.c_char_p
    if path is None:
        _LIB = lib
    return lib


def dtype_code(dtype) -> int:
    import torch
    return {torch.bfloat16: SMLA_BF16, torch.float8_e4m3fn: SMLA_FP8_E4M3FN,
            torch.float32: SMLA_FP32, torch.int32: SMLA_INT32,
            torch.float8_e8m0fnu: SMLA_E8M0}.get(dtype, UNKNOWN_DTYPE)


def describe(t) -> SmlaTensor | None:
    """smla_tensor view of a torch tensor (None stays None)."""
    if t is None:
        return None
    if t.dim() > 3:
        raise ValueError("at most 3 dims")
    d = SmlaTensor()
    d.data = t.data_ptr() if t.numel() > 0 or t.data_ptr() else None
    d.dtype = dtype_code(t.dtype)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(d):
    return ctypes.byref(d) if d is not None else None


def _stream_handle(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if any(t is not None and t.is_cuda for t in tensors):
        return torch.cuda.current_stream(tensors[0].device).cuda_stream
    return None


def last_error() -> str:
    return load().sparse_mla_last_error().decode()


def version() -> str:
    return load().sparse_mla_version().decode()


def _check(status: int):
    if status != SMLA_OK:
        raise SparseMLAError(status, last_error())


def _options(head_block=0, splits=0, remap=0, workspace=None, workspace_bytes=None, variant=0,
             q_scale=None, workgroups=0):
    o = SmlaOptions()
    o.head_block, o.splits, o.remap, o.variant = head_block, splits, remap, variant
    o.workgroups = workgroups
    if q_scale is not None:
        o.q_scale = q_scale.data_ptr()
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size() \
            if workspace_bytes is None else workspace_bytes
    return o


def sparse_mla_fwd(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream=None) -> None:
    """out[R,H,512] (bf16) and lse[R,H] (fp32) <- sparse MLA forward; raises on error."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, out, lse)]
    st = _stream_handle(stream, q, out)
    _check(lib.sparse_mla_fwd(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), _ptr(ds[3]),
                              float(sm_scale), _ptr(ds[4]), _ptr(ds[5]), st))


def sparse_mla_fwd_ex(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream=None,
                      head_block=0, splits=0, remap=0, workspace=None, workspace_bytes=None,
                      variant=0, q_scale=None,
                      workgroups=0) -> None:
    """sparse_mla_fwd with planner overrides (head_block 16/32/64, splits,
    remap 1 = XCD-aware / 2 = grid order, kernel variant) and an optional
    caller workspace."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, out, lse)]
    opt = _options(head_block, splits, remap, workspace, workspace_bytes, variant, q_scale,
                   workgroups)
    st = _stream_handle(stream, q, out)
    _check(lib.sparse_mla_fwd_ex(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), _ptr(ds[3]),
                                 float(sm_scale), _ptr(ds[4]), _ptr(ds[5]), st, ctypes.byref(opt)))


def sparse_mla_fwd_noalloc(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream=None,
                           head_block=0, splits=0, remap=0, variant=0, q_scale=None,
                           workgroups=0) -> None:
    """sparse_mla_fwd_ex without any device allocation: split partials go to
    the library's fixed per-device scratch (SMLA_NOALLOC_SCRATCH_BYTES)."""
    _check(status_of_fwd_noalloc(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream,
                                 head_block, splits, remap, variant, q_scale,
                                 workgroups=workgroups))


def status_of_fwd_noalloc(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream=None,
                          head_block=0, splits=0, remap=0, variant=0, q_scale=None,
                          workspace=None, workspace_bytes=None, workgroups=0) -> int:
    """Raw status of sparse_mla_fwd_noalloc (a workspace may be passed only to
    test its rejection)."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, out, lse)]
    opt = _options(head_block, splits, remap, workspace, workspace_bytes, variant, q_scale,
                   workgroups)
    st = _stream_handle(stream, q, out)
    return lib.sparse_mla_fwd_noalloc(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), _ptr(ds[3]),
                                      float(sm_scale), _ptr(ds[4]), _ptr(ds[5]), st,
                                      ctypes.byref(opt))


def workspace_bytes(device: int = 0) -> int:
    """Bytes of the library-owned split workspace held for `device`."""
    return int(load().sparse_mla_workspace_bytes(int(device)))


def status_of_fwd(q, kv_pool, kv_scale, indices, sm_scale, out, lse, stream=None) -> int:
    """Raw status of sparse_mla_fwd (for tests of the error paths)."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, out, lse)]
    return lib.sparse_mla_fwd(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), _ptr(ds[3]),
                              float(sm_scale), _ptr(ds[4]), _ptr(ds[5]), stream)


def status_of_fwd2(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices,
                   sm_scale, out, lse, stream=None) -> int:
    """Raw status of sparse_mla_fwd2 with no options (for tests of the error paths)."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale,
                                extra_indices, out, lse)]
    return lib.sparse_mla_fwd2(*[_ptr(d) for d in ds[:7]], float(sm_scale), _ptr(ds[7]),
                               _ptr(ds[8]), stream, None)


def sparse_mla_is_supported(q, kv_pool, indices) -> bool:
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, indices)]
    return bool(lib.sparse_mla_is_supported(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2])))


def sparse_mla_plan(q, kv_pool, indices, head_block=0, splits=0, remap=0, num_cus=0,
                    variant=0, workgroups=0) -> dict:
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, indices)]
    opt = _options(head_block, splits, remap, variant=variant, workgroups=workgroups)
    plan = SmlaPlan()
    _check(lib.sparse_mla_plan(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), ctypes.byref(opt),
                               int(num_cus), ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in SmlaPlan._fields_ if name != "reserved"}


def sparse_mla_fwd2(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices,
                    sm_scale, out, lse, stream=None, head_block=0, splits=0, remap=0,
                    workspace=None, workspace_bytes=None, variant=0, q_scale=None,
                    workgroups=0) -> None:
    """Two-segment forward: one softmax over the valid slots of `indices` into
    kv_pool (scale kv_scale) and of `extra_indices` into extra_pool (scale
    extra_kv_scale, or kv_scale when None for fp8 pools)."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale,
                                extra_indices, out, lse)]
    opt = _options(head_block, splits, remap, workspace, workspace_bytes, variant, q_scale,
                   workgroups)
    st = _stream_handle(stream, q, out)
    _check(lib.sparse_mla_fwd2(*[_ptr(d) for d in ds[:7]], float(sm_scale), _ptr(ds[7]),
                               _ptr(ds[8]), st, ctypes.byref(opt)))


def sparse_mla_plan2(q, kv_pool, indices, extra_pool, extra_indices, head_block=0, splits=0,
                     remap=0, num_cus=0, variant=0) -> tuple[dict, dict, int]:
    """Plans of both segments of sparse_mla_fwd2 and its workspace bytes."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, indices, extra_pool, extra_indices)]
    opt = _options(head_block, splits, remap, variant=variant)
    p1, p2, ws = SmlaPlan(), SmlaPlan(), ctypes.c_int64(0)
    _check(lib.sparse_mla_plan2(*[_ptr(d) for d in ds], ctypes.byref(opt), int(num_cus),
                                ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(ws)))
    as_dict = lambda pl: {n: getattr(pl, n) for n, _ in SmlaPlan._fields_ if n != "reserved"}
    return as_dict(p1), as_dict(p2), int(ws.value)


def sparse_mla_work_of(pid: int, grid: int, remap: int) -> int:
    return int(load().sparse_mla_work_of(pid, grid, remap))


def forward(q, kv_pool, kv_scale, indices, sm_scale, **options):
    """Allocate out/lse on q's device and run the forward (options go to _ex)."""
    import torch
    R, H = q.shape[0], q.shape[1]
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((R, H), dtype=torch.float32, device=q.device)
    if options:
        sparse_mla_fwd_ex(q, kv_pool, kv_scale, indices, sm_scale, out, lse, **options)
    else:
        sparse_mla_fwd(q, kv_pool, kv_scale, indices, sm_scale, out, lse)
    return out, lse


def forward2(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices, sm_scale,
             **options):
    """Allocate out/lse on q's device and run the two-segment forward."""
    import torch
    R, H = q.shape[0], q.shape[1]
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((R, H), dtype=torch.float32, device=q.device)
    sparse_mla_fwd2(q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale, extra_indices,
                    sm_scale, out, lse, **options)
    return out, lse


def _epilogue(rope_positions=None, rope_cos_sin=None, out_scale=None):
    """smla_epilogue and the descriptors it points at (kept alive together)."""
    ds = [describe(t) for t in (rope_positions, rope_cos_sin, out_scale)]
    epi = SmlaEpilogue()
    epi.rope_positions = ctypes.pointer(ds[0]) if ds[0] is not None else None
    epi.rope_cos_sin = ctypes.pointer(ds[1]) if ds[1] is not None else None
    epi.out_scale = ctypes.pointer(ds[2]) if ds[2] is not None else None
    return epi, ds


def sparse_mla_fwd_epi(q, kv_pool, kv_scale, indices, sm_scale, out, lse, rope_positions=None,
                       rope_cos_sin=None, out_scale=None, extra_pool=None, extra_kv_scale=None,
                       extra_indices=None, stream=None, head_block=0, splits=0, remap=0,
                       workspace=None, workspace_bytes=None, variant=0, q_scale=None,
                       workgroups=0) -> None:
    """Forward whose final store applies the output epilogue: inverse RoPE of
    columns 448..511 (rope_positions int32 [R], rope_cos_sin fp32 [P, 64]) and,
    with out_scale (float8_e8m0fnu [R, H, 16]), an MXFP8 store of float8_e4m3fn
    codes into out; else out is bf16."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, extra_pool, extra_kv_scale,
                                extra_indices, out, lse)]
    epi, _keep = _epilogue(rope_positions, rope_cos_sin, out_scale)
    opt = _options(head_block, splits, remap, workspace, workspace_bytes, variant, q_scale,
                   workgroups)
    st = _stream_handle(stream, q, out)
    _check(lib.sparse_mla_fwd_epi(*[_ptr(d) for d in ds[:7]], float(sm_scale), ctypes.byref(epi),
                                  _ptr(ds[7]), _ptr(ds[8]), st, ctypes.byref(opt)))


def sparse_mla_out_epilogue(rows, out, rope_positions=None, rope_cos_sin=None, out_scale=None,
                            stream=None) -> None:
    """The output epilogue as a pass of its own over bf16 rows [R, H, 512]."""
    lib = load()
    dr, do = describe(rows), describe(out)
    epi, _keep = _epilogue(rope_positions, rope_cos_sin, out_scale)
    st = _stream_handle(stream, rows, out)
    _check(lib.sparse_mla_out_epilogue(_ptr(dr), ctypes.byref(epi), _ptr(do), st))


def status_of_fwd_epi(q, kv_pool, kv_scale, indices, sm_scale, out, lse, rope_positions=None,
                      rope_cos_sin=None, out_scale=None, stream=None) -> int:
    """Raw status of sparse_mla_fwd_epi with one segment and no options (for
    tests of the error paths)."""
    lib = load()
    ds = [describe(t) for t in (q, kv_pool, kv_scale, indices, out, lse)]
    epi, _keep = _epilogue(rope_positions, rope_cos_sin, out_scale)
    return lib.sparse_mla_fwd_epi(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), _ptr(ds[3]), None, None,
                                  None, float(sm_scale), ctypes.byref(epi), _ptr(ds[4]),
                                  _ptr(ds[5]), stream, None)


def status_of_out_epilogue(rows, out, rope_positions=None, rope_cos_sin=None, out_scale=None,
                           stream=None) -> int:
    lib = load()
    dr, do = describe(rows), describe(out)
    epi, _keep = _epilogue(rope_positions, rope_cos_sin, out_scale)
    return lib.sparse_mla_out_epilogue(_ptr(dr), ctypes.byref(epi), _ptr(do), stream)


def status_of_indexer_logits(q, k, kv_scale, w, ks, ke, logits, clean=True, stream=None) -> int:
    """Raw status of sparse_mla_indexer_logits."""
    lib = load()
    ds = [describe(t) for t in (q, k, kv_scale, w, ks, ke, logits)]
    st = _stream_handle(stream, q, logits) if stream is None and q is not None and q.is_cuda else stream
    return lib.sparse_mla_indexer_logits(*[_ptr(d) for d in ds[:6]], int(bool(clean)), _ptr(ds[6]), st)


def sparse_mla_indexer_logits(q, k, kv_scale, w, ks, ke, logits, clean=True, stream=None) -> None:
    """Indexer logits: per key the sum over 32 heads of relu(q . k) * w, times
    the key's scale, inside [ks, ke) (-inf outside when clean)."""
    _check(status_of_indexer_logits(q, k, kv_scale, w, ks, ke, logits, clean, stream))


def status_of_indexer_topk(logits, ks, ke, k, indices, stream=None) -> int:
    lib = load()
    ds = [describe(t) for t in (logits, ks, ke, indices)]
    st = _stream_handle(stream, logits) if stream is None and logits is not None and logits.is_cuda else stream
    return lib.sparse_mla_indexer_topk(_ptr(ds[0]), _ptr(ds[1]), _ptr(ds[2]), int(k), _ptr(ds[3]), st)


def sparse_mla_indexer_topk(logits, ks, ke, k, indices, stream=None) -> None:
    """Per row the indices of the k largest logits inside [ks, ke), ascending,
    -1 padded."""
    _check(status_of_indexer_topk(logits, ks, ke, k, indices, stream))
