"""Seeded synthetic inputs for sparse MLA forward.

This module only draws data. It holds none of the attention arithmetic, so both
the HIP path's tests and the fp64 oracle can consume the same tensors without
sharing any of the method's code.

Every tensor is drawn on the CPU from one ``torch.Generator`` seeded per
workload, in a fixed order: q, pool, indices, invalid slots. The same seed
always gives the same bytes (``tensor_digest`` hashes them).

Shapes follow the workloads of "[Triton/Gluon] GFX950 sparse mla optimizations"
(aiter PR 6159, Technical Details tables): 5+1 speculative decode at C requests,
8K/16K-row prefill, 16 or 64 heads, DeepSeek-style top-k 512 and GLM-style
top-k 2048, 576-wide rows (512 latent + 64 rope) or 512-wide rope-free rows.
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import torch

FP8_MAX = 448.0  # largest finite float8_e4m3fn value


@dataclass(frozen=True)
class Workload:
    """One synthetic sparse-MLA call.

    ``index_mode`` says where each row's indices come from:
      * ``"uniform"``  - distinct, uniform over the whole pool;
      * ``"request"``  - row r belongs to request r // rows_per_request, which
        owns pool rows [ctx * b, ctx * b + ctx); distinct within that range;
      * ``"causal"``   - row i sits at position ``first_pos + i``; distinct
        from [0, pos].
    """

    name: str
    rows: int
    heads: int
    d_qk: int
    pool_rows: int
    topk: int
    kv_dtype: str  # "bf16" or "fp8"
    seed: int
    index_mode: str = "uniform"
    invalid_per_row: int = 0
    rows_per_request: int = 1
    ctx_per_request: int = 0
    first_pos: int = 0
    sm_scale: float | None = None
    pool_pitch: int | None = None  # elements between pool rows (>= d_qk)
    description: str = ""

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else self.d_qk ** -0.5

    @property
    def pitch(self) -> int:
        return self.pool_pitch if self.pool_pitch is not None else self.d_qk


# The five workloads. Where a workload leaves a detail open the plainest
# reading is taken: sm_scale = d_qk^-0.5, a decode request owns an equal slice
# of the pool, prefill rows are the last positions of one context.
WORKLOADS: dict[str, Workload] = {
    "tiny": Workload(
        name="tiny", rows=4, heads=16, d_qk=576, pool_rows=4096, topk=128,
        kv_dtype="bf16", seed=0, index_mode="uniform", invalid_per_row=2,
        description="4 rows x 16 heads, bf16 pool 4096x576, top-k 128, 2 invalid per row"),
    "decode_bf16": Workload(
        name="decode_bf16", rows=192, heads=64, d_qk=576, pool_rows=131072, topk=512,
        kv_dtype="bf16", seed=1, index_mode="request", invalid_per_row=26,
        rows_per_request=6, ctx_per_request=4096,
        description="DSv4-style decode: 32 requests x (5+1) rows, 64 heads, bf16 pool "
                    "131072x576, top-k 512 from the request's context, 5% invalid"),
    "decode_fp8": Workload(
        name="decode_fp8", rows=768, heads=16, d_qk=576, pool_rows=262144, topk=2048,
        kv_dtype="fp8", seed=2, index_mode="uniform",
        description="fp8 decode: 128 requests x (5+1) rows, 16 heads, fp8 pool "
                    "262144x576 + per-tensor scale, top-k 2048 uniform, no invalid"),
    "prefill_fp8": Workload(
        name="prefill_fp8", rows=8192, heads=64, d_qk=576, pool_rows=131072, topk=2048,
        kv_dtype="fp8", seed=3, index_mode="causal", first_pos=122880,
        description="fp8 prefill: 8192 rows at positions 122880..131071, 64 heads, "
                    "fp8 pool 131072x576, top-k 2048 causal"),
    "prefill_glm": Workload(
        name="prefill_glm", rows=16384, heads=64, d_qk=512, pool_rows=262144, topk=2048,
        kv_dtype="fp8", seed=4, index_mode="causal", first_pos=245760,
        sm_scale=512 ** -0.5,
        description="rope-free GLM-style prefill: 16384 rows, 64 heads, 512-wide fp8 "
                    "pool 262144x512, top-k 2048 causal"),
}


# Workloads beyond the five (the benchmark's MALL-sensitivity line; its GPU
# parity test checks sampled rows, since the pool below is 1.2 GB). decode_fp8 draws its indices over the whole 151 MB
# pool, which a cold call still finds largely in the 256 MB MALL after its
# first touches (every pool row is gathered about six times per call); here
# each request owns its own 16384-row context, as a serving pool of 128
# requests would, so the pool does not fit.
SENSITIVITY_WORKLOADS: dict[str, Workload] = {
    "decode_fp8_ctx": Workload(
        name="decode_fp8_ctx", rows=768, heads=16, d_qk=576, pool_rows=2097152, topk=2048,
        kv_dtype="fp8", seed=5, index_mode="request", rows_per_request=6,
        ctx_per_request=16384,
        description="fp8 decode, MALL sensitivity: 128 requests x (5+1) rows, 16 heads, fp8 "
                    "pool 2097152x576 (1.2 GB), each request's top-k 2048 from its own "
                    "16384-row context, no invalid"),
}


# The two decode workloads with their heads split over two GPUs (32 heads on
# each): one GPU's share of a head-parallel deployment, timed on its own.
HEAD_SHARE_WORKLOADS: dict[str, Workload] = {
    "decode_bf16_h32": Workload(
        name="decode_bf16_h32", rows=192, heads=32, d_qk=576, pool_rows=131072, topk=512,
        kv_dtype="bf16", seed=1, index_mode="request", invalid_per_row=26, rows_per_request=6,
        ctx_per_request=4096,
        description="decode_bf16 with 32 heads (one GPU's share of a two-way head split)"),
    "decode_fp8_h32": Workload(
        name="decode_fp8_h32", rows=768, heads=32, d_qk=576, pool_rows=262144, topk=2048,
        kv_dtype="fp8", seed=2, index_mode="uniform",
        description="decode_fp8 with 32 heads (one GPU's share of a two-way head split)"),
}


@dataclass
class Inputs:
    q: torch.Tensor          # bf16 [R, H, D]
    pool: torch.Tensor       # bf16 or float8_e4m3fn [N, pitch] (first d_qk used)
    kv_scale: torch.Tensor | None  # fp32 [1] or None for bf16 pools
    indices: torch.Tensor    # int32 [R, K]
    sm_scale: float
    workload: Workload
    extra: dict = field(default_factory=dict)


def _index_ranges(w: Workload) -> tuple[torch.Tensor, torch.Tensor]:
    r = torch.arange(w.rows, dtype=torch.int64)
    if w.index_mode == "uniform":
        lo = torch.zeros(w.rows, dtype=torch.int64)
        hi = torch.full((w.rows,), w.pool_rows, dtype=torch.int64)
    elif w.index_mode == "request":
        b = r // w.rows_per_request
        lo = b * w.ctx_per_request
        hi = lo + w.ctx_per_request
    elif w.index_mode == "causal":
        lo = torch.zeros(w.rows, dtype=torch.int64)
        hi = w.first_pos + r + 1
    else:
        raise ValueError(f"unknown index_mode {w.index_mode!r}")
    if int(hi.max()) > w.pool_rows or int((hi - lo).min()) < w.topk:
        raise ValueError(f"{w.name}: index ranges do not fit pool/top-k")
    return lo, hi


def distinct_indices(lo: torch.Tensor, hi: torch.Tensor, k: int,
                     gen: torch.Generator) -> torch.Tensor:
    """k distinct ints per row, uniform over [lo_r, hi_r), kept in draw order.

    Sampler: draw candidates lo + floor(u * (hi - lo)) with u ~ U[0,1) in fp64,
    keep the first occurrence of each value in draw order, and take the first k
    kept candidates. While any row has fewer than k distinct candidates another
    block of candidates is drawn for every row. The result is exactly a uniform
    draw without replacement (rejection of repeats).
    """
    rows = lo.shape[0]
    span = (hi - lo).to(torch.float64)
    if rows == 0:
        return torch.empty((0, k), dtype=torch.int32)
    # expected repeats among m draws from n values: about m^2 / (2n)
    n_min = float(span.min())
    extra = int(min(4 * k, 2 * k * k / n_min + 8 * math.sqrt(k * k / n_min + 1) + 32))
    cand = torch.empty((rows, 0), dtype=torch.int64)
    block = k + extra
    while True:
        u = torch.rand((rows, block), generator=gen, dtype=torch.float64)
        new = lo[:, None] + torch.floor(u * span[:, None]).to(torch.int64)
        cand = torch.cat([cand, new], dim=1)
        # first occurrence of each value within its row, in draw order
        sv, order = torch.sort(cand, dim=1, stable=True)
        dup_sorted = torch.zeros_like(sv, dtype=torch.bool)
        dup_sorted[:, 1:] = sv[:, 1:] == sv[:, :-1]
        keep = torch.empty_like(dup_sorted)
        keep.scatter_(1, order, ~dup_sorted)
        if int(keep.sum(dim=1).min()) >= k:
            break
        block = max(64, k // 4)
    rank = torch.cumsum(keep.to(torch.int64), dim=1) - 1
    sel = keep & (rank < k)
    out = cand[sel].view(rows, k)
    return out.to(torch.int32)


def set_invalid(indices: torch.Tensor, n_invalid: int, gen: torch.Generator) -> torch.Tensor:
    """Set n_invalid slots per row, at uniformly random distinct slots, to -1."""
    if n_invalid <= 0 or indices.numel() == 0:
        return indices
    rows, k = indices.shape
    slots = torch.argsort(torch.rand((rows, k), generator=gen), dim=1)[:, :n_invalid]
    out = indices.clone()
    out.scatter_(1, slots, -1)
    return out


def quantize_fp8(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-tensor e4m3fn codes: s = max|x| / 448, codes = clamp(x / s) in e4m3fn.

    The clamp keeps x / s inside the finite range (torch turns out-of-range
    values into NaN). This quantiser only makes test data; the method itself
    starts from the codes and the scale.
    """
    s = float(x.abs().max()) / FP8_MAX
    if s == 0.0:
        s = 1.0
    s32 = torch.tensor([s], dtype=torch.float32)
    codes = torch.clamp(x / s32, -FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, s32


def make_inputs(w: Workload | str, rows: int | None = None) -> Inputs:
    """Draw the workload's tensors on the CPU.

    ``rows`` (optional) keeps only the first ``rows`` query rows of q and of the
    indices *after* drawing the full workload, so a prefix of a big workload is
    byte-identical to the same rows of the full draw.
    """
    if isinstance(w, str):
        w = {**WORKLOADS, **SENSITIVITY_WORKLOADS, **HEAD_SHARE_WORKLOADS}[w]
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    q = torch.randn((w.rows, w.heads, w.d_qk), generator=gen, dtype=torch.float32)
    q = q.to(torch.bfloat16)
    x = torch.randn((w.pool_rows, w.d_qk), generator=gen, dtype=torch.float32)
    if w.kv_dtype == "bf16":
        vals, kv_scale = x.to(torch.bfloat16), None
    elif w.kv_dtype == "fp8":
        vals, kv_scale = quantize_fp8(x)
    else:
        raise ValueError(f"unknown kv dtype {w.kv_dtype!r}")
    del x
    if w.pitch != w.d_qk:
        pool = torch.zeros((w.pool_rows, w.pitch), dtype=vals.dtype)
        pool[:, : w.d_qk] = vals
    else:
        pool = vals
    lo, hi = _index_ranges(w)
    idx = distinct_indices(lo, hi, w.topk, gen)
    idx = set_invalid(idx, w.invalid_per_row, gen)
    if rows is not None:
        q = q[:rows].contiguous()
        idx = idx[:rows].contiguous()
    return Inputs(q=q, pool=pool, kv_scale=kv_scale, indices=idx, sm_scale=w.scale, workload=w)


@dataclass
class ExtraSegment:
    """The second segment of a two-segment call: its own pool (same dtype as
    the main one), its own fp8 scale (None for bf16) and its indices."""
    pool: torch.Tensor
    kv_scale: torch.Tensor | None
    indices: torch.Tensor  # int32 [R, window]


def window_ends(w: Workload) -> torch.Tensor:
    """Position of each query row in its own context, as the index modes
    place it: "request" rows are the last rows_per_request positions of their
    request's context slice, "causal" rows sit at first_pos + r, "uniform"
    rows at the end of the pool."""
    r = torch.arange(w.rows, dtype=torch.int64)
    if w.index_mode == "request":
        b = r // w.rows_per_request
        return b * w.ctx_per_request + (w.ctx_per_request - w.rows_per_request) + r % w.rows_per_request
    if w.index_mode == "causal":
        return w.first_pos + r
    return torch.full((w.rows,), w.pool_rows - 1, dtype=torch.int64)


def make_extra_segment(inp: Inputs, window: int, seed: int, value_std: float = 1.0,
                       invalid_per_row: int = 0, rows: int | None = None) -> ExtraSegment:
    """A sliding-window segment for ``inp``: an extra pool of the same shape
    and dtype as inp.pool, drawn N(0, value_std^2) (fp8: quantised with its
    own per-tensor scale), and for each query row the ``window`` consecutive
    pool rows ending at the row's position (window_ends). Positions before a
    request's context start (or below 0) are -1; ``invalid_per_row`` more
    slots per row are set to -1 at random. Seeded on its own generator."""
    w = inp.workload
    gen = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((w.pool_rows, w.d_qk), generator=gen, dtype=torch.float32) * value_std
    if w.kv_dtype == "bf16":
        vals, scale = x.to(torch.bfloat16), None
    else:
        vals, scale = quantize_fp8(x)
    del x
    if w.pitch != w.d_qk:
        pool = torch.zeros((w.pool_rows, w.pitch), dtype=vals.dtype)
        pool[:, : w.d_qk] = vals
    else:
        pool = vals
    end = window_ends(w)
    if w.index_mode == "request":
        start = (torch.arange(w.rows, dtype=torch.int64) // w.rows_per_request) * w.ctx_per_request
    else:
        start = torch.zeros(w.rows, dtype=torch.int64)
    pos = end[:, None] - torch.arange(window - 1, -1, -1, dtype=torch.int64)[None, :]
    idx = torch.where(pos >= start[:, None], pos, torch.full_like(pos, -1)).to(torch.int32)
    idx = set_invalid(idx, invalid_per_row, gen)
    n = inp.q.shape[0] if rows is None else rows
    return ExtraSegment(pool=pool, kv_scale=scale, indices=idx[:n].contiguous())


def custom_workload(name: str = "custom", **kw) -> Workload:
    """A Workload with the given fields (for tests of edge shapes)."""
    base = dict(name=name, rows=4, heads=16, d_qk=576, pool_rows=4096, topk=128,
                kv_dtype="bf16", seed=123)
    base.update(kw)
    return Workload(**base)


def tensor_digest(t: torch.Tensor) -> str:
    """SHA-256 of a CPU tensor's bytes (dtype-agnostic)."""
    t = t.contiguous()
    b = t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16 if t.element_size() == 2 else torch.int32)
    return hashlib.sha256(b.numpy().tobytes()).hexdigest()


# ------------------------------------------------------ output epilogue ---

@dataclass
class EpilogueInputs:
    """Inputs of the output epilogue: a position per query row and a cos/sin
    cache. ``cos_sin`` is fp32 [max_pos, 64]: row p holds the cosines of the
    32 pair angles at position p, then their sines (the layout of a serving
    stack's rotary cache); the angles are p * base^(-2j/64)."""
    positions: torch.Tensor   # int32 [R]
    cos_sin: torch.Tensor     # fp32 [max_pos, 64]


def make_rope_cache(max_pos: int, base: float = 10000.0) -> torch.Tensor:
    """fp32 [max_pos, 64] cos|sin table of the 32 rotary frequencies."""
    j = torch.arange(32, dtype=torch.float64)
    inv_freq = base ** (-2.0 * j / 64.0)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv_freq[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32)


def make_epilogue_inputs(rows: int, seed: int, max_pos: int = 131072,
                         first_pos: int | None = None) -> EpilogueInputs:
    """Positions drawn uniformly from [0, max_pos) (or first_pos + row, the
    positions of consecutive prefill rows), and the cache."""
    gen = torch.Generator("cpu").manual_seed(seed)
    if first_pos is None:
        pos = torch.randint(0, max_pos, (rows,), generator=gen, dtype=torch.int64)
    else:
        pos = (first_pos + torch.arange(rows, dtype=torch.int64)) % max_pos
    return EpilogueInputs(pos.to(torch.int32), make_rope_cache(max_pos))


def make_epilogue_rows(rows: int, heads: int, seed: int, std: float = 0.05) -> torch.Tensor:
    """bf16 [R, H, 512] rows shaped like attention outputs, N(0, std^2), with
    blocks that reach the MXFP8 edge cases: an all-zero 32-column block, a
    block whose largest magnitude sits just under and one just at a power of
    two, one block scaled up by 2^20 and one down by 2^-20 (e4m3 subnormals
    and flushes), and negative values that round to zero."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(rows, heads, 512, generator=gen, dtype=torch.float32) * std
    for r in range(rows):
        h = r % heads
        x[r, h, 0:32] = 0.0
        x[r, h, 32:64] *= 1.0 / x[r, h, 32:64].abs().max()          # amax = 1 exactly
        x[r, h, 64:96] *= (1.0 - 2.0 ** -8) / x[r, h, 64:96].abs().max()
        x[r, h, 96:128] *= 2.0 ** 20
        x[r, h, 128:160] *= 2.0 ** -20
        x[r, h, 160] = -1e-9                                          # rounds to -0 in e4m3
        x[r, h, 448:512] *= 4.0                                       # the rotated columns
    return x.to(torch.bfloat16)


# ------------------------------------------------------------- indexer ---

@dataclass(frozen=True)
class IndexerWorkload:
    """One synthetic indexer call: `rows` query rows of `requests` requests,
    each request's rows the last positions of its own `keys / requests`-key
    context (causal windows), 32 heads of 128 dims, top-k `topk`."""
    name: str
    rows: int
    keys: int
    requests: int = 1
    heads: int = 32
    dim: int = 128
    topk: int = 2048
    seed: int = 0
    description: str = ""


# The indexer shapes of "[HIP] [JIT] fp8_mqa_logits: v35w gfx950 prefill
# indexer logits kernel" (aiter PR 7183), its kernel-time table: causal
# chunks of one request, and of four requests per chunk.
INDEXER_WORKLOADS = {
    w.name: w for w in [
        IndexerWorkload("ix_tiny", rows=70, keys=600, requests=2, topk=64, seed=21,
                        description="small ragged case: 2 requests, 35 rows, 300 keys each"),
        IndexerWorkload("ix_causal_8k_8k", 8192, 8192, 1, seed=22,
                        description="causal, one request: s_q 8192, s_k 8192"),
        IndexerWorkload("ix_causal_4k_32k", 4096, 32768, 1, seed=23,
                        description="causal, one request: s_q 4096, s_k 32768"),
        IndexerWorkload("ix_causal_2k_64k", 2048, 65536, 1, seed=24,
                        description="causal, one request: s_q 2048, s_k 65536"),
        IndexerWorkload("ix_causal_1k_128k", 1024, 131072, 1, seed=25,
                        description="causal, one request: s_q 1024, s_k 131072"),
        IndexerWorkload("ix_multi_4k_32k", 4096, 32768, 4, seed=26,
                        description="causal, four requests per chunk: s_q 4096, s_k 32768"),
    ]
}


@dataclass
class IndexerInputs:
    workload: IndexerWorkload
    q: torch.Tensor         # float8_e4m3fn [M, H, D]
    k: torch.Tensor         # float8_e4m3fn [N, D]
    kv_scale: torch.Tensor  # fp32 [N]
    w: torch.Tensor         # fp32 [M, H]
    ks: torch.Tensor        # int32 [M]
    ke: torch.Tensor        # int32 [M]


def indexer_windows(w: IndexerWorkload) -> tuple[torch.Tensor, torch.Tensor]:
    """Request b owns rows [b M/B, (b+1) M/B) and keys [b N/B, (b+1) N/B); its
    local row i sits at key position N/B - M/B + i and sees the keys of its
    request up to and including that position."""
    B = w.requests
    mb, nb = w.rows // B, w.keys // B
    m = torch.arange(w.rows, dtype=torch.int64)
    b = torch.clamp(m // mb, max=B - 1)
    i = m - b * mb
    ks = b * nb
    ke = ks + (nb - mb) + i + 1
    return ks.to(torch.int32), ke.to(torch.int32)


def make_indexer_inputs(w: IndexerWorkload | str) -> IndexerInputs:
    """Draw order: q (N(0,1) to e4m3), k (N(0,1) per key, quantised with the
    key's own scale max|k|/448), w (N(0, 1/32))."""
    if isinstance(w, str):
        w = INDEXER_WORKLOADS[w]
    gen = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn(w.rows, w.heads, w.dim, generator=gen).clamp(-FP8_MAX, FP8_MAX)
    q = q.to(torch.float8_e4m3fn)
    kx = torch.randn(w.keys, w.dim, generator=gen)
    scale = kx.abs().amax(dim=1) / FP8_MAX
    k = (kx / scale[:, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    wt = torch.randn(w.rows, w.heads, generator=gen) * w.heads ** -0.5
    ks, ke = indexer_windows(w)
    return IndexerInputs(w, q, k, scale.to(torch.float32), wt.to(torch.float32), ks, ke)


def make_topk_logits(rows: int, keys: int, seed: int, k: int) -> tuple[torch.Tensor, torch.Tensor,
                                                                       torch.Tensor]:
    """fp32 logits [rows, keys] with windows [ks, ke) of every kind a top-k
    meets: empty, shorter than k, exactly k, longer; rows of continuous
    values, rows drawn from a handful of values (many ties at the k-th
    value), rows with negative zeros and huge magnitudes. Outside the window
    the values are NaN (a top-k must not read them)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(rows, keys, generator=gen)
    ks = torch.randint(0, max(1, keys // 4), (rows,), generator=gen)
    span = torch.randint(0, keys, (rows,), generator=gen)
    for r in range(rows):
        kind = r % 6
        if kind == 1:
            x[r] = torch.randint(-3, 4, (keys,), generator=gen).float()   # ties
        elif kind == 2:
            x[r] = torch.where(torch.rand(keys, generator=gen) < 0.5, -0.0, 0.0)
            x[r, ::7] = 1.0
        elif kind == 3:
            x[r] *= 1e30
        if r % 5 == 0:
            span[r] = 0                     # empty window
        elif r % 5 == 1:
            span[r] = k // 2                # shorter than k
        elif r % 5 == 2:
            span[r] = k                     # exactly k
    ke = torch.clamp(ks + span, max=keys)
    for r in range(rows):
        x[r, :ks[r]] = float("nan")
        x[r, ke[r]:] = float("nan")
    return x.to(torch.float32), ks.to(torch.int32), ke.to(torch.int32)


def make_fp8_q(inp: Inputs) -> tuple[torch.Tensor, torch.Tensor]:
    """An fp8 q for the same call: the workload's q quantised to e4m3fn with
    one per-tensor scale (max|q| / 448), the way the cache is."""
    return quantize_fp8(inp.q.to(torch.float32))
