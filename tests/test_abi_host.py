"""Host-side checks of libsparse_mla.so that need no GPU: the library loads and
exports every symbol include/sparse_mla.h declares, arguments are validated
before any HIP call, the planner's choices are legal, and the XCD-aware work
order is a bijection that gives each XCD one contiguous run of work ids.
No call here reaches a kernel."""

import ctypes
import os
import re

import pytest
import torch

from sparse_mla_attention_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SMLA_API\s+[\w\s\*]+?\b(sparse_mla_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert len(declared) >= 7
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.EXPORTED)
    assert _lib.version().count(".") == 2


def _args(R=4, H=16, D=576, N=256, K=64, pool_dtype=torch.bfloat16, width=None):
    q = torch.zeros(R, H, D, dtype=torch.bfloat16)
    pool = torch.zeros(N, width or D, dtype=pool_dtype)
    scale = torch.ones(1, dtype=torch.float32) if pool_dtype == torch.float8_e4m3fn else None
    idx = torch.zeros(R, K, dtype=torch.int32)
    out = torch.zeros(R, H, 512, dtype=torch.bfloat16)
    lse = torch.zeros(R, H, dtype=torch.float32)
    return dict(q=q, kv_pool=pool, kv_scale=scale, indices=idx, sm_scale=0.1, out=out, lse=lse)


def _status(a):
    return _lib.status_of_fwd(a["q"], a["kv_pool"], a["kv_scale"], a["indices"], a["sm_scale"],
                              a["out"], a["lse"])


INVALID, UNSUP = _lib.SMLA_ERR_INVALID_ARG, _lib.SMLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(q=a["q"].float()), UNSUP),
    (lambda a: a.update(q=torch.zeros(4, 16, 448, dtype=torch.bfloat16)), UNSUP),
    (lambda a: a.update(q=torch.zeros(4, 16, dtype=torch.bfloat16)), INVALID),
    (lambda a: a.update(kv_pool=a["kv_pool"].to(torch.float16)), UNSUP),
    (lambda a: a.update(kv_pool=torch.zeros(256, 576, dtype=torch.float8_e4m3fnuz),
                        kv_scale=torch.ones(1)), UNSUP),
    (lambda a: a.update(kv_pool=torch.zeros(256, 500, dtype=torch.bfloat16)), INVALID),
    (lambda a: a.update(kv_pool=torch.zeros(256, 580, dtype=torch.bfloat16)), UNSUP),  # 1160-B pitch
    (lambda a: a.update(indices=torch.zeros(5, 64, dtype=torch.int32)), INVALID),
    (lambda a: a.update(indices=torch.zeros(4, 64, dtype=torch.int64)), UNSUP),
    (lambda a: a.update(indices=torch.zeros(4, 0, dtype=torch.int32)), UNSUP),
    (lambda a: a.update(indices=torch.zeros(4, 128, dtype=torch.int32)[:, ::2]), UNSUP),
    (lambda a: a.update(out=torch.zeros(4, 16, 256, dtype=torch.bfloat16)), INVALID),
    (lambda a: a.update(out=torch.zeros(4, 16, 512, dtype=torch.float32)), UNSUP),
    (lambda a: a.update(lse=torch.zeros(4, 8, dtype=torch.float32)), INVALID),
    (lambda a: a.update(lse=torch.zeros(4, 16, dtype=torch.float64)), UNSUP),
    (lambda a: a.update(sm_scale=float("nan")), INVALID),
    (lambda a: a.update(kv_scale=torch.ones(1)), INVALID),          # scale given for bf16 pool
    (lambda a: a.update(kv_pool=torch.zeros(256, 576, dtype=torch.float8_e4m3fn)), INVALID),  # no scale
    (lambda a: a.update(q=torch.zeros(4, 2000, 576, dtype=torch.bfloat16),
                        out=torch.zeros(4, 2000, 512, dtype=torch.bfloat16),
                        lse=torch.zeros(4, 2000)), UNSUP),
    (lambda a: a.update(q=torch.zeros(4, 16, 580, dtype=torch.bfloat16)[:, :, :576]), UNSUP),
    (lambda a: a.update(out=a["q"][:, :, :512]), INVALID),           # out aliases q
])
def test_validation_rejects_before_any_hip_call(mutate, expected):
    a = _args()
    mutate(a)
    assert _status(a) == expected, _lib.last_error()
    assert _lib.last_error()


def test_fp8_pool_requires_fp32_scale():
    a = _args(pool_dtype=torch.float8_e4m3fn)
    a["kv_scale"] = torch.ones(1, dtype=torch.float64)
    assert _status(a) == UNSUP


def test_null_descriptor_is_invalid(lib):
    a = _args()
    d = [_lib.describe(a[k]) for k in ("q", "kv_pool", "indices", "out", "lse")]
    st = lib.sparse_mla_fwd(None, _lib._ptr(d[1]), None, _lib._ptr(d[2]), 0.1, _lib._ptr(d[3]),
                            _lib._ptr(d[4]), None)
    assert st == INVALID


def test_zero_rows_is_a_noop():
    a = _args(R=0)
    assert _status(a) == _lib.SMLA_OK


def test_is_supported():
    a = _args()
    assert _lib.sparse_mla_is_supported(a["q"], a["kv_pool"], a["indices"])
    assert not _lib.sparse_mla_is_supported(a["q"].float(), a["kv_pool"], a["indices"])
    b = _args(D=512, pool_dtype=torch.float8_e4m3fn)
    assert _lib.sparse_mla_is_supported(b["q"], b["kv_pool"], b["indices"])


# ------------------------------------------------------------------ planner

def _plan(R, H, D=576, K=2048, dtype=torch.float8_e4m3fn, **kw):
    a = _args(R=R, H=H, D=D, K=K, pool_dtype=dtype, N=16)
    return _lib.sparse_mla_plan(a["q"], a["kv_pool"], a["indices"], **kw)


@pytest.mark.parametrize("R,H,D,K", [
    (4, 16, 576, 128), (192, 64, 576, 512), (768, 16, 576, 2048), (8192, 64, 576, 2048),
    (16384, 64, 512, 2048), (1, 8, 576, 2048), (37, 8, 576, 100), (6, 16, 576, 2048),
    (3, 48, 512, 1), (2, 128, 576, 65), (100, 32, 576, 64),
])
def test_plan_is_legal(R, H, D, K):
    p = _plan(R, H, D, K)
    assert p["tile_slots"] in (16, 64, 128)
    tiles = -(-K // p["tile_slots"])
    assert p["head_block"] in (16, 32, 64)
    assert p["head_blocks"] == -(-H // p["head_block"])
    assert 1 <= p["splits"] <= 64
    assert p["splits"] * p["tiles_per_split"] >= tiles
    assert (p["splits"] - 1) * p["tiles_per_split"] < tiles  # no empty split
    assert p["grid"] == R * p["head_blocks"] * p["splits"]
    assert p["waves"] in (4, 8) and 0 < p["lds_bytes"] <= 160 * 1024
    if p["splits"] > 1:
        assert p["workspace_bytes"] >= p["splits"] * R * H * (512 + 1) * 4
    else:
        assert p["workspace_bytes"] == 0


def test_plan_head_block_choice_and_overrides():
    assert _plan(768, 16)["head_block"] == 16
    # 32 heads: two 16-head decode-kernel blocks over fp8 pools (measured
    # faster than the 32-head staged kernel), one 32-head block over bf16
    p = _plan(768, 32)
    assert (p["head_block"], p["head_blocks"], p["variant"], p["remap"]) == (16, 2, 0, 1)
    p = _plan(100, 32, dtype=torch.bfloat16)
    assert (p["head_block"], p["variant"]) == (32, 0)
    assert _plan(100, 48)["head_block"] == 64
    # 64 heads over bf16 pools: the staged-tile kernel unless overridden
    assert _plan(192, 64, K=512, dtype=torch.bfloat16)["variant"] == 1
    assert _plan(192, 64, K=512, dtype=torch.bfloat16, variant=2)["variant"] == 2
    # 64 heads over fp8 pools: the fp8-dot kernel (variant 3) for both row
    # widths; 4 forces the 4-wave kernel (reported as variant 0)
    assert _plan(8192, 64)["variant"] == 3
    assert _plan(8192, 64, D=512)["variant"] == 3
    assert _plan(8192, 64, D=512, variant=4)["variant"] == 0
    assert _plan(8192, 64)["head_block"] == 64
    assert _plan(8192, 64)["splits"] == 1
    assert _plan(4, 16, K=2048)["splits"] > 1      # a tiny launch gets split
    p = _plan(4, 16, K=2048, head_block=64, splits=8, remap=2)
    assert (p["head_block"], p["splits"], p["remap"]) == (64, 8, 0)
    p = _plan(4, 16, K=128, splits=8, dtype=torch.bfloat16)
    assert p["splits"] == 128 // p["tile_slots"]  # capped at the tile count
    with pytest.raises(_lib.SparseMLAError):
        _plan(4, 16, head_block=24)
    with pytest.raises(_lib.SparseMLAError):
        _plan(4, 16, splits=65)


def test_plan_counts_workgroups_per_cu():
    # The fp8 decode kernel fits two workgroups per CU. They share the CU's
    # memory traffic, so a launch that already gives every CU work stays
    # unsplit (768 rows on 256 CUs measured 176 us unsplit, 193 us with two
    # splits), while a launch that leaves CUs idle is still split.
    p = _plan(768, 16, num_cus=256)
    assert (p["head_block"], p["waves"], p["splits"]) == (16, 4, 1)
    assert 2 * p["lds_bytes"] <= 160 * 1024
    assert _plan(256, 16, num_cus=256)["splits"] == 1
    assert _plan(32, 16, num_cus=256)["splits"] > 1


@pytest.mark.parametrize("grid", [1, 7, 8, 9, 63, 64, 100, 513, 768, 1536])
def test_xcd_work_order_is_contiguous_bijection(grid):
    works = [_lib.sparse_mla_work_of(pid, grid, 1) for pid in range(grid)]
    assert sorted(works) == list(range(grid))
    for x in range(8):
        mine = [works[pid] for pid in range(x, grid, 8)]
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True
    assert [_lib.sparse_mla_work_of(pid, grid, 0) for pid in range(grid)] == list(range(grid))
    assert _lib.sparse_mla_work_of(grid, grid, 1) == -1


# ------------------------------------------------------------ two segments

def _args2(pool_dtype=torch.float8_e4m3fn, K2=32, D=576, N2=128):
    a = _args(pool_dtype=pool_dtype, D=D)
    a["extra_pool"] = torch.zeros(N2, D, dtype=pool_dtype)
    a["extra_kv_scale"] = torch.ones(1) if pool_dtype == torch.float8_e4m3fn else None
    a["extra_indices"] = torch.zeros(a["q"].shape[0], K2, dtype=torch.int32)
    return a


def _status2(a):
    return _lib.status_of_fwd2(a["q"], a["kv_pool"], a["kv_scale"], a["indices"], a["extra_pool"],
                               a["extra_kv_scale"], a["extra_indices"], a["sm_scale"], a["out"],
                               a["lse"])


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(extra_pool=torch.zeros(128, 576, dtype=torch.bfloat16)), UNSUP),  # dtype mismatch
    (lambda a: a.update(extra_pool=torch.zeros(128, 500, dtype=torch.float8_e4m3fn)), INVALID),  # too narrow
    (lambda a: a.update(extra_indices=torch.zeros(5, 32, dtype=torch.int32)), INVALID),  # rows
    (lambda a: a.update(extra_indices=torch.zeros(4, 32, dtype=torch.int64)), UNSUP),  # dtype
    (lambda a: a.update(extra_kv_scale=torch.ones(1, dtype=torch.float64)), UNSUP),
])
def test_two_segment_validation(mutate, expected):
    a = _args2()
    mutate(a)
    assert _status2(a) == expected, _lib.last_error()


def test_two_segment_bf16_rejects_extra_scale():
    a = _args2(pool_dtype=torch.bfloat16)
    a["extra_kv_scale"] = torch.ones(1)
    assert _status2(a) == INVALID


def test_two_segment_fp8_extra_scale_defaults_to_main():
    a = _args2()
    a["extra_kv_scale"] = None
    for k in ("q", "indices", "extra_indices", "out", "lse"):
        a[k] = a[k][:0]
    assert _status2(a) == 0


@pytest.mark.parametrize("H,K1,K2,dtype", [(16, 512, 128, torch.float8_e4m3fn),
                                            (64, 512, 128, torch.bfloat16),
                                            (64, 2048, 128, torch.float8_e4m3fn)])
def test_plan2_workspace_covers_both_segments(H, K1, K2, dtype):
    R = 192
    q = torch.zeros(R, H, 576, dtype=torch.bfloat16)
    pool = torch.zeros(1024, 576, dtype=dtype)
    i1 = torch.zeros(R, K1, dtype=torch.int32)
    i2 = torch.zeros(R, K2, dtype=torch.int32)
    p1, p2, ws = _lib.sparse_mla_plan2(q, pool, i1, pool, i2)
    whole = _lib.sparse_mla_plan(q, pool, torch.zeros(R, K1 + K2, dtype=torch.int32))
    if H == 16 and dtype == torch.float8_e4m3fn:
        # the decode kernel walks both segments in one launch
        assert whole["head_block"] == 16 and whole["variant"] == 0
        assert p1 == whole and p2["grid"] == 0
        S = p1["splits"] if p1["splits"] > 1 else 0
    elif dtype == torch.bfloat16 or H == 64:
        # the 64-head bf16 kernel and the 64-head fp8-dot kernel walk them
        # too, the main top-k padded to tiles
        K1p = (K1 + whole["tile_slots"] - 1) // whole["tile_slots"] * whole["tile_slots"]
        # (bf16: the 8-wave kernel, variant 2: the one-segment default is the
        # staged kernel, which would need a second launch)
        padded = _lib.sparse_mla_plan(q, pool, torch.zeros(R, K1p + K2, dtype=torch.int32),
                                      variant=2 if dtype == torch.bfloat16 else 0)
        assert p1 == padded and p2["grid"] == 0
        assert dtype == torch.bfloat16 or p1["variant"] == 3
        S = p1["splits"] if p1["splits"] > 1 else 0
    else:
        assert p1 == _lib.sparse_mla_plan(q, pool, i1)
        assert p2 == _lib.sparse_mla_plan(q, pool, i2)
        S = p1["splits"] + p2["splits"]
    o_bytes = S * R * H * 512 * 4
    assert ws == ((o_bytes + 255) // 256 * 256 + S * R * H * 4 if S else 0)


def test_plan2_fp8dot_composes_when_the_extra_pitch_is_out_of_reach():
    """The fp8-dot kernel addresses the second segment's pool through a
    structured buffer whose stride field holds 14 bits: an extra pool with a
    16 KB row pitch takes the two-launch composition."""
    R, H = 192, 64
    q = torch.zeros(R, H, 576, dtype=torch.bfloat16)
    pool = torch.zeros(1024, 576, dtype=torch.float8_e4m3fn)
    wide = torch.zeros(64, 16384, dtype=torch.float8_e4m3fn)[:, :576]
    i1 = torch.zeros(R, 2048, dtype=torch.int32)
    i2 = torch.zeros(R, 128, dtype=torch.int32)
    p1, p2, ws = _lib.sparse_mla_plan2(q, pool, i1, wide, i2)
    assert p1 == _lib.sparse_mla_plan(q, pool, i1) and p1["variant"] == 3
    assert p2 == _lib.sparse_mla_plan(q, wide, i2) and p2["grid"] > 0
    S = p1["splits"] + p2["splits"]
    assert ws == (S * R * H * 512 * 4 + 255) // 256 * 256 + S * R * H * 4


def test_plan2_fp8dot_walks_both_segments_over_a_paged_main_pool():
    """A paged main pool (pages a whole number of rows apart) keeps the
    fp8-dot kernel's one-launch walk; the second pool is 2-D."""
    R, H, rows_per_page = 192, 64, 64
    q = torch.zeros(R, H, 576, dtype=torch.bfloat16)
    flat = torch.zeros(16 * rows_per_page * 576, dtype=torch.float8_e4m3fn)
    paged = flat.as_strided((16, rows_per_page, 576), (rows_per_page * 576, 576, 1))
    extra = torch.zeros(1024, 576, dtype=torch.float8_e4m3fn)
    i1 = torch.zeros(R, 300, dtype=torch.int32)
    i2 = torch.zeros(R, 100, dtype=torch.int32)
    p1, p2, _ = _lib.sparse_mla_plan2(q, paged, i1, extra, i2)
    assert p1["variant"] == 3 and p2["grid"] == 0
    padded = _lib.sparse_mla_plan(q, paged, torch.zeros(R, 320 + 100, dtype=torch.int32))
    assert p1 == padded


# ------------------------------------------------------------ output epilogue

def _epi_args(R=4, H=16, mx=True, rope=True):
    a = _args(R=R, H=H)
    if mx:
        a["out"] = torch.zeros(R, H, 512, dtype=torch.float8_e4m3fn)
        a["out_scale"] = torch.zeros(R, H, 16, dtype=torch.uint8).view(torch.float8_e8m0fnu)
    else:
        a["out_scale"] = None
    a["rope_positions"] = torch.zeros(R, dtype=torch.int32) if rope else None
    a["rope_cos_sin"] = torch.zeros(64, 64, dtype=torch.float32) if rope else None
    return a


def _status_epi(a):
    return _lib.status_of_fwd_epi(a["q"], a["kv_pool"], a["kv_scale"], a["indices"], a["sm_scale"],
                                  a["out"], a["lse"], a["rope_positions"], a["rope_cos_sin"],
                                  a["out_scale"])


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(out=torch.zeros(4, 16, 512, dtype=torch.bfloat16)), UNSUP),   # MXFP8 needs fp8 codes
    (lambda a: a.update(out_scale=torch.zeros(4, 16, 8, dtype=torch.uint8).view(torch.float8_e8m0fnu)), INVALID),
    (lambda a: a.update(out_scale=torch.zeros(4, 16, 16, dtype=torch.uint8)), UNSUP),  # not E8M0
    (lambda a: a.update(rope_positions=torch.zeros(5, dtype=torch.int32)), INVALID),
    (lambda a: a.update(rope_positions=torch.zeros(4, dtype=torch.int64)), UNSUP),
    (lambda a: a.update(rope_cos_sin=None), INVALID),                                 # positions alone
    (lambda a: a.update(rope_positions=None), INVALID),                               # cache alone
    (lambda a: a.update(rope_cos_sin=torch.zeros(64, 32, dtype=torch.float32)), UNSUP),
    (lambda a: a.update(rope_cos_sin=torch.zeros(0, 64, dtype=torch.float32)), INVALID),
    (lambda a: a.update(rope_cos_sin=torch.zeros(64, 64, dtype=torch.bfloat16)), UNSUP),
    (lambda a: a.update(out_scale=torch.zeros(4, 16, 32, dtype=torch.uint8).view(torch.float8_e8m0fnu)[:, :, ::2]), UNSUP),
    (lambda a: a.update(out=torch.zeros(4, 16, 520, dtype=torch.float8_e4m3fn)[:, :, :512]), UNSUP),  # 520-B row
])
def test_epilogue_validation(mutate, expected):
    a = _epi_args()
    mutate(a)
    assert _status_epi(a) == expected, _lib.last_error()
    assert _lib.last_error()


def test_epilogue_outputs_must_not_alias():
    a = _epi_args()
    buf = torch.zeros(4 * 16 * 512 + 4 * 16 * 16, dtype=torch.uint8)
    a["out"] = buf[:4 * 16 * 512].view(4, 16, 512).view(torch.float8_e4m3fn)
    a["out_scale"] = buf[:4 * 16 * 16].view(4, 16, 16).view(torch.float8_e8m0fnu)  # overlaps out
    assert _status_epi(a) == INVALID
    a = _epi_args()
    a["rope_cos_sin"] = a["lse"].view(-1)[:64].view(1, 64)                             # lse aliases cache
    assert _status_epi(a) == INVALID


def test_epilogue_zero_rows_is_a_noop():
    for mx in (True, False):
        a = _epi_args(R=0, mx=mx)
        assert _status_epi(a) == _lib.SMLA_OK, _lib.last_error()
    rows = torch.zeros(0, 16, 512, dtype=torch.bfloat16)
    out = torch.zeros(0, 16, 512, dtype=torch.float8_e4m3fn)
    sc = torch.zeros(0, 16, 16, dtype=torch.uint8).view(torch.float8_e8m0fnu)
    assert _lib.status_of_out_epilogue(rows, out, out_scale=sc) == _lib.SMLA_OK


@pytest.mark.parametrize("mutate,expected", [
    (lambda r, o, k: k.update(out_scale=None), UNSUP),                              # fp8 out without scales
    (lambda r, o, k: k.update(rope_positions=torch.zeros(3, dtype=torch.int32)), INVALID),
    (lambda r, o, k: r.__setitem__(0, torch.zeros(4, 16, 256, dtype=torch.bfloat16)), INVALID),
    (lambda r, o, k: r.__setitem__(0, torch.zeros(4, 16, 512, dtype=torch.float32)), UNSUP),
    (lambda r, o, k: o.__setitem__(0, torch.zeros(4, 8, 512, dtype=torch.float8_e4m3fn)), INVALID),
])
def test_out_epilogue_pass_validation(mutate, expected):
    rows = [torch.zeros(4, 16, 512, dtype=torch.bfloat16)]
    out = [torch.zeros(4, 16, 512, dtype=torch.float8_e4m3fn)]
    kw = dict(rope_positions=torch.zeros(4, dtype=torch.int32),
              rope_cos_sin=torch.zeros(8, 64, dtype=torch.float32),
              out_scale=torch.zeros(4, 16, 16, dtype=torch.uint8).view(torch.float8_e8m0fnu))
    mutate(rows, out, kw)
    assert _lib.status_of_out_epilogue(rows[0], out[0], **kw) == expected, _lib.last_error()


# ------------------------------------------------------------------ indexer

def _ix_args(M=40, N=300):
    return dict(q=torch.zeros(M, 32, 128, dtype=torch.float8_e4m3fn),
                k=torch.zeros(N, 128, dtype=torch.float8_e4m3fn),
                kv_scale=torch.ones(N), w=torch.zeros(M, 32), ks=torch.zeros(M, dtype=torch.int32),
                ke=torch.zeros(M, dtype=torch.int32), logits=torch.zeros(M, N))


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(q=torch.zeros(40, 16, 128, dtype=torch.float8_e4m3fn)), UNSUP),
    (lambda a: a.update(q=torch.zeros(40, 32, 64, dtype=torch.float8_e4m3fn)), UNSUP),
    (lambda a: a.update(q=torch.zeros(40, 32, 128, dtype=torch.bfloat16)), UNSUP),
    (lambda a: a.update(k=torch.zeros(300, 64, dtype=torch.float8_e4m3fn)), UNSUP),
    (lambda a: a.update(kv_scale=torch.ones(299)), INVALID),
    (lambda a: a.update(w=torch.zeros(40, 16)), INVALID),
    (lambda a: a.update(w=torch.zeros(40, 34)[:, :32]), UNSUP),          # row stride 34
    (lambda a: a.update(ks=torch.zeros(39, dtype=torch.int32)), INVALID),
    (lambda a: a.update(ke=torch.zeros(40, dtype=torch.int64)), UNSUP),
    (lambda a: a.update(logits=torch.zeros(40, 299)), INVALID),
    (lambda a: a.update(logits=torch.zeros(40, 300, dtype=torch.float64)), UNSUP),
    (lambda a: a.update(k=torch.zeros(300, 136, dtype=torch.float8_e4m3fn)[:, :128]), UNSUP),  # 136-B rows
])
def test_indexer_logits_validation(mutate, expected):
    a = _ix_args()
    mutate(a)
    assert _lib.status_of_indexer_logits(**a) == expected, _lib.last_error()


def test_indexer_logits_alias_and_noop():
    a = _ix_args()
    buf = torch.zeros(40 * 300 + 40 * 32)
    a["w"] = buf[:40 * 32].view(40, 32)
    a["logits"] = buf[:40 * 300].view(40, 300)                       # overlaps w
    assert _lib.status_of_indexer_logits(**a) == INVALID
    assert _lib.status_of_indexer_logits(**_ix_args(M=0)) == _lib.SMLA_OK
    assert _lib.status_of_indexer_logits(**_ix_args(N=0)) == _lib.SMLA_OK
    assert _lib.status_of_indexer_topk(torch.zeros(0, 10), torch.zeros(0, dtype=torch.int32),
                                       torch.zeros(0, dtype=torch.int32), 4,
                                       torch.zeros(0, 4, dtype=torch.int32)) == _lib.SMLA_OK


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: a.update(k=0), UNSUP),
    (lambda a: a.update(k=70000), UNSUP),
    (lambda a: a.update(indices=torch.zeros(8, 32, dtype=torch.int32)), INVALID),
    (lambda a: a.update(indices=torch.zeros(8, 16, dtype=torch.int64)), UNSUP),
    (lambda a: a.update(ks=torch.zeros(7, dtype=torch.int32)), INVALID),
    (lambda a: a.update(logits=torch.zeros(8, 100, dtype=torch.bfloat16)), UNSUP),
])
def test_indexer_topk_validation(mutate, expected):
    a = dict(logits=torch.zeros(8, 100), ks=torch.zeros(8, dtype=torch.int32),
             ke=torch.zeros(8, dtype=torch.int32), k=16, indices=torch.zeros(8, 16, dtype=torch.int32))
    mutate(a)
    assert _lib.status_of_indexer_topk(**a) == expected, _lib.last_error()


# ------------------------------------------------- fp8 q and paged pools

def test_fp8_q_is_accepted_and_q_scale_needs_it(lib):
    a = _args(R=0)
    a["q"] = torch.zeros(0, 16, 576, dtype=torch.float8_e4m3fn)
    assert _status(a) == _lib.SMLA_OK, _lib.last_error()
    a = _args(R=0)
    qs = torch.ones(1)
    d = [_lib.describe(a[k]) for k in ("q", "kv_pool", "indices", "out", "lse")]
    opt = _lib._options(q_scale=qs)
    st = lib.sparse_mla_fwd_ex(_lib._ptr(d[0]), _lib._ptr(d[1]), None, _lib._ptr(d[2]), 0.1,
                               _lib._ptr(d[3]), _lib._ptr(d[4]), None, ctypes.byref(opt))
    assert st == INVALID and "q_scale" in _lib.last_error()


@pytest.mark.parametrize("pool,expected", [
    (lambda: torch.zeros(64, 4, 576, dtype=torch.bfloat16), _lib.SMLA_OK),
    (lambda: torch.zeros(64, 3, 576, dtype=torch.bfloat16), UNSUP),          # 3 rows a page
    (lambda: torch.zeros(64, 4 * 576 + 64, dtype=torch.bfloat16).as_strided(
        (64, 4, 576), (4 * 576 + 64, 576, 1)), _lib.SMLA_OK),                 # padded pages
    (lambda: torch.zeros(64 * 4 * 576, dtype=torch.bfloat16).as_strided(
        (64, 4, 576), (2 * 576, 576, 1)), INVALID),                          # pages overlap
    (lambda: torch.zeros(64, 4, 500, dtype=torch.bfloat16), INVALID),         # rows too narrow
])
def test_paged_pool_validation(pool, expected):
    a = _args(R=0)
    a["kv_pool"] = pool()
    assert _status(a) == expected, _lib.last_error()


def test_paged_extra_pool_is_rejected():
    a = _args2(pool_dtype=torch.bfloat16)
    a["extra_pool"] = torch.zeros(32, 4, 576, dtype=torch.bfloat16)
    for k in ("q", "indices", "extra_indices", "out", "lse"):
        a[k] = a[k][:0]
    assert _status2(a) == UNSUP


# ------------------------------------------------------- no-allocation entry

def test_noalloc_validates_before_any_hip_call():
    """The no-allocation forward takes the forward's checks, and a caller
    workspace is refused (its partials go to the library's fixed scratch)."""
    a = _args()
    ws = torch.zeros(1024, dtype=torch.uint8)
    st = _lib.status_of_fwd_noalloc(a["q"], a["kv_pool"], a["kv_scale"], a["indices"],
                                    a["sm_scale"], a["out"], a["lse"], workspace=ws)
    assert st == INVALID
    b = _args()
    st = _lib.status_of_fwd_noalloc(b["q"].float(), b["kv_pool"], b["kv_scale"], b["indices"],
                                    b["sm_scale"], b["out"], b["lse"])
    assert st == UNSUP
    c = _args(R=0)
    st = _lib.status_of_fwd_noalloc(c["q"], c["kv_pool"], c["kv_scale"], c["indices"],
                                    c["sm_scale"], c["out"], c["lse"])
    assert st == _lib.SMLA_OK                     # R == 0: a no-op, no HIP call


def test_workspace_query_without_a_gpu():
    assert _lib.workspace_bytes(-1) == -1
    assert _lib.workspace_bytes(64) == -1
    assert _lib.workspace_bytes(0) == 0           # nothing allocated without a split call


def test_plan_rejects_unknown_variants():
    with pytest.raises(_lib.SparseMLAError):
        _plan(64, 64, variant=5)
    with pytest.raises(_lib.SparseMLAError):
        _plan(64, 16, variant=2)                   # 2 is a 64-head kernel
    with pytest.raises(_lib.SparseMLAError):
        _plan(64, 16, variant=4)                   # 4 is a 64-head fp8 kernel
    with pytest.raises(_lib.SparseMLAError):
        _plan(64, 64, dtype=torch.bfloat16, variant=4)
    assert _plan(64, 64, variant=4)["variant"] == 0
    assert _plan(64, 64, variant=2)["variant"] == 2
    assert _plan(64, 16, variant=1)["variant"] == 1


def test_plan_rejects_negative_workgroups():
    """The workgroup cap of kernels that walk several items per workgroup:
    0 = one per compute unit, positive = at most that many, negative is an
    error (the plan itself does not depend on it)."""
    with pytest.raises(_lib.SparseMLAError):
        _plan(8192, 64, variant=3, workgroups=-1)
    assert _plan(8192, 64, variant=3, workgroups=3) == _plan(8192, 64, variant=3)


def test_plan_fp8_dot_kernel_eligibility():
    """Variant 3 (the fp8-dot 64-head kernel) addresses pool rows through a
    structured buffer: 64-head blocks over fp8 pools only, row pitch under
    16 KB, pages a whole number of rows apart; other layouts take variant 0."""
    assert _plan(64, 64, variant=3)["variant"] == 3
    with pytest.raises(_lib.SparseMLAError):
        _plan(64, 64, dtype=torch.bfloat16, variant=3)
    q = torch.zeros(8, 64, 576, dtype=torch.bfloat16)
    idx = torch.zeros(8, 256, dtype=torch.int32)
    flat = torch.zeros(4096, 576, dtype=torch.float8_e4m3fn)
    paged_ok = torch.zeros(64 * 65 * 576, dtype=torch.float8_e4m3fn).as_strided(
        (64, 64, 576), (65 * 576, 576, 1))
    paged_odd = torch.zeros(64 * (64 * 576 + 1024), dtype=torch.float8_e4m3fn).as_strided(
        (64, 64, 576), (64 * 576 + 1024, 576, 1))
    wide = torch.zeros(16, 20000, dtype=torch.float8_e4m3fn)[:, :576]
    assert _lib.sparse_mla_plan(q, flat, idx, variant=3)["variant"] == 3
    assert _lib.sparse_mla_plan(q, paged_ok, idx, variant=3)["variant"] == 3
    assert _lib.sparse_mla_plan(q, paged_odd, idx, variant=3)["variant"] == 0
    assert _lib.sparse_mla_plan(q, wide, idx, variant=3)["variant"] == 0


def _call_args(src, start):
    """Top-level comma-separated arguments of the call whose '(' is at start."""
    depth, args, cur = 0, [], ""
    for ch in src[start:]:
        if ch == "(":
            depth += 1
            if depth == 1:
                continue
        elif ch == ")":
            depth -= 1
            if depth == 0:
                args.append(cur.strip())
                return args
        if ch == "," and depth == 1:
            args.append(cur.strip())
            cur = ""
        else:
            cur += ch
    raise AssertionError("unbalanced call")


def test_buffer_loads_keep_offsets_range_checked():
    """Every buffer load or store in the kernels passes its offset in the
    vector (or immediate) operand and 0 as the scalar offset: the hardware
    range check that turns out-of-range slots into zeros does not cover the
    scalar offset, so an offset there can read past a tensor's end."""
    csrc = os.path.join(os.path.dirname(_lib.__file__), "csrc")
    n = 0
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h")):
            continue
        src = open(os.path.join(csrc, name)).read()
        for m in re.finditer(r"__builtin_amdgcn_raw_buffer_(load|store)_\w+\s*\(", src):
            args = _call_args(src, m.end() - 1)
            soff = args[2] if m.group(1) == "load" else args[3]
            assert soff in ("0", "0u"), f"{name}: scalar offset {soff!r} in {m.group(0)}"
            n += 1
        for m in re.finditer(r"buffer_(load|store)_dword\w*\s+%\d+,\s*%\d+,\s*(\S+)", src):
            assert m.group(2) == "0", f"{name}: scalar offset {m.group(2)!r} in inline asm"
            n += 1
    assert n > 10
