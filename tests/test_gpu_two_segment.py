"""GPU parity of the two-segment forward (sparse_mla_fwd2, through the C ABI)
against the fp64 two-segment oracle.

Same bar as the one-segment parity tests: max |out - ref| <= 2e-2 and
||out - ref||_F / ||ref||_F <= 5e-3 for the bf16 output, |lse - ref| <= 1e-3
on rows with a valid slot in either segment, and exactly out = 0, lse = -inf
on rows with none. Outputs start NaN-poisoned.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_05_amd import _lib
from sparse_mla_attention_05_amd.inputs import custom_workload, make_extra_segment, make_inputs
from test_gpu_parity import assert_parity

pytestmark = pytest.mark.gpu


def _workload(kv, d_qk, heads, topk, mode, rows=12, seed=41):
    if mode == "request":
        w = custom_workload(rows=rows, heads=heads, d_qk=d_qk, pool_rows=(rows // 6 + 1) * 4096,
                            topk=topk, kv_dtype=kv, seed=seed, index_mode="request",
                            rows_per_request=6, ctx_per_request=4096, invalid_per_row=5)
    elif mode == "causal":
        w = custom_workload(rows=rows, heads=heads, d_qk=d_qk, pool_rows=8192, topk=topk,
                            kv_dtype=kv, seed=seed, index_mode="causal", first_pos=4000,
                            invalid_per_row=5)
    else:
        w = custom_workload(rows=rows, heads=heads, d_qk=d_qk, pool_rows=8192, topk=topk,
                            kv_dtype=kv, seed=seed, invalid_per_row=5)
    return make_inputs(w)


def run_gpu2(inp, ex, extra_scale="own", pool=None, **opts):
    q, idx = inp.q.cuda(), inp.indices.cuda()
    pool = inp.pool.cuda() if pool is None else pool
    s1 = inp.kv_scale.cuda() if inp.kv_scale is not None else None
    es = ex.kv_scale if extra_scale == "own" else extra_scale
    s2 = es.cuda() if es is not None else None
    R, H = q.shape[0], q.shape[1]
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    _lib.sparse_mla_fwd2(q, pool, s1, idx, ex.pool.cuda(), s2, ex.indices.cuda(), inp.sm_scale,
                         out, lse, **opts)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle2(inp, ex, extra_scale="own", rows=None):
    es = ex.kv_scale if extra_scale == "own" else extra_scale
    return oracle.sparse_mla_fwd_2seg_torch(inp.q, inp.pool, inp.kv_scale, inp.indices, ex.pool, es,
                                            ex.indices, inp.sm_scale, rows=rows)


def _both(inp, ex):
    return torch.cat([inp.indices, ex.indices], dim=1)


CASES = [
    # kv, d_qk, heads, top-k, window, index mode, planner overrides
    ("fp8", 576, 16, 512, 128, "request", {}),
    ("bf16", 576, 64, 512, 128, "request", {}),
    ("fp8", 576, 64, 2048, 128, "causal", {}),
    ("fp8", 512, 64, 2048, 128, "causal", {}),
    ("fp8", 576, 16, 2048, 100, "uniform", {}),
    ("bf16", 512, 32, 300, 64, "causal", {}),
    ("fp8", 576, 16, 1000, 128, "request", dict(head_block=16, splits=3)),
    ("bf16", 576, 64, 512, 128, "request", dict(head_block=64, splits=2)),
    ("fp8", 576, 80, 512, 128, "request", {}),
    # 16-head fp8 decode kernel walking both segments, splits across the
    # segment boundary and one split holding only second-segment slots
    ("fp8", 576, 16, 512, 128, "uniform", dict(head_block=16, splits=5)),
    ("fp8", 512, 16, 2048, 128, "causal", {}),
    # the same shape through the composition (another 16-head instance)
    ("fp8", 576, 16, 512, 128, "request", dict(variant=1)),
    # 64-head bf16 kernel walking both segments: main top-k padded to whole
    # tiles, splits across the boundary; and the composition for comparison
    ("bf16", 576, 64, 300, 100, "causal", {}),
    ("bf16", 512, 64, 1000, 128, "uniform", dict(head_block=64, splits=3)),
    ("bf16", 576, 64, 512, 128, "request", dict(variant=1)),
    # 64-head fp8-dot kernel walking both segments: ragged last tiles in both,
    # splits that straddle the segment boundary; the 4-wave kernel composes
    # the two segments through the combine kernel
    ("fp8", 576, 64, 300, 100, "causal", {}),
    ("fp8", 512, 64, 300, 100, "uniform", dict(head_block=64, splits=3)),
    ("fp8", 576, 64, 1000, 128, "request", dict(variant=4)),
]


@pytest.mark.parametrize("kv,d_qk,heads,topk,window,mode,opts", CASES)
def test_two_segment_parity(kv, d_qk, heads, topk, window, mode, opts):
    print(f"\n[two-segment] kv={kv} d_qk={d_qk} H={heads} K={topk} W={window} {mode} {opts}",
          flush=True)
    inp = _workload(kv, d_qk, heads, topk, mode)
    ex = make_extra_segment(inp, window, seed=77, value_std=0.7, invalid_per_row=3)
    # row 1: no valid main slot; row 2: no valid extra slot; row 3: neither
    inp.indices[1] = -1
    inp.indices[3] = -1
    ex.indices[2] = -1
    ex.indices[3] = -1
    out, lse = run_gpu2(inp, ex, **opts)
    ref_out, ref_lse = run_oracle2(inp, ex)
    stats = assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex))
    print(f"[two-segment] {stats}", flush=True)


def test_two_segment_default_extra_scale():
    """extra_kv_scale NULL: the extra segment uses kv_scale."""
    inp = _workload("fp8", 576, 16, 512, "request")
    ex = make_extra_segment(inp, 128, seed=5, value_std=0.7)
    out, lse = run_gpu2(inp, ex, extra_scale=None)
    ref_out, ref_lse = run_oracle2(inp, ex, extra_scale=None)
    assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex))


def test_two_segment_caller_workspace_is_bitwise_equal():
    inp = _workload("bf16", 576, 64, 512, "request")
    ex = make_extra_segment(inp, 128, seed=6)
    q, pool, idx = inp.q.cuda(), inp.pool.cuda(), inp.indices.cuda()
    xp, xi = ex.pool.cuda(), ex.indices.cuda()
    _, _, ws_bytes = _lib.sparse_mla_plan2(q, pool, idx, xp, xi)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = []
    for kw in ({}, dict(workspace=ws, workspace_bytes=ws_bytes)):
        out = torch.full((12, 64, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((12, 64), float("nan"), dtype=torch.float32, device="cuda")
        _lib.sparse_mla_fwd2(q, pool, None, idx, xp, None, xi, inp.sm_scale, out, lse, **kw)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    small = torch.empty(ws_bytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.SparseMLAError):
        out = torch.empty((12, 64, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((12, 64), dtype=torch.float32, device="cuda")
        _lib.sparse_mla_fwd2(q, pool, None, idx, xp, None, xi, inp.sm_scale, out, lse,
                             workspace=small, workspace_bytes=ws_bytes - 256)


@pytest.mark.parametrize("name,window,every", [("decode_bf16", 128, 1), ("decode_fp8", 128, 8)])
def test_two_segment_on_decode_workloads(name, window, every):
    """The decode workloads with a 128-slot sliding window as the extra
    segment (its own pool and fp8 scale); every `every`-th row is checked."""
    print(f"\n[two-segment] workload={name} window={window}", flush=True)
    inp = make_inputs(name)
    ex = make_extra_segment(inp, window, seed=1001, value_std=0.7, invalid_per_row=2)
    out, lse = run_gpu2(inp, ex)
    R = inp.q.shape[0]
    rows = np.unique(np.r_[np.arange(0, R, every), R - 1])
    ref_out, ref_lse = run_oracle2(inp, ex, rows=rows)
    stats = assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex), rows=torch.from_numpy(rows))
    print(f"[two-segment] {name}: {stats}", flush=True)


def test_fp8dot_two_segments_streaming_on_sampled_rows():
    """600 rows of 64 heads in one split: the fp8-dot kernel's workgroups walk
    several rows each as one stream of tiles (3 main tiles, then 2 of the
    second segment, so the next row's first tiles, fetched ahead, include
    second-segment ones). The oracle checks every 16th row plus the last."""
    print("\n[two-segment] fp8-dot streaming, 600 rows, K=192, W=128", flush=True)
    inp = _workload("fp8", 576, 64, 192, "causal", rows=600, seed=43)
    ex = make_extra_segment(inp, 128, seed=78, value_std=0.7, invalid_per_row=3)
    p1, p2, _ = _lib.sparse_mla_plan2(inp.q, inp.pool, inp.indices, ex.pool, ex.indices, splits=1)
    assert p1["variant"] == 3 and p1["splits"] == 1 and p2["grid"] == 0
    out, lse = run_gpu2(inp, ex, splits=1)
    R = inp.q.shape[0]
    rows = np.unique(np.r_[np.arange(0, R, 16), R - 1])
    ref_out, ref_lse = run_oracle2(inp, ex, rows=rows)
    stats = assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex), rows=torch.from_numpy(rows))
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    print(f"[two-segment] {stats}", flush=True)


@pytest.mark.parametrize("ratio", [16.0, 1.0 / 16.0])
def test_fp8dot_two_segments_scale_ratio(ratio):
    """A second-segment scale about 16 times (or 1/16 of) the main one, with
    its codes divided by the same factor (clamped to the e4m3 range), so
    that keys and values keep their magnitudes (and the absolute bounds
    their meaning) while the fp8-dot kernel's one launch weighs the two
    segments' codes by scales far apart."""
    inp = _workload("fp8", 576, 64, 512, "causal", seed=44)
    ex = make_extra_segment(inp, 128, seed=79, value_std=0.7, invalid_per_row=3)
    ex.pool = (ex.pool.float() / ratio).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    s2 = (ex.kv_scale.float() * ratio).reshape(1)
    out, lse = run_gpu2(inp, ex, extra_scale=s2)
    ref_out, ref_lse = run_oracle2(inp, ex, extra_scale=s2)
    print(f"\n[two-segment] ratio {ratio}: {assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex))}",
          flush=True)


@pytest.mark.parametrize("d_qk,page_rows,pad", [(576, 64, 576), (512, 32, 512)])
def test_fp8dot_two_segments_paged_main_pool(d_qk, page_rows, pad):
    """A paged main pool (pages a whole number of rows apart) in the fp8-dot
    kernel's two-segment launch gives the flat pool's result bit for bit (same
    plan, only the main rows' addresses differ), and so the oracle's."""
    from test_gpu_variants import paged_pool

    inp = _workload("fp8", d_qk, 64, 300, "causal", seed=45)
    ex = make_extra_segment(inp, 100, seed=80, value_std=0.7, invalid_per_row=3)
    flat_out, flat_lse = run_gpu2(inp, ex)
    _keep, paged = paged_pool(inp.pool, page_rows, pad)
    p1, p2, _ = _lib.sparse_mla_plan2(inp.q, paged, inp.indices, ex.pool, ex.indices)
    assert p1["variant"] == 3 and p2["grid"] == 0
    out, lse = run_gpu2(inp, ex, pool=paged)
    assert torch.equal(out, flat_out) and torch.equal(lse, flat_lse)
    ref_out, ref_lse = run_oracle2(inp, ex)
    print(f"\n[two-segment paged] {assert_parity(out, lse, ref_out, ref_lse, _both(inp, ex))}",
          flush=True)
