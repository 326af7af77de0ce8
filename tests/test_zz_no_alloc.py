"""GPU check of sparse_mla_fwd_noalloc, the forward for callers that cannot
allocate device memory (its split partials live in a fixed per-device
scratch array instead of a hipMalloc'ed workspace).

Through the C ABI, its output must equal sparse_mla_fwd_ex's on the same
inputs and plan bit for bit (the same kernels run; only the partials' buffer
differs), and both must meet the parity bar against the fp64 oracle. Two
calls in a row, the second with a smaller input, show that the scratch's
stale contents from the first call do not leak into the second. A plan whose
partials exceed the scratch is rejected before any launch.
"""

import pytest
import torch

from sparse_mla_attention_05_amd import _lib
from sparse_mla_attention_05_amd.inputs import custom_workload, make_inputs

from test_gpu_parity import _dev, assert_parity, run_oracle

pytestmark = pytest.mark.gpu

SCRATCH = 32 * 1024 * 1024


def _nan_out(R, H):
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def _pair(inp, **opts):
    """(noalloc out, lse), (fwd_ex out, lse) on the same inputs and options."""
    q, pool, scale, idx = _dev(inp)
    R, H = q.shape[0], q.shape[1]
    o1, l1 = _nan_out(R, H)
    _lib.sparse_mla_fwd_noalloc(q, pool, scale, idx, inp.sm_scale, o1, l1, **opts)
    torch.cuda.synchronize()
    o2, l2 = _nan_out(R, H)
    _lib.sparse_mla_fwd_ex(q, pool, scale, idx, inp.sm_scale, o2, l2, **opts)
    torch.cuda.synchronize()
    return (o1.cpu(), l1.cpu()), (o2.cpu(), l2.cpu())


def _same(a, b):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), "out differs from fwd_ex"
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)), "lse differs from fwd_ex"


CALLS = [
    # the larger input first, then a smaller one: 16-head fp8 decode kernel
    # with 4 splits, then the 64-head fp8 kernel with 3 splits and an empty row
    (dict(rows=40, heads=16, d_qk=576, topk=2048, pool_rows=20000, kv_dtype="fp8",
          invalid_per_row=100, seed=71), dict(splits=4)),
    (dict(rows=5, heads=64, d_qk=512, topk=700, pool_rows=4000, kv_dtype="fp8",
          invalid_per_row=33, seed=72), dict(splits=3, head_block=64)),
]


def test_noalloc_matches_fwd_ex_on_two_calls():
    for i, (shape, opts) in enumerate(CALLS):
        print(f"\n[noalloc] call {i}: {shape} {opts}", flush=True)
        inp = make_inputs(custom_workload(**shape))
        if i == 1:
            idx = inp.indices.clone()
            idx[2, :] = -1
            inp.indices = idx
        q, pool, _, idx = _dev(inp)
        plan = _lib.sparse_mla_plan(q, pool, idx, **opts)
        assert plan["splits"] > 1 and 0 < plan["workspace_bytes"] <= SCRATCH, plan
        na, ex = _pair(inp, **opts)
        _same(na, ex)
        ref_out, ref_lse = run_oracle(inp)
        stats = assert_parity(na[0], na[1], ref_out, ref_lse, inp.indices)
        print(f"[noalloc] call {i}: bitwise equal to fwd_ex; {stats}", flush=True)


def test_noalloc_unsplit_and_rejections():
    inp = make_inputs(custom_workload(rows=9, heads=16, d_qk=576, topk=512, pool_rows=4000,
                                      kv_dtype="fp8", invalid_per_row=20, seed=73))
    print("\n[noalloc] unsplit call", flush=True)
    na, ex = _pair(inp, splits=1)
    _same(na, ex)
    q, pool, scale, idx = _dev(inp)
    out, lse = _nan_out(q.shape[0], q.shape[1])
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    st = _lib.status_of_fwd_noalloc(q, pool, scale, idx, inp.sm_scale, out, lse, workspace=ws)
    assert st == _lib.SMLA_ERR_INVALID_ARG, st
    # partials past the scratch: 300 rows x 64 heads x 8 splits x 2052 B
    big = make_inputs(custom_workload(rows=300, heads=64, d_qk=512, topk=1024, pool_rows=4000,
                                      kv_dtype="fp8", seed=74))
    q, pool, scale, idx = _dev(big)
    plan = _lib.sparse_mla_plan(q, pool, idx, splits=8, head_block=64)
    assert plan["workspace_bytes"] > SCRATCH
    out, lse = _nan_out(q.shape[0], q.shape[1])
    print("[noalloc] oversize plan", flush=True)
    st = _lib.status_of_fwd_noalloc(q, pool, scale, idx, big.sm_scale, out, lse, splits=8,
                                    head_block=64)
    assert st == _lib.SMLA_ERR_UNSUPPORTED, st
    assert "scratch" in _lib.last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a rejected call must launch nothing"
