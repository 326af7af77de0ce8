"""The seeded generators: determinism and the structure each workload promises."""

import torch

from sparse_mla_attention_05_amd.inputs import (
    WORKLOADS, custom_workload, distinct_indices, make_inputs, quantize_fp8, tensor_digest)


def test_same_seed_same_bytes():
    a, b = make_inputs("tiny"), make_inputs("tiny")
    for x, y in ((a.q, b.q), (a.pool, b.pool), (a.indices, b.indices)):
        assert tensor_digest(x) == tensor_digest(y)
    c = make_inputs(custom_workload(seed=1))
    assert tensor_digest(c.q) != tensor_digest(a.q)


def test_tiny_structure():
    inp = make_inputs("tiny")
    w = WORKLOADS["tiny"]
    assert inp.q.shape == (4, 16, 576) and inp.q.dtype == torch.bfloat16
    assert inp.pool.shape == (4096, 576) and inp.pool.dtype == torch.bfloat16
    assert inp.indices.shape == (4, 128) and inp.indices.dtype == torch.int32
    assert inp.kv_scale is None and abs(inp.sm_scale - 576 ** -0.5) < 1e-15
    for r in range(4):
        row = inp.indices[r]
        assert int((row == -1).sum()) == w.invalid_per_row
        v = row[row >= 0]
        assert v.unique().numel() == v.numel() and int(v.max()) < 4096


def test_distinct_indices_ranges_and_uniqueness():
    g = torch.Generator().manual_seed(0)
    lo = torch.tensor([0, 100, 5000])
    hi = torch.tensor([300, 400, 5300])
    idx = distinct_indices(lo, hi, 256, g)
    for r in range(3):
        v = idx[r].to(torch.int64)
        assert v.unique().numel() == 256
        assert int(v.min()) >= int(lo[r]) and int(v.max()) < int(hi[r])


def test_distinct_indices_full_range():
    """k equal to the range size must return a permutation of the range."""
    g = torch.Generator().manual_seed(1)
    idx = distinct_indices(torch.tensor([10]), torch.tensor([74]), 64, g)
    assert sorted(idx[0].tolist()) == list(range(10, 74))


def test_fp8_quantiser():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(1000, 64, generator=g)
    codes, s = quantize_fp8(x)
    assert codes.dtype == torch.float8_e4m3fn and s.dtype == torch.float32
    v = codes.to(torch.float32)
    assert torch.isfinite(v).all() and float(v.abs().max()) == 448.0
    assert float((v * s - x).abs().max()) < float(x.abs().max()) / 16


def test_prefix_rows_match_full_draw():
    w = custom_workload(rows=10, topk=64, pool_rows=2048, invalid_per_row=3, seed=5)
    full = make_inputs(w)
    part = make_inputs(w, rows=4)
    assert torch.equal(part.q, full.q[:4]) and torch.equal(part.indices, full.indices[:4])


def test_causal_and_request_ranges():
    w = custom_workload(rows=12, topk=32, pool_rows=600, index_mode="causal", first_pos=200, seed=3)
    inp = make_inputs(w)
    for i in range(12):
        assert int(inp.indices[i].max()) <= 200 + i
    w2 = custom_workload(rows=12, topk=40, pool_rows=4 * 64, index_mode="request",
                         rows_per_request=3, ctx_per_request=64, invalid_per_row=2, seed=4)
    inp2 = make_inputs(w2)
    for r in range(12):
        v = inp2.indices[r][inp2.indices[r] >= 0]
        b = r // 3
        assert int(v.min()) >= 64 * b and int(v.max()) < 64 * (b + 1)
