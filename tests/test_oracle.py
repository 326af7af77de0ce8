"""Pins for the fp64 oracle: each checks it against something other than itself.

CPU only. Sizes are tiny (R <= 8, H <= 16, K <= 256) so the whole file runs in
seconds. The pins are chosen so a plausible mistake (a dropped rope term, a
wrong sign, log2 instead of ln, a transposed operand, a mishandled invalid or
duplicate slot) fails at least one of them; ``test_planted_mistakes_are_caught``
checks that claim by planting such mistakes in copies of the oracle.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sparse_mla_oracle as orc
from sparse_mla_attention_05_amd.inputs import custom_workload, make_extra_segment, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(inp, rows=None, fn=None):
    fn = fn or oracle.sparse_mla_fwd_torch
    return fn(inp.q, inp.pool, inp.kv_scale, inp.indices, inp.sm_scale, rows=rows)


def _brute_force(inp):
    """Dense attention over the materialised gathered rows, per query row, using
    torch's own dtype conversions and scaled_dot_product_attention in fp64."""
    R, H, D = inp.q.shape
    sm = float(np.float32(inp.sm_scale))
    if inp.pool.dtype == torch.float8_e4m3fn:
        pool = inp.pool[:, :D].to(torch.float64) * float(inp.kv_scale[0])
    else:
        pool = inp.pool[:, :D].to(torch.float64)
    outs, lses = [], []
    for r in range(R):
        idx = inp.indices[r].to(torch.int64)
        idx = idx[idx >= 0]
        if idx.numel() == 0:
            outs.append(torch.zeros(H, 512, dtype=torch.float64))
            lses.append(torch.full((H,), -math.inf, dtype=torch.float64))
            continue
        g = pool[idx]                                          # [n, D]
        qr = inp.q[r].to(torch.float64)                        # [H, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qr[:, None, :], g[None].expand(H, -1, -1), g[None, :, :512].expand(H, -1, -1), scale=sm)
        outs.append(o[:, 0, :])
        lses.append(torch.logsumexp(sm * torch.mm(qr, g.t()), dim=1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _small(kv_dtype="bf16", d_qk=576, invalid=5, seed=7, rows=6, heads=16, topk=96, pool_rows=512):
    w = custom_workload(rows=rows, heads=heads, d_qk=d_qk, pool_rows=pool_rows, topk=topk,
                        kv_dtype=kv_dtype, seed=seed, invalid_per_row=invalid)
    return make_inputs(w)


# ------------------------------------------------------------------ decoding

def test_e4m3fn_table_matches_torch_all_codes():
    lut = oracle.e4m3fn_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_lut, nan_ref = np.isnan(lut), np.isnan(ref)
    assert np.array_equal(nan_lut, nan_ref)
    assert set(np.nonzero(nan_lut)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(lut[~nan_lut], ref[~nan_ref])
    assert np.array_equal(np.signbit(lut[~nan_lut]), np.signbit(ref[~nan_ref]))
    assert lut[0x7E] == 448.0 and lut[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(4096, generator=g) * torch.exp(torch.randn(4096, generator=g) * 8)).to(torch.bfloat16)
    assert np.array_equal(oracle.bf16_bits_to_f64(_bits(x)), x.to(torch.float64).numpy())


# ------------------------------------------------------- whole-result pins

@pytest.mark.parametrize("kv_dtype,d_qk", [("bf16", 576), ("bf16", 512), ("fp8", 576), ("fp8", 512)])
def test_matches_dense_sdpa(kv_dtype, d_qk):
    inp = _small(kv_dtype, d_qk)
    out, lse = _run(inp)
    bo, bl = _brute_force(inp)
    assert _rel(out, bo) < 1e-12
    assert np.max(np.abs(lse - bl)) < 1e-12


def test_large_scores_are_stable():
    inp = _small()
    inp.q = (inp.q.to(torch.float32) * 60).to(torch.bfloat16)
    out, lse = _run(inp)
    bo, bl = _brute_force(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert _rel(out, bo) < 1e-12
    assert np.max(np.abs(lse - bl) / np.abs(bl)) < 1e-12


def test_lse_ties_halves_to_whole():
    """Splitting each row's slots into two disjoint sets: the LSE-weighted mix of
    the halves' outputs is the whole output, and ln(e^lse_a + e^lse_b) the whole
    LSE. This ties the LSE (base, scale, shift) to the SDPA-pinned outputs and
    pins lse_combine."""
    inp = _small(invalid=0, topk=128)
    out, lse = _run(inp)
    g = torch.Generator().manual_seed(3)
    perm = torch.argsort(torch.rand(inp.indices.shape, generator=g), dim=1)
    shuffled = torch.gather(inp.indices, 1, perm)
    parts_o, parts_l = [], []
    for half in (shuffled[:, :50], shuffled[:, 50:]):
        a = make_inputs(custom_workload(rows=1))
        a.q, a.pool, a.kv_scale, a.indices, a.sm_scale = inp.q, inp.pool, inp.kv_scale, half.contiguous(), inp.sm_scale
        o, l_ = _run(a)
        parts_o.append(o)
        parts_l.append(l_)
    lse_mix = np.logaddexp(parts_l[0], parts_l[1])
    w0 = np.exp(parts_l[0] - lse_mix)[..., None]
    w1 = np.exp(parts_l[1] - lse_mix)[..., None]
    assert _rel(w0 * parts_o[0] + w1 * parts_o[1], out) < 1e-12
    assert np.max(np.abs(lse_mix - lse)) < 1e-12
    co, cl = oracle.lse_combine(np.stack(parts_o), np.stack(parts_l))
    assert _rel(co, out) < 1e-12 and np.max(np.abs(cl - lse)) < 1e-12


def test_lse_combine_all_invalid_and_empty_splits():
    po = np.random.default_rng(0).standard_normal((3, 2, 512))
    pl = np.array([[-np.inf, 0.5], [-np.inf, -np.inf], [-np.inf, 1.5]])
    o, l_ = oracle.lse_combine(po, pl)
    assert np.all(o[0] == 0) and l_[0] == -np.inf
    ref_l = np.logaddexp(0.5, 1.5)
    assert abs(l_[1] - ref_l) < 1e-15
    assert np.allclose(o[1], np.exp(0.5 - ref_l) * po[0, 1] + np.exp(1.5 - ref_l) * po[2, 1], rtol=0, atol=1e-15)


# ------------------------------------------------------------- invariants

def test_softmax_weights_sum_to_one():
    s = np.random.default_rng(1).standard_normal((16, 300)) * 30
    w, m, l = oracle.softmax_weights(s)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-12
    assert np.all(w >= 0)


def test_constant_values_give_constant_output():
    """If every gathered V row is the same constant vector, O equals it whatever
    the weights (they sum to 1)."""
    inp = _small(invalid=3)
    pool = inp.pool.clone()
    pool[:, :512] = torch.tensor(0.375, dtype=torch.bfloat16)
    inp.pool = pool
    out, _ = _run(inp)
    assert np.max(np.abs(out - 0.375)) < 1e-12


def test_all_invalid_rows_exact():
    inp = _small()
    idx = inp.indices.clone()
    idx[1] = -1
    idx[4] = -7  # any negative index is invalid
    inp.indices = idx
    out, lse = _run(inp)
    for r in (1, 4):
        assert np.all(out[r] == 0.0) and np.all(lse[r] == -np.inf)
    assert np.all(np.isfinite(lse[[0, 2, 3, 5]]))


def test_compaction_invariance():
    inp = _small(invalid=20)
    out, lse = _run(inp)
    rows = []
    for r in range(inp.indices.shape[0]):
        v = inp.indices[r][inp.indices[r] >= 0]
        rows.append(v[:76])
    inp.indices = torch.stack(rows)
    assert inp.indices.shape[1] == 76
    out2, lse2 = _run(inp)
    assert np.max(np.abs(out - out2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


def test_permutation_invariance():
    inp = _small(invalid=9)
    out, lse = _run(inp)
    g = torch.Generator().manual_seed(5)
    perm = torch.argsort(torch.rand(inp.indices.shape, generator=g), dim=1)
    inp.indices = torch.gather(inp.indices, 1, perm).contiguous()
    out2, lse2 = _run(inp)
    assert np.max(np.abs(out - out2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


# ---------------------------------------------------------- special cases

def test_single_valid_slot():
    inp = _small(kv_dtype="fp8")
    idx = torch.full_like(inp.indices, -1)
    idx[:, 17] = inp.indices[:, 17].abs()
    inp.indices = idx
    out, lse = _run(inp)
    s = float(inp.kv_scale[0])
    for r in range(idx.shape[0]):
        row = inp.pool[int(idx[r, 17])].to(torch.float64).numpy() * s
        assert np.array_equal(out[r], np.broadcast_to(row[:512], out[r].shape))
        q = inp.q[r].to(torch.float64).numpy()
        sc = float(np.float32(inp.sm_scale)) * (q @ row[:576])
        assert np.max(np.abs(lse[r] - sc)) < 1e-12


def test_zero_query_gives_mean_and_log_count():
    inp = _small(invalid=7)
    inp.q = torch.zeros_like(inp.q)
    out, lse = _run(inp)
    pool = inp.pool.to(torch.float64).numpy()
    for r in range(inp.indices.shape[0]):
        v = inp.indices[r][inp.indices[r] >= 0].numpy()
        assert np.max(np.abs(out[r] - pool[v, :512].mean(axis=0))) < 1e-13
        assert np.max(np.abs(lse[r] - math.log(len(v)))) < 1e-13


def test_identical_rows_give_that_row():
    inp = _small(invalid=4)
    pool = inp.pool.clone()
    pool[:] = pool[3]
    inp.pool = pool
    out, lse = _run(inp)
    row = pool[3].to(torch.float64).numpy()
    sm = float(np.float32(inp.sm_scale))
    for r in range(inp.indices.shape[0]):
        kv = int((inp.indices[r] >= 0).sum())
        s = sm * (inp.q[r].to(torch.float64).numpy() @ row)
        assert np.max(np.abs(out[r] - row[:512])) < 1e-13
        assert np.max(np.abs(lse[r] - (s + math.log(kv)))) < 1e-12


def test_duplicate_slot_counts_twice():
    inp = _small(rows=1, heads=2, topk=5, invalid=0, pool_rows=64)
    idx = torch.tensor([[10, 20, 10, -1, 30]], dtype=torch.int32)
    inp.indices = idx
    out, lse = _run(inp)
    pool = inp.pool.to(torch.float64).numpy()
    sm = float(np.float32(inp.sm_scale))
    q = inp.q[0].to(torch.float64).numpy()
    for h in range(2):
        s = {j: sm * (q[h] @ pool[j]) for j in (10, 20, 30)}
        wts = {10: 2 * math.exp(s[10]), 20: math.exp(s[20]), 30: math.exp(s[30])}
        z = sum(wts.values())
        ref = sum(wts[j] * pool[j, :512] for j in wts) / z
        assert np.max(np.abs(out[0, h] - ref)) < 1e-13
        assert abs(lse[0, h] - math.log(z)) < 1e-12


def test_fp8_scale_folding_identity():
    """oracle(fp8 codes C, scale s, sm) == s * oracle(bf16 pool holding C, sm * s).
    s is a power of two so that sm * s is exact in fp32."""
    inp = _small(kv_dtype="fp8", invalid=3)
    s = 2.0 ** -5
    inp.kv_scale = torch.tensor([s], dtype=torch.float32)
    out8, lse8 = _run(inp)
    b = make_inputs(custom_workload(rows=1))
    b.q, b.indices = inp.q, inp.indices
    b.pool = inp.pool.to(torch.float32).to(torch.bfloat16)  # e4m3 values are exact in bf16
    assert torch.equal(b.pool.to(torch.float32), inp.pool.to(torch.float32))
    b.kv_scale = None
    b.sm_scale = float(np.float32(inp.sm_scale)) * s
    outb, lseb = _run(b)
    assert np.max(np.abs(out8 - s * outb)) < 1e-15
    assert np.max(np.abs(lse8 - lseb)) < 1e-13


def test_index_beyond_pool_raises():
    inp = _small()
    idx = inp.indices.clone()
    idx[2, 5] = inp.pool.shape[0]
    inp.indices = idx
    with pytest.raises(IndexError):
        _run(inp)


def test_padded_pitch_pool_same_result():
    w = custom_workload(rows=3, heads=16, pool_rows=300, topk=40, seed=9, pool_pitch=640, invalid_per_row=2)
    inp = make_inputs(w)
    assert inp.pool.shape == (300, 640)
    out, lse = _run(inp)
    inp2 = make_inputs(w)
    inp2.pool = inp.pool[:, :576].contiguous()
    out2, lse2 = _run(inp2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# --------------------------------------------------------- two segments

def _two_seg(kv_dtype="fp8", d_qk=576, window=40, invalid=3, extra_invalid=2, std=1.7, seed=21):
    inp = _small(kv_dtype, d_qk, invalid=invalid, seed=seed)
    w = inp.workload
    inp.workload = custom_workload(**{**w.__dict__, "index_mode": "uniform"})
    ex = make_extra_segment(inp, window, seed=seed + 1, value_std=std, invalid_per_row=extra_invalid)
    return inp, ex


def _run2(inp, ex, extra_scale="own"):
    es = ex.kv_scale if extra_scale == "own" else extra_scale
    return oracle.sparse_mla_fwd_2seg_torch(inp.q, inp.pool, inp.kv_scale, inp.indices, ex.pool, es,
                                            ex.indices, inp.sm_scale)


def _concat(inp, ex, pool):
    """One-segment inputs over [main pool; extra pool] with the extra indices
    shifted past the main pool (invalid slots stay -1)."""
    n1 = inp.pool.shape[0]
    shifted = torch.where(ex.indices >= 0, ex.indices + n1, ex.indices)
    c = make_inputs(custom_workload(rows=1))
    c.q, c.sm_scale = inp.q, inp.sm_scale
    c.indices = torch.cat([inp.indices, shifted], dim=1).contiguous()
    c.pool = pool
    return c


def test_two_segment_equal_scales_is_one_concatenated_pool():
    """Extra scale left out (it defaults to kv_scale): the same as attention
    over the concatenated fp8 pools with all slots in one index row."""
    inp, ex = _two_seg("fp8")
    out2, lse2 = _run2(inp, ex, extra_scale=None)
    c = _concat(inp, ex, torch.cat([inp.pool, ex.pool]))
    c.kv_scale = inp.kv_scale
    out1, lse1 = _run(c)
    assert np.max(np.abs(out2 - out1)) < 1e-15 and np.max(np.abs(lse2 - lse1)) < 1e-13


@pytest.mark.parametrize("d_qk", [576, 512])
def test_two_segment_scale_folding(d_qk):
    """Scales 2^-6 (main) and 2^-4 (extra), sm = 2^-4: the two-segment result
    is 2^-6 times one-segment attention over one bf16 pool holding the main
    codes and 4x the extra codes (all exact in bf16), with sm * 2^-6."""
    inp, ex = _two_seg("fp8", d_qk=d_qk)
    inp.kv_scale = torch.tensor([2.0 ** -6], dtype=torch.float32)
    ex.kv_scale = torch.tensor([2.0 ** -4], dtype=torch.float32)
    inp.sm_scale = 2.0 ** -4
    out2, lse2 = _run2(inp, ex)
    main = inp.pool.to(torch.float32)
    extra = ex.pool.to(torch.float32) * 4
    pool = torch.cat([main, extra]).to(torch.bfloat16)
    assert torch.equal(pool.to(torch.float32), torch.cat([main, extra]))
    c = _concat(inp, ex, pool)
    c.kv_scale = None
    c.sm_scale = 2.0 ** -10
    out1, lse1 = _run(c)
    assert np.max(np.abs(out2 - 2.0 ** -6 * out1)) < 1e-15
    assert np.max(np.abs(lse2 - lse1)) < 1e-13


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_two_segment_empty_segment_leaves_the_other(kv_dtype):
    inp, ex = _two_seg(kv_dtype)
    main_out, main_lse = _run(inp)
    none = torch.full_like(ex.indices, -1)
    ex_empty = type(ex)(pool=ex.pool, kv_scale=ex.kv_scale, indices=none)
    out, lse = _run2(inp, ex_empty)
    assert np.array_equal(out, main_out) and np.array_equal(lse, main_lse)
    only = make_inputs(custom_workload(rows=1))
    only.q, only.pool, only.kv_scale, only.indices, only.sm_scale = (
        inp.q, ex.pool, ex.kv_scale, ex.indices, inp.sm_scale)
    ex_out, ex_lse = _run(only)
    inp_empty = make_inputs(custom_workload(rows=1))
    inp_empty.q, inp_empty.pool, inp_empty.kv_scale, inp_empty.sm_scale = inp.q, inp.pool, inp.kv_scale, inp.sm_scale
    inp_empty.indices = torch.full_like(inp.indices, -1)
    out, lse = _run2(inp_empty, ex)
    assert np.array_equal(out, ex_out) and np.array_equal(lse, ex_lse)
    both = type(ex)(pool=ex.pool, kv_scale=ex.kv_scale, indices=none)
    out, lse = _run2(inp_empty, both)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_two_segment_matches_dense_sdpa():
    """Brute force with torch's own conversions over the union of both
    segments' gathered rows, each pool scaled by its own factor."""
    inp, ex = _two_seg("fp8", std=0.6)
    out2, lse2 = _run2(inp, ex)
    sm = float(np.float32(inp.sm_scale))
    D = inp.q.shape[2]
    p1 = inp.pool[:, :D].to(torch.float64) * float(inp.kv_scale[0])
    p2 = ex.pool[:, :D].to(torch.float64) * float(ex.kv_scale[0])
    for r in range(inp.q.shape[0]):
        i1 = inp.indices[r].to(torch.int64)
        i2 = ex.indices[r].to(torch.int64)
        g = torch.cat([p1[i1[i1 >= 0]], p2[i2[i2 >= 0]]])
        qr = inp.q[r].to(torch.float64)
        H = qr.shape[0]
        o = torch.nn.functional.scaled_dot_product_attention(
            qr[:, None, :], g[None].expand(H, -1, -1), g[None, :, :512].expand(H, -1, -1), scale=sm)
        assert _rel(out2[r], o[:, 0, :].numpy()) < 1e-12
        l_ = torch.logsumexp(sm * torch.mm(qr, g.t()), dim=1).numpy()
        assert np.max(np.abs(lse2[r] - l_)) < 1e-12


# --------------------------------------------------------------- golden

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_form_golden(case):
    R, H, D, N = case["rows"], case["heads"], case["d_qk"], case["pool_rows"]
    q = torch.zeros(R, H, D)
    for r, h, d, v in case["q"]:
        q[r, h, d] = v
    pool = torch.zeros(N, D)
    for n, d, v in case["pool"]:
        pool[n, d] = v
    qb, pb = q.to(torch.bfloat16), pool.to(torch.bfloat16)
    assert torch.equal(qb.float(), q) and torch.equal(pb.float(), pool)
    idx = np.array(case["indices"], dtype=np.int32)
    out, lse = oracle.sparse_mla_fwd(_bits(qb), _bits(pb), "bf16", None, idx, case["sm_scale"])
    exp_out = np.zeros((R, H, 512))
    for r, h, d, v in case["expected_out"]:
        exp_out[r, h, d] = v
    assert np.max(np.abs(out - exp_out)) < 1e-15
    for r, h, c, arg in case["expected_lse"]:
        if c == "-inf":
            assert lse[r, h] == -np.inf
        else:
            a = 1 + math.exp(-2) if arg == "1+e^-2" else float(arg)
            assert abs(lse[r, h] - (c + math.log(a))) < 1e-15


# ------------------------------------------------- planted mistakes caught

def _mutant_attend(kind):
    def attend(q_row, gathered, sm):
        if kind == "drop_rope":
            scores = sm * (q_row[:, :512] @ gathered[:, :512].T)
        elif kind == "sign":
            scores = -sm * (q_row @ gathered.T)
        elif kind == "no_scale":
            scores = q_row @ gathered.T
        else:
            scores = sm * (q_row @ gathered.T)
        p, m, l = orc.softmax_weights(scores)
        out = p @ gathered[:, :512]
        lse = m + (np.log2(l) if kind == "log2" else np.log(l))
        if kind == "no_shift":
            lse = np.log(l)
        return out, lse
    return attend


@pytest.mark.parametrize("kind", ["drop_rope", "sign", "no_scale", "log2", "no_shift"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    inp = _small(invalid=4)
    monkeypatch.setattr(orc, "attend_row", _mutant_attend(kind))
    out, lse = _run(inp)
    bo, bl = _brute_force(inp)
    caught = _rel(out, bo) > 1e-6 or np.max(np.abs(lse - bl)) > 1e-6
    assert caught, f"mutation {kind} not caught by the dense-attention pin"


def test_planted_mask_mistake_is_caught(monkeypatch):
    """Treating index 0 as invalid (a plausible off-by-one in the mask) must fail
    the compaction pin's comparison against dense attention."""
    inp = _small(invalid=4)
    idx = inp.indices.clone()
    idx[0, 3] = 0
    inp.indices = idx
    real = orc.sparse_mla_fwd

    def mutant(q_bits, pool_raw, kv_dtype, kv_scale, indices, sm_scale, rows=None, q_scale=None):
        ind = np.where(indices == 0, -1, indices)
        return real(q_bits, pool_raw, kv_dtype, kv_scale, ind, sm_scale, rows=rows, q_scale=q_scale)

    monkeypatch.setattr(orc, "sparse_mla_fwd", mutant)
    out, _ = orc.sparse_mla_fwd_torch(inp.q, inp.pool, inp.kv_scale, inp.indices, inp.sm_scale)
    bo, _ = _brute_force(inp)
    assert _rel(out, bo) > 1e-6


# ------------------------------------------------------------------ fp8 q

def test_fp8_q_is_scale_folding_of_a_bf16_q():
    """An fp8 q with scale s attends like a bf16 q holding the codes' values
    (every e4m3fn value is a bf16 value) with sm_scale * s."""
    from sparse_mla_attention_05_amd.inputs import make_fp8_q
    inp = make_inputs(custom_workload(rows=5, heads=16, d_qk=576, pool_rows=2000, topk=100,
                                      kv_dtype="fp8", seed=8, invalid_per_row=3))
    q8, _ = make_fp8_q(inp)
    qs = torch.tensor([2.0 ** -5])   # a power of two: sm_scale * s stays exact in fp32
    a_out, a_lse = oracle.sparse_mla_fwd_torch(q8, inp.pool, inp.kv_scale, inp.indices,
                                               inp.sm_scale, q_scale=qs)
    q_as_bf16 = q8.to(torch.float32).to(torch.bfloat16)          # exact
    assert torch.equal(q_as_bf16.to(torch.float32), q8.to(torch.float32))
    sm = float(np.float32(inp.sm_scale)) * float(qs[0])
    b_out, b_lse = oracle.sparse_mla_fwd_torch(q_as_bf16, inp.pool, inp.kv_scale, inp.indices, sm)
    assert np.allclose(a_out, b_out, rtol=1e-12, atol=1e-14)
    assert np.allclose(a_lse, b_lse, rtol=1e-12, atol=1e-14)


def test_fp8_q_brute_force():
    from sparse_mla_attention_05_amd.inputs import make_fp8_q
    inp = make_inputs(custom_workload(rows=4, heads=16, d_qk=512, pool_rows=1500, topk=80,
                                      kv_dtype="bf16", seed=9, invalid_per_row=2))
    q8, qs = make_fp8_q(inp)
    got, got_lse = oracle.sparse_mla_fwd_torch(q8, inp.pool, None, inp.indices, inp.sm_scale,
                                               q_scale=qs)
    q = q8.to(torch.float64) * float(qs[0])
    sm = float(np.float32(inp.sm_scale))
    for r in range(4):
        idx = inp.indices[r][inp.indices[r] >= 0].long()
        kv = inp.pool[idx, :512].to(torch.float64)
        s = sm * (q[r] @ kv.T)
        w = torch.softmax(s, dim=-1)
        assert np.allclose(got[r], (w @ kv).numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(got_lse[r], torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12)
