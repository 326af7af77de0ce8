"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (per element over the whole output): max |out - ref| <= 2e-2 and
||out - ref||_F / ||ref||_F <= 5e-3 for the bf16 output; |lse - ref| <= 1e-3 on
every (row, head) with a valid slot; rows without a valid slot exactly out = 0
and lse = -inf. Every call writes into NaN-poisoned out/lse buffers, so an
element the kernel forgets to write fails the check.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_05_amd import _lib
from sparse_mla_attention_05_amd.inputs import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

OUT_MAX_ABS = 2e-2
OUT_REL_FRO = 5e-3
LSE_ABS = 1e-3


def _dev(inp):
    q = inp.q.cuda()
    pool = inp.pool.cuda()
    scale = inp.kv_scale.cuda() if inp.kv_scale is not None else None
    idx = inp.indices.cuda()
    return q, pool, scale, idx


def run_gpu(inp, dev=None, out_like=None, **opts):
    q, pool, scale, idx = dev or _dev(inp)
    R, H = q.shape[0], q.shape[1]
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    if out_like is not None:
        out = out_like
        out.fill_(float("nan"))
    if opts:
        _lib.sparse_mla_fwd_ex(q, pool, scale, idx, inp.sm_scale, out, lse, **opts)
    else:
        _lib.sparse_mla_fwd(q, pool, scale, idx, inp.sm_scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle(inp, rows=None):
    return oracle.sparse_mla_fwd_torch(inp.q, inp.pool, inp.kv_scale, inp.indices, inp.sm_scale,
                                       rows=rows)


def assert_parity(out, lse, ref_out, ref_lse, indices, rows=None):
    """out/lse: GPU results for `rows` (all rows if None); ref_*: oracle."""
    if rows is not None:
        out, lse, indices = out[rows], lse[rows], indices[rows]
    o = out.to(torch.float64).numpy()
    l_ = lse.to(torch.float64).numpy()
    assert not np.isnan(o).any(), "NaN in output (unwritten or poisoned element)"
    assert not np.isnan(l_).any(), "NaN in lse"
    has_valid = (indices >= 0).any(dim=1).numpy()
    empty = ~has_valid
    if empty.any():
        assert np.all(o[empty] == 0.0), "row without valid slot must give out = 0"
        assert np.all(l_[empty] == -np.inf), "row without valid slot must give lse = -inf"
    if has_valid.any():
        d = o[has_valid] - ref_out[has_valid]
        max_abs = float(np.max(np.abs(d)))
        rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref_out[has_valid]), 1e-30))
        lse_err = float(np.max(np.abs(l_[has_valid] - ref_lse[has_valid])))
        assert max_abs <= OUT_MAX_ABS, f"max abs {max_abs}"
        assert rel <= OUT_REL_FRO, f"relative Frobenius {rel}"
        assert lse_err <= LSE_ABS, f"lse error {lse_err}"
        return dict(max_abs=max_abs, rel_fro=rel, lse_err=lse_err)
    return {}


def _check(inp, **opts):
    out, lse = run_gpu(inp, **opts)
    ref_out, ref_lse = run_oracle(inp)
    return assert_parity(out, lse, ref_out, ref_lse, inp.indices)


# ---------------------------------------------------------- the workloads

@pytest.mark.parametrize("name", ["tiny", "decode_bf16", "decode_fp8", "decode_bf16_h32",
                                  "decode_fp8_h32"])
def test_workload_full_parity(name):
    print(f"\n[parity] workload={name}", flush=True)
    inp = make_inputs(name)
    stats = _check(inp)
    print(f"[parity] {name}: {stats}", flush=True)


@pytest.mark.parametrize("variant", [0, 3, 4])
@pytest.mark.parametrize("name", ["prefill_fp8", "prefill_glm"])
def test_prefill_parity_on_sampled_rows(name, variant):
    """The whole workload runs in the launch the benchmark times (variant 0,
    the planner's choice); the oracle checks every 64th row plus the last
    one. Variants 3 and 4 force the fp8-dot and the 4-wave 64-head kernels."""
    print(f"\n[parity] workload={name} variant={variant} (sampled rows)", flush=True)
    inp = make_inputs(name)
    out, lse = run_gpu(inp, **({"variant": variant} if variant else {}))
    R = inp.q.shape[0]
    rows = np.unique(np.r_[np.arange(0, R, 64), R - 1])
    ref_out, ref_lse = run_oracle(inp, rows=rows)
    stats = assert_parity(out, lse, ref_out, ref_lse, inp.indices, rows=torch.from_numpy(rows))
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    print(f"[parity] {name}: {stats}", flush=True)


def test_decode_past_the_mall_on_sampled_rows():
    """decode_fp8_ctx: the headline decode over a 1.2 GB pool (2,097,152 rows,
    each request's top-k from its own 16,384-row context), in the launch the
    benchmark times; pool offsets reach about 1.2e9 bytes. The oracle checks
    every 8th row plus the last one."""
    print("\n[parity] workload=decode_fp8_ctx (sampled rows)", flush=True)
    inp = make_inputs("decode_fp8_ctx")
    out, lse = run_gpu(inp)
    R = inp.q.shape[0]
    rows = np.unique(np.r_[np.arange(0, R, 8), R - 1])
    ref_out, ref_lse = run_oracle(inp, rows=rows)
    stats = assert_parity(out, lse, ref_out, ref_lse, inp.indices, rows=torch.from_numpy(rows))
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    assert int(inp.indices.max()) > 2_000_000   # rows near the pool's end are read
    print(f"[parity] decode_fp8_ctx: {stats}", flush=True)


def test_library_workspace_grows_by_doubling():
    """Three split calls with growing partials: the library-owned workspace
    grows to at least twice its size when it grows, so the last two calls
    reallocate at most once."""
    dev = torch.cuda.current_device()
    b0 = _lib.workspace_bytes(dev)
    sizes = []
    rows0 = max(8, b0 // (16 * 4 * 513 * 4) + 1)   # partials past the current buffer
    for i, rows in enumerate([rows0, rows0 + rows0 // 4, rows0 + rows0 // 2]):
        inp = _case(rows=int(rows), heads=16, topk=256, pool_rows=2000, kv_dtype="fp8", seed=90 + i)
        dev_inp = _dev(inp)
        need = _lib.sparse_mla_plan(dev_inp[0], dev_inp[1], dev_inp[3], splits=4)["workspace_bytes"]
        run_gpu(inp, dev=dev_inp, splits=4)
        sizes.append((need, _lib.workspace_bytes(dev)))
    print(f"\n[workspace] start {b0}, (need, held) per call: {sizes}", flush=True)
    (n1, b1), (n2, b2), (n3, b3) = sizes
    assert b1 >= n1 and b1 >= 2 * b0
    assert b2 >= n2 and (b2 == b1 or b2 >= 2 * b1)
    assert n3 <= 2 * n1 and b3 == b2, "the third call must fit what the growth left"


# ------------------------------------------------------------- edge cases

def _case(**kw):
    base = dict(rows=6, heads=16, d_qk=576, pool_rows=3000, topk=256, kv_dtype="bf16", seed=31)
    base.update(kw)
    return make_inputs(custom_workload(**base))


@pytest.mark.parametrize("valid", [1, 2, 63, 64, 65, 127, 128, 129, 191, 192])
def test_valid_count_on_tile_edges(valid):
    inp = _case(topk=192, seed=valid)
    idx = inp.indices.clone()
    idx[:, valid:] = -1
    inp.indices = idx
    _check(inp)


@pytest.mark.parametrize("topk", [1, 31, 63, 64, 65, 129, 300])
def test_topk_on_tile_edges(topk):
    _check(_case(topk=topk, pool_rows=4096, seed=topk, invalid_per_row=min(3, topk - 1)))


def test_invalid_every_other_slot_and_leading_tiles():
    inp = _case(topk=384, kv_dtype="fp8")
    idx = inp.indices.clone()
    idx[0:3, ::2] = -1             # every other slot
    idx[3:5, :192] = -1            # 192 leading slots (whole leading tiles)
    idx[5, :] = -5                 # a row with no valid slot
    inp.indices = idx
    _check(inp)
    _check(inp, splits=3)


def test_all_invalid_split_and_rows():
    inp = _case(topk=512)
    idx = inp.indices.clone()
    idx[1, 128:256] = -1           # split 1 of 4 empty
    idx[2, :384] = -1              # splits 0-2 empty
    idx[4, :] = -1                 # whole row empty
    inp.indices = idx
    for s in (1, 4, 8):
        _check(inp, splits=s)


@pytest.mark.parametrize("heads", [1, 8, 16, 24, 32, 48, 64, 80])
@pytest.mark.parametrize("d_qk,kv", [(576, "bf16"), (576, "fp8"), (512, "fp8"), (512, "bf16")])
def test_heads_widths_dtypes(heads, d_qk, kv):
    _check(_case(heads=heads, d_qk=d_qk, kv_dtype=kv, rows=5, topk=200, invalid_per_row=7,
                 seed=heads + d_qk))


@pytest.mark.parametrize("head_block", [16, 32, 64])
@pytest.mark.parametrize("splits", [1, 2, 8])
@pytest.mark.parametrize("remap", [1, 2])
def test_forced_plans(head_block, splits, remap):
    inp = _case(heads=40, rows=5, topk=640, kv_dtype="fp8", invalid_per_row=11, seed=head_block)
    _check(inp, head_block=head_block, splits=splits, remap=remap)


def test_caller_workspace():
    inp = _case(rows=7, topk=512)
    ws = torch.empty(8 * 7 * 16 * 513 + 1024, dtype=torch.float32, device="cuda")
    _check(inp, splits=8, workspace=ws)


def test_guard_row_before_pool_is_never_read():
    """The pool view starts one row into a buffer whose first row is NaN; a read
    of index -1 would pull the NaN row into the output."""
    inp = _case(topk=256, invalid_per_row=40, kv_dtype="bf16")
    q, pool, scale, idx = _dev(inp)
    big = torch.empty((pool.shape[0] + 1, pool.shape[1]), dtype=pool.dtype, device="cuda")
    big[0] = float("nan")
    big[1:] = pool
    out, lse = run_gpu(inp, dev=(q, big[1:], scale, idx))
    ref_out, ref_lse = run_oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, inp.indices)


def test_fp8_guard_row_and_padded_pitch():
    w = custom_workload(rows=4, heads=16, d_qk=576, pool_rows=2000, topk=320, kv_dtype="fp8",
                        seed=77, pool_pitch=640, invalid_per_row=33)
    inp = make_inputs(w)
    q, pool, scale, idx = _dev(inp)
    big = torch.empty((pool.shape[0] + 1, pool.shape[1]), dtype=torch.uint8, device="cuda")
    big[0] = 0x7F  # e4m3fn NaN code
    big[1:] = pool.view(torch.uint8)
    out, lse = run_gpu(inp, dev=(q, big[1:].view(torch.float8_e4m3fn), scale, idx))
    ref_out, ref_lse = run_oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, inp.indices)


def test_strided_q_and_out():
    inp = _case(rows=5, heads=16, topk=130)
    q, pool, scale, idx = _dev(inp)
    qbig = torch.zeros((5, 20, 584), dtype=torch.bfloat16, device="cuda")
    qbig[:, 2:18, :576] = q
    qv = qbig[:, 2:18, :576]
    outbig = torch.full((5, 17, 520), float("nan"), dtype=torch.bfloat16, device="cuda")
    outv = outbig[:, :16, :512]
    lse = torch.full((5, 16), float("nan"), dtype=torch.float32, device="cuda")
    _lib.sparse_mla_fwd(qv, pool, scale, idx, inp.sm_scale, outv, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(inp)
    assert_parity(outv.cpu(), lse.cpu(), ref_out, ref_lse, inp.indices)
    assert torch.isnan(outbig[:, 16].float()).all() and torch.isnan(outbig[:, :16, 512:].float()).all()


def test_fp8_widening_is_exact_for_every_code():
    """One valid slot per row: out is that pool row exactly (scale 1), so each
    finite e4m3fn code must widen to its exact value."""
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    pool = torch.zeros((2, 576), dtype=torch.uint8)
    pool[0, :254] = codes
    pool[1, :254] = codes.flip(0)
    pool[1, 254:508] = codes
    inp = make_inputs(custom_workload(rows=2, heads=16, d_qk=576, pool_rows=2, topk=2,
                                      kv_dtype="fp8", seed=1))
    inp.pool = pool.view(torch.float8_e4m3fn)
    inp.kv_scale = torch.ones(1, dtype=torch.float32)
    inp.indices = torch.tensor([[0, -1], [-1, 1]], dtype=torch.int32)
    out, lse = run_gpu(inp)
    ref = pool.view(torch.float8_e4m3fn)[:, :512].to(torch.float32)
    assert torch.equal(out[0].float(), ref[0].expand(16, -1))
    assert torch.equal(out[1].float(), ref[1].expand(16, -1))
    ref_out, ref_lse = run_oracle(inp)
    assert_parity(out, lse, ref_out, ref_lse, inp.indices)


def test_deterministic_repeat_and_permutation():
    inp = _case(rows=8, topk=512, kv_dtype="fp8", invalid_per_row=20)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
    g = torch.Generator().manual_seed(2)
    perm = torch.argsort(torch.rand(inp.indices.shape, generator=g), dim=1)
    inp2 = _case(rows=8, topk=512, kv_dtype="fp8", invalid_per_row=20)
    inp2.indices = torch.gather(inp.indices, 1, perm).contiguous()
    c = run_gpu(inp2)
    ref_out, ref_lse = run_oracle(inp)
    assert_parity(c[0], c[1], ref_out, ref_lse, inp2.indices)


def test_large_scores_stay_finite():
    inp = _case(rows=4, topk=256)
    inp.q = (inp.q.float() * 30).to(torch.bfloat16)
    _check(inp)


def test_zero_rows_noop():
    inp = _case(rows=1)
    q, pool, scale, idx = _dev(inp)
    out = torch.empty((0, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    _lib.sparse_mla_fwd(q[:0], pool, scale, idx[:0], inp.sm_scale, out, lse)
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("topk,splits", [(2048, 1), (1000, 1), (129, 1), (17, 1), (1000, 3), (2048, 5)])
def test_decode_fp8_variants(variant, topk, splits):
    """The two 16-head fp8 kernels (the decode kernel; the staged-tile kernel
    with 4 waves over 64-slot tiles) on ragged top-k, with and without
    splits."""
    inp = _case(rows=7, heads=16, topk=topk, pool_rows=8192, kv_dtype="fp8", invalid_per_row=37,
                seed=topk + splits)
    idx = inp.indices.clone()
    idx[2, : min(topk, 300)] = -1   # leading tiles of a row invalid
    idx[5, :] = -1                  # a row with no valid slot
    inp.indices = idx
    _check(inp, variant=variant, splits=splits)


@pytest.mark.parametrize("topk,splits,heads,d_qk", [
    (5000, 1, 16, 576), (5000, 2, 12, 576), (4097, 1, 16, 512), (2049, 3, 5, 576), (6144, 4, 16, 512)])
def test_decode_index_chunks(topk, splits, heads, d_qk):
    """The fp8 decode kernel stages a row's indices 2048 at a time and merges
    its four waves a quarter of the columns at a time: top-k past one and two
    chunks, splits that straddle chunk boundaries, partial head blocks."""
    print(f"\n[parity] decode chunks topk={topk} splits={splits} heads={heads} d_qk={d_qk}", flush=True)
    inp = _case(rows=6, heads=heads, d_qk=d_qk, topk=topk, pool_rows=16384, kv_dtype="fp8",
                invalid_per_row=50, seed=topk + heads)
    idx = inp.indices.clone()
    idx[1, 2040:2060] = -1          # invalid slots across the first chunk boundary
    idx[4, :] = -1                  # a row with no valid slot
    inp.indices = idx
    _check(inp, variant=0, splits=splits)


VARIANT_SHAPES = [(v, d, kv, h) for v in (0, 1, 2, 3, 4)
                  for d, kv, h in [(576, "fp8", 64), (512, "fp8", 80), (576, "bf16", 64)]
                  if not (v >= 3 and kv == "bf16")]


@pytest.mark.parametrize("variant,d_qk,kv,heads", VARIANT_SHAPES)
@pytest.mark.parametrize("topk,splits", [(2048, 1), (1000, 1), (17, 1), (1000, 3), (300, 2)])
def test_64head_variants(variant, d_qk, kv, heads, topk, splits):
    """The 64-head kernels (variant 0: the planner's choice; 1: the
    single-buffered staged-tile kernel; 2: the 8-wave kernel; 3: the fp8-dot
    kernel and 4: the 4-wave kernel, fp8 pools only) on ragged
    top-k, odd tile counts, a partial head block, leading invalid tiles and
    an empty row, with and without splits."""
    inp = _case(rows=5, heads=heads, d_qk=d_qk, topk=topk, pool_rows=8192, kv_dtype=kv,
                invalid_per_row=29, seed=topk + splits + d_qk)
    idx = inp.indices.clone()
    idx[1, : min(topk, 200)] = -1   # leading tiles of a row invalid
    idx[3, :] = -1                  # a row with no valid slot
    inp.indices = idx
    print(f"\n[parity] 64-head variant={variant} d={d_qk} kv={kv} H={heads} K={topk} S={splits}",
          flush=True)
    _check(inp, variant=variant, splits=splits, head_block=64)


@pytest.mark.parametrize("kv,variant", [("fp8", 0), ("bf16", 0), ("fp8", 2), ("fp8", 3)])
@pytest.mark.parametrize("splits", [1, 2])
def test_score_jump_after_first_tile(kv, variant, splits):
    """Every head's first 64 slots point at near-zero keys and later slots at
    keys whose scores are ~138 higher in the log2 domain, so a reference max
    taken from the first tile would overflow P: the kernels must move their
    reference (rescale, or a second walk from the row max)."""
    R, H, D, K, N = 3, 64, 576, 320, 600
    inp = _case(rows=R, heads=H, d_qk=D, topk=K, pool_rows=N, kv_dtype=kv, seed=5)
    g = torch.Generator().manual_seed(11)
    pool = torch.randn((N, D), generator=g) * 0.01
    pool[300:] = 1.0 + 0.05 * torch.randn((N - 300, D), generator=g)
    q = torch.full((R, H, D), 4.0) + 0.1 * torch.randn((R, H, D), generator=g)
    inp.q = q.to(torch.bfloat16)
    if kv == "fp8":
        from sparse_mla_attention_05_amd.inputs import quantize_fp8
        inp.pool, inp.kv_scale = quantize_fp8(pool)
    else:
        inp.pool = pool.to(torch.bfloat16)
    idx = torch.empty((R, K), dtype=torch.int32)
    for r in range(R):
        idx[r, :64] = torch.randperm(300, generator=g)[:64].to(torch.int32)
        idx[r, 64:] = (300 + torch.randperm(N - 300, generator=g)[: K - 64]).to(torch.int32)
    idx[1, 100:110] = -1
    inp.indices = idx
    print(f"\n[parity] score jump kv={kv} variant={variant} splits={splits}", flush=True)
    _check(inp, splits=splits, **({"variant": variant, "head_block": 64} if variant else {}))
