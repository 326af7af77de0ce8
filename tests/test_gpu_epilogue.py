"""GPU checks of the output epilogue (inverse RoPE of columns 448..511 and the
MXFP8 store), through the C ABI.

1. The separate pass (sparse_mla_out_epilogue) on seeded synthetic bf16 rows
   equals the oracle's epilogue bit for bit: the pages fix its arithmetic
   (bf16 rows, fp32 products rounded one by one, the OCP MX scale rule), so
   both sides take every rounding and every e4m3 decision in the same
   precision.
2. The fused store of every kernel path (decode, 64-head fp8 and bf16, the
   8-wave kernel over fp8, the staged-tile kernel, split-K through the combine
   kernel, both two-segment routes) equals the same call's plain bf16 output
   run through the separate pass, bit for bit.
3. The fused output against the fp64 attention oracle followed by the
   oracle's epilogue. bf16 output: the parity bar of the plain forward
   (max abs 2e-2 * sqrt(2), since a rotated column mixes two columns'
   errors; relative Frobenius 5e-3, which the rotation preserves). MXFP8:
   both sides quantise values that differ by the attention error, so an
   element may land one e4m3 step apart and a block scale one binade apart:
   per element |deq_gpu - deq_ref| <= sqrt(2) * 2e-2 + one step of the
   coarser grid, relative Frobenius <= 3e-2 (one-step flips at a rate of
   error/step, each one step: sqrt(2e-3 * 2^-3) = 1.6e-2 expected), scale
   codes within 1.
Outputs start poisoned (NaN bf16, e4m3 NaN codes 0x7F, E8M0 NaN 0xFF), so an
element a kernel forgets to store fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import out_epilogue as ep
from sparse_mla_attention_05_amd import _lib
from sparse_mla_attention_05_amd.inputs import (custom_workload, make_epilogue_inputs,
                                                make_epilogue_rows, make_extra_segment,
                                                make_inputs)

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2 * math.sqrt(2)
REL_FRO_BF16 = 5e-3
REL_FRO_MX = 3e-2
E8M0 = torch.float8_e8m0fnu


def _u8(t):
    return t.cpu().view(torch.uint8).numpy()


def _bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _poisoned(R, H, mx):
    if mx:
        out = torch.full((R, H, 512), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        sc = torch.full((R, H, 16), 0xFF, dtype=torch.uint8, device="cuda").view(E8M0)
        return out, sc
    return torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda"), None


def _epi_kw(e, rope):
    if not rope:
        return {}
    return dict(rope_positions=e.positions.cuda(), rope_cos_sin=e.cos_sin.cuda())


# ------------------------------------------------ 1. the pass vs the oracle

@pytest.mark.parametrize("R,H", [(37, 16), (5, 64), (3, 20)])
@pytest.mark.parametrize("mx,rope", [(True, True), (False, True), (True, False)])
def test_pass_equals_oracle_bitwise(R, H, mx, rope):
    print(f"\n[epilogue pass] R={R} H={H} mx={mx} rope={rope}", flush=True)
    rows = make_epilogue_rows(R, H, seed=100 + R)
    e = make_epilogue_inputs(R, seed=200 + R)
    out, sc = _poisoned(R, H, mx)
    _lib.sparse_mla_out_epilogue(rows.cuda(), out, out_scale=sc, **_epi_kw(e, rope))
    torch.cuda.synchronize()
    pos = e.positions.numpy() if rope else None
    ref = ep.out_epilogue(_bits(rows), pos, e.cos_sin.numpy(), mxfp8=mx)
    if mx:
        assert np.array_equal(_u8(out), ref[0]), "e4m3 codes differ"
        assert np.array_equal(_u8(sc), ref[1]), "E8M0 scales differ"
    else:
        assert np.array_equal(_bits(out), ref)


def test_pass_strided_rows_and_outputs():
    """Row and head strides that are not the dense ones, for rows, the
    codes and the scales."""
    R, H = 6, 8
    rows_big = make_epilogue_rows(R, 2 * H, seed=7)
    rows = rows_big.cuda()[:, ::2]
    e = make_epilogue_inputs(R, seed=8)
    big = torch.full((R, H + 1, 528), 0x7F, dtype=torch.uint8, device="cuda")
    out = big[:, 1:, :512].view(torch.float8_e4m3fn)
    sbig = torch.full((R, H, 32), 0xFF, dtype=torch.uint8, device="cuda")
    sc = sbig[:, :, :16].view(E8M0)
    _lib.sparse_mla_out_epilogue(rows, out, out_scale=sc, **_epi_kw(e, True))
    torch.cuda.synchronize()
    ref = ep.out_epilogue(_bits(rows_big[:, ::2]), e.positions.numpy(), e.cos_sin.numpy(), True)
    assert np.array_equal(_u8(out), ref[0]) and np.array_equal(_u8(sc), ref[1])
    assert np.all(_u8(big)[:, 0] == 0x7F) and np.all(_u8(big)[:, :, 512:] == 0x7F)
    assert np.all(_u8(sbig)[:, :, 16:] == 0xFF)


# ------------------------------------- 2./3. fused stores of every kernel path

def _workload(kv, d_qk, heads, topk, rows=12, seed=61):
    w = custom_workload(rows=rows, heads=heads, d_qk=d_qk, pool_rows=6000, topk=topk,
                        kv_dtype=kv, seed=seed, index_mode="causal", first_pos=5000,
                        invalid_per_row=5)
    inp = make_inputs(w)
    inp.indices[1] = -1  # one row with no valid slot
    return inp


def _dev(inp):
    s = inp.kv_scale.cuda() if inp.kv_scale is not None else None
    return inp.q.cuda(), inp.pool.cuda(), s, inp.indices.cuda()


def run_fused(inp, e, mx, rope, ex=None, **opts):
    q, pool, s, idx = _dev(inp)
    R, H = q.shape[0], q.shape[1]
    out, sc = _poisoned(R, H, mx)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    extra = {}
    if ex is not None:
        extra = dict(extra_pool=ex.pool.cuda(), extra_indices=ex.indices.cuda(),
                     extra_kv_scale=ex.kv_scale.cuda() if ex.kv_scale is not None else None)
    _lib.sparse_mla_fwd_epi(q, pool, s, idx, inp.sm_scale, out, lse, out_scale=sc,
                            **_epi_kw(e, rope), **extra, **opts)
    torch.cuda.synchronize()
    return out, sc, lse


def run_unfused(inp, e, mx, rope, ex=None, **opts):
    """Plain bf16 forward of the same call, then the separate pass."""
    q, pool, s, idx = _dev(inp)
    R, H = q.shape[0], q.shape[1]
    plain = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    if ex is None:
        _lib.sparse_mla_fwd_ex(q, pool, s, idx, inp.sm_scale, plain, lse, **opts)
    else:
        _lib.sparse_mla_fwd2(q, pool, s, idx, ex.pool.cuda(),
                             ex.kv_scale.cuda() if ex.kv_scale is not None else None,
                             ex.indices.cuda(), inp.sm_scale, plain, lse, **opts)
    out, sc = _poisoned(R, H, mx)
    _lib.sparse_mla_out_epilogue(plain, out, out_scale=sc, **_epi_kw(e, rope))
    torch.cuda.synchronize()
    return out, sc, lse


def oracle_fused(inp, e, mx, rope, ex=None, rows=None):
    if ex is None:
        ref, ref_lse = oracle.sparse_mla_fwd_torch(inp.q, inp.pool, inp.kv_scale, inp.indices,
                                                   inp.sm_scale, rows=rows)
    else:
        ref, ref_lse = oracle.sparse_mla_fwd_2seg_torch(inp.q, inp.pool, inp.kv_scale, inp.indices,
                                                        ex.pool, ex.kv_scale, ex.indices,
                                                        inp.sm_scale, rows=rows)
    pos = e.positions.numpy() if rope else None
    if rows is not None and pos is not None:
        pos = pos[rows]
    return ep.fwd_with_epilogue(ref, pos, e.cos_sin.numpy(), mxfp8=mx), ref_lse


def _e4m3_step(a):
    """Spacing of the e4m3 grid at magnitude a (in units of the block scale)."""
    a = np.maximum(np.abs(a), 2.0 ** -6)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 3)


def assert_mx_close(codes, scales, ref_codes, ref_scales):
    c, s = np.asarray(codes), np.asarray(scales)
    assert not np.any((c & 0x7F) == 0x7F), "NaN code (unwritten element)"
    assert not np.any(s == 0xFF), "NaN scale (unwritten block)"
    ds = np.abs(s.astype(np.int64) - ref_scales.astype(np.int64))
    assert ds.max() <= 1, f"scale codes {ds.max()} apart"
    deq = ep.mxfp8_dequantize(c, s)
    deq_r = ep.mxfp8_dequantize(ref_codes, ref_scales)
    x = np.repeat(np.ldexp(1.0, np.maximum(s, ref_scales).astype(np.int64) - 127), 32, axis=-1)
    step = _e4m3_step(np.maximum(np.abs(deq), np.abs(deq_r)) / x) * x
    err = np.abs(deq - deq_r)
    assert np.all(err <= MAX_ABS + step), f"max excess {np.max(err - MAX_ABS - step)}"
    rel = float(np.linalg.norm(deq - deq_r) / max(np.linalg.norm(deq_r), 1e-30))
    assert rel <= REL_FRO_MX, f"relative Frobenius {rel}"
    flips = float(np.mean(c != ref_codes))
    return dict(rel_fro=rel, code_mismatch=flips, scale_mismatch=float(np.mean(ds != 0)))


def assert_bf16_close(out_bits, ref_bits):
    o = ep.bf16_value(out_bits).astype(np.float64)
    r = ep.bf16_value(ref_bits).astype(np.float64)
    assert not np.isnan(o).any(), "NaN in output (unwritten element)"
    d = np.abs(o - r)
    rel = float(np.linalg.norm(o - r) / max(np.linalg.norm(r), 1e-30))
    assert d.max() <= MAX_ABS, f"max abs {d.max()}"
    assert rel <= REL_FRO_BF16, f"relative Frobenius {rel}"
    return dict(max_abs=float(d.max()), rel_fro=rel)


PATHS = [
    # kv, d_qk, heads, top-k, planner overrides: which kernel stores
    ("fp8", 576, 16, 512, {}),                                  # decode kernel
    ("fp8", 512, 16, 300, dict(head_block=16, splits=3)),       # decode, split-K: combine
    ("fp8", 576, 20, 256, {}),                                  # 16-head blocks, one partial
    ("fp8", 576, 64, 512, {}),                                  # 64-head fp8 default (fp8-dot)
    ("fp8", 512, 64, 300, dict(variant=4)),                     # 4-wave 64-head fp8 kernel
    ("fp8", 576, 64, 512, dict(variant=4)),
    ("fp8", 576, 64, 512, dict(variant=2)),                     # 8-wave kernel over fp8
    ("fp8", 576, 64, 512, dict(variant=3)),                     # fp8-dot kernel
    ("fp8", 512, 64, 300, dict(variant=3, head_block=64, splits=2)),  # fp8-dot, combine
    ("fp8", 576, 64, 512, dict(variant=1)),                     # staged-tile kernel, 64 heads
    ("bf16", 576, 64, 512, {}),                                 # 8-wave kernel over bf16
    ("bf16", 512, 64, 700, dict(head_block=64, splits=2)),      # split-K: combine
    ("bf16", 576, 16, 200, {}),                                 # staged-tile kernel, 16 heads
    ("bf16", 576, 32, 200, {}),                                 # staged-tile kernel, 32 heads
    ("bf16", 576, 80, 300, {}),                                 # 64 + 16 heads
]
MODES = [(True, True), (False, True), (True, False)]


@pytest.mark.parametrize("kv,d_qk,heads,topk,opts", PATHS)
@pytest.mark.parametrize("mx,rope", MODES)
def test_fused_store(kv, d_qk, heads, topk, opts, mx, rope):
    print(f"\n[epilogue fused] kv={kv} d_qk={d_qk} H={heads} K={topk} {opts} mx={mx} rope={rope}",
          flush=True)
    inp = _workload(kv, d_qk, heads, topk)
    e = make_epilogue_inputs(inp.q.shape[0], seed=heads + topk)
    f_out, f_sc, f_lse = run_fused(inp, e, mx, rope, **opts)
    u_out, u_sc, u_lse = run_unfused(inp, e, mx, rope, **opts)
    if mx:
        assert np.array_equal(_u8(f_out), _u8(u_out)), "fused codes != plain output + pass"
        assert np.array_equal(_u8(f_sc), _u8(u_sc)), "fused scales != plain output + pass"
    else:
        assert np.array_equal(_bits(f_out), _bits(u_out)), "fused bf16 != plain output + pass"
    assert torch.equal(f_lse.cpu(), u_lse.cpu())
    ref, ref_lse = oracle_fused(inp, e, mx, rope)
    if mx:
        stats = assert_mx_close(_u8(f_out), _u8(f_sc), ref[0], ref[1])
    else:
        stats = assert_bf16_close(_bits(f_out), ref)
    valid = (inp.indices >= 0).any(dim=1).numpy()
    lse = f_lse.cpu().numpy().astype(np.float64)
    assert np.all(lse[~valid] == -np.inf)
    assert np.max(np.abs(lse[valid] - ref_lse[valid])) <= 1e-3
    print(f"[epilogue fused] {stats}", flush=True)


@pytest.mark.parametrize("kv,heads,opts", [("fp8", 16, {}), ("fp8", 64, {}), ("bf16", 64, {}),
                                           ("fp8", 16, dict(variant=1)), ("fp8", 64, dict(splits=1)),
                                           ("fp8", 64, dict(variant=4))])
def test_fused_store_two_segments(kv, heads, opts):
    """Both two-segment routes: one launch walking both segments (16-head fp8
    decode kernel, 64-head bf16 kernel, 64-head fp8-dot kernel; with one
    split the store of that launch applies the epilogue) and the composition
    (each segment's partials, then the combine kernel's store; the 4-wave
    64-head fp8 kernel)."""
    print(f"\n[epilogue two-segment] kv={kv} H={heads} {opts}", flush=True)
    inp = _workload(kv, 576, heads, 512)
    ex = make_extra_segment(inp, 128, seed=71, value_std=0.7, invalid_per_row=3)
    e = make_epilogue_inputs(inp.q.shape[0], seed=3)
    f_out, f_sc, _ = run_fused(inp, e, True, True, ex=ex, **opts)
    u_out, u_sc, _ = run_unfused(inp, e, True, True, ex=ex, **opts)
    assert np.array_equal(_u8(f_out), _u8(u_out)) and np.array_equal(_u8(f_sc), _u8(u_sc))
    ref, _ = oracle_fused(inp, e, True, True, ex=ex)
    print(f"[epilogue two-segment] {assert_mx_close(_u8(f_out), _u8(f_sc), ref[0], ref[1])}",
          flush=True)


@pytest.mark.parametrize("name,every", [("decode_bf16", 1), ("decode_fp8", 8)])
def test_fused_store_on_decode_workloads(name, every):
    """The decode workloads with rope and MXFP8, in the launch the benchmark
    times: fused == plain + pass on every row, the oracle on every
    `every`-th row."""
    print(f"\n[epilogue] workload={name}", flush=True)
    inp = make_inputs(name)
    R = inp.q.shape[0]
    e = make_epilogue_inputs(R, seed=11)
    f_out, f_sc, _ = run_fused(inp, e, True, True)
    u_out, u_sc, _ = run_unfused(inp, e, True, True)
    assert np.array_equal(_u8(f_out), _u8(u_out)) and np.array_equal(_u8(f_sc), _u8(u_sc))
    rows = np.unique(np.r_[np.arange(0, R, every), R - 1])
    ref, _ = oracle_fused(inp, e, True, True, rows=rows)
    stats = assert_mx_close(_u8(f_out)[rows], _u8(f_sc)[rows], ref[0], ref[1])
    print(f"[epilogue] {name}: {stats}", flush=True)
