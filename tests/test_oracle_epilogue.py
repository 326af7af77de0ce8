"""Pins for the output-epilogue oracle (inverse RoPE + MXFP8), each against
something other than the oracle's own formula: closed forms, complex
multiplication, torch's float8 conversion, the e4m3 code table, and the
properties the OCP MX scale rule guarantees. CPU only, seconds."""

import math

import numpy as np
import pytest
import torch

from oracle import out_epilogue as ep
from oracle.sparse_mla_oracle import e4m3fn_table
from sparse_mla_attention_05_amd.inputs import make_epilogue_inputs, make_epilogue_rows


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _rows_f32(bits):
    return ep.bf16_value(bits)


# ------------------------------------------------------------- rotation ---

def test_zero_angle_is_identity_bitwise():
    rows = make_epilogue_rows(3, 4, seed=1)
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32] = 1.0
    out = ep.out_epilogue(_bits(rows), np.zeros(3, np.int32), cs)
    assert np.array_equal(out, _bits(rows))


def test_quarter_turn_closed_form():
    """Angle pi/2 on pair j (cos 0, sin 1): (x, y) -> (y, -x); other pairs
    keep angle 0. Columns before 448 never move."""
    rows = make_epilogue_rows(2, 3, seed=2)
    cs = np.zeros((5, 64), np.float32)
    cs[:, :32] = 1.0
    j = 7
    cs[4, j], cs[4, 32 + j] = 0.0, 1.0
    pos = np.array([4, 0], np.int32)
    out = _rows_f32(ep.out_epilogue(_bits(rows), pos, cs))
    src = _rows_f32(_bits(rows))
    x, y = 448 + 2 * j, 449 + 2 * j
    assert np.array_equal(out[0, :, x], src[0, :, y])
    assert np.array_equal(out[0, :, y], -src[0, :, x])
    keep = np.ones(512, bool)
    keep[[x, y]] = False
    assert np.array_equal(out[0][:, keep], src[0][:, keep])
    assert np.array_equal(out[1], src[1])


def test_rotation_is_complex_multiplication():
    """Pair j as z = x + i y; the inverse rotation is z * e^(-i angle), here in
    complex128 against the oracle's fp32 arithmetic (so a swapped cos/sin, a
    wrong sign or a wrong pairing fails)."""
    R, H = 6, 5
    rows = make_epilogue_rows(R, H, seed=3)
    e = make_epilogue_inputs(R, seed=4, max_pos=4096)
    cs = e.cos_sin.numpy().astype(np.float64)
    pos = e.positions.numpy()
    src = _rows_f32(_bits(rows)).astype(np.float64)
    z = src[:, :, 448::2] + 1j * src[:, :, 449::2]
    rot = np.exp(-1j * np.arctan2(cs[pos, 32:], cs[pos, :32]))[:, None, :]
    want = z * rot
    got32 = ep.inverse_rope(_rows_f32(_bits(rows)), pos, e.cos_sin.numpy())
    got = got32[:, :, 448::2] + 1j * got32[:, :, 449::2]
    scale = np.abs(z).max()
    assert np.abs(got - want).max() <= 4 * 2.0 ** -24 * scale + 1e-7 * scale
    assert np.array_equal(got32[:, :, :448], src[:, :, :448].astype(np.float32))


def test_rotation_preserves_norm():
    rows = make_epilogue_rows(4, 8, seed=5)
    e = make_epilogue_inputs(4, seed=6)
    src = _rows_f32(_bits(rows)).astype(np.float64)
    got = ep.inverse_rope(_rows_f32(_bits(rows)), e.positions.numpy(), e.cos_sin.numpy())
    n0 = np.linalg.norm(src[:, :, 448:], axis=-1)
    n1 = np.linalg.norm(got[:, :, 448:].astype(np.float64), axis=-1)
    assert np.allclose(n0, n1, rtol=1e-6, atol=0)


def test_forward_then_inverse_returns_the_row():
    """A forward RoPE written as the complex product z * e^(+i angle) in fp64,
    then the oracle's inverse: back to the start within fp32 rounding."""
    R, H = 3, 4
    gen = np.random.default_rng(7)
    z0 = gen.standard_normal((R, H, 32)) + 1j * gen.standard_normal((R, H, 32))
    e = make_epilogue_inputs(R, seed=8)
    pos = e.positions.numpy()
    ang = np.arctan2(e.cos_sin.numpy()[pos, 32:].astype(np.float64),
                     e.cos_sin.numpy()[pos, :32].astype(np.float64))
    z1 = z0 * np.exp(1j * ang)[:, None, :]
    rows = np.zeros((R, H, 512), np.float32)
    rows[:, :, 448::2] = z1.real
    rows[:, :, 449::2] = z1.imag
    back = ep.inverse_rope(rows, pos, e.cos_sin.numpy())
    z2 = back[:, :, 448::2].astype(np.float64) + 1j * back[:, :, 449::2]
    assert np.abs(z2 - z0).max() < 1e-5


# -------------------------------------------------------------- e4m3 codes ---

def test_e4m3_encode_matches_torch_in_range():
    gen = torch.Generator().manual_seed(9)
    x = torch.cat([torch.randn(20000, generator=gen) * 40,
                   torch.randn(20000, generator=gen) * 2.0 ** -7,
                   (torch.rand(2000, generator=gen) * 2 - 1) * 447.9])
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = ep.e4m3_encode(x.numpy().astype(np.float64))
    inside = np.abs(x.numpy()) < 448
    assert np.array_equal(got[inside], want[inside])


def test_e4m3_encode_table_round_trip_midpoints_and_saturation():
    t = e4m3fn_table()
    finite = [c for c in range(256) if not math.isnan(t[c])]
    vals = t[finite]
    codes = ep.e4m3_encode(vals)
    # every value encodes to its own code, except -0 which keeps its sign bit
    assert np.array_equal(codes, np.array(finite, np.uint8))
    mags = t[:0x7F]
    mid = (mags[:-1] + mags[1:]) / 2
    got = ep.e4m3_encode(mid)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    assert list(ep.e4m3_encode(np.array([448.0, 460.0, 480.0, 1e9, -500.0]))) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert ep.e4m3_encode(np.array([2.0 ** -10]))[0] == 0            # tie between 0 and 2^-9: even
    assert ep.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 2        # tie between 2^-9 and 2^-8
    assert ep.e4m3_encode(np.array([-1e-9]))[0] == 0x80


# ---------------------------------------------------------------- MXFP8 ---

def test_mx_scale_puts_every_block_max_in_the_top_binade():
    """OCP MX rule: after dividing by X the block max lies in [256, 512), so
    its code is 256..448 after saturation; all-zero blocks get code 0."""
    rows = make_epilogue_rows(5, 6, seed=10)
    f = _rows_f32(_bits(rows))
    codes, scales = ep.mxfp8_quantize(f)
    blocks = f.astype(np.float64).reshape(5, 6, 16, 32)
    amax = np.abs(blocks).max(-1)
    x = np.ldexp(1.0, scales.astype(np.int64) - 127)
    nz = amax > 0
    assert np.all((amax[nz] / x[nz] >= 256) & (amax[nz] / x[nz] < 512))
    assert np.all(scales[~nz] == 0)
    top = np.abs(ep.mxfp8_dequantize(codes, scales)).reshape(5, 6, 16, 32).max(-1)
    assert np.all((top[nz] / x[nz] >= 256) & (top[nz] / x[nz] <= 448))
    # amax exactly 1.0 (bf16 1.0) gives 2^-8; just under 1 gives 2^-9
    assert scales[0, 0, 1] == 127 - 8 and scales[0, 0, 2] == 127 - 9


def test_mx_dequantised_error_within_half_a_step():
    rows = make_epilogue_rows(4, 4, seed=11)
    f = _rows_f32(_bits(rows)).astype(np.float64)
    codes, scales = ep.mxfp8_quantize(f.astype(np.float32))
    deq = ep.mxfp8_dequantize(codes, scales)
    x = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    a = np.abs(f) / x
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 2.0 ** -6))).astype(np.int64) - 3))
    err = np.abs(deq - f) / x
    sat = a > 448
    assert np.all(err[~sat] <= step[~sat] / 2)
    assert np.all(np.abs(deq[sat]) / x[sat] == 448)


def test_bf16_round_matches_torch():
    gen = torch.Generator().manual_seed(12)
    x = torch.randn(50000, generator=gen, dtype=torch.float64) * 3
    x[:10] = torch.tensor([0.0, -0.0, 1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2.0 ** -130, -1e-40, 5e37, 1e-45, 7.0])
    want = x.to(torch.float32).to(torch.bfloat16)    # x is exact in fp32 here except noted
    exact32 = x.to(torch.float32).to(torch.float64) == x
    got = ep.bf16_round_bits(x.numpy())
    assert np.array_equal(got[exact32.numpy()], _bits(want)[exact32.numpy()])


def test_epilogue_of_mxfp8_equals_rotation_then_quantisation():
    rows = make_epilogue_rows(3, 2, seed=13)
    e = make_epilogue_inputs(3, seed=14)
    codes, scales = ep.out_epilogue(_bits(rows), e.positions.numpy(), e.cos_sin.numpy(), mxfp8=True)
    rot = ep.inverse_rope(_rows_f32(_bits(rows)), e.positions.numpy(), e.cos_sin.numpy())
    c2, s2 = ep.mxfp8_quantize(rot)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # without a rotation only bf16 rows are quantised
    c3, _ = ep.out_epilogue(_bits(rows), None, None, mxfp8=True)
    assert not np.array_equal(c3[:, :, 448:], codes[:, :, 448:])
    assert np.array_equal(c3[:, :, :448], codes[:, :, :448])


@pytest.mark.parametrize("mistake", ["swap_cos_sin", "sign", "neox_pairs", "scale_emax"])
def test_planted_mistakes_are_caught(mistake, monkeypatch):
    """Plant a plausible mistake in a copy of the oracle's arithmetic and check
    that one of the pins above fails."""
    orig_rope, orig_exp = ep.inverse_rope, ep.e8m0_exponent

    def bad_rope(rows, positions, cos_sin):
        rows = np.asarray(rows, np.float32)
        cs = np.asarray(cos_sin, np.float32)[positions]
        if mistake == "swap_cos_sin":
            cs = np.concatenate([cs[:, 32:], cs[:, :32]], axis=1)
        out = rows.copy()
        c, s = cs[:, None, :32], cs[:, None, 32:]
        if mistake == "neox_pairs":
            x, y = rows[:, :, 448:480], rows[:, :, 480:512]
            out[:, :, 448:480] = x * c + y * s
            out[:, :, 480:512] = y * c - x * s
            return out
        x, y = rows[:, :, 448::2], rows[:, :, 449::2]
        sg = -1.0 if mistake == "sign" else 1.0
        out[:, :, 448::2] = x * c + sg * y * s
        out[:, :, 449::2] = y * c - sg * x * s
        return out

    def bad_exp(amax):
        return orig_exp(amax) + (1 if mistake == "scale_emax" else 0)

    monkeypatch.setattr(ep, "inverse_rope", bad_rope)
    monkeypatch.setattr(ep, "e8m0_exponent", bad_exp)
    pins = [test_rotation_is_complex_multiplication, test_quarter_turn_closed_form,
            test_mx_scale_puts_every_block_max_in_the_top_binade]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
