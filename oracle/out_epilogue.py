"""CPU oracle of the forward's output epilogue: inverse RoPE of the trailing 64
columns of each output row, then either a bf16 store or an MXFP8 store
(float8_e4m3fn codes with one E8M0 power-of-two scale per 32 columns).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
package smoke check and the benchmark's CPU-baseline leg may call it, the
library never does, and it shares no code with the HIP path.

Source: "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159), the
commit notes on the fused epilogue. Before the output projection the serving
path rotates the last 64 lanes of every attention output row back (inverse
RoPE) and, for an MXFP8 projection, quantises the row to e4m3 with one E8M0
scale per 32 lanes. The kernel that stores the output does both: the
attention kernel without split-K, the split reduce with it. The rows are
rounded to bf16 first, and each product of the rotation is rounded to fp32 on
its own, so that the result equals the separate pass run on the bf16 rows.

The pages fix the precision here (bf16 rows, fp32 products rounded one by
one), so this oracle computes in that precision, not in fp64: numpy float32
arithmetic rounds every operation to nearest even, exactly as stated.

Readings where the pages are silent:
  * Pairing: the rotation pairs are adjacent columns (448 + 2j, 449 + 2j),
    j = 0..31. The pages keep "the rotation pairs and the scale groups" in
    registers of a thread that holds 32 consecutive columns, which only
    adjacent pairs (not columns 32 apart) allow.
  * cos/sin cache: fp32 [P, 64]; row p holds cos(angle_j(p)) in column j and
    sin(angle_j(p)) in column 32 + j. A row's position selects its row.
  * Inverse rotation of a pair (x, y) by its angle: x' = x*cos + y*sin,
    y' = y*cos - x*sin, each product rounded, then the sum.
  * E8M0 scale of a 32-column block (the OCP Microscaling Formats (MX) v1.0
    conversion): X = 2^(floor(log2(amax)) - 8), 8 being the exponent of the
    largest power of two in e4m3; the exponent is clamped to [-127, 127],
    amax = 0 gives the smallest scale 2^-127 (code 0). Code = exponent + 127.
  * Elements: v / X rounded to the nearest e4m3fn value, ties to the even
    code, magnitudes past 448 saturated to 448; the sign of v is kept (a
    negative value that rounds to zero is code 0x80).

Parity pins (tests/test_oracle_epilogue.py, CPU): a quarter-turn and a zero
angle as closed forms, the rotation against complex multiplication by
e^(-i angle) in fp64, norm preservation, the e4m3 encoder against torch's
float8_e4m3fn conversion and against the code table (round trip, midpoints
to even, saturation, subnormals), the scale range of every block, and the
dequantised error within half an e4m3 step.
"""

from __future__ import annotations

import math

import numpy as np

from .sparse_mla_oracle import e4m3fn_table

D_V = 512
ROPE_DIM = 64
ROPE_START = D_V - ROPE_DIM   # first rotated column
MX_BLOCK = 32                 # columns per E8M0 scale
E4M3_EMAX = 8                 # exponent of the largest power of two in e4m3fn
E4M3_MAX = 448.0


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float values, round to nearest even, computed from
    the value itself (no fp32 step, so no double rounding): the value is
    scaled by the spacing of its binade and rounded half-to-even."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                                  # |x| = m * 2^e, m in [0.5, 1)
    spacing_exp = np.maximum(e - 8, -133)               # 8 significant bits; subnormal floor
    spacing = np.ldexp(1.0, spacing_exp)
    q = np.rint(x / spacing) * spacing                  # np.rint: half to even
    q = np.where(x == 0, x, q)                          # keep the sign of zero
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """float32 value of bf16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def inverse_rope(rows: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """Rotate columns 448..511 of each row back by the angles of its position.

    rows: float32 [R, H, 512] (bf16 values); positions: int [R];
    cos_sin: float32 [P, 64]. Pairs are (448 + 2j, 449 + 2j); every product
    is a float32 product and the sum a float32 sum.
    """
    rows = np.asarray(rows, dtype=np.float32)
    out = rows.copy()
    cs = np.asarray(cos_sin, dtype=np.float32)[np.asarray(positions, dtype=np.int64)]  # [R, 64]
    c = cs[:, None, :ROPE_DIM // 2]                     # [R, 1, 32]
    s = cs[:, None, ROPE_DIM // 2:]
    x = rows[:, :, ROPE_START::2]                       # [R, H, 32] columns 448, 450, ...
    y = rows[:, :, ROPE_START + 1::2]
    xc = np.multiply(x, c, dtype=np.float32)
    ys = np.multiply(y, s, dtype=np.float32)
    yc = np.multiply(y, c, dtype=np.float32)
    xs = np.multiply(x, s, dtype=np.float32)
    out[:, :, ROPE_START::2] = np.add(xc, ys, dtype=np.float32)
    out[:, :, ROPE_START + 1::2] = np.subtract(yc, xs, dtype=np.float32)
    return out


def _e4m3_magnitudes() -> np.ndarray:
    """Values of codes 0x00..0x7E (the non-negative finite e4m3fn values),
    increasing with the code."""
    t = e4m3fn_table()[:0x7F]
    assert np.all(np.diff(t) > 0)
    return t


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float8_e4m3fn code of each value: nearest representable magnitude, ties
    to the even code, saturated at 448, sign of v kept."""
    v = np.asarray(v, dtype=np.float64)
    mags = _e4m3_magnitudes()
    a = np.abs(v)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, len(mags) - 1)
    lo = hi - 1
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(a <= 0, 0, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e8m0_exponent(amax: float) -> int:
    """Shared exponent of a block with largest magnitude amax."""
    if amax == 0.0:
        return -127
    _, e = math.frexp(amax)                              # amax = m * 2^e, m in [0.5, 1)
    return max(-127, min(127, (e - 1) - E4M3_EMAX))


def mxfp8_quantize(rows: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 of float32 rows [R, H, 512]: e4m3fn codes [R, H, 512] and E8M0
    scale codes [R, H, 16]."""
    rows = np.asarray(rows, dtype=np.float32)
    R, H, D = rows.shape
    blocks = rows.astype(np.float64).reshape(R, H, D // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    exps = np.vectorize(e8m0_exponent, otypes=[np.int64])(amax)
    scale = np.ldexp(1.0, exps)[..., None]
    codes = e4m3_encode(blocks / scale).reshape(R, H, D)
    return codes, (exps + 127).astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values of MXFP8 codes [.., 512] with E8M0 scales [.., 16]."""
    t = e4m3fn_table()
    v = t[np.asarray(codes, dtype=np.uint8)]
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v.reshape(*v.shape[:-1], -1, MX_BLOCK) * x[..., None]).reshape(v.shape)


def out_epilogue(row_bits: np.ndarray, positions=None, cos_sin=None, mxfp8: bool = False):
    """The epilogue on bf16 output rows (bit patterns uint16 [R, H, 512]).

    Returns bf16 bit patterns [R, H, 512], or (e4m3fn codes [R, H, 512],
    E8M0 codes [R, H, 16]) when mxfp8 is set. positions None: no rotation.
    """
    rows = bf16_value(row_bits)
    if positions is not None:
        rows = inverse_rope(rows, positions, cos_sin)
    if mxfp8:
        return mxfp8_quantize(rows)
    return bf16_round_bits(rows.astype(np.float64))


def fwd_with_epilogue(out_f64: np.ndarray, positions=None, cos_sin=None, mxfp8: bool = False):
    """The forward's output (fp64 [R, H, 512] from the attention oracle) through
    the epilogue: rounded to bf16 first, then out_epilogue."""
    return out_epilogue(bf16_round_bits(out_f64), positions, cos_sin, mxfp8)
