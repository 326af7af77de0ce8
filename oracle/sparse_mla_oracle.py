"""fp64 CPU oracle for sparse multi-head latent attention (MLA) forward.

TEST INFRASTRUCTURE ONLY. This module is the correctness reference that the
HIP kernels are checked against. Only the tests, the package's smoke check and
the benchmark's CPU-baseline leg may import it; the library never calls it.
It shares no code with the HIP path (no kernels, headers, helpers or tables).

What it computes (the plain definition, written out in fp64 with no blocking,
fusion or reordering). For query row r, head h, and the row's int32 top-k slot
indices idx[r, 0..K) into a KV pool, where a negative index marks an invalid
slot:

    J        = { j : idx[r, j] >= 0 }            (slots, duplicates kept)
    s_j      = sm_scale * q[r, h, :] . K[idx[r, j], :D_qk]
    O[r, h]  = sum_j softmax(s)_j * V[idx[r, j]]   with V = K[:, :512]
    LSE[r,h] = ln sum_j exp(s_j)                   (natural log)

and for a row with J empty: O = 0 and LSE = -inf.

Sources on the pages:
  * "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159):
    Technical Details (576-wide rows = 512 latent + 64 rope, 512-wide
    rope-free rows, per-tensor fp8 or bf16 KV, 2,048 or 512 indices per row);
    commit notes on the 64-head program (the rope part of the key is dotted
    after the latent part, so the QK dot runs over all D_qk columns), on the
    per-tensor fp8 two-loop route (a per-tensor scale on the cache; the V scale
    comes off in the epilogue, i.e. value = code * kv_scale for K and V alike),
    and on the walk's sentinel slots (masked slots).
  * The method as stated for this library fixes what the pages leave open:
    -1 slots are invalid and masked, V is the first 512 columns of the
    gathered rows, LSE is returned per (r, h), an all-invalid row gives O = 0
    and LSE = -inf.

Readings where the pages are silent:
  * LSE is the natural log of the sum of exp of the sm_scale-scaled scores.
  * Any negative index is invalid; an index >= pool rows is a caller error and
    the oracle raises.
  * Duplicate indices count once per slot; slot order does not matter.
  * fp8 is OCP float8_e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals at exponent field 0, codes 0x7F/0xFF are NaN, no inf).
  * sm_scale is used as the fp32 value the kernel receives.

Parity pins (tests/test_oracle.py, all CPU): brute-force dense attention via
torch's scaled_dot_product_attention in fp64 over the same gathered rows,
softmax weights summing to 1, all-invalid rows, slot-permutation and
compaction invariance, closed-form special cases, the e4m3fn table against
torch's own float8 conversion, and the fp8 scale-folding identity. The
two-segment forward is pinned to the one-segment one: with equal scales it
equals attention over the concatenated pools, with a power-of-two scale ratio
it equals attention over one bf16 pool holding the rescaled codes exactly
(scale folding), an all-invalid segment leaves the other segment's result,
and brute force covers it directly.
"""

from __future__ import annotations

import numpy as np

D_V = 512  # value width: the first 512 columns of every gathered row


# ---------------------------------------------------------------- decoding ---

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 bits are the top half of fp32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16) if b.dtype.itemsize == 2 else b.astype(np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 float8_e4m3fn codes, from the OCP definition.

    code = s eeee mmm.  exponent field e in 1..15: (-1)^s * 2^(e-7) * (1 + m/8);
    e == 0 (subnormal): (-1)^s * 2^-6 * (m/8); e == 15 and m == 7: NaN.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            table[code] = np.nan
        elif e == 0:
            table[code] = sign * (2.0 ** -6) * (m / 8.0)
        else:
            table[code] = sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return table


_E4M3FN = e4m3fn_table()


def decode_rows(pool_raw: np.ndarray, rows: np.ndarray, d_qk: int, kv_dtype: str,
                kv_scale: float | None) -> np.ndarray:
    """fp64 values of pool rows ``rows`` (first d_qk columns).

    bf16 pools hold bit patterns (uint16); fp8 pools hold e4m3fn codes (uint8)
    whose value is code * kv_scale, kv_scale being the fp32 per-tensor scale.
    """
    raw = pool_raw[rows, :d_qk]
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        if kv_scale is None:
            raise ValueError("fp8 pool needs kv_scale")
        s = float(np.float32(kv_scale))
        return _E4M3FN[np.asarray(raw, dtype=np.uint8)] * s
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


# ------------------------------------------------------------- attention ---

def softmax_weights(scores: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row-wise softmax of fp64 scores [H, n] with its max and sum.

    Returns (w / l, m, l) where m = max_j s_j, w_j = exp(s_j - m), l = sum_j w_j.
    """
    m = scores.max(axis=1)
    w = np.exp(scores - m[:, None])
    l = w.sum(axis=1)
    return w / l[:, None], m, l


def attend_row(q_row: np.ndarray, gathered: np.ndarray, sm: float) -> tuple[np.ndarray, np.ndarray]:
    """One query row against its gathered rows.

    q_row: fp64 [H, D_qk]; gathered: fp64 [n, D_qk] with n >= 1.
    Returns O [H, 512] and LSE [H].
    """
    scores = sm * (q_row @ gathered.T)             # [H, n]
    p, m, l = softmax_weights(scores)
    out = p @ gathered[:, :D_V]                    # [H, 512]
    lse = m + np.log(l)
    return out, lse


def decode_q(q_raw: np.ndarray, q_scale: float | None) -> np.ndarray:
    """fp64 values of q: bf16 bit patterns (uint16), or float8_e4m3fn codes
    (uint8) times the per-tensor q scale ("an fp8 q is widened in the
    kernel", commit notes on the two-loop route of "[Triton/Gluon] GFX950
    sparse mla optimizations"; value = code * q_scale, as for the cache)."""
    q_raw = np.asarray(q_raw)
    if q_raw.dtype == np.uint8:
        return e4m3fn_table()[q_raw] * (1.0 if q_scale is None else float(np.float32(q_scale)))
    return bf16_bits_to_f64(q_raw)


def sparse_mla_fwd(q_bits: np.ndarray, pool_raw: np.ndarray, kv_dtype: str,
                   kv_scale: float | None, indices: np.ndarray, sm_scale: float,
                   rows: np.ndarray | None = None,
                   q_scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Sparse MLA forward in fp64.

    q_bits   : uint16 [R, H, D_qk] bf16 bit patterns of q, or uint8 e4m3fn
               codes of an fp8 q (value = code * q_scale)
    pool_raw : uint16 [N, >=D_qk] bf16 bits, or uint8 [N, >=D_qk] e4m3fn codes
    kv_dtype : "bf16" or "fp8"
    kv_scale : fp32 per-tensor scale for fp8 pools (None for bf16)
    indices  : int32 [R, K]; negative = invalid slot
    sm_scale : softmax scale (used as its fp32 value)
    rows     : optional subset of query rows to compute (for big workloads)
    q_scale  : fp32 per-tensor scale of an fp8 q (None: 1)

    Returns (out fp64 [len(rows), H, 512], lse fp64 [len(rows), H]).
    """
    q_bits = np.asarray(q_bits)
    indices = np.asarray(indices)
    R, H, d_qk = q_bits.shape
    if d_qk < D_V:
        raise ValueError("D_qk must be at least 512")
    n_pool = pool_raw.shape[0]
    sm = float(np.float32(sm_scale))
    sel = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(sel), H, D_V), dtype=np.float64)
    lse = np.full((len(sel), H), -np.inf, dtype=np.float64)
    for i, r in enumerate(sel):
        idx = indices[r]
        valid = idx[idx >= 0].astype(np.int64)
        if valid.size == 0:
            continue
        if valid.max() >= n_pool:
            raise IndexError(f"row {r}: index {int(valid.max())} >= pool rows {n_pool}")
        gathered = decode_rows(pool_raw, valid, d_qk, kv_dtype, kv_scale)
        out[i], lse[i] = attend_row(decode_q(q_bits[r], q_scale), gathered, sm)
    return out, lse


def _q_raw(q):
    import torch  # local: the oracle itself is numpy-only
    if q.dtype == torch.float8_e4m3fn:
        return q.contiguous().view(torch.uint8).numpy()
    return q.contiguous().view(torch.int16).numpy().view(np.uint16)


def sparse_mla_fwd_torch(q, pool, kv_scale, indices, sm_scale, rows=None, q_scale=None):
    """Convenience wrapper taking CPU torch tensors (bf16 or e4m3fn q with
    q_scale; bf16 or e4m3fn pool).

    Only views raw bytes; all arithmetic is in ``sparse_mla_fwd``.
    """
    import torch  # local: the oracle itself is numpy-only

    q_bits = _q_raw(q)
    qs = None if q_scale is None else float(q_scale.reshape(-1)[0])
    if pool.dtype == torch.bfloat16:
        kv_dtype, raw, s = "bf16", pool.view(torch.int16).numpy().view(np.uint16), None
    elif pool.dtype == torch.float8_e4m3fn:
        kv_dtype, raw = "fp8", pool.view(torch.uint8).numpy()
        s = float(kv_scale.reshape(-1)[0])
    else:
        raise ValueError(f"unsupported pool dtype {pool.dtype}")
    return sparse_mla_fwd(q_bits, raw, kv_dtype, s, indices.numpy(), sm_scale, rows=rows,
                          q_scale=qs)


# ------------------------------------------------------------ two segments ---

def sparse_mla_fwd_2seg(q_bits: np.ndarray, pool_raw: np.ndarray, kv_dtype: str,
                        kv_scale: float | None, indices: np.ndarray,
                        extra_raw: np.ndarray, extra_scale: float | None,
                        extra_indices: np.ndarray, sm_scale: float,
                        rows: np.ndarray | None = None,
                        q_scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Two-segment sparse MLA forward in fp64 (q as for sparse_mla_fwd).

    After "[Triton/Gluon] GFX950 sparse mla optimizations" (aiter PR 6159),
    commit notes on the per-tensor fp8 two-loop route: a row attends under
    one softmax to the valid slots of its main indices (into pool_raw, value =
    code * kv_scale for fp8) and of its extra indices (into extra_raw, value =
    code * extra_scale; the extra scale defaults to kv_scale). Written as the
    plain definition: the gathered rows of both segments, each decoded with
    its own scale, form one set of slots. Both pools have the same dtype.

    Returns (out fp64 [len(rows), H, 512], lse fp64 [len(rows), H]).
    """
    q_bits = np.asarray(q_bits)
    indices = np.asarray(indices)
    extra_indices = np.asarray(extra_indices)
    R, H, d_qk = q_bits.shape
    if d_qk < D_V:
        raise ValueError("D_qk must be at least 512")
    if kv_dtype == "fp8" and extra_scale is None:
        extra_scale = kv_scale
    sm = float(np.float32(sm_scale))
    sel = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(sel), H, D_V), dtype=np.float64)
    lse = np.full((len(sel), H), -np.inf, dtype=np.float64)
    for i, r in enumerate(sel):
        parts = []
        for raw, scale, idx in ((pool_raw, kv_scale, indices[r]),
                                (extra_raw, extra_scale, extra_indices[r])):
            valid = idx[idx >= 0].astype(np.int64)
            if valid.size == 0:
                continue
            if valid.max() >= raw.shape[0]:
                raise IndexError(f"row {r}: index {int(valid.max())} >= pool rows {raw.shape[0]}")
            parts.append(decode_rows(raw, valid, d_qk, kv_dtype, scale))
        if not parts:
            continue
        out[i], lse[i] = attend_row(decode_q(q_bits[r], q_scale), np.concatenate(parts), sm)
    return out, lse


def sparse_mla_fwd_2seg_torch(q, pool, kv_scale, indices, extra_pool, extra_scale,
                              extra_indices, sm_scale, rows=None, q_scale=None):
    """Wrapper of ``sparse_mla_fwd_2seg`` taking CPU torch tensors. Only views
    raw bytes; all arithmetic is in ``sparse_mla_fwd_2seg``."""
    import torch  # local: the oracle itself is numpy-only

    q_bits = _q_raw(q)
    qs = None if q_scale is None else float(q_scale.reshape(-1)[0])
    if pool.dtype == torch.bfloat16:
        kv_dtype = "bf16"
        raw = pool.view(torch.int16).numpy().view(np.uint16)
        xraw = extra_pool.view(torch.int16).numpy().view(np.uint16)
        s1 = s2 = None
    elif pool.dtype == torch.float8_e4m3fn:
        kv_dtype = "fp8"
        raw, xraw = pool.view(torch.uint8).numpy(), extra_pool.view(torch.uint8).numpy()
        s1 = float(kv_scale.reshape(-1)[0])
        s2 = None if extra_scale is None else float(extra_scale.reshape(-1)[0])
    else:
        raise ValueError(f"unsupported pool dtype {pool.dtype}")
    return sparse_mla_fwd_2seg(q_bits, raw, kv_dtype, s1, indices.numpy(), xraw, s2,
                               extra_indices.numpy(), sm_scale, rows=rows, q_scale=qs)


# ----------------------------------------------------- split combination ---

def lse_combine(partial_out: np.ndarray, partial_lse: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Combine attention over disjoint slot subsets (splits), in fp64.

    partial_out [S, ..., 512] holds each split's normalised output and
    partial_lse [S, ...] its LSE (-inf for a split with no valid slot).
    lse = ln sum_s exp(lse_s); O = sum_s exp(lse_s - lse) O_s. All -inf gives
    O = 0, lse = -inf. Exact in real arithmetic: softmax over a union of
    disjoint sets is the LSE-weighted mix of the per-set softmaxes.
    """
    m = partial_lse.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(partial_lse), np.exp(partial_lse - m_safe), 0.0)
    total = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    scale = np.where(finite, 1.0 / np.where(finite, total, 1.0), 0.0)
    out = np.einsum("s...,s...d->...d", w, partial_out) * scale[..., None]
    return out, lse
