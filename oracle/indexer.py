"""CPU oracle of the indexer that produces the sparse attention's index rows:
fp8 MQA logits, then a per-row top-k.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
package smoke check and the benchmark's CPU-baseline leg may call it, the
library never does, and it shares no code with the HIP path.

Logits (the formula of "[HIP] [JIT] fp8_mqa_logits: v35w gfx950 prefill
indexer logits kernel" (aiter PR 7183), Motivation): for query row m and key
n, with H = 32 heads of 128 dims,

    logits[m, n] = sum_h relu(Q[m, h, :] . K[n, :]) * w[m, h] * kv_scale[n]
                   for n in [ks[m], ke[m]),  -inf elsewhere

Q and K are float8_e4m3fn codes (decoded exactly), kv_scale fp32 per key, w
fp32 per (row, head). Written out in fp64: every product of two e4m3 values
and their 128-term sum is exact in fp64, so only the head sum and the scales
round.

Top-k (the pages give no selection algorithm; the plainest reading of "the
indices of the k largest logits"): for row m, among n in [ks[m], ke[m]) the k
keys with the largest logits; a window with fewer than k keys gives all of
them and -1 for the rest. Ties at the k-th value may be broken either way;
the selected multiset of values is unique.

Readings where the pages are silent:
  * ks and ke are clipped to [0, N]; ke <= ks is an empty window (all -inf).
  * Q carries no scale of its own (a producer folds it into w).
  * The order of the returned indices does not matter to the attention (slot
    order is irrelevant there); the oracle returns them ascending.

Parity pins (tests/test_oracle_indexer.py, CPU): brute force through torch's
float8 decoding and an einsum in fp64, one-hot head weights against a single
relu'd dot, windows against explicit masks, the e4m3 decoding against
torch's, and the top-k against a full sort.
"""

from __future__ import annotations

import numpy as np

from .sparse_mla_oracle import e4m3fn_table


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """fp64 values of float8_e4m3fn codes (exact)."""
    return e4m3fn_table()[np.asarray(codes, dtype=np.uint8)]


def clip_window(ks: int, ke: int, n: int) -> tuple[int, int]:
    lo = min(max(int(ks), 0), n)
    hi = min(max(int(ke), 0), n)
    return lo, max(lo, hi)


def mqa_logits(q_codes: np.ndarray, k_codes: np.ndarray, kv_scale: np.ndarray, w: np.ndarray,
               ks: np.ndarray, ke: np.ndarray, rows=None) -> np.ndarray:
    """fp64 logits [len(rows), N] (rows: all rows when None).

    q_codes uint8 [M, H, D]; k_codes uint8 [N, D]; kv_scale fp32 [N];
    w fp32 [M, H]; ks, ke int [M].
    """
    q_codes = np.asarray(q_codes, dtype=np.uint8)
    k = decode_e4m3(k_codes)                       # [N, D]
    N = k.shape[0]
    scale = np.asarray(kv_scale, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    rows = np.arange(q_codes.shape[0]) if rows is None else np.asarray(rows)
    out = np.full((len(rows), N), -np.inf)
    for i, m in enumerate(rows):
        lo, hi = clip_window(ks[m], ke[m], N)
        if hi == lo:
            continue
        q = decode_e4m3(q_codes[m])                # [H, D]
        s = q @ k[lo:hi].T                         # [H, n], exact
        out[i, lo:hi] = (np.maximum(s, 0.0) * w[m][:, None]).sum(axis=0) * scale[lo:hi]
    return out


def topk_indices(logits: np.ndarray, ks: np.ndarray, ke: np.ndarray, k: int) -> np.ndarray:
    """int32 [R, k]: per row the indices of the k largest logits inside the
    row's window, ascending, -1 padded. logits [R, N] (any float dtype);
    ties at the k-th value go to the lower index."""
    logits = np.asarray(logits)
    R, N = logits.shape
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        lo, hi = clip_window(ks[r], ke[r], N)
        n = np.arange(lo, hi)
        if len(n) <= k:
            sel = n
        else:
            v = logits[r, lo:hi].astype(np.float64)
            order = np.lexsort((n, -v))            # by value descending, then index ascending
            sel = np.sort(n[order[:k]])
        out[r, :len(sel)] = sel
    return out
