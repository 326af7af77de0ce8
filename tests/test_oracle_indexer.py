"""Pins for the indexer oracle (fp8 MQA logits and the per-row top-k), each
against something other than the oracle's own formula: torch's float8
decoding and einsum in fp64, closed-form special cases, explicit window
masks, and a full sort. CPU only, seconds."""

import numpy as np
import pytest
import torch

from oracle import indexer as ix
from sparse_mla_attention_05_amd.inputs import (IndexerWorkload, make_indexer_inputs,
                                                make_topk_logits)


def _codes(t):
    return t.view(torch.uint8).numpy()


def _brute(inp, rows=None):
    """torch: decode through torch's own float8 conversion, einsum in fp64,
    relu, weights, per-key scale, window mask."""
    q = inp.q.to(torch.float64)
    k = inp.k.to(torch.float64)
    s = torch.einsum("mhd,nd->mhn", q, k)
    lg = (torch.relu(s) * inp.w.double()[:, :, None]).sum(1) * inp.kv_scale.double()[None, :]
    n = torch.arange(k.shape[0])[None, :]
    inside = (n >= inp.ks.long()[:, None]) & (n < inp.ke.long()[:, None])
    lg = torch.where(inside, lg, torch.full_like(lg, -float("inf")))
    return lg.numpy() if rows is None else lg.numpy()[rows]


def _run(inp, rows=None):
    return ix.mqa_logits(_codes(inp.q), _codes(inp.k), inp.kv_scale.numpy(), inp.w.numpy(),
                         inp.ks.numpy(), inp.ke.numpy(), rows=rows)


def test_logits_match_brute_force():
    inp = make_indexer_inputs("ix_tiny")
    got, want = _run(inp), _brute(inp)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == -np.inf)
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12 * np.abs(want[fin]).max())


def test_rows_argument_selects_rows():
    inp = make_indexer_inputs("ix_tiny")
    rows = np.array([0, 17, 69])
    assert np.array_equal(_run(inp, rows=rows), _run(inp)[rows])


def test_one_hot_head_is_one_relu_dot():
    """w = e_j, kv_scale = 1: the logit is relu(q_j . k_n) of the decoded codes."""
    inp = make_indexer_inputs("ix_tiny")
    j = 5
    inp.w = torch.zeros_like(inp.w)
    inp.w[:, j] = 1.0
    inp.kv_scale = torch.ones_like(inp.kv_scale)
    got = _run(inp)
    q = inp.q.to(torch.float64)[:, j, :]
    want = torch.relu(q @ inp.k.to(torch.float64).T).numpy()
    fin = np.isfinite(got)
    assert np.array_equal(got[fin], want[fin])
    assert (got[fin] >= 0).all() and (got[fin] == 0).any()


def test_windows_are_half_open_and_clipped():
    w = IndexerWorkload("t", rows=6, keys=40, requests=1, topk=8, seed=3)
    inp = make_indexer_inputs(w)
    inp.ks = torch.tensor([0, 5, 10, -7, 30, 20], dtype=torch.int32)
    inp.ke = torch.tensor([1, 5, 11, 3, 99, 10], dtype=torch.int32)
    got = _run(inp)
    fin = np.isfinite(got)
    assert fin[0].nonzero()[0].tolist() == [0]
    assert not fin[1].any() and not fin[5].any()           # ke == ks, ke < ks: empty
    assert fin[2].nonzero()[0].tolist() == [10]
    assert fin[3].nonzero()[0].tolist() == [0, 1, 2]       # ks < 0 clipped
    assert fin[4].nonzero()[0].tolist() == list(range(30, 40))  # ke > N clipped


def test_windows_of_the_workloads():
    inp = make_indexer_inputs("ix_tiny")
    ks, ke = inp.ks.numpy(), inp.ke.numpy()
    assert ks[0] == 0 and ke[0] == 300 - 35 + 1 and ke[34] == 300
    assert ks[35] == 300 and ke[69] == 600


# ---------------------------------------------------------------- top-k ---

def _sorted_topk(x, lo, hi, k):
    n = np.arange(lo, hi)
    v = x[lo:hi].astype(np.float64)
    order = sorted(range(len(n)), key=lambda i: (-v[i], n[i]))   # plain Python sort
    return sorted(n[order[:k]].tolist())


def test_topk_matches_a_full_sort():
    k = 64
    x, ks, ke = make_topk_logits(30, 500, seed=4, k=k)
    got = ix.topk_indices(x.numpy(), ks.numpy(), ke.numpy(), k)
    for r in range(30):
        lo, hi = int(ks[r]), int(ke[r])
        want = _sorted_topk(x[r].numpy(), lo, hi, k)
        row = got[r]
        assert row[:len(want)].tolist() == want
        assert np.all(row[len(want):] == -1)


def test_topk_ties_go_to_the_lower_index_and_short_windows_pad():
    x = np.zeros((3, 10), np.float32)
    x[0] = [1, 5, 5, 5, 0, 5, 2, 2, 2, 9]
    got = ix.topk_indices(x, np.array([0, 2, 4]), np.array([10, 5, 4]), 4)
    assert got[0].tolist() == [1, 2, 3, 9]          # 9, then three of the 5s: the lowest
    assert got[1].tolist() == [2, 3, 4, -1]
    assert got[2].tolist() == [-1, -1, -1, -1]      # empty window


@pytest.mark.parametrize("mistake", ["relu_after_sum", "no_kv_scale", "inclusive_ke", "no_relu"])
def test_planted_mistakes_are_caught(mistake, monkeypatch):
    orig = ix.mqa_logits

    def bad(q_codes, k_codes, kv_scale, w, ks, ke, rows=None):
        if mistake == "no_kv_scale":
            return orig(q_codes, k_codes, np.ones_like(kv_scale), w, ks, ke, rows)
        if mistake == "inclusive_ke":
            return orig(q_codes, k_codes, kv_scale, w, ks, np.asarray(ke) + 1, rows)
        k = ix.decode_e4m3(k_codes)
        out = np.full((q_codes.shape[0], k.shape[0]), -np.inf)
        for m in range(q_codes.shape[0]):
            lo, hi = ix.clip_window(ks[m], ke[m], k.shape[0])
            s = ix.decode_e4m3(q_codes[m]) @ k[lo:hi].T
            if mistake == "relu_after_sum":
                out[m, lo:hi] = np.maximum((s * w[m][:, None]).sum(0), 0) * kv_scale[lo:hi]
            else:
                out[m, lo:hi] = (s * w[m][:, None]).sum(0) * kv_scale[lo:hi]
        return out

    monkeypatch.setattr(ix, "mqa_logits", bad)
    failed = 0
    for pin in (test_logits_match_brute_force, test_one_hot_head_is_one_relu_dot,
                test_windows_are_half_open_and_clipped):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
