"""Pins of the oracle's router top-k against values fixed by the mathematics.

The router's fp32 expert scores feed a top-k choice of experts (HPC-Ops x
SGLang blog, section "Router GEMM"); the layer then runs the chosen experts
with the renormalised softmax weights, and fused shared experts appear as
extra expert ids of weight 1 (SGLang fused-MoE tuning guide, model-config
section).  Each test below checks the oracle against something other than
its own formula: closed-form weights, a brute-force ranking written
independently, the full softmax at k = E, the ratio and shift laws of the
softmax, and torch's stable sort + softmax.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def brute_ids(row, k):
    """Ranking by (descending value, ascending id), NaN as -inf, by a plain sort."""
    key = [(-(v if not math.isnan(v) else -math.inf), e) for e, v in enumerate(row)]
    return [e for _, e in sorted(key)[:k]]


def test_closed_form_log_logits():
    # logits log 1, log 2, log 3, log 4: softmax = (1, 2, 3, 4) / 10
    l = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    for k, want_ids, want_w in [
        (1, [3], [1.0]),
        (2, [3, 2], [4 / 7, 3 / 7]),
        (3, [3, 2, 1], [4 / 9, 3 / 9, 2 / 9]),
        (4, [3, 2, 1, 0], [0.4, 0.3, 0.2, 0.1]),
    ]:
        ids, w = oracle.router_topk(l, k)
        assert ids[0].tolist() == want_ids
        # the fp32 rounding of log(n) moves the weights by about 1e-7
        np.testing.assert_allclose(w[0], want_w, rtol=0, atol=3e-7)
        ids, w = oracle.router_topk(l, k, renormalize=False)
        assert ids[0].tolist() == want_ids
        np.testing.assert_allclose(w[0], [v / 10 for v in (4, 3, 2, 1)][:k], rtol=0, atol=3e-7)


def test_two_experts_is_sigmoid():
    # k = 2 of E = 2: w0 = 1 / (1 + exp(l1 - l0)) exactly (the logistic function)
    g = np.random.default_rng(3)
    l = g.normal(0.0, 3.0, size=(200, 2)).astype(np.float32)
    ids, w = oracle.router_topk(l, 2)
    hi = np.maximum(l[:, 0], l[:, 1]).astype(np.float64)
    lo = np.minimum(l[:, 0], l[:, 1]).astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(lo - hi)), rtol=1e-14)
    np.testing.assert_allclose(w[:, 1], 1.0 / (1.0 + np.exp(hi - lo)), rtol=1e-14)
    assert (ids[:, 0] == np.where(l[:, 1] > l[:, 0], 1, 0)).all()


def test_equal_logits_take_lowest_ids_equal_weights():
    for E in (1, 3, 8, 64, 256):
        for k in sorted({1, min(2, E), min(8, E), min(16, E)}):
            l = np.full((3, E), 0.75, dtype=np.float32)
            ids, w = oracle.router_topk(l, k)
            assert (ids == np.arange(k)).all()
            np.testing.assert_allclose(w, 1.0 / k, rtol=1e-15)
            _, w = oracle.router_topk(l, k, renormalize=False)
            np.testing.assert_allclose(w, 1.0 / E, rtol=1e-14)


def test_brute_force_every_tiny_case():
    # every row over a 3-value alphabet (ties everywhere), E <= 5, every k
    for E in range(1, 6):
        rows = np.array(list(itertools.product([-1.0, 0.0, 0.5], repeat=E)), dtype=np.float32)
        for k in range(1, E + 1):
            ids, w = oracle.router_topk(rows, k)
            for r in range(rows.shape[0]):
                assert ids[r].tolist() == brute_ids(rows[r].tolist(), k)
            assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_nan_ranks_last():
    l = np.array([[np.nan, 1.0, np.nan, -5.0, 2.0]], dtype=np.float32)
    ids, _ = oracle.router_topk(l, 5)
    assert ids[0].tolist() == [4, 1, 3, 0, 2] == brute_ids(l[0].tolist(), 5)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (128, 8), (256, 8), (37, 16)])
def test_full_softmax_ratio_and_shift(E, k):
    g = np.random.default_rng(E * 31 + k)
    l = g.normal(0.0, 1.0, size=(64, E)).astype(np.float32)
    # k = E, renormalised: exactly the softmax over all experts
    ids, w = oracle.router_topk(l, E)
    ld = l.astype(np.float64)
    sm = np.exp(ld - ld.max(axis=1, keepdims=True))
    sm /= sm.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(sm, ids.astype(np.int64), 1), rtol=1e-13)
    # without renormalisation the k selected weights are those softmax values
    ids, w = oracle.router_topk(l, k, renormalize=False)
    np.testing.assert_allclose(w, np.take_along_axis(sm, ids.astype(np.int64), 1), rtol=1e-13)
    # ratio law: w_i / w_j = exp(l_i - l_j); weights sum to one; descending
    ids, w = oracle.router_topk(l, k)
    sel = np.take_along_axis(ld, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w / w[:, :1], np.exp(sel - sel[:, :1]), rtol=1e-13)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    assert (np.diff(sel, axis=1) <= 0).all()
    # shift law: adding an exactly representable constant changes nothing
    lq = (np.round(l * 64) / 64).astype(np.float32)
    ids0, w0 = oracle.router_topk(lq, k)
    ids1, w1 = oracle.router_topk(lq + np.float32(8.0), k)
    assert (ids0 == ids1).all()
    np.testing.assert_allclose(w0, w1, rtol=1e-14)


def test_matches_torch_sort_and_softmax():
    # an independent ranking and softmax: torch's stable descending sort and
    # torch.softmax in fp64 over the selected logits
    g = torch.Generator().manual_seed(5)
    for E, k in [(8, 2), (64, 8), (128, 8), (256, 8), (200, 13)]:
        l = torch.randn(500, E, generator=g)
        l[::7] = torch.round(l[::7] * 2) / 2          # rows with many ties
        order = torch.sort(l, dim=1, descending=True, stable=True).indices[:, :k]
        want_w = torch.softmax(torch.gather(l, 1, order).double(), dim=1)
        ids, w = oracle.router_topk(l.numpy(), k)
        assert (ids == order.numpy()).all()
        np.testing.assert_allclose(w, want_w.numpy(), rtol=1e-13)


def test_shared_columns():
    g = np.random.default_rng(9)
    l = g.normal(size=(33, 16)).astype(np.float32)
    ids0, w0 = oracle.router_topk(l, 4)
    for ns in (1, 2):
        ids, w = oracle.router_topk(l, 4, n_shared=ns)
        assert ids.shape == (33, 4 + ns)
        assert (ids[:, :4] == ids0).all() and (w[:, :4] == w0).all()
        assert (ids[:, 4:] == np.arange(16, 16 + ns)).all()
        assert (w[:, 4:] == 1.0).all()


def test_empty():
    ids, w = oracle.router_topk(np.zeros((0, 8), dtype=np.float32), 2, n_shared=1)
    assert ids.shape == (0, 3) and w.shape == (0, 3)
