"""Pins of the oracle's precision-aware router GEMM.

The blog's "Router GEMM" section splits fp32 router weights into a bf16 part
cut by truncation and a bf16 part holding the residual scaled by 256, and
forms the scores as two bf16 products combined with the scale in the
epilogue.  The checks below tie the oracle to the definitions (torch's own
bf16 values and RNE cast), to exact cases, and to the approximation bound
that the split guarantees, and reproduce the point of the method on the
pages' shape (K = 4096, N = 192): the split's error against an fp32-weight
product stays below the blog's 0.00177, plain bf16 weights do not.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_testlib import golden
from moe_inputs import router_hidden, router_weight


def bf16_vals(codes):
    return torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).double().numpy()


def rand_w(shape, seed, std=0.02):
    return router_weight(shape[0], shape[1], seed, std)


def test_split_exact_cases():
    w = np.array([[1.0, 1.0 + 2 ** -10, -0.5, 3.0, 0.0, -(1.0 + 2 ** -20)]], dtype=np.float32)
    hi, lo = oracle.router_split(w)
    hv, lv = bf16_vals(hi), bf16_vals(lo)
    assert hv[0].tolist() == [1.0, 1.0, -0.5, 3.0, 0.0, -1.0]
    # residuals: 0, 2^-10 * 256 = 1/4, 0, 0, 0, -2^-20 * 256 = -2^-12 (all exact in bf16)
    assert lv[0].tolist() == [0.0, 0.25, 0.0, 0.0, 0.0, -(2.0 ** -12)]


def test_high_part_is_truncation():
    w = rand_w((64, 512), 1).numpy()
    hi, _ = oracle.router_split(w)
    hv = bf16_vals(hi)
    # same sign, not larger in magnitude, and the next bf16 away from zero overshoots
    nxt = bf16_vals((hi.astype(np.int32) + 1).astype(np.uint16))
    aw = np.abs(w.astype(np.float64))
    assert (np.abs(hv) <= aw).all()
    assert (np.abs(nxt) > aw).all()
    assert ((hv == 0) | (np.sign(hv) == np.sign(w))).all()


def test_low_part_is_rne_of_exact_residual():
    w = rand_w((64, 512), 2, std=1.0)
    hi, lo = oracle.router_split(w.numpy())
    resid = (w - torch.from_numpy(bf16_vals(hi)).float()) * 256.0      # exact in fp32
    want = resid.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert (lo == want).all()


def test_split_bound():
    # bf16 keeps 8 significant bits: RNE is off by at most 2^-8 of the value,
    # truncation by less than 2^-7, so
    # |W - (W_high + W_low/256)| <= 2^-8 |W - W_high| < 2^-15 |W|
    w = rand_w((128, 1024), 3, std=1.0).numpy().astype(np.float64)
    hi, lo = oracle.router_split(w.astype(np.float32))
    approx = bf16_vals(hi) + bf16_vals(lo) / 256.0
    err = np.abs(w - approx)
    assert (err <= 2.0 ** -8 * np.abs(w - bf16_vals(hi)) + 1e-300).all()
    assert (err < 2.0 ** -15 * np.abs(w) + 1e-300).all()
    # ... and the bound is nearly reached (a dropped low part would be ~2^-7)
    assert err.max() > 2.0 ** -18 * np.abs(w).max()


def test_scores_unit_vectors_and_linearity():
    N, K = 24, 96
    w = rand_w((N, K), 4).numpy()
    hi, lo = oracle.router_split(w)
    x = torch.zeros(K, K, dtype=torch.bfloat16)
    x[torch.arange(K), torch.arange(K)] = 1.0
    s = oracle.router_scores(x, hi, lo)
    np.testing.assert_array_equal(s, (bf16_vals(hi) + bf16_vals(lo) / 256.0).T)
    g = torch.Generator().manual_seed(5)
    a = torch.randn(3, K, generator=g).bfloat16()
    sa = oracle.router_scores(a, hi, lo)
    s2 = oracle.router_scores((a.float() * 2).bfloat16(), hi, lo)     # exact doubling
    np.testing.assert_array_equal(s2, 2 * sa)
    neg = oracle.router_scores((-a.float()).bfloat16(), hi, lo)
    np.testing.assert_array_equal(neg, -sa)
    assert (oracle.router_scores(torch.zeros(2, K).bfloat16(), hi, lo) == 0).all()


def test_scores_against_fp32_weights_within_bound():
    T, N, K = 16, 64, 2048
    w = rand_w((N, K), 6)
    x = torch.randn(T, K, generator=torch.Generator().manual_seed(7)).bfloat16()
    hi, lo = oracle.router_split(w.numpy())
    s = oracle.router_scores(x, hi, lo)
    exact = x.double() @ w.double().T
    bound = 2.0 ** -15 * (x.double().abs() @ w.double().abs().T)
    assert (np.abs(s - exact.numpy()) <= bound.numpy()).all()


def test_pages_shape_error_target():
    # the blog's sweep shape: K = 4096, N = 192; fp32 weights of a typical
    # router init (N(0, 0.02)); the error target is 0.00177 max abs error
    # against the fp32-weight product
    tgt = golden("router_gemm_error_target")
    T, N, K = 256, tgt["N"], tgt["K"]
    w = rand_w((N, K), 8)
    x = router_hidden(T, K, 9)
    hi, lo = oracle.router_split(w.numpy())
    s = oracle.router_scores(x, hi, lo)
    exact = (x.double() @ w.double().T).numpy()
    err_split = float(np.abs(s - exact).max())
    err_bf16 = float(np.abs((x.double() @ w.bfloat16().double().T).numpy() - exact).max())
    print(f"max|err| split {err_split:.3e}, plain bf16 weights {err_bf16:.3e}")
    assert err_split <= tgt["max_abs_error"]
    assert err_bf16 > tgt["max_abs_error"]
