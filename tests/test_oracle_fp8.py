"""Pins of the oracle's fp8 w8a8 forward.

The HPC-Ops MoE runs with BF16 hidden states and FP8 E4M3 expert weights,
and requantises the SiLU-and-mul output to FP8 before the down GEMM
(HPC-Ops x SGLang blog, section "MoE", gate-up & activation; operator
table).  The oracle applies the same quantisation steps; here it is pinned
against a dense torch fp64 evaluation whose quantisation uses torch's own
float8_e4m3fn cast, and the claim that e4m3 x e4m3 dot products are exact in
fp64 is checked against integer arithmetic.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, quantize_weight_rows


def torch_quant_rows(v32):
    amax = v32.abs().amax(dim=-1)
    s = torch.where(amax > 0, (amax.double() / 448.0).float(), torch.ones_like(amax))
    inv = torch.where(amax > 0, (448.0 / amax.double()).float(), torch.ones_like(amax))
    q = (v32 * inv.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q, s


def torch_fp8_reference(x, w, ids, W1q, s1, W2q, s2):
    T, H = x.shape
    E, I2, _ = W1q.shape
    I = I2 // 2
    xq, sx = torch_quant_rows(x.float())
    xd = xq.double()
    W1d = W1q.view(torch.float8_e4m3fn).double()
    W2d = W2q.view(torch.float8_e4m3fn).double()
    out = torch.zeros(T, H, dtype=torch.float64)
    hqs = {}
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not (0 <= e < E):
                continue
            g = (sx[t].double() * s1[e, :I].double()) * (W1d[e, :I] @ xd[t])
            u = (sx[t].double() * s1[e, I:].double()) * (W1d[e, I:] @ xd[t])
            a = (F.silu(g) * u).float()
            hq, sh = torch_quant_rows(a.unsqueeze(0))
            hqs[(t, j)] = hq.view(torch.uint8)[0]
            y = (sh[0].double() * s2[e].double()) * (W2d[e] @ hq[0].double())
            out[t] += w[t, j].double() * y
    return out.numpy(), xq.view(torch.uint8).numpy(), sx.numpy(), hqs


@pytest.mark.parametrize("T,E,H,I,k", [(5, 8, 128, 64, 2), (9, 16, 256, 96, 4)])
def test_fp8_forward_matches_torch_quantised_reference(T, E, H, I, k):
    wl = custom_workload(E, H, I, k, dtype="fp8", seed=21)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, T, seed=31)
    ids[0, 0] = -1                                         # one dropped pair
    out, (xq, sx, hq, sh) = oracle.forward_fp8(x, w, ids, W["w1"], W["w1_scale"], W["w2"],
                                               W["w2_scale"], want_quant=True)
    ref, rxq, rsx, rhq = torch_fp8_reference(x, w, ids, W["w1"], W["w1_scale"], W["w2"],
                                             W["w2_scale"])
    assert np.array_equal(xq, rxq) and np.array_equal(sx, rsx)
    total = flips = 0
    for (t, j), codes in rhq.items():
        total += codes.numel()
        flips += int((torch.from_numpy(hq[t, j]) != codes).sum())
    # the intermediate is an fp32 rounding of an fp64 value; silu() of the two
    # sides may differ in the last ulp, which can move a code across a
    # rounding boundary very rarely
    assert flips <= max(1, total // 1000)
    err = np.max(np.abs(out - ref)) / np.max(np.abs(ref))
    assert err < (1e-12 if flips == 0 else 1e-2)


def test_fp8_zero_token_row():
    wl = custom_workload(8, 128, 64, 2, dtype="fp8", seed=22)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 3, seed=5)
    x[1] = 0
    out, (xq, sx, hq, sh) = oracle.forward_fp8(x, w, ids, W["w1"], W["w1_scale"], W["w2"],
                                               W["w2_scale"], want_quant=True)
    assert sx[1] == 1.0 and not xq[1].any()
    assert sh[1].tolist() == [1.0, 1.0] and not hq[1].any()     # silu(0)*0 = 0 rows
    assert not out[1].any() and out[0].any() and out[2].any()


def test_fp8_dot_products_are_exact_in_fp64():
    # every e4m3 value is an integer multiple of 2^-9 below 2^9, so a product
    # is a multiple of 2^-18 below 2^18 and a 7168-term sum needs < 53 bits
    rng = np.random.default_rng(1)
    H = 7168
    for trial in range(4):
        a = rng.integers(0, 256, H).astype(np.uint8)
        b = rng.integers(0, 256, H).astype(np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x7E                    # no NaN codes
        b[(b & 0x7F) == 0x7F] = 0x7E
        if trial == 0:
            a[:] = 0x7E
            b[:] = 0x7E                                 # worst case: 448*448*H
        va = np.array([oracle.e4m3_value(c) for c in a])
        vb = np.array([oracle.e4m3_value(c) for c in b])
        s = 0.0
        for i in range(H):
            s += va[i] * vb[i]
        exact = sum(int(round(x * 512)) * int(round(y * 512)) for x, y in zip(va, vb))
        assert s * 2.0 ** 18 == float(exact) and int(s * 2.0 ** 18) == exact


def test_generator_weight_quantisation_is_per_output_channel():
    wl = custom_workload(4, 128, 64, 2, dtype="fp8", seed=23)
    W = make_weights(wl)
    s1 = W["w1_scale"]
    dec = W["w1"].view(torch.float8_e4m3fn).float()
    # every row reaches +-448 at its amax
    assert torch.all(dec.abs().amax(dim=-1) == 448.0)
    assert s1.shape == (4, 128) and W["w2_scale"].shape == (4, 128)
    # round trip of a row through quantize_weight_rows reproduces its codes
    q, s = quantize_weight_rows(dec[0, :3] * s1[0, :3, None])
    assert torch.equal(q, W["w1"][0, :3])
