"""Pins of the oracle's MXFP8 (OCP Microscaling, 32-element blocks) path.

The SGLang tuning guide notes that gfx95 devices keep MXFP8's [1, 32] block
shape; the OCP MX format gives every 32 consecutive K values one E8M0 scale
2^s, s = floor(log2(amax)) - 8, and E4M3 elements.  The quantiser is pinned
to worked cases of that rule and to an independent torch implementation
(frexp for the exponent, torch's RNE e4m3 cast); the forward pass to a
dense torch reference built on that implementation.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, quantize_weight_mx


def torch_mx(v):
    """(codes, scale codes) of fp32 rows by the OCP rule, in torch."""
    v = torch.as_tensor(v, dtype=torch.float32)
    R, n = v.shape
    b = v.reshape(R, n // 32, 32)
    amax = b.abs().amax(-1)
    _, e = torch.frexp(amax)
    s = torch.where(amax > 0, e - 9, torch.full_like(e, -127)).clamp(-127, 127)
    q = (b * torch.exp2(-s.float()).unsqueeze(-1)).clamp(-448, 448).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, n).numpy(), (s + 127).to(torch.uint8).numpy()


def test_worked_cases():
    rows = np.zeros((6, 32), dtype=np.float32)
    rows[0, 0], rows[0, 1:] = 448.0, 1.0      # amax 448: s = 0, values unchanged
    rows[1, :] = 1.0                            # amax 1: s = -8, 1 -> 256
    rows[2, 0] = 500.0                          # amax 500: s = 0, 500 saturates to 448
    rows[3, :] = 0.0                            # zero block: s = -127, codes 0
    rows[4, 0], rows[4, 1] = 0.75, -0.001       # amax 0.75: s = -9; -0.001 * 512 = -0.512
    rows[5, 0] = 1e-40                          # subnormal amax: s clamps to -127
    c, s = oracle.mx_quant_rows(rows)
    assert s[:, 0].tolist() == [127, 119, 127, 0, 118, 0]
    assert c[0, 0] == 0x7E and c[0, 1] == 0x38
    assert c[1, 0] == 0x78                      # 256 = 2^8
    assert c[2, 0] == 0x7E                      # saturated to 448
    assert not c[3].any()
    assert c[4, 0] == torch.tensor(0.75 * 512).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert c[4, 1] == torch.tensor(-0.512).to(torch.float8_e4m3fn).view(torch.uint8).item()


@pytest.mark.parametrize("scale", [1e-6, 1e-2, 1.0, 300.0, 1e6])
def test_against_torch_rule(scale):
    g = torch.Generator().manual_seed(int(scale * 7) % 1000 + 1)
    v = torch.randn(64, 256, generator=g) * scale
    v[3, :32] = 0.0                             # one zero block
    v[5, 40] = 512.0 * scale                    # an outlier
    c, s = oracle.mx_quant_rows(v.numpy())
    tc, ts = torch_mx(v)
    assert (s == ts).all()
    assert (c == tc).all()


def test_dequantisation_bound():
    g = torch.Generator().manual_seed(2)
    v = torch.randn(32, 512, generator=g).numpy().astype(np.float32)
    c, s = oracle.mx_quant_rows(v)
    d = oracle.mx_values(c, s)
    X = np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=-1) - 127)
    # not saturated: RNE error within half a step of E4M3 (3 mantissa bits)
    # at the value's binade, never below the subnormal step 2^-9 X
    step = np.maximum(np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(v) / X, 1e-30))).astype(int) - 3),
                      2.0 ** -9) * X
    sat = np.abs(v) / X > 448
    assert (np.abs(d - v)[~sat] <= 0.5 * step[~sat] + 1e-30).all()
    assert (np.abs(d[sat]) == 448 * X[sat]).all()


def test_bf16_rows_match_float_rows():
    x = (torch.randn(5, 256, generator=torch.Generator().manual_seed(3)) * 3).bfloat16()
    c1, s1 = oracle.mx_quant_rows_bf16(x)
    c2, s2 = oracle.mx_quant_rows(x.float().numpy())
    assert (c1 == c2).all() and (s1 == s2).all()


def dense_reference(x, ids, w, W):
    """Dense fp64 MX layer built on the torch quantiser: every expert on every
    token, combined by the scattered routing weights."""
    T, H = x.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    xc, xs = torch_mx(x.float())
    xv = oracle.mx_values(xc, xs)
    W1 = oracle.mx_values(W["w1"].numpy().reshape(-1, H), W["w1_scale"].numpy().reshape(-1, H // 32)).reshape(E, I2, H)
    W2 = oracle.mx_values(W["w2"].numpy().reshape(-1, I), W["w2_scale"].numpy().reshape(-1, I // 32)).reshape(E, H, I)
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            gu = W1[e] @ xv[t]
            g, u = gu[:I], gu[I:]
            h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
            hc, hs = torch_mx(h[None, :])
            out[t] += float(w[t, j]) * (W2[e] @ oracle.mx_values(hc, hs)[0])
    return out


@pytest.mark.parametrize("k", [1, 3])
def test_forward_against_dense_reference(k):
    wl = custom_workload(6, 128, 96, k, dtype="mxfp8", seed=4)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 7, seed=11)
    ids[2, 0] = -1                                 # a dropped pair
    xb = x.bfloat16()
    got = oracle.forward_mxfp8(xb, w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    ref = dense_reference(xb, ids.numpy(), w.numpy(), W)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_forward_quant_outputs():
    wl = custom_workload(4, 64, 64, 2, dtype="mxfp8", seed=5)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 3, seed=12)
    out, xq, sx, hq, sh = oracle.forward_mxfp8(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"],
                                               W["w2_scale"], want_quant=True)
    c, s = oracle.mx_quant_rows_bf16(x.bfloat16())
    assert (xq == c).all() and (sx == s).all()
    assert hq.shape == (3, 2, 64) and sh.shape == (3, 2, 2)


def test_generator_weights_follow_the_rule():
    v = torch.randn(3, 16, 64, generator=torch.Generator().manual_seed(6)) * 0.05
    q, s = quantize_weight_mx(v)
    c, so = oracle.mx_quant_rows(v.reshape(-1, 64).numpy())
    assert (q.reshape(-1, 64).numpy() == c).all() and (s.reshape(-1, 2).numpy() == so).all()
