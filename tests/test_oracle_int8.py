"""Pins of the oracle's int8 w8a8 path (SGLang tuning guide: int8_w8a8 with
per-channel quantisation).  The per-row rule (scale amax/127, codes
rounded half to even and clamped to +-127) is pinned to worked cases and to
an independent torch quantiser; the forward pass to a dense torch reference
whose integer dot products are exact int64 matmuls.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, quantize_weight_int8


def torch_int8(v):
    v = torch.as_tensor(v, dtype=torch.float32).reshape(-1)
    amax = float(v.abs().max())
    if amax == 0.0:
        return np.zeros(v.numel(), dtype=np.int8), 1.0
    inv = torch.tensor(127.0 / amax, dtype=torch.float64).float()
    q = torch.round(v * inv).clamp(-127, 127).to(torch.int8)
    return q.numpy(), float(np.float32(amax / 127.0))


def test_worked_cases():
    q, s = oracle.int8_quant_row(np.array([127, -127, 0.5, 1.5, 2.5, -0.5, 64, 3], dtype=np.float32))
    assert s == 1.0 and q.tolist() == [127, -127, 0, 2, 2, 0, 64, 3]
    q, s = oracle.int8_quant_row(np.zeros(8, dtype=np.float32))
    assert s == 1.0 and not q.any()
    q, s = oracle.int8_quant_row(np.array([2.0, -1.0, 0.5], dtype=np.float32))   # inv = 63.5
    assert s == np.float32(2.0 / 127.0) and q.tolist() == [127, -64, 32]       # -63.5 -> -64 (even)


@pytest.mark.parametrize("scale", [1e-5, 1.0, 3e4])
def test_against_torch_rule(scale):
    g = torch.Generator().manual_seed(int(scale) % 97 + 3)
    for r in range(20):
        v = torch.randn(257, generator=g) * scale
        q, s = oracle.int8_quant_row(v.numpy())
        tq, ts = torch_int8(v)
        assert (q == tq).all() and s == ts


def test_bf16_rows():
    x = torch.randn(4, 96, generator=torch.Generator().manual_seed(1)).bfloat16()
    q, s = oracle.int8_quant_rows_bf16(x)
    for t in range(4):
        tq, ts = torch_int8(x[t].float())
        assert (q[t] == tq).all() and s[t] == ts


def dense_reference(x, ids, w, W):
    T, H = x.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    W1 = W["w1"].to(torch.int64)
    W2 = W["w2"].to(torch.int64)
    s1 = W["w1_scale"].double()
    s2 = W["w2_scale"].double()
    out = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        xq, sx = torch_int8(x[t].float())
        xq = torch.from_numpy(xq).to(torch.int64)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            gu = sx * s1[e] * (W1[e] @ xq).double()
            h = (gu[:I] / (1 + torch.exp(-gu[:I])) * gu[I:]).float()
            hq, sh = torch_int8(h)
            y = sh * s2[e] * (W2[e] @ torch.from_numpy(hq).to(torch.int64)).double()
            out[t] += float(w[t, j]) * y
    return out.numpy()


@pytest.mark.parametrize("k", [1, 3])
def test_forward_against_dense_reference(k):
    wl = custom_workload(6, 128, 96, k, dtype="int8", seed=4)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 7, seed=11)
    ids[2, 0] = -1
    xb = x.bfloat16()
    got = oracle.forward_int8(xb, w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    ref = dense_reference(xb, ids, w, W)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_generator_weights_follow_the_rule():
    v = torch.randn(3, 8, 64, generator=torch.Generator().manual_seed(6)) * 0.05
    q, s = quantize_weight_int8(v)
    amax = v.abs().amax(-1)
    assert torch.allclose(s, amax / 127)
    assert q.abs().max() == 127
    deq = q.float() * s.unsqueeze(-1)
    assert (deq - v).abs().max() <= 0.5 * s.max() + 1e-7
