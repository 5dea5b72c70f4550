"""Pins of the oracle's block-scaled fp8 path (SGLang tuning guide:
block_shape [128, 128], DeepSeek-V3's quantisation): weights with one fp32
scale per 128 x 128 block, activations with one per 128-value group of a
row.  The group quantiser is pinned to the per-row rule (itself pinned to
torch's e4m3 cast) on each group; the forward pass to a dense torch
reference on dequantised weights and activations.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, quantize_weight_block_fp8


def test_groups_are_rows():
    g = torch.Generator().manual_seed(1)
    v = torch.randn(512, generator=g) * torch.tensor([1.0, 30.0, 0.01, 0.0]).repeat_interleave(128)
    codes, sc = oracle.quant_groups(v.numpy())
    for j in range(4):
        c, s = oracle.quant_row(v[128 * j:128 * (j + 1)].numpy())
        assert (codes[128 * j:128 * (j + 1)] == c).all() and sc[j] == s
    assert sc[3] == 1.0 and not codes[384:].any()


def test_generator_block_scales():
    w = torch.randn(2, 256, 384, generator=torch.Generator().manual_seed(2)) * 0.03
    q, s = quantize_weight_block_fp8(w)
    assert q.shape == (2, 256, 384) and s.shape == (2, 2, 3)
    amax = w.reshape(2, 2, 128, 3, 128).abs().amax(dim=(2, 4))
    assert torch.equal(s, (amax / 448.0).float())
    deq = q.view(torch.float8_e4m3fn).float() * s.repeat_interleave(128, 1).repeat_interleave(128, 2)
    assert ((deq - w).abs() <= 2.0 ** -4 * w.abs() + s.max() * 2.0 ** -9).all()


def e4m3(codes):
    return torch.as_tensor(codes).view(torch.float8_e4m3fn).double()


def dense_reference(x, ids, w, W):
    T, H = x.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    W1 = e4m3(W["w1"]) * W["w1_scale"].double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    W2 = e4m3(W["w2"]) * W["w2_scale"].double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    out = np.zeros((T, H))
    for t in range(T):
        xc, xs = oracle.quant_groups(x[t].float().numpy())
        xv = e4m3(xc) * torch.from_numpy(xs).double().repeat_interleave(128)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            gu = W1[e] @ xv
            h = (gu[:I] / (1 + torch.exp(-gu[:I])) * gu[I:]).float()
            hc, hs = oracle.quant_groups(h.numpy())
            hv = e4m3(hc) * torch.from_numpy(hs).double().repeat_interleave(128)
            out[t] += float(w[t, j]) * (W2[e] @ hv).numpy()
    return out


@pytest.mark.parametrize("k", [1, 3])
def test_forward_against_dense_reference(k):
    wl = custom_workload(6, 256, 128, k, dtype="fp8b", seed=4)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 5, seed=11)
    ids[1, 0] = -1
    xb = x.bfloat16()
    got = oracle.forward_fp8_block(xb, w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    ref = dense_reference(xb, ids, w, W)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())
