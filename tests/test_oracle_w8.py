"""Pins of the oracle's int8 w8a16 path (SGLang tuning guide dtype list:
int8_w8a16): int8 weight codes with one fp32 scale per weight row, bf16
activations.  Where every dequantised weight is a bf16 value (power-of-two
scales) the layer is exactly the pinned bf16 layer on those weights; in
general it equals a dense torch reference on the dequantised weights.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, random_ids, random_weights_w


def test_reduces_to_bf16_layer():
    # |q| <= 128 has at most 8 significant bits and the scales are powers of
    # two, so q * s is a bf16 value: the w8a16 layer is the bf16 layer on it
    E, H, I, k, T = 4, 256, 128, 2, 6
    g = torch.Generator().manual_seed(5)
    W1 = torch.randint(-128, 128, (E, 2 * I, H), generator=g, dtype=torch.int8)
    W2 = torch.randint(-128, 128, (E, H, I), generator=g, dtype=torch.int8)
    W1[0, 0, :256] = torch.arange(-128, 128, dtype=torch.int8)   # every code once
    s1 = torch.pow(2.0, torch.randint(-12, -6, (E, 2 * I), generator=g).float())
    s2 = torch.pow(2.0, torch.randint(-12, -6, (E, H), generator=g).float())
    x = torch.randn(T, H, generator=g).bfloat16()
    ids = random_ids(T, k, E, seed=6, p_drop=0.1)
    w = random_weights_w(T, k, seed=7)
    d1 = (W1.float() * s1[..., None]).bfloat16()
    d2 = (W2.float() * s2[..., None]).bfloat16()
    assert torch.equal(d1.float(), W1.float() * s1[..., None])           # exact in bf16
    got = oracle.forward_w8a16(x, w, ids, W1, s1, W2, s2)
    ref = oracle.forward_bf16(x, w, ids, d1, d2)
    np.testing.assert_array_equal(got, ref)


def dense_reference(x, ids, w, W):
    T, H = x.shape
    W1 = W["w1"].double() * W["w1_scale"].double()[..., None]
    W2 = W["w2"].double() * W["w2_scale"].double()[..., None]
    E, I2, _ = W1.shape
    I = I2 // 2
    xv = x.double()
    gate = torch.zeros(T, E, dtype=torch.float64)   # routing weights scattered to a dense gate matrix
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if 0 <= e < E:
                gate[t, e] += float(w[t, j])
    out = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        gu = xv @ W1[e].T
        h = gu[:, :I] / (1 + torch.exp(-gu[:, :I])) * gu[:, I:]
        out += gate[:, e:e + 1] * (h @ W2[e].T)
    return out.numpy()


@pytest.mark.parametrize("k", [1, 3])
def test_forward_against_dense_reference(k):
    wl = custom_workload(6, 192, 128, k, dtype="int8w", seed=4)
    W = make_weights(wl)
    assert W["w1"].dtype == torch.int8 and W["w1_scale"].shape == (6, 256)
    x, ids, w = make_tokens(wl, 5, seed=11)
    ids[1, 0] = -1
    xb = x.bfloat16()
    got = oracle.forward_w8a16(xb, w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    ref = dense_reference(xb, ids, w, W)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_scale_is_per_row():
    # doubling the scale of one up row doubles that h column only: the
    # output moves by exactly the W2 column times the added h
    wl = custom_workload(2, 128, 64, 1, dtype="int8w", seed=8)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, 1, seed=9)
    ids = torch.tensor([[1]], dtype=torch.int32)
    w = torch.tensor([[1.0]])
    base = oracle.forward_w8a16(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    s1 = W["w1_scale"].clone()
    s1[1, 64 + 5] *= 2                     # up row 5 of expert 1
    moved = oracle.forward_w8a16(x.bfloat16(), w, ids, W["w1"], s1, W["w2"], W["w2_scale"])
    xv = x.bfloat16().double()[0]
    W1 = W["w1"][1].double() * W["w1_scale"][1].double()[:, None]
    g, u = W1[5] @ xv, W1[64 + 5] @ xv
    h5 = g / (1 + torch.exp(-g)) * u
    col = W["w2"][1, :, 5].double() * W["w2_scale"][1].double()
    np.testing.assert_allclose(moved - base, (h5 * col).numpy()[None], rtol=1e-9, atol=1e-12)
