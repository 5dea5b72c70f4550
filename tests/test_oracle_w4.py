"""Pins of the oracle's int4 w4a16 path (SGLang tuning guide dtype list:
int4_w4a16): int4 weights with one fp32 scale per 128 K values of a row,
bf16 activations.  The nibble order and sign are pinned to torch bit
operations and hand-made bytes; the forward pass to a dense torch reference
on the dequantised weights.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, quantize_weight_int4


def torch_unpack(codes, scales):
    c = torch.as_tensor(codes).to(torch.int16)
    lo = c & 0xF
    hi = (c >> 4) & 0xF
    q = torch.stack([lo, hi], dim=-1).reshape(*c.shape[:-1], c.shape[-1] * 2)
    q = torch.where(q >= 8, q - 16, q).double()
    s = torch.as_tensor(scales).double().repeat_interleave(128, dim=-1)
    return (q * s).numpy()


def test_exact_bytes():
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 0] = 0x7F        # k=0 -> -1 (0xF), k=1 -> 7
    codes[0, 1] = 0x88        # k=2 -> -8, k=3 -> -8
    codes[0, 2] = 0x21        # k=4 -> 1, k=5 -> 2
    scales = np.array([[0.5]], dtype=np.float32)
    v = oracle.w4_dequant(codes, scales)
    assert v[0, :6].tolist() == [-0.5, 3.5, -4.0, -4.0, 0.5, 1.0]
    assert not v[0, 6:].any()


def test_against_torch_unpack():
    g = torch.Generator().manual_seed(2)
    codes = torch.randint(0, 256, (9, 192), generator=g, dtype=torch.uint8).numpy()
    scales = torch.rand(9, 3, generator=g).numpy().astype(np.float32)
    np.testing.assert_array_equal(oracle.w4_dequant(codes, scales), torch_unpack(codes, scales))


def test_generator_quantiser():
    w = torch.randn(4, 16, 256, generator=torch.Generator().manual_seed(3)) * 0.02
    w[0, 0, :128] = 0.0                                   # an all-zero group
    q, s = quantize_weight_int4(w)
    assert q.shape == (4, 16, 128) and s.shape == (4, 16, 2)
    assert s[0, 0, 0] == 1.0
    deq = oracle.w4_dequant(q.reshape(-1, 128).numpy(), s.reshape(-1, 2).numpy()).reshape(4, 16, 256)
    err = np.abs(deq - w.double().numpy())
    bound = s.double().numpy().repeat(128, axis=-1) / 2
    assert (err <= bound * (1 + 1e-6)).all()
    amax = w.abs().reshape(4, 16, 2, 128).amax(-1)
    assert torch.allclose(s[amax > 0], (amax / 7)[amax > 0])


def dense_reference(x, ids, w, W):
    T, H = x.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    W1 = torch_unpack(W["w1"].numpy(), W["w1_scale"].numpy())
    W2 = torch_unpack(W["w2"].numpy(), W["w2_scale"].numpy())
    xv = x.double().numpy()
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            gu = W1[e] @ xv[t]
            h = gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]
            out[t] += float(w[t, j]) * (W2[e] @ h)
    return out


@pytest.mark.parametrize("k", [1, 3])
def test_forward_against_dense_reference(k):
    wl = custom_workload(6, 256, 128, k, dtype="int4", seed=4)
    W = make_weights(wl)
    x, ids, w = make_tokens(wl, 5, seed=11)
    ids[1, 0] = -1
    xb = x.bfloat16()
    got = oracle.forward_w4a16(xb, w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])
    ref = dense_reference(xb, ids, w, W)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())
