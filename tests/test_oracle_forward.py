"""Pins of the oracle's forward pass.

The layer's result is the plain routed SwiGLU mixture (HPC-Ops x SGLang
blog, section "MoE"): out[t] = sum_j w[t][j] W2[e_j] (SiLU(gate) * up).  The
oracle is pinned against dense fp64 torch matmuls that evaluate every
expert on every token and combine them with a gate matrix scattered from
(ids, w), against the k=1 single-expert FFN, against the k=E mean of all
experts, and by structural invariants (token permutation, zero weights,
linearity in w, idle experts never read).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from moe_inputs import WORKLOADS, make_tokens, make_weights, random_ids, random_weights_w


def dense_ref(x, w, ids, W1, W2):
    """Every expert on every token in fp64, combined through a dense gate matrix."""
    x = torch.as_tensor(x).double()
    W1 = torch.as_tensor(W1).double()
    W2 = torch.as_tensor(W2).double()
    ids = torch.as_tensor(ids).long()
    w = torch.as_tensor(w).double()
    T, H = x.shape
    E, I2, _ = W1.shape
    I = I2 // 2
    gate = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if 0 <= e < E:
                gate[t, e] += w[t, j]
    out = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        g = x @ W1[e, :I].T
        u = x @ W1[e, I:].T
        y = (F.silu(g) * u) @ W2[e].T
        out += gate[:, e:e + 1] * y
    return out.numpy()


def tiny_case(T=4, seed=None):
    wl = WORKLOADS["tiny"]
    x, ids, w = make_tokens(wl, T, seed=seed)
    W = make_weights(wl)
    return x, ids, w, W["w1"], W["w2"]


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_tiny_workload_matches_dense_reference():
    x, ids, w, W1, W2 = tiny_case()
    got = oracle.forward_f32(x, w, ids, W1, W2)
    ref = dense_ref(x, w, ids, W1, W2)
    assert rel_err(got, ref) < 1e-12


def test_tiny_many_tokens_with_drops_and_duplicates():
    wl = WORKLOADS["tiny"]
    W = make_weights(wl)
    T = 40
    x, _, _ = make_tokens(wl, T, seed=77)
    ids = random_ids(T, 3, wl.E, seed=5, p_drop=0.2)
    ids[3] = torch.tensor([2, 2, 5], dtype=torch.int32)       # duplicate expert
    w = random_weights_w(T, 3, seed=6)
    got = oracle.forward_f32(x, w, ids, W["w1"], W["w2"])
    ref = dense_ref(x, w, ids, W["w1"], W["w2"])
    assert rel_err(got, ref) < 1e-12


def test_k1_weight1_is_single_expert_ffn():
    x, _, _, W1, W2 = tiny_case(T=9, seed=3)
    E = W1.shape[0]
    I = W1.shape[1] // 2
    ids = torch.tensor([[t % E] for t in range(9)], dtype=torch.int32)
    w = torch.ones(9, 1)
    got = oracle.forward_f32(x, w, ids, W1, W2)
    xd = x.double()
    for t in range(9):
        e = t % E
        g = W1[e, :I].double() @ xd[t]
        u = W1[e, I:].double() @ xd[t]
        y = W2[e].double() @ (F.silu(g) * u)
        assert np.max(np.abs(got[t] - y.numpy())) <= 1e-12 * np.max(np.abs(y.numpy()))


def test_k_equals_E_uniform_weight_is_expert_mean():
    x, _, _, W1, W2 = tiny_case(T=5, seed=4)
    E = W1.shape[0]
    I = W1.shape[1] // 2
    ids = torch.stack([torch.randperm(E, generator=torch.Generator().manual_seed(t)) for t in range(5)]).int()
    w = torch.full((5, E), 1.0 / E)
    got = oracle.forward_f32(x, w, ids, W1, W2)
    xd, W1d, W2d = x.double(), W1.double(), W2.double()
    g = torch.einsum("eih,th->tei", W1d[:, :I], xd)
    u = torch.einsum("eih,th->tei", W1d[:, I:], xd)
    y = torch.einsum("ehi,tei->teh", W2d, F.silu(g) * u)
    ref = (y * torch.tensor(1.0 / E, dtype=torch.float64)).sum(dim=1).numpy()
    assert rel_err(got, ref) < 1e-12


def test_gate_up_halves_are_not_interchangeable():
    # a mistaken gate/up order would be invisible if both halves were equal;
    # make them differ strongly and compare with the dense reference.
    x, ids, w, W1, W2 = tiny_case(T=6, seed=8)
    I = W1.shape[1] // 2
    W1 = W1.clone()
    W1[:, I:] *= 3.0
    W1[:, :I] += 0.5
    got = oracle.forward_f32(x, w, ids, W1, W2)
    ref = dense_ref(x, w, ids, W1, W2)
    swapped = torch.cat([W1[:, I:], W1[:, :I]], dim=1)
    ref_swapped = dense_ref(x, w, ids, swapped, W2)
    assert rel_err(got, ref) < 1e-12
    assert rel_err(got, ref_swapped) > 1e-2


def test_token_permutation_permutes_output_exactly():
    x, ids, w, W1, W2 = tiny_case(T=4)
    x2, ids2, w2 = make_tokens(WORKLOADS["tiny"], 12, seed=9)
    perm = torch.randperm(12, generator=torch.Generator().manual_seed(2))
    a = oracle.forward_f32(x2, w2, ids2, W1, W2)
    b = oracle.forward_f32(x2[perm], w2[perm], ids2[perm], W1, W2)
    assert np.array_equal(a[perm.numpy()], b)


def test_zero_weight_equals_dropped_pair():
    x, ids, w, W1, W2 = tiny_case(T=4)
    w0 = w.clone()
    w0[1, 0] = 0.0
    ids_d = ids.clone()
    ids_d[1, 0] = -1
    a = oracle.forward_f32(x, w0, ids, W1, W2)
    b = oracle.forward_f32(x, w0, ids_d, W1, W2)
    assert np.array_equal(a, b)


def test_linear_in_routing_weights():
    x, ids, w, W1, W2 = tiny_case(T=4)
    a = oracle.forward_f32(x, w, ids, W1, W2)
    b = oracle.forward_f32(x, w * 2, ids, W1, W2)      # scaling by 2 is exact
    assert np.array_equal(2 * a, b)
    c = oracle.forward_f32(x, w * 3, ids, W1, W2)       # 3*w rounds once in fp32
    assert rel_err(c, 3 * a) < 2 ** -22


def test_split_pair_into_two_halves():
    x, ids, w, W1, W2 = tiny_case(T=4)
    ids3 = torch.cat([ids, ids[:, :1]], dim=1)
    w3 = torch.cat([w, w[:, :1] / 2], dim=1)
    w3[:, 0] = w[:, 0] / 2
    a = oracle.forward_f32(x, w, ids, W1, W2)
    b = oracle.forward_f32(x, w3, ids3, W1, W2)
    assert rel_err(b, a) < 1e-14


def test_idle_experts_are_never_read():
    x, ids, w, W1, W2 = tiny_case(T=4)
    used = set(ids.reshape(-1).tolist())
    W1n, W2n = W1.clone(), W2.clone()
    for e in range(W1.shape[0]):
        if e not in used:
            W1n[e] = float("nan")
            W2n[e] = float("nan")
    a = oracle.forward_f32(x, w, ids, W1, W2)
    b = oracle.forward_f32(x, w, ids, W1n, W2n)
    assert np.all(np.isfinite(b)) and np.array_equal(a, b)


def test_bf16_entry_equals_f64_on_torch_decoded_values():
    wl = WORKLOADS["tiny"]
    x, ids, w = make_tokens(wl, 6, seed=10)
    W = make_weights(wl)
    xb, W1b, W2b = x.bfloat16(), W["w1"].bfloat16(), W["w2"].bfloat16()
    a = oracle.forward_bf16(xb, w, ids, W1b, W2b)
    b = oracle.forward_f64(xb.double(), w, ids, W1b.double(), W2b.double())
    assert np.array_equal(a, b)
    assert rel_err(a, dense_ref(xb, w, ids, W1b, W2b)) < 1e-12


def test_row_subset_matches_full():
    x, ids, w, W1, W2 = tiny_case(T=4)
    full = oracle.forward_f32(x, w, ids, W1, W2)
    sub = oracle.forward_f32(x, w, ids, W1, W2, rows=[3, 0])
    assert np.array_equal(sub, full[[3, 0]])


def test_all_pairs_dropped_gives_zero():
    x, ids, w, W1, W2 = tiny_case(T=4)
    ids = torch.full_like(ids, -1)
    out = oracle.forward_f32(x, w, ids, W1, W2)
    assert not out.any()
