"""GPU parity of the int8 w8a16 path (SGLang tuning guide dtype list:
int8_w8a16): int8 weights with one fp32 scale per weight row, converted to
bf16 in registers, bf16 activations, fp32 accumulation.  The layer output
against the oracle's fp64 layer on the dequantised weights, within the bf16
bound max|err| <= 1e-2 max|ref| + 1e-3 (h and the down rows are stored as
bf16, as on the bf16 path), over shapes spanning several tiles and ragged
tails (16-, 32- and 64-row tiles, odd step counts per wave), dropped pairs,
one token, every code value, the Mixtral-8x7B shape at decode sizes, and a
replayed HIP graph.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, custom_workload, make_tokens, make_weights, random_ids, random_weights_w
from moe_testlib import check_tol, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def run(lib, x, ids, w, W):
    packed = lib.pack_weights({k: v.cuda() for k, v in W.items()}, "int8w")
    out, routing, ws = lib.moe_layer(x.cuda().bfloat16().contiguous(), ids.cuda().contiguous(),
                                     w.cuda().float().contiguous(), packed, dtype="int8w")
    torch.cuda.synchronize()
    return out


def ref_out(x, ids, w, W):
    return oracle.forward_w8a16(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"])


SHAPES = [
    # E, H, I, k, T, p_drop
    (8, 256, 256, 2, 5, 0.0),
    (16, 512, 384, 4, 33, 0.1),
    (64, 1024, 640, 8, 100, 0.05),
    (32, 256, 128, 8, 1, 0.0),
    (1, 256, 256, 1, 70, 0.0),          # one expert: 64-row tiles
    (4, 384, 256, 2, 40, 0.0),          # 32-row tiles (20 rows per expert)
    (8, 320, 192, 2, 12, 0.0),          # 5 and 3 K steps: one step per wave
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop", SHAPES)
def test_int8w_layer_parity(lib, E, H, I, k, T, p_drop):
    log(f"int8w layer E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    wl = custom_workload(E, H, I, k, dtype="int8w", seed=E + T)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 1)
    ids = random_ids(T, k, E, seed=T + 2, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 3)
    out = run(lib, x, ids, w, W)
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "bf16", f"int8w E={E} T={T}")


def test_int8w_every_code(lib):
    # weights cycling through all 256 codes (including -128, which the quantiser never makes)
    E, H, I, k, T = 4, 256, 128, 2, 9
    wl = custom_workload(E, H, I, k, dtype="int8w", seed=3)
    W = make_weights(wl)
    g = torch.Generator().manual_seed(4)
    for key in ("w1", "w2"):
        W[key] = torch.randint(-128, 128, W[key].shape, generator=g, dtype=torch.int8)
    W["w1"][0, 0, :256] = torch.arange(-128, 128, dtype=torch.int8)
    for key in ("w1_scale", "w2_scale"):
        W[key] = (torch.rand(W[key].shape, generator=g) * 0.0005 + 0.0001).float()
    x, _, _ = make_tokens(wl, T, seed=5)
    ids = random_ids(T, k, E, seed=6)
    ids[0, 0] = 0
    w = random_weights_w(T, k, seed=7)
    out = run(lib, x, ids, w, W)
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "bf16", "int8w every code")


def test_int8w_mixtral_shape_decode(lib):
    wl = WORKLOADS["mixtral8"]
    W = make_weights(wl, device="cuda")
    packed = lib.pack_weights(W, "int8w")
    Wc = {kk: v.cpu() for kk, v in W.items()}
    del W
    for T in (1, 16):
        x, ids, w = make_tokens(wl, T)
        out, _, _ = lib.moe_layer(x.cuda(), ids.cuda(), w.cuda(), packed, dtype="int8w")
        torch.cuda.synchronize()
        ref = oracle.forward_w8a16(x, w, ids, Wc["w1"], Wc["w1_scale"], Wc["w2"], Wc["w2_scale"])
        check_tol(out.float().cpu().numpy(), ref, "bf16", f"mixtral8 T={T}")


def test_int8w_graph_replay(lib):
    E, H, I, k, T = 32, 512, 256, 4, 64
    wl = custom_workload(E, H, I, k, dtype="int8w", seed=13)
    W = make_weights(wl)
    packed = lib.pack_weights({kk: v.cuda() for kk, v in W.items()}, "int8w")
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    routing = lib.alloc_routing(T, k, E, H, I, "int8w")
    ws = lib.alloc_workspace(T, k, E, H, I, "int8w")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step():
        lib.moe_build_routing_int8_w8a16(ids, E, H, I, routing)
        lib.moe_forward_int8_w8a16(x, w, routing, packed["w1"], packed["w1_scale"], packed["w2"],
                                   packed["w2_scale"], ws, out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        xh, _, _ = make_tokens(wl, T, seed=20 + rep)
        idh = random_ids(T, k, E, seed=30 + rep, p_drop=0.05)
        wh = random_weights_w(T, k, seed=40 + rep)
        x.copy_(xh.bfloat16().cuda())
        ids.copy_(idh.cuda())
        w.copy_(wh.cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        step()
        torch.cuda.synchronize()
        assert torch.equal(out.float().cpu(), torch.from_numpy(got)), "graph replay != eager"
        check_tol(got, ref_out(xh, idh, wh, W), "bf16", f"int8w graph replay {rep}")
