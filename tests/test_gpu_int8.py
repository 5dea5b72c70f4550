"""GPU parity of the int8 w8a8 path with per-channel weight scales (SGLang
tuning guide: int8_w8a8 with per-channel quantisation, as for channel-INT8
DeepSeek checkpoints).

* x's per-token int8 quantisation is decided on exact inputs on both sides:
  codes and scales bit-exact.
* The integer products are exact on both sides (int32 on the GPU, int64 in
  the oracle); the layer output against the oracle within the fp8 bound
  max|err| <= 4e-2 max|ref|, over shapes spanning several tiles and ragged
  tails, dropped pairs, one token, the tuning guide's TP=16 slice of the
  DeepSeek-V3 shape (I = 2048/16), and in a replayed HIP graph.
* The requantised intermediate (fp32 on the GPU, fp64 in the oracle
  before its rounding): at least 99% of codes equal, none more than one
  apart, scales within 1e-6.
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
    packed = lib.pack_weights({k: v.cuda() for k, v in W.items()}, "int8")
    out, routing, ws = lib.moe_layer(x.cuda().bfloat16().contiguous(), ids.cuda().contiguous(),
                                     w.cuda().float().contiguous(), packed, dtype="int8")
    torch.cuda.synchronize()
    return out, routing, ws


def ref_out(x, ids, w, W, want_quant=False):
    return oracle.forward_int8(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"],
                               want_quant=want_quant)


SHAPES = [
    # E, H, I, k, T, p_drop
    (8, 256, 256, 2, 5, 0.0),
    (16, 512, 192, 4, 33, 0.1),
    (64, 1024, 640, 8, 100, 0.05),
    (32, 256, 128, 8, 1, 0.0),
    (1, 256, 256, 1, 70, 0.0),
    (256, 7168, 128, 8, 16, 0.0),       # DeepSeek-V3 shape, TP=16 slice
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop", SHAPES)
def test_int8_layer_parity(lib, E, H, I, k, T, p_drop):
    log(f"int8 layer E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    wl = custom_workload(E, H, I, k, dtype="int8", seed=E + T)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 1)
    ids = random_ids(T, k, E, seed=T + 2, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 3)
    out, _, _ = run(lib, x, ids, w, W)
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "int8", f"int8 E={E} T={T}")


# Strips (from 24 mean rows per expert): 64-, 128- and 192-row tiles, the
# down reduction unsplit or split into fp32 partial sums (2 and 8 slices).
STRIP_SHAPES = [
    # E, H, I, k, T, p_drop, block_m, split_k2
    (128, 512, 512, 8, 400, 0.02, 64, 1),
    (16, 256, 256, 8, 100, 0.0, 128, 1),
    (64, 512, 512, 8, 1200, 0.0, 192, 2),
    (32, 256, 2048, 4, 200, 0.05, 64, 8),
    (64, 512, 1024, 8, 960, 0.0, 160, 2),     # 120 rows per expert: 160-row tiles
    (64, 1024, 1024, 8, 960, 0.02, 160, 1),
    (16, 2048, 2048, 2, 1000, 0.0, 160, 2),   # 16 gate-up strips with rotated K loops
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop,bm,s2", STRIP_SHAPES)
def test_int8_strip_shapes(lib, E, H, I, k, T, p_drop, bm, s2):
    log(f"int8 strips E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    L = lib.moe_workspace_layout(T, k, E, H, I, "int8")
    assert L["tiling"] == 2 and L["split_k1"] == 1 and L["split_k2"] == s2
    assert lib.moe_routing_layout(T, k, E, H, I, "int8")["block_m"] == bm
    wl = custom_workload(E, H, I, k, dtype="int8", seed=E + T + 5)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 6)
    ids = random_ids(T, k, E, seed=T + 7, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 8)
    out, routing, ws = run(lib, x, ids, w, W)
    ref, _, _, hq_ref, sh_ref = ref_out(x, ids, w, W, want_quant=True)
    # the requantised intermediate, at the rows of the valid pairs
    R = lib.read_routing(routing, T, k, E, H, I, "int8")
    pos = R["pos"].numpy().reshape(T, k)
    valid = (ids.numpy() >= 0) & (ids.numpy() < E)
    b = ws.cpu()
    P = T * k
    hq = b[L["h"]:L["h"] + P * I].view(torch.int8).numpy().reshape(P, I)[pos[valid]]
    sh = b[L["h_scale"]:L["h_scale"] + 4 * P].view(torch.float32).numpy()[pos[valid]]
    hr = hq_ref.reshape(T, k, I)[valid]
    sr = sh_ref.reshape(T, k)[valid]
    same = (hq == hr).mean()
    log(f"  h codes equal {same:.4f}, max scale rel diff {np.abs(sh / sr - 1).max():.2e}")
    assert same >= 0.99
    assert np.abs(hq.astype(int) - hr.astype(int)).max() <= 1
    assert np.abs(sh / sr - 1).max() <= 1e-6
    check_tol(out.float().cpu().numpy(), ref, "int8", f"int8 strips E={E} T={T}")


def test_int8_quant_and_requant(lib):
    E, H, I, k, T = 16, 512, 256, 4, 24
    wl = custom_workload(E, H, I, k, dtype="int8", seed=9)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=10)
    x[3] = 0.0                                         # an all-zero row
    x[5, 0] = 3000.0                                   # an outlier
    ids = random_ids(T, k, E, seed=11)
    w = random_weights_w(T, k, seed=12)
    out, routing, ws = run(lib, x, ids, w, W)
    L = lib.moe_workspace_layout(T, k, E, H, I, "int8")
    b = ws.cpu()
    xq = b[L["xq"]:L["xq"] + T * H].view(torch.int8).numpy().reshape(T, H)
    sx = b[L["x_scale"]:L["x_scale"] + 4 * T].view(torch.float32).numpy()
    rq, rs = oracle.int8_quant_rows_bf16(x.bfloat16())
    assert (xq == rq).all() and (sx == rs).all(), "x quantisation differs"
    _, _, _, hq_ref, sh_ref = ref_out(x, ids, w, W, want_quant=True)
    R = lib.read_routing(routing, T, k, E, H, I, "int8")
    pos = R["pos"].numpy()
    P = T * k
    hq = b[L["h"]:L["h"] + P * I].view(torch.int8).numpy().reshape(P, I)[pos].reshape(T, k, I)
    sh = b[L["h_scale"]:L["h_scale"] + 4 * P].view(torch.float32).numpy()[pos].reshape(T, k)
    same = (hq == hq_ref).mean()
    log(f"  h codes equal {same:.4f}, max scale rel diff {np.abs(sh / sh_ref - 1).max():.2e}")
    assert same >= 0.99
    assert np.abs(hq.astype(int) - hq_ref.astype(int)).max() <= 1
    assert np.abs(sh / sh_ref - 1).max() <= 1e-6
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "int8", "int8 quant case")


def test_int8_dsv3_shape_decode(lib):
    wl = WORKLOADS["dsv3i8"]
    W = make_weights(wl, device="cuda")
    packed = lib.pack_weights(W, "int8")
    Wc = {kk: v.cpu() for kk, v in W.items()}
    del W
    for T in (1, 16):
        x, ids, w = make_tokens(wl, T)
        out, _, _ = lib.moe_layer(x.cuda(), ids.cuda(), w.cuda(), packed, dtype="int8")
        torch.cuda.synchronize()
        ref = oracle.forward_int8(x, w, ids, Wc["w1"], Wc["w1_scale"], Wc["w2"], Wc["w2_scale"])
        check_tol(out.float().cpu().numpy(), ref, "int8", f"dsv3i8 T={T}")


def test_int8_graph_replay(lib):
    E, H, I, k, T = 32, 512, 256, 4, 64
    wl = custom_workload(E, H, I, k, dtype="int8", seed=13)
    W = make_weights(wl)
    packed = lib.pack_weights({kk: v.cuda() for kk, v in W.items()}, "int8")
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    routing = lib.alloc_routing(T, k, E, H, I, "int8")
    ws = lib.alloc_workspace(T, k, E, H, I, "int8")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step():
        lib.moe_build_routing_int8(ids, E, H, I, routing)
        lib.moe_forward_int8(x, w, routing, packed["w1"], packed["w1_scale"], packed["w2"],
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
        check_tol(got, ref_out(xh, idh, wh, W), "int8", f"int8 graph replay {rep}")
