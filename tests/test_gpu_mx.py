"""GPU parity of the MXFP8 path (OCP microscaling, 32-value blocks; SGLang
tuning guide: gfx95 devices keep MXFP8's [1, 32] block shape).

* x's MX quantisation (e4m3 codes and e8m0 scale codes) is decided on exact
  inputs on both sides: bit-exact.
* The layer output against the oracle's fp64 MX layer, within the fp8 bound
  max|err| <= 4e-2 max|ref|, over shapes that span several tiles and ragged
  tails, dropped pairs, one token, one expert per token, a hot expert, and
  in a replayed HIP graph.
* The requantised intermediate: its scale codes and e4m3 codes against the
  oracle's (computed from fp64 rather than fp32 sums, so a code may sit one
  step away at a rounding boundary: at least 99% equal, none more than one
  step apart).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import custom_workload, make_tokens, make_weights, random_ids, random_weights_w
from moe_testlib import check_tol, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def run(lib, x, ids, w, W):
    packed = lib.pack_weights({k: v.cuda() for k, v in W.items()}, "mxfp8")
    out, routing, ws = lib.moe_layer(x.cuda().bfloat16().contiguous(), ids.cuda().contiguous(),
                                     w.cuda().float().contiguous(), packed, dtype="mxfp8")
    torch.cuda.synchronize()
    return out, routing, ws


def ref_out(x, ids, w, W, want_quant=False):
    return oracle.forward_mxfp8(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"],
                                want_quant=want_quant)


SHAPES = [
    # E, H, I, k, T, p_drop
    (8, 256, 256, 2, 5, 0.0),
    (16, 512, 384, 4, 33, 0.1),
    (64, 1024, 640, 8, 100, 0.05),
    (32, 256, 128, 8, 1, 0.0),
    (4, 128, 128, 1, 3, 0.0),
    (1, 256, 256, 1, 70, 0.0),          # one expert: several 64-row tiles
    (256, 384, 256, 8, 40, 0.02),
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop", SHAPES)
def test_mx_layer_parity(lib, E, H, I, k, T, p_drop):
    log(f"mx layer E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    wl = custom_workload(E, H, I, k, dtype="mxfp8", seed=E + T)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 1)
    ids = random_ids(T, k, E, seed=T + 2, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 3)
    out, _, ws = run(lib, x, ids, w, W)
    ref = ref_out(x, ids, w, W)
    check_tol(out.float().cpu().numpy(), ref, "mxfp8", f"mx E={E} T={T}")


def test_mx_quant_and_requant(lib):
    E, H, I, k, T = 16, 512, 256, 4, 24
    wl = custom_workload(E, H, I, k, dtype="mxfp8", seed=9)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=10)
    x[3, 64:96] = 0.0                                  # an all-zero block
    x[5, 0] = 3000.0                                   # an outlier
    ids = random_ids(T, k, E, seed=11)
    w = random_weights_w(T, k, seed=12)
    out, routing, ws = run(lib, x, ids, w, W)
    L = lib.moe_workspace_layout(T, k, E, H, I, "mxfp8")
    b = ws.cpu().numpy()
    xq = b[L["xq"]:L["xq"] + T * H].reshape(T, H)
    sx = b[L["x_scale"]:L["x_scale"] + T * H // 32].reshape(T, H // 32)
    rc, rs = oracle.mx_quant_rows_bf16(x.bfloat16())
    assert (xq == rc).all() and (sx == rs).all(), "x quantisation differs"
    # intermediate rows, sorted order: row pos[t*k+j] holds pair (t, j)
    _, _, _, hq_ref, sh_ref = ref_out(x, ids, w, W, want_quant=True)
    R = lib.read_routing(routing, T, k, E, H, I, "mxfp8")
    pos = R["pos"].numpy()
    P = T * k
    hq = b[L["h"]:L["h"] + P * I].reshape(P, I)[pos].reshape(T, k, I)
    sh = b[L["h_scale"]:L["h_scale"] + P * I // 32].reshape(P, I // 32)[pos].reshape(T, k, I // 32)
    same_s = (sh == sh_ref).mean()
    vals = oracle.mx_values(hq.reshape(-1, I), sh.reshape(-1, I // 32))
    vals_ref = oracle.mx_values(hq_ref.reshape(-1, I), sh_ref.reshape(-1, I // 32))
    same_c = (hq == hq_ref).mean()
    log(f"  h scale codes equal {same_s:.4f}, e4m3 codes equal {same_c:.4f}")
    assert same_s >= 0.99 and same_c >= 0.99
    # where both scales agree, codes are at most one e4m3 step apart
    ok = np.repeat((sh == sh_ref).reshape(-1, I // 32), 32, axis=1)
    d = np.abs(vals - vals_ref)[ok]
    step = np.maximum(np.abs(vals_ref)[ok] / 8, np.ldexp(1.0, np.repeat(sh_ref.reshape(-1, I // 32).astype(int), 32, axis=1)[ok] - 127 - 9))
    assert (d <= step * 1.0001).all()
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "mxfp8", "mx quant case")


def test_mx_dsv3_shape_decode(lib):
    # DeepSeek-V3-shaped MXFP8 layer at T=1 and T=16, every output row
    from moe_inputs import WORKLOADS
    wl = WORKLOADS["dsv3mx"]
    W = make_weights(wl, device="cuda")
    packed = lib.pack_weights(W, "mxfp8")
    Wc = {kk: v.cpu() for kk, v in W.items()}
    del W
    for T in (1, 16):
        x, ids, w = make_tokens(wl, T)
        out, _, _ = lib.moe_layer(x.cuda(), ids.cuda(), w.cuda(), packed, dtype="mxfp8")
        torch.cuda.synchronize()
        ref = oracle.forward_mxfp8(x, w, ids, Wc["w1"], Wc["w1_scale"], Wc["w2"], Wc["w2_scale"])
        check_tol(out.float().cpu().numpy(), ref, "mxfp8", f"dsv3mx T={T}")


def test_mx_graph_replay(lib):
    E, H, I, k, T = 32, 512, 256, 4, 64
    wl = custom_workload(E, H, I, k, dtype="mxfp8", seed=13)
    W = make_weights(wl)
    packed = lib.pack_weights({kk: v.cuda() for kk, v in W.items()}, "mxfp8")
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    routing = lib.alloc_routing(T, k, E, H, I, "mxfp8")
    ws = lib.alloc_workspace(T, k, E, H, I, "mxfp8")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step():
        lib.moe_build_routing_mxfp8(ids, E, H, I, routing)
        lib.moe_forward_mxfp8(x, w, routing, packed["w1"], packed["w1_scale"], packed["w2"],
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
        check_tol(got, ref_out(xh, idh, wh, W), "mxfp8", f"mx graph replay {rep}")
