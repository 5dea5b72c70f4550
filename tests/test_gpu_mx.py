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


def dense_h_mx(xq, sx, ids, W):
    """fp64 intermediate silu(gate) * up of every pair from the quantised x
    and the MX weights, and a bound on the error of the GPU's fp32 value:
    the fp8 MFMA's unit sums are off by less than 7 * 2^-13 * sum of a^ b^
    (a^ = max(|a|, 2^-6) times the block scale; the truncation model measured
    on the device for the same datapath), carried through silu(g) * u
    (|silu'| < 1.1), plus 2^-20 |h| for the fp32 sums and SiLU."""
    T, H = xq.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    k = ids.shape[1]
    e4 = np.array([oracle.lib().oracle_e4m3_value(i) for i in range(256)])
    xs = np.ldexp(1.0, np.repeat(sx.astype(np.int64), 32, axis=-1) - 127)
    x = e4[xq] * xs
    xhat = np.maximum(np.abs(e4[xq]), 2.0 ** -6) * xs
    h = np.zeros((T, k, I))
    bound = np.zeros((T, k, I))
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            if e not in cache:
                c = W["w1"][e].numpy()
                ws_ = np.ldexp(1.0, np.repeat(W["w1_scale"][e].numpy().astype(np.int64), 32, axis=-1) - 127)
                cache[e] = (e4[c] * ws_, np.maximum(np.abs(e4[c]), 2.0 ** -6) * ws_)
            wd, wb = cache[e]
            gu = wd @ x[t]
            ab = wb @ xhat[t]
            g, u = gu[:I], gu[I:]
            sg = g / (1 + np.exp(-g))
            h[t, j] = sg * u
            bound[t, j] = 2.0 ** -10 * (1.1 * np.abs(u) * ab[:I] + np.abs(sg) * ab[I:]) + 2.0 ** -20 * np.abs(h[t, j])
    return h, bound


def check_mx_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, what):
    """x codes and scales bit-exact; for the valid pairs, the fp32
    intermediate within the MFMA's summation bound of the fp64 one, its MX
    requantisation bit-exact to the oracle's rule applied to that fp32 row,
    and codes at least 99% equal to the oracle's own; the layer output."""
    L = lib.moe_workspace_layout(T, k, E, H, I, "mxfp8")
    b = ws.cpu().numpy()
    xq = b[L["xq"]:L["xq"] + T * H].reshape(T, H)
    sx = b[L["x_scale"]:L["x_scale"] + T * H // 32].reshape(T, H // 32)
    rc, rs = oracle.mx_quant_rows_bf16(x.bfloat16())
    assert (xq == rc).all() and (sx == rs).all(), "x quantisation differs"
    # intermediate rows, sorted order: row pos[t*k+j] holds pair (t, j)
    ref, _, _, hq_ref, sh_ref = ref_out(x, ids, w, W, want_quant=True)
    R = lib.read_routing(routing, T, k, E, H, I, "mxfp8")
    pos = R["pos"].numpy()
    P = T * k
    valid = ((ids.numpy() >= 0) & (ids.numpy() < E)).reshape(T, k)
    h32 = b[L["g"]:L["g"] + 4 * P * I].view(np.float32).reshape(P, I)[pos].reshape(T, k, I)
    hq = b[L["h"]:L["h"] + P * I].reshape(P, I)[pos].reshape(T, k, I)[valid]
    sh = b[L["h_scale"]:L["h_scale"] + P * I // 32].reshape(P, I // 32)[pos].reshape(T, k, I // 32)[valid]
    # the fp32 intermediate against fp64 products of the same codes
    h64, hbound = dense_h_mx(rc, rs, ids, W)
    dh = np.abs(h32 - h64)[valid]
    ratio = (dh / np.maximum(hbound[valid], 1e-300)).max() if dh.size else 0.0
    log(f"  h max |err|/bound {ratio:.3e}")
    assert (dh <= hbound[valid]).all(), "intermediate outside the summation bound"
    # the requantisation: the MX rule on the GPU's own fp32 rows, exactly
    qc, qs = oracle.mx_quant_rows(h32[valid])
    assert (qc == hq).all() and (qs == sh).all(), "MX requantisation differs from the rule"
    same_s = (sh == sh_ref.reshape(T, k, I // 32)[valid]).mean()
    same_c = (hq == hq_ref.reshape(T, k, I)[valid]).mean()
    log(f"  h scale codes equal {same_s:.4f}, e4m3 codes equal {same_c:.4f} (against the oracle's fp64 rows)")
    assert same_s >= 0.99 and same_c >= 0.99
    check_tol(out.float().cpu().numpy(), ref, "mxfp8", what)


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
    check_mx_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, "mx quant case")


# Strips (from 12 mean rows per expert): the scaled instruction with the rows'
# and weights' e8m0 codes copied per stage; 64-, 128- and 192-row tiles, the
# down reduction unsplit or split into fp32 partial sums (2 and 8 slices).
STRIP_SHAPES = [
    # E, H, I, k, T, p_drop, block_m, split_k2
    (128, 512, 512, 8, 400, 0.02, 64, 1),
    (16, 256, 256, 8, 100, 0.0, 128, 1),
    (32, 256, 2048, 4, 200, 0.05, 64, 8),
    (128, 256, 512, 8, 1700, 0.01, 192, 2),
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop,bm,s2", STRIP_SHAPES)
def test_mx_strip_shapes(lib, E, H, I, k, T, p_drop, bm, s2):
    log(f"mx strips E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    L = lib.moe_workspace_layout(T, k, E, H, I, "mxfp8")
    assert L["tiling"] == 2 and L["split_k1"] == 1 and L["split_k2"] == s2
    assert lib.moe_routing_layout(T, k, E, H, I, "mxfp8")["block_m"] == bm
    wl = custom_workload(E, H, I, k, dtype="mxfp8", seed=E + T + 5)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 6)
    ids = random_ids(T, k, E, seed=T + 7, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 8)
    out, routing, ws = run(lib, x, ids, w, W)
    check_mx_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, f"mx strips E={E} T={T}")


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
