"""GPU parity of the block-scaled fp8 path (SGLang tuning guide: block_shape
[128, 128], DeepSeek-V3's fp8 quantisation): e4m3 weights with one fp32
scale per 128 x 128 block, activations quantised per 128-value group of a
row.

* x's group quantisation is decided on exact inputs on both sides: codes
  and scales bit-exact.
* Each 128-value unit sum comes from one fp8 MFMA (whose own summation is
  coarser than fp32, see dense_h) and is rescaled in fp32; the layer is
  checked against the oracle within the fp8 bound
  max|err| <= 4e-2 max|ref|, over shapes spanning several tiles and ragged
  tails, dropped pairs, one token, the DeepSeek-V3 expert shape (at a TP=8
  slice and whole), and in a replayed HIP graph.
* The fp32 intermediate silu(gate) * up within the MFMA's summation bound
  of an fp64 evaluation on the same codes; its requantisation (fp64 in the
  oracle before its rounding): at least 99% of codes equal, none more than
  one code apart, each group scale within the group's largest
  intermediate error / 448.
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
    packed = lib.pack_weights({k: v.cuda() for k, v in W.items()}, "fp8b")
    out, routing, ws = lib.moe_layer(x.cuda().bfloat16().contiguous(), ids.cuda().contiguous(),
                                     w.cuda().float().contiguous(), packed, dtype="fp8b")
    torch.cuda.synchronize()
    return out, routing, ws


def ref_out(x, ids, w, W, want_quant=False):
    return oracle.forward_fp8_block(x.bfloat16(), w, ids, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"],
                                    want_quant=want_quant)


def e4m3_order(codes):
    """Signed position of e4m3 codes on the number line (adjacent codes of
    one sign differ by one; +0 and -0 coincide)."""
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e4m3_spacing(mag):
    """Distance to the next e4m3 code above magnitude code mag (0..126):
    2^-9 for subnormals (exponent field 0), else 2^(e - 10)."""
    e = (np.asarray(mag).astype(np.int32) >> 3)
    return np.where(e == 0, 2.0 ** -9, np.exp2(e.astype(np.float64) - 10.0))


def e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()


def dense_h(xq, sx, ids, W):
    """fp64 intermediate silu(gate) * up of every pair from the quantised x
    (codes and group scales) and the block-scaled weights, and a bound on
    the error of the GPU's evaluation.

    The gfx950 fp8 MFMA does not sum a unit's 128 products exactly: measured
    on the device, each run of 8 consecutive products is aligned to the
    largest exponent sum e_a + e_b among them (e = the code's exponent, -6
    for subnormals) and cut to multiples of 2^(e_max - 13), so a unit sum
    is off by less than 7 * 2^-13 * sum of a^ b^ with a^ = max(|a|, 2^-6).
    The bound takes 2^-10 times those sums (scaled) for gate and up, carried
    through silu(g) * u (|silu'| < 1.1), plus 2^-20 |h| for the fp32
    rescales, sums and SiLU."""
    T, H = xq.shape
    E, I2, _ = W["w1"].shape
    I = I2 // 2
    k = ids.shape[1]
    xs = torch.from_numpy(sx).double().repeat_interleave(128, dim=1)
    xv = e4m3_values(xq)
    x = xv * xs
    xhat = xv.abs().clamp_min(2.0 ** -6) * xs
    s1 = W["w1_scale"].double().repeat_interleave(128, dim=1).repeat_interleave(128, dim=2)
    h = np.zeros((T, k, I))
    bound = np.zeros((T, k, I))
    cache = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            if e not in cache:   # the expert's dequantised weights and their bound weights
                wv = e4m3_values(W["w1"][e].numpy())
                cache[e] = (wv * s1[e], wv.abs().clamp_min(2.0 ** -6) * s1[e])
            wd, wb = cache[e]
            gu = (wd @ x[t]).numpy()
            ab = (wb @ xhat[t]).numpy()
            g, u = gu[:I], gu[I:]
            sg = g / (1 + np.exp(-g))
            h[t, j] = sg * u
            bound[t, j] = 2.0 ** -10 * (1.1 * np.abs(u) * ab[:I] + np.abs(sg) * ab[I:]) + 2.0 ** -20 * np.abs(h[t, j])
    return h, bound


SHAPES = [
    # E, H, I, k, T, p_drop
    (8, 256, 256, 2, 5, 0.0),
    (16, 512, 256, 4, 33, 0.1),
    (64, 1024, 640, 8, 100, 0.05),
    (32, 256, 128, 8, 1, 0.0),
    (1, 256, 256, 1, 70, 0.0),
    (256, 7168, 256, 8, 16, 0.0),       # DeepSeek-V3 shape, TP=8 slice
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop", SHAPES)
def test_fp8b_layer_parity(lib, E, H, I, k, T, p_drop):
    log(f"fp8b layer E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    wl = custom_workload(E, H, I, k, dtype="fp8b", seed=E + T)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 1)
    ids = random_ids(T, k, E, seed=T + 2, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 3)
    out, _, _ = run(lib, x, ids, w, W)
    check_tol(out.float().cpu().numpy(), ref_out(x, ids, w, W), "fp8b", f"fp8b E={E} T={T}")


def check_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, what):
    """x codes and scales bit-exact, their copies at the sorted rows, the
    fp32 intermediate within the MFMA's summation bound, its group
    requantisation (codes and scales), and the layer output."""
    L = lib.moe_workspace_layout(T, k, E, H, I, "fp8b")
    b = ws.cpu()
    xq = b[L["xq"]:L["xq"] + T * H].numpy().reshape(T, H)
    sx = b[L["x_scale"]:L["x_scale"] + 4 * T * H // 128].view(torch.float32).numpy().reshape(T, H // 128)
    ref, xq_ref, sx_ref, hq_ref, sh_ref = ref_out(x, ids, w, W, want_quant=True)
    assert (xq == xq_ref).all() and (sx == sx_ref).all(), "x quantisation differs"
    R = lib.read_routing(routing, T, k, E, H, I, "fp8b")
    pos = R["pos"].numpy()
    P = T * k
    valid = ((ids.numpy() >= 0) & (ids.numpy() < E)).reshape(T, k)
    # the scales of x, spread unit-major over the sorted rows of each pair
    sxr = b[L["x_scale_rows"]:L["x_scale_rows"] + 4 * P * H // 128].view(torch.float32).numpy()
    sxr = sxr.reshape(H // 128, P)[:, pos].T.reshape(T, k, H // 128)
    assert (sxr[valid] == np.broadcast_to(sx_ref[:, None, :], sxr.shape)[valid]).all(), "x scales at sorted rows"
    # the fp32 intermediate against fp64 products of the same codes, each
    # error within the MFMA's summation bound
    h32 = b[L["g"]:L["g"] + 4 * P * I].view(torch.float32).numpy().reshape(P, I)[pos].reshape(T, k, I)
    h64, hbound = dense_h(xq_ref, sx_ref, ids, W)
    dh = np.where(valid[..., None], np.abs(h32 - h64), 0.0)
    ratio = np.where(hbound > 0, dh / np.where(hbound > 0, hbound, 1.0), np.where(dh > 0, np.inf, 0.0))
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    log(f"  h max |err|/bound {ratio.max():.3e} at {worst}: gpu {h32[worst]!r} fp64 {h64[worst]!r} "
        f"bound {hbound[worst]:.3e}")
    assert (dh <= hbound).all(), "intermediate outside the summation bound"
    hq = b[L["h"]:L["h"] + P * I].numpy().reshape(P, I)[pos].reshape(T, k, I)
    sh = b[L["h_scale"]:L["h_scale"] + 4 * P * I // 128].view(torch.float32).numpy()
    sh = sh.reshape(I // 128, P)[:, pos].T.reshape(T, k, I // 128)
    same = (hq[valid] == hq_ref[valid]).mean()
    log(f"  h codes equal {same:.4f}, max scale rel diff {np.abs(sh[valid] / sh_ref[valid] - 1).max():.2e}")
    assert same >= 0.99
    # A code is decided on the fp32 intermediate here and on fp64 in the
    # oracle; the two differ by at most dh.  Where an e4m3 step is larger
    # than that (normal codes) the codes are at most one apart; in the
    # subnormal range a step (2^-9 of the scale) can be smaller than dh, so
    # the gate is on values: one step at the larger code plus dh.
    step = e4m3_spacing(np.maximum(hq & 0x7F, hq_ref & 0x7F))
    shx = np.repeat(sh, 128, axis=-1)
    shrx = np.repeat(sh_ref, 128, axis=-1)
    vdev = np.abs(e4m3_values(hq).numpy() * shx - e4m3_values(hq_ref).numpy() * shrx)
    allowed = dh + step * np.maximum(shx, shrx) * (1 + 1e-6)
    far = np.abs(e4m3_order(hq) - e4m3_order(hq_ref)) > 1
    log(f"  codes more than one apart: {int(far[valid].sum())}, all subnormal: "
        f"{bool(((np.maximum(hq & 0x7F, hq_ref & 0x7F) < 8) | ~far)[valid].all())}")
    assert (vdev <= allowed)[valid].all(), "requantised values beyond one step plus the intermediate error"
    # a group's scale is its max |h| / 448: it moves by at most the group's
    # largest intermediate error / 448 (plus the scale's own rounding)
    gerr = dh.reshape(T, k, I // 128, 128).max(-1) / 448.0
    assert (np.abs(sh - sh_ref)[valid] <= (gerr * (1 + 1e-6) + 2 * np.spacing(sh_ref))[valid]).all()
    check_tol(out.float().cpu().numpy(), ref, "fp8b", what)


def test_fp8b_quant_and_requant(lib):
    E, H, I, k, T = 16, 512, 256, 4, 24
    wl = custom_workload(E, H, I, k, dtype="fp8b", seed=9)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=10)
    x[3] = 0.0                                         # an all-zero row
    x[5, 0] = 3000.0                                   # an outlier in one group
    x[6, 128:256] = 0.0                                # an all-zero group
    ids = random_ids(T, k, E, seed=11)
    w = random_weights_w(T, k, seed=12)
    out, routing, ws = run(lib, x, ids, w, W)
    L = lib.moe_workspace_layout(T, k, E, H, I, "fp8b")
    xq = ws.cpu()[L["xq"]:L["xq"] + T * H].numpy().reshape(T, H)
    sx = ws.cpu()[L["x_scale"]:L["x_scale"] + 4 * T * H // 128].view(torch.float32).numpy().reshape(T, H // 128)
    for t in range(T):                                 # the oracle's rule, restated per row
        for gi in range(H // 128):
            qc, qs = oracle.quant_groups(x[t, gi * 128:(gi + 1) * 128].bfloat16().float().numpy())
            assert (qc == xq[t, gi * 128:(gi + 1) * 128]).all() and qs[0] == sx[t, gi]
    check_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, "fp8b quant case")


# Strips (from 12 mean rows per expert): each 128-value unit rescaled by its
# row group and weight block scales; 64-, 128- and 192-row tiles, the down
# reduction unsplit or split into fp32 partial sums (2 and 8 slices).
STRIP_SHAPES = [
    # E, H, I, k, T, p_drop, block_m, split_k2
    (128, 512, 512, 8, 400, 0.02, 64, 1),
    (16, 256, 256, 8, 100, 0.0, 128, 1),
    (32, 256, 2048, 4, 200, 0.05, 64, 8),
    (128, 256, 512, 8, 1700, 0.01, 192, 2),
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop,bm,s2", STRIP_SHAPES)
def test_fp8b_strip_shapes(lib, E, H, I, k, T, p_drop, bm, s2):
    log(f"fp8b strips E={E} H={H} I={I} k={k} T={T} p_drop={p_drop}")
    L = lib.moe_workspace_layout(T, k, E, H, I, "fp8b")
    assert L["tiling"] == 2 and L["split_k1"] == 1 and L["split_k2"] == s2
    assert lib.moe_routing_layout(T, k, E, H, I, "fp8b")["block_m"] == bm
    wl = custom_workload(E, H, I, k, dtype="fp8b", seed=E + T + 5)
    W = make_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 6)
    ids = random_ids(T, k, E, seed=T + 7, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 8)
    out, routing, ws = run(lib, x, ids, w, W)
    check_intermediates(lib, x, ids, w, W, E, H, I, k, T, out, routing, ws, f"fp8b strips E={E} T={T}")


def test_fp8b_dsv3_shape_decode(lib):
    wl = WORKLOADS["dsv3b"]
    W = make_weights(wl, device="cuda")
    packed = lib.pack_weights(W, "fp8b")
    Wc = {kk: v.cpu() for kk, v in W.items()}
    del W
    for T in (1, 16):
        x, ids, w = make_tokens(wl, T)
        out, _, _ = lib.moe_layer(x.cuda(), ids.cuda(), w.cuda(), packed, dtype="fp8b")
        torch.cuda.synchronize()
        ref = oracle.forward_fp8_block(x, w, ids, Wc["w1"], Wc["w1_scale"], Wc["w2"], Wc["w2_scale"])
        check_tol(out.float().cpu().numpy(), ref, "fp8b", f"dsv3b T={T}")


def test_fp8b_graph_replay(lib):
    E, H, I, k, T = 32, 512, 256, 4, 64
    wl = custom_workload(E, H, I, k, dtype="fp8b", seed=13)
    W = make_weights(wl)
    packed = lib.pack_weights({kk: v.cuda() for kk, v in W.items()}, "fp8b")
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    w = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    routing = lib.alloc_routing(T, k, E, H, I, "fp8b")
    ws = lib.alloc_workspace(T, k, E, H, I, "fp8b")
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step():
        lib.moe_build_routing_fp8_block(ids, E, H, I, routing)
        lib.moe_forward_fp8_block(x, w, routing, packed["w1"], packed["w1_scale"], packed["w2"],
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
        check_tol(got, ref_out(xh, idh, wh, W), "fp8b", f"fp8b graph replay {rep}")
