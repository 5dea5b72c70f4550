"""GPU parity of the router top-k kernel against the oracle.

The router's fp32 scores pick the experts through a top-k choice (HPC-Ops x
SGLang blog, section "Router GEMM"); shared experts are fused as extra
expert ids (SGLang tuning guide, model-config section).  The ranking
compares fp32 logits on both sides, so ids are checked bit-exactly, ties
included; weights are fp32 on the GPU against fp64 in the oracle, within
|err| <= 2e-6 (a few fp32 roundings of exp, one sum of at most 256 terms
and one division, on values in [0, 1]).

Cases: every width of the lane group (E from 1 to 256), k from 1 to 16,
renormalised and plain softmax weights, 0-2 shared experts, rows with
ties, equal rows, 1e30-wide and NaN-sprinkled rows, the unaligned-row
path, the workloads' own shapes at full size, and router -> routing build
-> forward end to end (with a fused shared expert, up to 257 experts),
eagerly and replayed from one HIP graph.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, custom_workload, make_router_inputs, make_weights, router_logits
from moe_testlib import check_tol, log

pytestmark = pytest.mark.gpu

W_TOL = 2e-6


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def compare(lib, logits, k, renorm=True, ns=0, what="", logits_dev=None):
    T, E = logits.shape
    log(f"router {what}: T={T} E={E} k={k} renorm={int(renorm)} n_shared={ns}")
    dev = logits.cuda() if logits_dev is None else logits_dev
    ids, w = lib.moe_router_topk(dev, k, renormalize=renorm, n_shared=ns)
    torch.cuda.synchronize()
    rid, rw = oracle.router_topk(logits, k, renormalize=renorm, n_shared=ns)
    gid = ids.cpu().numpy()
    gw = w.cpu().numpy().astype(np.float64)
    bad = np.argwhere(gid != rid)
    assert bad.size == 0, f"ids differ at {bad[:5].tolist()}: gpu {gid[tuple(bad[0])]} oracle {rid[tuple(bad[0])]}"
    fin = np.isfinite(rw)
    if fin.any():
        err = float(np.max(np.abs(gw[fin] - rw[fin])))
        assert err <= W_TOL, f"weights differ by {err}"
    return gid, gw


SHAPES = [(1, 1), (2, 2), (3, 1), (3, 3), (5, 2), (8, 2), (8, 8), (12, 5), (16, 16), (17, 4),
          (32, 8), (37, 16), (64, 8), (100, 6), (128, 8), (129, 3), (200, 13), (256, 1),
          (256, 8), (256, 16)]


@pytest.mark.parametrize("E,k", SHAPES)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_router_parity(lib, E, k, kind):
    T = 301
    l = router_logits(T, E, seed=E * 100 + k, kind=kind)
    compare(lib, l, k, True, 0, kind)
    compare(lib, l, k, False, 0, kind)
    if k + 2 <= 16:
        compare(lib, l, k, True, 2 if E % 2 else 1, kind)


@pytest.mark.parametrize("kind", ["const", "wide", "nan"])
@pytest.mark.parametrize("E,k", [(8, 2), (37, 5), (64, 8), (256, 8), (256, 16)])
def test_router_special_rows(lib, kind, E, k):
    l = router_logits(129, E, seed=7 + E, kind=kind)
    gid, gw = compare(lib, l, k, True, 0, kind)
    if kind == "const":
        assert (gid == np.arange(k)).all()
        assert np.allclose(gw, 1.0 / k, atol=W_TOL)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (256, 8)])
def test_router_unaligned_rows(lib, E, k):
    # rows that start 4 bytes past a 16-byte boundary take the per-element loads
    T = 77
    l = router_logits(T, E, seed=3, kind="ties")
    flat = torch.zeros(T * E + 1, dtype=torch.float32, device="cuda")
    flat[1:] = l.reshape(-1).cuda()
    dev = flat[1:].view(T, E)
    assert dev.data_ptr() % 16 == 4
    compare(lib, l, k, True, 1, "unaligned", logits_dev=dev)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 1000])
def test_router_token_counts(lib, T):
    # groups per workgroup: 256 / L tokens; counts around the block edges
    for E in (8, 64, 256):
        compare(lib, router_logits(T, E, seed=T, kind="ties"), min(8, E), True, 1, "tokens")


@pytest.mark.parametrize("name,T", [("mixtral", 64), ("qwen3", 256), ("qwen2", 4096), ("dsv3", 4096),
                                    ("dsv3", 1)])
def test_router_workloads_full_size(lib, name, T):
    wl = WORKLOADS[name]
    _, l = make_router_inputs(wl, T)
    compare(lib, l, wl.k, True, 0, name)
    compare(lib, l, wl.k, True, 1, name + " +shared")


def test_router_empty(lib):
    ids, w = lib.moe_router_topk(torch.zeros(0, 8, device="cuda"), 2, n_shared=1)
    torch.cuda.synchronize()
    assert ids.shape == (0, 3) and w.shape == (0, 3)


def _layer_oracle(x, l, k, ns, Wd, dtype):
    rid, rw = oracle.router_topk(l, k, renormalize=True, n_shared=ns)
    ids = torch.from_numpy(rid)
    w = torch.from_numpy(rw.astype(np.float32))
    xb = x.bfloat16()
    if dtype == "bf16":
        return oracle.forward_bf16(xb, w, ids, Wd["w1"].cpu(), Wd["w2"].cpu())
    return oracle.forward_fp8(xb, w, ids, Wd["w1"].cpu(), Wd["w1_scale"].cpu(), Wd["w2"].cpu(),
                              Wd["w2_scale"].cpu())


@pytest.mark.parametrize("E,H,I,k,T,dtype", [
    (32, 512, 256, 4, 100, "bf16"),
    (32, 512, 256, 4, 100, "fp8"),
    (256, 256, 128, 8, 64, "bf16"),     # 256 routed + 1 shared = 257 experts
    (256, 256, 128, 8, 600, "fp8"),
    (8, 256, 192, 2, 1, "bf16"),
])
def test_router_to_layer_with_shared_expert(lib, E, H, I, k, T, dtype):
    ns = 1
    wl = custom_workload(E + ns, H, I, k + ns, dtype=dtype, seed=E + T)
    Wd = make_weights(wl, device="cpu")
    packed = lib.pack_weights({kk: v.cuda() for kk, v in Wd.items()}, dtype)
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(T)).bfloat16()
    l = router_logits(T, E, seed=T + 1, kind="normal")
    log(f"router->layer: E={E}+{ns} H={H} I={I} k={k}+{ns} T={T} {dtype}")
    ids, w = lib.moe_router_topk(l.cuda(), k, renormalize=True, n_shared=ns)
    out, _, _ = lib.moe_layer(x.cuda(), ids, w, packed, dtype=dtype)
    torch.cuda.synchronize()
    ref = _layer_oracle(x, l, k, ns, Wd, dtype)
    check_tol(out.float().cpu().numpy(), ref, dtype, f"router->layer {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_router_and_layer_in_one_graph(lib, dtype):
    # router top-k + routing build + forward captured once, replayed on new logits
    E, H, I, k, T, ns = 64, 512, 256, 6, 48, 1
    wl = custom_workload(E + ns, H, I, k + ns, dtype=dtype, seed=5)
    Wd = make_weights(wl, device="cpu")
    packed = lib.pack_weights({kk: v.cuda() for kk, v in Wd.items()}, dtype)
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(2)).bfloat16().cuda()
    logits = torch.zeros(T, E, device="cuda")
    ids = torch.empty(T, k + ns, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k + ns, dtype=torch.float32, device="cuda")
    routing = lib.alloc_routing(T, k + ns, E + ns, H, I, dtype)
    ws = lib.alloc_workspace(T, k + ns, E + ns, H, I, dtype)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    build = lib.moe_build_routing_bf16 if dtype == "bf16" else lib.moe_build_routing_fp8

    def step():
        lib.moe_router_topk(logits, k, True, ns, topk_ids=ids, topk_w=w)
        build(ids, E + ns, H, I, routing)
        if dtype == "bf16":
            lib.moe_forward_bf16(x, w, routing, packed["w1"], packed["w2"], ws, out)
        else:
            lib.moe_forward_fp8(x, w, routing, packed["w1"], packed["w1_scale"], packed["w2"],
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
        l = router_logits(T, E, seed=40 + rep, kind="ties" if rep == 1 else "normal")
        logits.copy_(l.cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rid, _ = oracle.router_topk(l, k, True, ns)
        assert (ids.cpu().numpy() == rid).all()
        got = out.float().cpu().numpy()
        step()                                   # eager run on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(out.float().cpu(), torch.from_numpy(got)), "graph replay != eager"
        check_tol(got, _layer_oracle(x.cpu(), l, k, ns, Wd, dtype), dtype, f"graph replay {rep}")
