"""The routing build and the forward pass in one call (moe_route_forward_bf16
/ _fp8 / _int8 / _fp8_block / _mxfp8 / _int4 / _int8_w8a16).  For a decode batch of at most 64 token-expert pairs the routing
build runs inside the forward's first kernel (bf16 activations: the gate-up
GEMM; quantised activations: the x quantisation), whose workgroup 0 writes
the routing buffer.

Checked on every case:
- the routing buffer holds the same bytes as after moe_build_routing_* (both
  buffers start from the same poison, so a part one path leaves unwritten
  would differ), and its parts equal the oracle's routing;
- the output and the workspace equal those of the two separate calls bit
  for bit: the same kernels' arithmetic runs on the same rows;
- the output is within the forward tolerance of the oracle (bf16: max|err|
  <= 1e-2*max|ref| + 1e-3; fp8: 4e-2*max|ref|).
Cases: k from 1 to 16, dropped ids, every pair dropped, an expert named
twice, E = 1, batches of up to 64 pairs with a hot expert cut into several
row tiles, batches just past 64 pairs (the routing build launched first),
the full-size bf16 and fp8 workloads at every swept T with at most 64 pairs
in the launch configuration the benchmark times, graph capture with new ids
between replays.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, custom_workload, make_tokens, random_ids, random_weights_w
from moe_testlib import check_tol, device_weights, log, oracle_rows, path_dtype, workload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def separate(lib, ids, x, w, Wp, dtype, E, H, I, routing, ws, out):
    lib.build_routing(ids, E, H, I, routing, dtype)
    if dtype == "bf16":
        lib.moe_forward_bf16(x, w, routing, Wp["w1"], Wp["w2"], ws, out)
    else:
        fwd = {"fp8": lib.moe_forward_fp8, "int8": lib.moe_forward_int8, "fp8b": lib.moe_forward_fp8_block,
               "mxfp8": lib.moe_forward_mxfp8, "int4": lib.moe_forward_int4,
               "int8w": lib.moe_forward_int8_w8a16}[dtype]
        fwd(x, w, routing, Wp["w1"], Wp["w1_scale"], Wp["w2"], Wp["w2_scale"], ws, out)


def combined(lib, ids, x, w, Wp, dtype, routing, ws, out):
    lib.route_forward(ids, x, w, routing, Wp, ws, out, dtype)


def buffers(lib, T, k, E, H, I, dtype):
    routing = lib.alloc_routing(T, k, E, H, I, dtype)
    routing.fill_(0xAB)
    ws = lib.alloc_workspace(T, k, E, H, I, dtype)
    ws.fill_(0x5C)
    out = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
    return routing, ws, out


def check_case(lib, x, ids, w, Wp, Wc, E, H, I, dtype, what, oracle_check=True):
    T, k = ids.shape
    x = x.cuda().bfloat16().contiguous()
    idd = ids.cuda().contiguous()
    wd = w.cuda().float().contiguous()
    r0, ws0, out0 = buffers(lib, T, k, E, H, I, dtype)
    r1, ws1, out1 = buffers(lib, T, k, E, H, I, dtype)
    separate(lib, idd, x, wd, Wp, dtype, E, H, I, r0, ws0, out0)
    combined(lib, idd, x, wd, Wp, dtype, r1, ws1, out1)
    torch.cuda.synchronize()
    log(f"route+forward {what}: T={T} k={k} E={E} H={H} I={I} {dtype}")
    assert torch.equal(r1, r0), "routing buffer differs from the routing build's"
    assert torch.equal(out1, out0), "output differs from the separate calls'"
    assert torch.equal(ws1, ws0), "workspace differs from the separate calls'"
    R = lib.read_routing(r1, T, k, E, H, I, dtype)
    ref = oracle.route(ids.cpu().numpy(), E, R["layout"]["block_m"])
    assert np.array_equal(R["offsets"].numpy(), ref["offsets"]), "expert offsets"
    assert np.array_equal(R["sorted"].numpy(), ref["sorted"]), "sorted_pairs"
    assert np.array_equal(R["pos"].numpy(), ref["pos"]), "pair_pos"
    assert R["num_tasks"] == ref["num_tasks"] and R["num_dropped"] == ref["num_dropped"]
    assert np.array_equal(R["tasks"].numpy(), ref["tasks"]), "task map"
    if oracle_check:
        ref_out = oracle_rows(x, ids, w, Wc, dtype)
        if not np.abs(ref_out).sum():
            assert not out1.float().abs().sum().item()
        else:
            check_tol(out1.float().cpu().double().numpy(), ref_out, dtype, what)


DECODE = [
    # E, H, I, k
    (1, 256, 128, 4),
    (8, 256, 192, 1),
    (8, 512, 256, 2),
    (16, 320, 576, 3),
    (64, 1024, 640, 8),
    (32, 256, 128, 16),
    (256, 512, 256, 8),
]


# shapes for the dtypes with 128-value groups (H and I multiples of 128)
DECODE_Q = [
    (1, 256, 128, 4),
    (8, 256, 256, 1),
    (16, 512, 256, 3),
    (64, 1024, 512, 8),
    (32, 256, 128, 16),
]
QUANT = ["int8", "fp8b", "mxfp8", "int4", "int8w"]


@pytest.mark.parametrize("E,H,I,k,dtype", [(*sh, dt) for dt in ("bf16", "fp8") for sh in DECODE] +
                         [(*sh, dt) for dt in QUANT for sh in DECODE_Q])
@pytest.mark.parametrize("case", ["plain", "dropped", "all_dropped", "repeated"])
def test_one_token(lib, E, H, I, k, case, dtype):
    assert lib.moe_workspace_layout(1, k, E, H, I, dtype)["tiling"] == 0
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=E + H + I + k + 5)
    Wr = device_weights(wl)
    Wp = lib.pack_weights(Wr, dtype)
    Wc = {n: v.cpu() for n, v in Wr.items()}
    x, _, _ = make_tokens(wl, 1, seed=k + 50)
    ids = random_ids(1, k, E, seed=k + 51)
    if case == "dropped" and k > 1:
        ids[0, k // 2] = E + 3
        ids[0, 0] = -2
    elif case == "all_dropped":
        ids[0, :] = -1
    elif case == "repeated" and k > 1:
        ids[0, k - 1] = ids[0, 0]
    w = random_weights_w(1, k, seed=k + 52)
    check_case(lib, x, ids, w, Wp, Wc, E, H, I, dtype, case)


SEVERAL = [
    # T, k, E, case: pairs up to 64 take the folded build, more the launched one
    (2, 4, 16, "plain"), (3, 5, 16, "dropped"), (2, 8, 64, "plain"), (4, 16, 32, "hot"),
    (8, 8, 16, "hot"), (16, 4, 8, "dropped"), (32, 2, 8, "hot"), (8, 8, 1, "plain"),
    (9, 8, 16, "plain"), (5, 13, 16, "hot"), (64, 4, 16, "dropped"),
]


@pytest.mark.parametrize("T,k,E,case", SEVERAL)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"] + QUANT)
def test_several_tokens(lib, T, k, E, case, dtype):
    H, I = 512, 256
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=T + k + 60)
    Wr = device_weights(wl)
    Wp = lib.pack_weights(Wr, dtype)
    Wc = {n: v.cpu() for n, v in Wr.items()}
    x, _, _ = make_tokens(wl, T, seed=T + 61)
    ids = random_ids(T, k, E, seed=T + k + 62, p_drop=0.1 if case == "dropped" else 0.0)
    if case == "hot":          # one expert takes three pairs of every token: several row tiles
        ids[:, :min(3, k)] = 0
    w = random_weights_w(T, k, seed=T + 63)
    check_case(lib, x, ids, w, Wp, Wc, E, H, I, dtype, f"T={T} {case}")


FULL_DECODE = [(n, T) for n in ("mixtral", "qwen3", "qwen2", "dsv3", "dsv3i8", "dsv3b", "dsv3mx", "mixtral4",
                                 "mixtral8")
               for T in sorted(set([1] + [t for t in WORKLOADS[n].Ts if t * WORKLOADS[n].k <= 64]))]


@pytest.mark.parametrize("name,T", FULL_DECODE)
def test_full_size_decode(lib, name, T):
    wl = WORKLOADS[name]
    dtype = path_dtype(wl)
    Wp, Wc = workload_weights(name)
    x, ids, w = make_tokens(wl, T)
    check_case(lib, x, ids, w, Wp, Wc, wl.E, wl.H, wl.I, dtype, f"{name} T={T}")


@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (8, "bf16"), (1, "fp8"), (8, "fp8"), (1, "int8"),
                                     (8, "mxfp8"), (2, "fp8b"), (1, "int4"), (4, "int8w")])
def test_graph_capture_new_ids_between_replays(lib, T, dtype):
    E, H, I, k = 64, 1024, 512, 8
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=70)
    Wr = device_weights(wl)
    Wp = lib.pack_weights(Wr, dtype)
    x, _, _ = make_tokens(wl, T, seed=71)
    x = x.cuda().bfloat16().contiguous()
    ids = random_ids(T, k, E, seed=72).cuda()
    w = random_weights_w(T, k, seed=73).cuda()
    routing, ws, out = buffers(lib, T, k, E, H, I, dtype)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        combined(lib, ids, x, w, Wp, dtype, routing, ws, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        combined(lib, ids, x, w, Wp, dtype, routing, ws, out)
    draws = [random_ids(T, k, E, seed=74 + r) for r in range(3)]
    draws[1][:, 3] = draws[1][:, 0]        # an expert named twice
    draws[1][:, 2] = 5                     # and one in every token (T = 8: 8 pairs)
    draws[2][0, 1] = -1                    # a dropped pair
    for r, new in enumerate(draws):
        ids.copy_(new.cuda())
        out.fill_(0)
        routing.fill_(0xAB)
        g.replay()
        torch.cuda.synchronize()
        r0, ws0, out0 = buffers(lib, T, k, E, H, I, dtype)
        separate(lib, ids, x, w, Wp, dtype, E, H, I, r0, ws0, out0)
        torch.cuda.synchronize()
        assert torch.equal(out, out0), f"replay {r}: output"
        assert torch.equal(routing, r0), f"replay {r}: routing buffer"
