"""GPU parity of the routing & index build: bit-exact against the oracle.

Compared: expert offsets, the route index (sorted_pairs and its inverse
pair_pos), the task map up to num_tasks, num_tasks and num_dropped, for the
five workloads at every token count they are swept over, and for edge
cases (one pair, dropped ids, a single hot expert, duplicates, the maximum
of 65536 pairs, E = 1 and E = 256).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, make_tokens, random_ids
from moe_testlib import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def gpu_route(lib, ids, E, H, I, dtype):
    T, k = ids.shape
    routing = lib.alloc_routing(T, k, E, H, I, dtype)
    routing.fill_(0xAB)           # poison: every compared word must be written
    lib.build_routing(ids.cuda().contiguous(), E, H, I, routing, dtype)
    torch.cuda.synchronize()
    return lib.read_routing(routing, T, k, E, H, I, dtype)


def check_route(lib, ids, E, H, I, dtype, what):
    log(f"route {what}: T={ids.shape[0]} k={ids.shape[1]} E={E} {dtype}")
    got = gpu_route(lib, ids, E, H, I, dtype)
    ref = oracle.route(ids.cpu().numpy(), E, got["layout"]["block_m"])
    assert got["block_m"] == got["layout"]["block_m"]
    assert np.array_equal(got["offsets"].numpy(), ref["offsets"]), "expert offsets"
    assert np.array_equal(got["sorted"].numpy(), ref["sorted"]), "sorted_pairs"
    assert np.array_equal(got["pos"].numpy(), ref["pos"]), "pair_pos"
    assert got["num_tasks"] == ref["num_tasks"], "num_tasks"
    assert got["num_dropped"] == ref["num_dropped"], "num_dropped"
    assert np.array_equal(got["tasks"].numpy(), ref["tasks"]), "task map"
    hdr = got["header"].numpy()
    assert hdr[3] == ids.numel() and hdr[4] == E and hdr[5] == got["layout"]["max_tasks"]
    tiles = np.bincount(ref["tasks"][:, 0], minlength=1) if ref["num_tasks"] else np.zeros(1)
    assert hdr[6] == int(tiles.max()), "largest number of tiles of one expert"
    assert not hdr[7:].any()


CASES = [(name, T) for name, wl in WORKLOADS.items() for T in wl.Ts]


@pytest.mark.parametrize("name,T", CASES)
def test_routing_workloads(lib, name, T):
    wl = WORKLOADS[name]
    _, ids, _ = make_tokens(wl, T)
    dtype = wl.dtype if wl.dtype in ("fp8", "fp8b", "mxfp8", "int8", "int4", "int8w") else "bf16"
    check_route(lib, ids, wl.E, wl.H, wl.I, dtype, name)


@pytest.mark.parametrize("T,k,E,p_drop,seed", [
    (1, 1, 1, 0.0, 1), (1, 8, 256, 0.0, 2), (3, 4, 5, 0.5, 3), (777, 3, 17, 0.1, 4),
    (8192, 8, 256, 0.02, 5), (4096, 16, 256, 0.0, 6), (5000, 13, 200, 0.3, 7),
    (1000, 2, 1, 0.5, 8),
])
@pytest.mark.parametrize("H,I", [(128, 64), (4096, 14336)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_routing_edge_cases(lib, T, k, E, p_drop, seed, H, I, dtype):
    ids = random_ids(T, k, E, seed=seed, p_drop=p_drop)
    check_route(lib, ids, E, H, I, dtype, f"random seed={seed}")


def test_routing_max_pairs_hot_expert(lib):
    T, k, E = 4096, 16, 64               # P = 65536, the maximum
    ids = random_ids(T, k, E, seed=9)
    ids[::2, 0] = 0
    ids[:, 5] = 0                         # expert 0 appears twice in many tokens
    check_route(lib, ids, E, 3584, 640, "bf16", "max pairs")


def test_routing_all_dropped(lib):
    ids = torch.full((10, 4), -1, dtype=torch.int32)
    ids[3, 2] = 99
    check_route(lib, ids, 8, 128, 64, "bf16", "all dropped")


def test_routing_is_deterministic(lib):
    ids = random_ids(3000, 8, 128, seed=10, p_drop=0.05)
    a = gpu_route(lib, ids, 128, 2048, 768, "bf16")
    for _ in range(3):
        b = gpu_route(lib, ids, 128, 2048, 768, "bf16")
        for key in ("offsets", "sorted", "pos", "tasks", "header"):
            assert torch.equal(a[key], b[key])
