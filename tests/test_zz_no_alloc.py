"""moe_forward_fp8_noalloc, the fp8 forward for callers that cannot allocate
(its workspace is the library's fixed per-GPU array): called through the C
ABI, its output equals moe_forward_fp8's on the same inputs, bit for bit (the
same kernels on the same plan), on two calls in a row with the second one
smaller, on register-streaming and strip tilings; and both are within the fp8
bound of the oracle.  Sizes beyond the array are refused before any launch."""
import pytest
import torch

from moe_inputs import custom_workload, make_tokens, random_ids, random_weights_w
from moe_testlib import check_tol, device_weights, log, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def test_noalloc_matches_the_workspace_entry_point(lib):
    E, H, I, k = 64, 1024, 512, 8
    wl = custom_workload(E, H, I, k, dtype="fp8", seed=71)
    W = device_weights(wl)
    Wp = lib.pack_weights(W, "fp8")
    # strips, then register streaming on a smaller batch, then strips again
    for T, seed in ((300, 72), (16, 73), (64, 74)):
        L = lib.moe_workspace_layout(T, k, E, H, I, "fp8")
        log(f"noalloc fp8 E={E} H={H} I={I} k={k} T={T} tiling={L['tiling']} "
            f"workspace={L['total_bytes']} B")
        assert L["total_bytes"] <= lib.STATIC_WORKSPACE_BYTES
        x, _, _ = make_tokens(wl, T, seed=seed)
        x = x.cuda()
        ids = random_ids(T, k, E, seed=seed + 1, p_drop=0.05).cuda()
        w = random_weights_w(T, k, seed=seed + 2).cuda()
        routing = lib.alloc_routing(T, k, E, H, I, "fp8")
        lib.moe_build_routing_fp8(ids, E, H, I, routing)
        ws = lib.alloc_workspace(T, k, E, H, I, "fp8")
        ref = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        lib.moe_forward_fp8(x, w, routing, Wp["w1"], Wp["w1_scale"], Wp["w2"], Wp["w2_scale"], ws, ref)
        out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        lib.moe_forward_fp8_noalloc(x, w, routing, Wp["w1"], Wp["w1_scale"], Wp["w2"], Wp["w2_scale"], out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"T={T}: differs from moe_forward_fp8"
        check_tol(out.float().cpu().double().numpy(), oracle_rows(x, ids, w, W, "fp8"), "fp8",
                  f"noalloc T={T}")


def test_noalloc_refuses_sizes_beyond_its_array(lib):
    E, H, I, k, T = 256, 7168, 2048, 8, 1024    # DeepSeek-V3 shape: about 0.6 GB of workspace
    L = lib.moe_workspace_layout(T, k, E, H, I, "fp8")
    assert L["total_bytes"] > lib.STATIC_WORKSPACE_BYTES
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    out = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    routing = torch.zeros(16, dtype=torch.uint8, device="cuda")
    w1 = lib.moe_describe_packed_weights(torch.zeros(E, 2 * I, H, dtype=torch.uint8, device="cuda"), "fp8")
    w2 = lib.moe_describe_packed_weights(torch.zeros(E, H, I, dtype=torch.uint8, device="cuda"), "fp8")
    s1 = torch.zeros(E, 2 * I, dtype=torch.float32, device="cuda")
    s2 = torch.zeros(E, H, dtype=torch.float32, device="cuda")
    with pytest.raises(lib.MoeError) as ei:
        lib.moe_forward_fp8_noalloc(x, w, routing, w1, s1, w2, s2, out)
    assert ei.value.status == -3
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item()          # nothing was launched
