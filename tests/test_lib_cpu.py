"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function include/moe.h declares, and
reject bad arguments on the host with the documented status codes before
enqueueing any work.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def m():
    import mixture_experts_layer_lds_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_all_exported(m):
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(m.EXPORTS)


def test_status_strings(m):
    assert m.status_string(0) == "ok"
    assert m.status_string(-3) == "buffer too small"


def test_routing_layout_sizes(m):
    L = m.moe_routing_layout(4, 2, 8, 128, 64, "bf16")
    assert L["header"] == 0 and L["expert_offsets"] == 64
    assert L["block_m"] in (16, 32, 64)
    assert L["max_tasks"] == 8 // L["block_m"] + min(8, 8)
    for key in ("expert_offsets", "sorted_pairs", "pair_pos", "tasks", "total_bytes"):
        assert L[key] % 16 == 0
    assert L["tasks"] + 16 * L["max_tasks"] <= L["total_bytes"]
    big = m.moe_routing_layout(4096, 8, 64, 3584, 640, "bf16")
    assert big["sorted_pairs"] + 4 * 32768 <= big["pair_pos"]


def test_workspace_layout(m):
    # register streaming (DeepSeek-V3 decode): fp32 h rows for the requantisation,
    # bf16 down rows, per-sorted-row x scales
    W = m.moe_workspace_layout(16, 8, 256, 7168, 2048, "fp8")
    P = 128
    assert W["tiling"] == 0 and W["split_k1"] == 1 and W["split_k2"] == 1
    assert W["xq"] == 0 and W["x_scale"] >= 16 * 7168
    assert W["x_scale_rows"] >= W["x_scale"] + 4 * 16
    assert W["g"] >= W["x_scale_rows"] + 4 * (P + 16)
    assert W["h"] >= W["g"] + 4 * P * 2048
    assert W["h_scale"] >= W["h"] + P * 2048
    assert W["y"] >= W["h_scale"] + 4 * P
    assert W["y"] + 2 * P * 7168 <= W["total_bytes"]
    for key in ("xq", "x_scale", "x_scale_rows", "g", "h", "h_scale", "y"):
        assert W[key] % 256 == 0
    # strips (T=1024): one gate-up slice, so fp32 SiLU(gate)*up and the
    # per-sorted-row x scales for its epilogue; down rows bf16 or fp32 partials
    S = m.moe_workspace_layout(1024, 8, 256, 7168, 2048, "fp8")
    P = 8192
    assert S["tiling"] == 2 and S["split_k1"] == 1
    assert S["g"] >= S["x_scale_rows"] + 4 * (P + 16)
    assert S["h"] >= S["g"] + 4 * P * 2048
    ybytes = 2 * P * 7168 if S["split_k2"] == 1 else 4 * S["split_k2"] * P * 7168
    assert S["y"] + ybytes <= S["total_bytes"]
    Wb = m.moe_workspace_layout(16, 8, 256, 7168, 2048, "bf16")
    assert Wb["xq"] == 2 ** 64 - 1 and Wb["h_scale"] == 2 ** 64 - 1
    # one token: the down launch adds the top-k rows, no down rows in memory
    # (bf16 and fp8 whenever an I row is an even number of 64-byte steps)
    for dt, I in (("fp8", 2048), ("bf16", 768), ("bf16", 576)):
        D = m.moe_workspace_layout(1, 8, 256, 7168, I, dt)
        assert D["tiling"] == 0 and D["y"] == 2 ** 64 - 1 and D["h"] < D["total_bytes"]
    # ... but not with an odd number (fp8, I = 576: 9 steps) or another dtype
    assert m.moe_workspace_layout(1, 3, 16, 320, 576, "fp8")["y"] != 2 ** 64 - 1
    assert m.moe_workspace_layout(1, 8, 256, 7168, 2048, "int8")["y"] == 2 ** 64 - 1
    assert m.moe_workspace_layout(1, 8, 256, 7168, 2048, "mxfp8")["y"] != 2 ** 64 - 1
    assert m.moe_workspace_layout(2, 8, 256, 7168, 2048, "fp8")["y"] != 2 ** 64 - 1


@pytest.mark.parametrize("args,code", [
    ((-1, 2, 8, 128, 64), -1), ((4, 0, 8, 128, 64), -1), ((4, 17, 8, 128, 64), -1),
    ((4, 2, 0, 128, 64), -1), ((4, 2, 512, 128, 64), -1), ((4, 2, 8, 0, 64), -1),
    ((4, 2, 8, 96, 64), -2), ((4, 2, 8, 128, 100), -2), ((8193, 8, 8, 128, 64), -2),
    ((4, 2, 8, 128 * 1024, 64), -2),
])
def test_layout_rejects_bad_shapes(m, args, code):
    lib = m._lib
    L = m.RoutingLayout()
    assert lib.moe_routing_layout(*args, 0, ctypes.byref(L)) == code
    W = m.WorkspaceLayout()
    assert lib.moe_workspace_layout(*args, 0, ctypes.byref(W)) == code
    assert lib.moe_routing_layout(4, 2, 8, 128, 64, 7, ctypes.byref(L)) == -1


def describe(m, addr, E, rows, cols, dtype):
    """Descriptor of (fake) packed bytes at addr, made by the library on the host."""
    d = m.PackedWeightsDesc()
    rc = m._lib.moe_describe_packed_weights(ctypes.c_void_p(addr), E, rows, cols, m.DTYPES[dtype],
                                            ctypes.byref(d))
    assert rc == 0
    return d


def test_calls_reject_bad_arguments_without_launching(m):
    lib = m._lib
    fake = ctypes.c_void_p(4096)            # never dereferenced: every call fails its checks
    odd = ctypes.c_void_p(4097)
    w1 = ctypes.byref(describe(m, 4096, 8, 128, 128, "bf16"))   # E=8, 2I=128, H=128
    w2 = ctypes.byref(describe(m, 4096, 8, 128, 64, "bf16"))    # H=128, I=64
    f1 = ctypes.byref(describe(m, 4096, 8, 128, 128, "fp8"))
    f2 = ctypes.byref(describe(m, 4096, 8, 128, 64, "fp8"))
    L = m.moe_routing_layout(4, 2, 8, 128, 64, "bf16")
    n = L["total_bytes"]
    # null ids / routing
    assert lib.moe_build_routing_bf16(None, 4, 2, 8, 128, 64, fake, n, None) == -1
    assert lib.moe_build_routing_fp8(fake, 4, 2, 8, 128, 64, None, n, None) == -1
    # routing buffer too small
    assert lib.moe_build_routing_bf16(fake, 4, 2, 8, 128, 64, fake, n - 1, None) == -3
    # misaligned routing buffer
    assert lib.moe_build_routing_bf16(fake, 4, 2, 8, 128, 64, odd, n, None) == -1
    # bad shape wins over everything
    assert lib.moe_build_routing_bf16(fake, 4, 2, 8, 100, 64, fake, n, None) == -2
    # T == 0 is a no-op success, even with null pointers
    assert lib.moe_build_routing_bf16(None, 0, 2, 8, 128, 64, None, 0, None) == 0
    assert lib.moe_forward_bf16(None, None, None, None, None, 0, 2, 8, 128, 64, None, 0, None, None) == 0
    W = m.moe_workspace_layout(4, 2, 8, 128, 64, "bf16")["total_bytes"]
    args = [fake, fake, fake, w1, w2, 4, 2, 8, 128, 64, fake, W, fake, None]
    a = list(args)
    a[0] = None
    assert lib.moe_forward_bf16(*a) == -1                 # null x
    a = list(args)
    a[11] = W - 1
    assert lib.moe_forward_bf16(*a) == -3                 # workspace too small
    a = list(args)
    a[10] = ctypes.c_void_p(4096 + 16)
    assert lib.moe_forward_bf16(*a) == -1                 # workspace not 256-byte aligned
    Wf = m.moe_workspace_layout(4, 2, 8, 128, 64, "fp8")["total_bytes"]
    fargs = [fake, fake, fake, f1, fake, f2, fake, 4, 2, 8, 128, 64, fake, Wf, fake, None]
    a = list(fargs)
    a[4] = None
    assert lib.moe_forward_fp8(*a) == -1                  # null w1_scale
    a = list(fargs)
    a[13] = Wf - 1
    assert lib.moe_forward_fp8(*a) == -3


def test_expert_limit_is_nine_bit_keys(m):
    # 511 experts plus the dropped bucket: the routing sort's keys fit nine bits
    L = m.RoutingLayout()
    assert m._lib.moe_routing_layout(4, 2, 511, 128, 64, 0, ctypes.byref(L)) == 0
    assert m._lib.moe_routing_layout(4, 2, 257, 128, 64, 1, ctypes.byref(L)) == 0


@pytest.mark.parametrize("args,code", [
    ((-1, 8, 2, 1, 0), -1),     # T < 0
    ((4, 0, 1, 1, 0), -1),      # E < 1
    ((4, 8, 0, 1, 0), -1),      # k < 1
    ((4, 8, 9, 1, 0), -1),      # k > E
    ((4, 8, 2, 2, 0), -1),      # renormalize not 0/1
    ((4, 8, 2, 1, -1), -1),     # n_shared < 0
    ((4, 257, 8, 1, 0), -2),    # E beyond one wave's 256 logits
    ((4, 64, 16, 1, 1), -2),    # k + n_shared > 16
    ((4, 256, 8, 1, 256), -2),  # k + n_shared > 16 (and E + n_shared > 511)
])
def test_router_rejects_bad_arguments(m, args, code):
    lib = m._lib
    fake = ctypes.c_void_p(4096)
    T, E, k, renorm, ns = args
    assert lib.moe_router_topk(fake, T, E, k, renorm, ns, fake, fake, None) == code


def test_router_pointer_checks(m):
    lib = m._lib
    fake = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4098)
    assert lib.moe_router_topk(None, 4, 8, 2, 1, 0, fake, fake, None) == -1
    assert lib.moe_router_topk(fake, 4, 8, 2, 1, 0, None, fake, None) == -1
    assert lib.moe_router_topk(fake, 4, 8, 2, 1, 0, fake, None, None) == -1
    assert lib.moe_router_topk(odd, 4, 8, 2, 1, 0, fake, fake, None) == -1
    assert lib.moe_router_topk(fake, 4, 8, 2, 1, 0, fake, odd, None) == -1
    # T == 0: no launch, null pointers accepted
    assert lib.moe_router_topk(None, 0, 8, 2, 1, 1, None, None, None) == 0


def test_stage_event_hook_argument_checks(m):
    lib = m._lib
    assert lib.moe_set_stage_events(None, 0) == 0
    arr = (ctypes.c_void_p * 4)(*[1, 2, 3, 4])
    assert lib.moe_set_stage_events(arr, 4) == -1
    arr = (ctypes.c_void_p * 10)(*([1] * 9 + [0]))
    assert lib.moe_set_stage_events(arr, 10) == -1      # half a pair
    arr = (ctypes.c_void_p * 10)(*([0] * 10))
    assert lib.moe_set_stage_events(arr, 10) == -1      # nothing to record
    arr = (ctypes.c_void_p * 10)(*([0, 0, 1, 2] + [0] * 6))
    assert lib.moe_set_stage_events(arr, 10) == 0       # gate-up only
    assert lib.moe_set_stage_events(None, 0) == 0


def test_forward_takes_only_packed_weight_descriptors(m):
    """Row-major weights cannot reach the kernels: the forward calls take
    descriptors that moe_pack_weights (or moe_describe_packed_weights) made
    for the call's dtype, expert count and matrix shapes, and reject every
    other one with MOE_ERR_INVALID_ARG before launching anything."""
    lib = m._lib
    fake = ctypes.c_void_p(4096)
    E, H, I, T, k = 8, 128, 64, 4, 2
    W = m.moe_workspace_layout(T, k, E, H, I, "bf16")["total_bytes"]
    good1 = describe(m, 1 << 20, E, 2 * I, H, "bf16")
    good2 = describe(m, 1 << 21, E, H, I, "bf16")

    def fwd(d1, d2, ws=W):
        return lib.moe_forward_bf16(fake, fake, fake, d1, d2, T, k, E, H, I, fake, ws, fake, None)

    # with good descriptors the call gets past them (and then fails on the
    # too-small workspace, so that nothing is launched)
    assert fwd(ctypes.byref(good1), ctypes.byref(good2), W - 1) == -3
    # row-major weights: a descriptor not made by the library
    raw = m.PackedWeightsDesc(data=1 << 20, dtype=0, experts=E, rows=2 * I, cols=H, check=0)
    assert fwd(ctypes.byref(raw), ctypes.byref(good2)) == -1
    assert fwd(None, ctypes.byref(good2)) == -1
    assert fwd(ctypes.byref(m.PackedWeightsDesc()), ctypes.byref(good2)) == -1
    # a library descriptor with any field changed afterwards
    for field, val in (("data", 1 << 22), ("dtype", 1), ("experts", 16), ("rows", 256), ("cols", 256)):
        d = m.PackedWeightsDesc.from_buffer_copy(good1)
        setattr(d, field, val)
        assert fwd(ctypes.byref(d), ctypes.byref(good2)) == -1, field
    # the right kind of descriptor in the wrong place or for another call
    assert fwd(ctypes.byref(good2), ctypes.byref(good1)) == -1          # W1 and W2 swapped
    fp8_1 = describe(m, 1 << 20, E, 2 * I, H, "fp8")
    assert fwd(ctypes.byref(fp8_1), ctypes.byref(good2)) == -1          # packed for another dtype
    other = describe(m, 1 << 20, 16, 2 * I, H, "bf16")
    assert fwd(ctypes.byref(other), ctypes.byref(good2)) == -1          # another expert count
    # describe checks the same size rules as the pack
    d = m.PackedWeightsDesc()
    assert lib.moe_describe_packed_weights(ctypes.c_void_p(4096), E, 24, H, 0, ctypes.byref(d)) == -2
    assert lib.moe_describe_packed_weights(ctypes.c_void_p(4100), E, 32, H, 0, ctypes.byref(d)) == -1
    assert lib.moe_describe_packed_weights(ctypes.c_void_p(4096), E, 32, H, 0, None) == -1


def test_binding_refuses_unpacked_tensors(m):
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    w = torch.zeros(4, 2, dtype=torch.float32)
    raw1 = torch.zeros(8, 128, 128, dtype=torch.bfloat16)
    raw2 = torch.zeros(8, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="PackedWeight"):
        m.moe_forward_bf16(x, w, torch.zeros(16, dtype=torch.uint8), raw1, raw2,
                           torch.zeros(256, dtype=torch.uint8), torch.zeros(4, 128, dtype=torch.bfloat16))


def test_measurement_aids_reject_bad_arguments(m):
    """moe_stream_read and moe_tile_copy_read check their arguments on the host
    before anything else (no device query, no launch)."""
    lib = m._lib
    fake = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4097)
    assert lib.moe_stream_read(None, 1024, fake, 8, None) == -1          # null buffer
    assert lib.moe_stream_read(fake, 1000, fake, 8, None) == -1          # bytes not a multiple of 16
    assert lib.moe_stream_read(fake, 1024, fake, 0, None) == -1          # no sink words
    for pattern in (-1, 3):
        assert lib.moe_tile_copy_read(pattern, fake, 1 << 24, 8192, 1, fake, 256, None) == -1
    assert lib.moe_tile_copy_read(0, None, 1 << 24, 8192, 1, fake, 256, None) == -1     # null buffer
    assert lib.moe_tile_copy_read(0, odd, 1 << 24, 8192, 1, fake, 256, None) == -1      # misaligned buffer
    assert lib.moe_tile_copy_read(1, fake, 1 << 24, 7168, 1, fake, 256, None) == -1     # rows not 2 KiB multiples
    assert lib.moe_tile_copy_read(2, fake, 1 << 24, 8192, -1, fake, 256, None) == -1    # negative passes
    assert lib.moe_tile_copy_read(2, fake, 1 << 24, 8192, 1, None, 256, None) == -1     # null sink
