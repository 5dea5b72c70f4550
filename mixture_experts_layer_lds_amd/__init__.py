"""Python binding of libmoe.so, the MI355X fused Mixture-of-Experts layer.

The binding only marshals arguments: every step of the layer runs in the
HIP kernels of libmoe.so (see include/moe.h).  PyTorch provides device
memory and streams.  There is no fallback path: if the library is missing
or cannot be loaded, importing this module raises.

Functions carry the C names:

    moe_pack_weights(w, dtype)                          -> PackedWeight (packed copy + descriptor, one-time)
    moe_routing_layout(T, k, E, H, I, dtype)            -> dict (host only)
    moe_workspace_layout(T, k, E, H, I, dtype)          -> dict (host only)
    moe_router_split_weights(w)                         -> split fp32 router weight pair (one-time)
    moe_router_gemm(x, w_pair, N)                       -> fp32 router scores
    moe_router_gemm_topk(x, w_pair, E, k, ...)          -> (topk_ids, topk_w[, scores])
    moe_router_topk(logits, k, renormalize, n_shared)    -> (topk_ids, topk_w)
    moe_build_routing_bf16(topk_ids, E, H, I, routing)  -> None
    moe_build_routing_fp8(topk_ids, E, H, I, routing)   -> None
    moe_forward_bf16(x, topk_w, routing, w1, w2, workspace, out) -> out
    moe_forward_fp8(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out) -> out
    moe_build_routing_mxfp8 / moe_forward_mxfp8 (as the fp8 pair, e8m0 block-scale codes)
    moe_build_routing_int8 / moe_forward_int8   (as the fp8 pair, int8 codes)
    moe_build_routing_int4 / moe_forward_int4   (int4 weights + group scales, bf16 activations)
    moe_build_routing_fp8_block / moe_forward_fp8_block (128x128 weight blocks, 1x128 token groups)
    moe_build_routing_int8_w8a16 / moe_forward_int8_w8a16 (int8 weights + row scales, bf16 activations)

plus allocation helpers (alloc_routing, alloc_workspace), pack_weights() for a
whole weight dict, and a convenience moe_layer() that runs routing + forward
with freshly allocated buffers.  The forward calls take W1/W2 packed by
moe_pack_weights (a one-time byte permutation into MFMA-fragment order).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that libmoe.so binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_DTYPE_BF16 = 0
MOE_DTYPE_FP8_W8A8 = 1
MOE_DTYPE_MXFP8 = 2
MOE_DTYPE_INT8_W8A8 = 3
MOE_DTYPE_INT4_W4A16 = 4
MOE_DTYPE_FP8_BLOCK = 5
MOE_DTYPE_INT8_W8A16 = 6
DTYPES = {"bf16": MOE_DTYPE_BF16, "fp8": MOE_DTYPE_FP8_W8A8, "mxfp8": MOE_DTYPE_MXFP8,
          "int8": MOE_DTYPE_INT8_W8A8, "int4": MOE_DTYPE_INT4_W4A16, "fp8b": MOE_DTYPE_FP8_BLOCK,
          "int8w": MOE_DTYPE_INT8_W8A16}


class MoeError(RuntimeError):
    def __init__(self, name, status):
        self.status = status
        super().__init__(f"{name} failed: {status} ({status_string(status)})")


class RoutingLayout(ctypes.Structure):
    _fields_ = [("header", ctypes.c_size_t), ("expert_offsets", ctypes.c_size_t),
                ("sorted_pairs", ctypes.c_size_t), ("pair_pos", ctypes.c_size_t),
                ("tasks", ctypes.c_size_t), ("scratch", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t),
                ("block_m", ctypes.c_int32), ("max_tasks", ctypes.c_int32)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_size_t), ("x_scale", ctypes.c_size_t),
                ("x_scale_rows", ctypes.c_size_t), ("g", ctypes.c_size_t),
                ("h", ctypes.c_size_t), ("h_scale", ctypes.c_size_t), ("y", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t), ("split_k1", ctypes.c_int32),
                ("split_k2", ctypes.c_int32), ("tiling", ctypes.c_int32)]


class PackedWeightsDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("check", ctypes.c_uint64)]


class PackedWeight:
    """A weight tensor packed by moe_pack_weights together with the
    library's descriptor of it, which the forward calls take.  `tensor` is
    the packed device tensor (same shape and dtype as the row-major one)."""

    def __init__(self, tensor, desc):
        self.tensor = tensor
        self.desc = desc

    shape = property(lambda self: self.tensor.shape)
    dtype = property(lambda self: self.tensor.dtype)
    device = property(lambda self: self.tensor.device)

    def clone(self):
        """A device copy of the packed bytes, with its own descriptor."""
        return moe_describe_packed_weights(self.tensor.clone(), self.desc.dtype)

    def numel(self):
        return self.tensor.numel()

    def element_size(self):
        return self.tensor.element_size()


EXPORTS = ("moe_status_string", "moe_pack_weights", "moe_describe_packed_weights", "moe_routing_layout",
           "moe_workspace_layout",
           "moe_router_topk", "moe_router_pair_bytes", "moe_router_split_weights",
           "moe_router_workspace_bytes", "moe_router_gemm", "moe_router_gemm_topk",
           "moe_build_routing_bf16", "moe_build_routing_fp8", "moe_build_routing_mxfp8",
           "moe_build_routing_int8", "moe_build_routing_int4", "moe_forward_bf16",
           "moe_forward_fp8", "moe_forward_mxfp8", "moe_forward_int8", "moe_forward_int4",
           "moe_build_routing_fp8_block", "moe_forward_fp8_block",
           "moe_build_routing_int8_w8a16", "moe_forward_int8_w8a16", "moe_set_stage_events", "moe_device_cu_count",
           "moe_stream_read", "moe_forward_fp8_noalloc", "moe_route_forward_bf16", "moe_route_forward_fp8",
           "moe_route_forward_int8", "moe_route_forward_fp8_block", "moe_route_forward_mxfp8",
           "moe_route_forward_int4", "moe_route_forward_int8_w8a16", "moe_tile_copy_read")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mixture_experts_layer_lds_amd/build.py` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    i, P, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [i]
    L.moe_pack_weights.restype = i
    L.moe_pack_weights.argtypes = [P, i, i, i, i, P, ctypes.POINTER(PackedWeightsDesc), P]
    L.moe_describe_packed_weights.restype = i
    L.moe_describe_packed_weights.argtypes = [P, i, i, i, i, ctypes.POINTER(PackedWeightsDesc)]
    L.moe_routing_layout.restype = i
    L.moe_routing_layout.argtypes = [i, i, i, i, i, i, ctypes.POINTER(RoutingLayout)]
    L.moe_workspace_layout.restype = i
    L.moe_workspace_layout.argtypes = [i, i, i, i, i, i, ctypes.POINTER(WorkspaceLayout)]
    for n in ("moe_build_routing_bf16", "moe_build_routing_fp8"):
        f = getattr(L, n)
        f.restype = i
        f.argtypes = [P, i, i, i, i, i, P, sz, P]
    L.moe_router_topk.restype = i
    L.moe_router_pair_bytes.restype = i
    L.moe_router_pair_bytes.argtypes = [i, i, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_router_split_weights.restype = i
    L.moe_router_split_weights.argtypes = [P, i, i, P, sz, P]
    L.moe_router_workspace_bytes.restype = i
    L.moe_router_workspace_bytes.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_router_gemm.restype = i
    L.moe_router_gemm.argtypes = [P, P, i, i, i, P, sz, P, P]
    L.moe_router_gemm_topk.restype = i
    L.moe_router_gemm_topk.argtypes = [P, P, i, i, i, i, i, i, P, sz, P, P, P, P]
    L.moe_router_topk.argtypes = [P, i, i, i, i, i, P, P, P]
    L.moe_forward_bf16.restype = i
    D = ctypes.POINTER(PackedWeightsDesc)
    L.moe_forward_bf16.argtypes = [P, P, P, D, D, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_fp8.restype = i
    L.moe_forward_fp8.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_mxfp8.restype = i
    L.moe_forward_mxfp8.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_fp8_block.restype = i
    L.moe_forward_fp8_block.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_int4.restype = i
    L.moe_forward_int4.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_int8.restype = i
    L.moe_forward_int8.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_forward_int8_w8a16.restype = i
    L.moe_forward_int8_w8a16.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    L.moe_set_stage_events.restype = i
    L.moe_set_stage_events.argtypes = [ctypes.POINTER(P), i]
    L.moe_device_cu_count.restype = i
    L.moe_device_cu_count.argtypes = []
    L.moe_forward_fp8_noalloc.restype = i
    L.moe_forward_fp8_noalloc.argtypes = [P, P, P, D, P, D, P, i, i, i, i, i, P, P]
    L.moe_stream_read.restype = i
    L.moe_stream_read.argtypes = [P, sz, P, sz, P]
    L.moe_tile_copy_read.restype = i
    L.moe_tile_copy_read.argtypes = [i, P, sz, i, i, P, sz, P]
    L.moe_route_forward_bf16.restype = i
    L.moe_route_forward_bf16.argtypes = [P, P, P, P, sz, D, D, i, i, i, i, i, P, sz, P, P]
    L.moe_route_forward_fp8.restype = i
    L.moe_route_forward_fp8.argtypes = [P, P, P, P, sz, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    for f in (L.moe_route_forward_int8, L.moe_route_forward_fp8_block, L.moe_route_forward_mxfp8,
              L.moe_route_forward_int4, L.moe_route_forward_int8_w8a16):
        f.restype = i
        f.argtypes = [P, P, P, P, sz, D, P, D, P, i, i, i, i, i, P, sz, P, P]
    return L


_lib = _load()


def status_string(status: int) -> str:
    return _lib.moe_status_string(int(status)).decode()


def _check(name, rc):
    if rc != 0:
        raise MoeError(name, rc)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def moe_pack_weights(w, dtype="bf16", out=None, stream=None):
    """Packed copy of a row-major [E][rows][cols] weight tensor (bf16; uint8
    e4m3 codes for dtype "fp8", "fp8b" and "mxfp8"; int8 codes for "int8"; uint8 bytes
    of two int4 codes for "int4", whose K length is twice the byte count), as a
    PackedWeight (the packed tensor and its descriptor for the forward calls)."""
    want = {"bf16": torch.bfloat16, "int8": torch.int8, "int8w": torch.int8}.get(dtype, torch.uint8)
    if w.dtype != want or w.dim() != 3 or not w.is_contiguous():
        raise ValueError(f"moe_pack_weights: expected contiguous {want} [E][rows][cols]")
    E, rows, cols = w.shape
    if dtype == "int4":
        cols *= 2
    if out is None:
        out = torch.empty_like(w)
    desc = PackedWeightsDesc()
    _check("moe_pack_weights", _lib.moe_pack_weights(_ptr(w), E, rows, cols, DTYPES[dtype],
                                                     _ptr(out), ctypes.byref(desc), _stream(stream)))
    return PackedWeight(out, desc)


def moe_describe_packed_weights(packed, dtype):
    """PackedWeight for a tensor that already holds packed bytes (a copy of a
    packed tensor, or packed weights loaded from storage); dtype is a name of
    DTYPES or its code."""
    code = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    E, rows, cols = packed.shape
    if code == MOE_DTYPE_INT4_W4A16:
        cols *= 2
    desc = PackedWeightsDesc()
    _check("moe_describe_packed_weights",
           _lib.moe_describe_packed_weights(_ptr(packed), E, rows, cols, code, ctypes.byref(desc)))
    return PackedWeight(packed, desc)


def pack_weights(weights, dtype="bf16", stream=None):
    """Weight dict with w1/w2 packed for the forward calls (scales copied by reference)."""
    out = dict(weights)
    out["w1"] = moe_pack_weights(weights["w1"], dtype, stream=stream)
    out["w2"] = moe_pack_weights(weights["w2"], dtype, stream=stream)
    return out


def moe_routing_layout(T, k, E, H, I, dtype="bf16") -> dict:
    L = RoutingLayout()
    _check("moe_routing_layout", _lib.moe_routing_layout(T, k, E, H, I, DTYPES[dtype], ctypes.byref(L)))
    return {f: getattr(L, f) for f, _ in RoutingLayout._fields_}


def moe_workspace_layout(T, k, E, H, I, dtype="bf16") -> dict:
    W = WorkspaceLayout()
    _check("moe_workspace_layout", _lib.moe_workspace_layout(T, k, E, H, I, DTYPES[dtype], ctypes.byref(W)))
    return {f: getattr(W, f) for f, _ in WorkspaceLayout._fields_}


def alloc_routing(T, k, E, H, I, dtype="bf16", device="cuda"):
    n = moe_routing_layout(T, k, E, H, I, dtype)["total_bytes"]
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def alloc_workspace(T, k, E, H, I, dtype="bf16", device="cuda"):
    n = moe_workspace_layout(T, k, E, H, I, dtype)["total_bytes"]
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_router_topk(logits, k, renormalize=True, n_shared=0, topk_ids=None, topk_w=None,
                    stream=None):
    """Router top-k of fp32 logits [T][E] into (topk_ids int32, topk_w fp32),
    both [T][k + n_shared]; the last n_shared columns are the fused shared
    experts (ids E.., weight 1)."""
    if logits.dtype != torch.float32 or logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous fp32 [T][E] tensor")
    T, E = logits.shape
    ncol = k + n_shared
    if topk_ids is None:
        topk_ids = torch.empty(T, ncol, dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty(T, ncol, dtype=torch.float32, device=logits.device)
    _check_tensor("topk_ids", topk_ids, torch.int32, (T, ncol))
    _check_tensor("topk_w", topk_w, torch.float32, (T, ncol))
    _check("moe_router_topk", _lib.moe_router_topk(
        _ptr(logits), T, E, k, int(bool(renormalize)), n_shared, _ptr(topk_ids), _ptr(topk_w),
        _stream(stream)))
    return topk_ids, topk_w


def moe_router_pair_bytes(N, K) -> int:
    n = ctypes.c_size_t()
    _check("moe_router_pair_bytes", _lib.moe_router_pair_bytes(N, K, ctypes.byref(n)))
    return n.value


def moe_router_workspace_bytes(T, N, K) -> int:
    n = ctypes.c_size_t()
    _check("moe_router_workspace_bytes", _lib.moe_router_workspace_bytes(T, N, K, ctypes.byref(n)))
    return n.value


def moe_router_split_weights(w, out=None, stream=None):
    """Split pair (uint8 tensor of moe_router_pair_bytes) of fp32 router weights [N][K]."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous fp32 [N][K] tensor")
    N, K = w.shape
    nbytes = moe_router_pair_bytes(N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check("moe_router_split_weights", _lib.moe_router_split_weights(
        _ptr(w), N, K, _ptr(out), out.numel() * out.element_size(), _stream(stream)))
    return out


def _router_ws(T, N, K, workspace, device):
    n = moe_router_workspace_bytes(T, N, K)
    if workspace is None:
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
    return workspace


def moe_router_gemm(x, w_pair, N, scores=None, workspace=None, stream=None):
    """fp32 scores [T][N] of bf16 x [T][K] against a split router weight pair."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T][K] tensor")
    T, K = x.shape
    workspace = _router_ws(T, N, K, workspace, x.device)
    if scores is None:
        scores = torch.empty(T, N, dtype=torch.float32, device=x.device)
    _check_tensor("scores", scores, torch.float32, (T, N))
    _check("moe_router_gemm", _lib.moe_router_gemm(
        _ptr(x), _ptr(w_pair), T, N, K, _ptr(workspace), workspace.numel(), _ptr(scores),
        _stream(stream)))
    return scores


def moe_router_gemm_topk(x, w_pair, E, k, renormalize=True, n_shared=0, want_scores=False,
                         topk_ids=None, topk_w=None, scores=None, workspace=None, stream=None):
    """Router GEMM + top-k: (topk_ids, topk_w) [T][k + n_shared], plus the fp32
    scores [T][E] when want_scores (or a scores tensor is given)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [T][K] tensor")
    T, K = x.shape
    ncol = k + n_shared
    workspace = _router_ws(T, E, K, workspace, x.device)
    if topk_ids is None:
        topk_ids = torch.empty(T, ncol, dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty(T, ncol, dtype=torch.float32, device=x.device)
    if scores is None and want_scores:
        scores = torch.empty(T, E, dtype=torch.float32, device=x.device)
    if scores is not None:
        _check_tensor("scores", scores, torch.float32, (T, E))
    _check_tensor("topk_ids", topk_ids, torch.int32, (T, ncol))
    _check_tensor("topk_w", topk_w, torch.float32, (T, ncol))
    _check("moe_router_gemm_topk", _lib.moe_router_gemm_topk(
        _ptr(x), _ptr(w_pair), T, E, K, k, int(bool(renormalize)), n_shared, _ptr(workspace),
        workspace.numel(), _ptr(scores), _ptr(topk_ids), _ptr(topk_w), _stream(stream)))
    return (topk_ids, topk_w, scores) if scores is not None else (topk_ids, topk_w)


def _shape_tk(topk_ids):
    if topk_ids.dim() != 2 or topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous int32 [T][k] tensor")
    return topk_ids.shape


def _build_routing(fn, name, topk_ids, E, H, I, routing, stream):
    T, k = _shape_tk(topk_ids)
    _check(name, fn(_ptr(topk_ids), T, k, E, H, I, _ptr(routing), routing.numel(), _stream(stream)))


def moe_build_routing_bf16(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_bf16, "moe_build_routing_bf16", topk_ids, E, H, I, routing, stream)


def moe_build_routing_fp8(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_fp8, "moe_build_routing_fp8", topk_ids, E, H, I, routing, stream)


def moe_build_routing_mxfp8(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_mxfp8, "moe_build_routing_mxfp8", topk_ids, E, H, I, routing,
                   stream)


def moe_build_routing_int8(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_int8, "moe_build_routing_int8", topk_ids, E, H, I, routing,
                   stream)


def moe_build_routing_int4(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_int4, "moe_build_routing_int4", topk_ids, E, H, I, routing,
                   stream)


def moe_build_routing_int8_w8a16(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_int8_w8a16, "moe_build_routing_int8_w8a16", topk_ids, E, H, I,
                   routing, stream)


def moe_build_routing_fp8_block(topk_ids, E, H, I, routing, stream=None):
    _build_routing(_lib.moe_build_routing_fp8_block, "moe_build_routing_fp8_block", topk_ids, E, H, I,
                   routing, stream)


def build_routing(topk_ids, E, H, I, routing, dtype="bf16", stream=None):
    """The routing build of the given dtype's forward."""
    {"bf16": moe_build_routing_bf16, "fp8": moe_build_routing_fp8,
     "mxfp8": moe_build_routing_mxfp8, "int8": moe_build_routing_int8,
     "int4": moe_build_routing_int4, "fp8b": moe_build_routing_fp8_block,
     "int8w": moe_build_routing_int8_w8a16}[dtype](
        topk_ids, E, H, I, routing, stream)


def _check_tensor(name, t, dtype, shape):
    if isinstance(t, PackedWeight):
        t = t.tensor
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _desc(name, w):
    """The library descriptor of a packed weight (forward calls take nothing else)."""
    if not isinstance(w, PackedWeight):
        raise TypeError(f"{name}: expected a PackedWeight from moe_pack_weights / pack_weights, "
                        f"got {type(w).__name__} (the forward calls take packed weights only)")
    return ctypes.byref(w.desc)


def moe_forward_bf16(x, topk_w, routing, w1, w2, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.bfloat16, (E, 2 * I, H))
    _check_tensor("w2", w2, torch.bfloat16, (E, H, I))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_bf16", _lib.moe_forward_bf16(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _desc("w2", w2), T, k, E, H, I,
        _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_forward_fp8(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I))
    _check_tensor("w2", w2, torch.uint8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_fp8", _lib.moe_forward_fp8(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_route_forward_bf16(topk_ids, x, topk_w, routing, w1, w2, workspace, out, stream=None):
    """moe_build_routing_bf16 + moe_forward_bf16 in one call (one token:
    the routing build runs inside the gate-up launch)."""
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("topk_ids", topk_ids, torch.int32, (T, k))
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.bfloat16, (E, 2 * I, H))
    _check_tensor("w2", w2, torch.bfloat16, (E, H, I))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_route_forward_bf16", _lib.moe_route_forward_bf16(
        _ptr(topk_ids), _ptr(x), _ptr(topk_w), _ptr(routing), routing.numel(), _desc("w1", w1), _desc("w2", w2),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_route_forward_fp8(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                          stream=None):
    """moe_build_routing_fp8 + moe_forward_fp8 in one call (one token: the
    routing build runs inside the x-quantisation launch)."""
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("topk_ids", topk_ids, torch.int32, (T, k))
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I))
    _check_tensor("w2", w2, torch.uint8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_route_forward_fp8", _lib.moe_route_forward_fp8(
        _ptr(topk_ids), _ptr(x), _ptr(topk_w), _ptr(routing), routing.numel(), _desc("w1", w1), _ptr(w1_scale),
        _desc("w2", w2), _ptr(w2_scale), T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out),
        _stream(stream)))
    return out


def _route_forward_q(fn, name, topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                     stream, scale_dtype, scale_shape):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("topk_ids", topk_ids, torch.int32, (T, k))
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1_scale", w1_scale, scale_dtype, scale_shape(E, 2 * I, H))
    _check_tensor("w2_scale", w2_scale, scale_dtype, scale_shape(E, H, I))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check(name, fn(_ptr(topk_ids), _ptr(x), _ptr(topk_w), _ptr(routing), routing.numel(), _desc("w1", w1),
                    _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale), T, k, E, H, I, _ptr(workspace),
                    workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_route_forward_int8(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                           stream=None):
    """moe_build_routing_int8 + moe_forward_int8 in one call."""
    return _route_forward_q(_lib.moe_route_forward_int8, "moe_route_forward_int8", topk_ids, x, topk_w, routing,
                            w1, w1_scale, w2, w2_scale, workspace, out, stream, torch.float32,
                            lambda E, N, K: (E, N))


def moe_route_forward_fp8_block(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                                stream=None):
    """moe_build_routing_fp8_block + moe_forward_fp8_block in one call."""
    return _route_forward_q(_lib.moe_route_forward_fp8_block, "moe_route_forward_fp8_block", topk_ids, x, topk_w,
                            routing, w1, w1_scale, w2, w2_scale, workspace, out, stream, torch.float32,
                            lambda E, N, K: (E, N // 128, K // 128))


def moe_route_forward_mxfp8(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                            stream=None):
    """moe_build_routing_mxfp8 + moe_forward_mxfp8 in one call."""
    return _route_forward_q(_lib.moe_route_forward_mxfp8, "moe_route_forward_mxfp8", topk_ids, x, topk_w,
                            routing, w1, w1_scale, w2, w2_scale, workspace, out, stream, torch.uint8,
                            lambda E, N, K: (E, N, K // 32))


def moe_route_forward_int4(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                           stream=None):
    """moe_build_routing_int4 + moe_forward_int4 in one call."""
    return _route_forward_q(_lib.moe_route_forward_int4, "moe_route_forward_int4", topk_ids, x, topk_w, routing,
                            w1, w1_scale, w2, w2_scale, workspace, out, stream, torch.float32,
                            lambda E, N, K: (E, N, K // 128))


def moe_route_forward_int8_w8a16(topk_ids, x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out,
                                 stream=None):
    """moe_build_routing_int8_w8a16 + moe_forward_int8_w8a16 in one call."""
    return _route_forward_q(_lib.moe_route_forward_int8_w8a16, "moe_route_forward_int8_w8a16", topk_ids, x,
                            topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream, torch.float32,
                            lambda E, N, K: (E, N))


def route_forward(topk_ids, x, topk_w, routing, weights, workspace, out, dtype="bf16", stream=None):
    """Routing build + forward in one library call, any dtype."""
    W = weights
    if dtype == "bf16":
        return moe_route_forward_bf16(topk_ids, x, topk_w, routing, W["w1"], W["w2"], workspace, out, stream)
    fn = {"fp8": moe_route_forward_fp8, "int8": moe_route_forward_int8, "fp8b": moe_route_forward_fp8_block,
          "mxfp8": moe_route_forward_mxfp8, "int4": moe_route_forward_int4,
          "int8w": moe_route_forward_int8_w8a16}[dtype]
    return fn(topk_ids, x, topk_w, routing, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"], workspace, out, stream)


STATIC_WORKSPACE_BYTES = 64 << 20


def moe_forward_fp8_noalloc(x, topk_w, routing, w1, w1_scale, w2, w2_scale, out, stream=None):
    """moe_forward_fp8 on the library's fixed per-GPU workspace (no workspace
    argument, nothing allocated); sizes whose workspace exceeds
    STATIC_WORKSPACE_BYTES raise MoeError (MOE_ERR_BUFFER_TOO_SMALL)."""
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I))
    _check_tensor("w2", w2, torch.uint8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_fp8_noalloc", _lib.moe_forward_fp8_noalloc(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2),
        _ptr(w2_scale), T, k, E, H, I, _ptr(out), _stream(stream)))
    return out


def moe_forward_mxfp8(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.uint8, (E, 2 * I, H // 32))
    _check_tensor("w2", w2, torch.uint8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.uint8, (E, H, I // 32))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_mxfp8", _lib.moe_forward_mxfp8(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_forward_fp8_block(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I // 128, H // 128))
    _check_tensor("w2", w2, torch.uint8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H // 128, I // 128))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_fp8_block", _lib.moe_forward_fp8_block(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_forward_int8_w8a16(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.int8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I))
    _check_tensor("w2", w2, torch.int8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_int8_w8a16", _lib.moe_forward_int8_w8a16(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_forward_int4(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.uint8, (E, 2 * I, H // 2))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I, H // 128))
    _check_tensor("w2", w2, torch.uint8, (E, H, I // 2))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H, I // 128))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_int4", _lib.moe_forward_int4(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_forward_int8(x, topk_w, routing, w1, w1_scale, w2, w2_scale, workspace, out, stream=None):
    T, H = x.shape
    k = topk_w.shape[1]
    E, I2, _ = w1.shape
    I = I2 // 2
    _check_tensor("x", x, torch.bfloat16, (T, H))
    _check_tensor("topk_w", topk_w, torch.float32, (T, k))
    _check_tensor("w1", w1, torch.int8, (E, 2 * I, H))
    _check_tensor("w1_scale", w1_scale, torch.float32, (E, 2 * I))
    _check_tensor("w2", w2, torch.int8, (E, H, I))
    _check_tensor("w2_scale", w2_scale, torch.float32, (E, H))
    _check_tensor("out", out, torch.bfloat16, (T, H))
    _check("moe_forward_int8", _lib.moe_forward_int8(
        _ptr(x), _ptr(topk_w), _ptr(routing), _desc("w1", w1), _ptr(w1_scale), _desc("w2", w2), _ptr(w2_scale),
        T, k, E, H, I, _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream)))
    return out


def moe_set_stage_events(events):
    """events: list of 10 entries, each a torch.cuda.Event(enable_timing=True)
    (already recorded once) or None (stage s is recorded when entries 2s and
    2s+1 are events), or None to switch the hook off."""
    if events is None:
        _check("moe_set_stage_events", _lib.moe_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event if e is not None else None
                                             for e in events])
    _check("moe_set_stage_events", _lib.moe_set_stage_events(arr, len(events)))


def moe_device_cu_count() -> int:
    n = _lib.moe_device_cu_count()
    if n < 0:
        raise MoeError("moe_device_cu_count", n)
    return n


def moe_stream_read(buf, sink, stream=None):
    """Measurement aid: one streaming read of the device tensor `buf` (its
    whole storage) into per-workgroup words of the uint32/int32 tensor `sink`."""
    nbytes = buf.numel() * buf.element_size()
    _check("moe_stream_read", _lib.moe_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(),
                                                   _stream(stream)))


def moe_tile_copy_read(pattern, buf, row_bytes, reps, sink, stream=None):
    """Measurement aid: token-tile copies into LDS in one of three lane
    patterns (0 contiguous, 1 MFMA lane order, 2 a row per lane quad) from the
    device tensor `buf` (its whole storage); one word per workgroup into the
    uint32/int32 tensor `sink`."""
    nbytes = buf.numel() * buf.element_size()
    _check("moe_tile_copy_read", _lib.moe_tile_copy_read(pattern, _ptr(buf), nbytes, row_bytes, reps, _ptr(sink),
                                                         sink.numel(), _stream(stream)))


def moe_layer(x, topk_ids, topk_w, weights, dtype="bf16", out=None, stream=None):
    """Routing + forward with freshly allocated routing buffer and workspace.

    weights: {"w1", "w2"} (bf16) or {"w1", "w1_scale", "w2", "w2_scale"} (fp8),
    with w1/w2 already packed (pack_weights).  Returns (out, routing, workspace)."""
    T, H = x.shape
    k = topk_ids.shape[1]
    E, I2, _ = weights["w1"].shape
    I = I2 // 2
    routing = alloc_routing(T, k, E, H, I, dtype, x.device)
    ws = alloc_workspace(T, k, E, H, I, dtype, x.device)
    if out is None:
        out = torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
    build_routing(topk_ids, E, H, I, routing, dtype, stream)
    if dtype == "bf16":
        moe_forward_bf16(x, topk_w, routing, weights["w1"], weights["w2"], ws, out, stream)
    else:
        fwd = {"fp8": moe_forward_fp8, "mxfp8": moe_forward_mxfp8, "int8": moe_forward_int8,
               "int4": moe_forward_int4, "fp8b": moe_forward_fp8_block,
               "int8w": moe_forward_int8_w8a16}[dtype]
        fwd(x, topk_w, routing, weights["w1"], weights["w1_scale"], weights["w2"],
            weights["w2_scale"], ws, out, stream)
    return out, routing, ws


def read_routing(routing, T, k, E, H, I, dtype="bf16") -> dict:
    """Copy a routing buffer's parts to host int32 tensors (for tests and tools)."""
    L = moe_routing_layout(T, k, E, H, I, dtype)
    b = routing.cpu()
    P = T * k

    def part(off, n):
        return b[off:off + 4 * n].view(torch.int32).clone()

    hdr = part(L["header"], 16)
    nt = int(hdr[0])
    return {"header": hdr, "num_tasks": nt, "num_dropped": int(hdr[1]), "block_m": int(hdr[2]),
            "offsets": part(L["expert_offsets"], E + 1), "sorted": part(L["sorted_pairs"], P),
            "pos": part(L["pair_pos"], P), "tasks": part(L["tasks"], 4 * nt).view(nt, 4),
            "layout": L}
