"""Helpers shared by the GPU parity tests: run the HIP layer, run the oracle
on the same bytes, compare with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from moe_inputs import WORKLOADS, make_tokens, make_weights

BF16_REL, BF16_ABS = 1e-2, 1e-3      # max|err| <= 1e-2*max|ref| + 1e-3
FP8_REL = 4e-2                        # max|err| <= 4e-2*max|ref|


# One line per full-size parity case, printed at the end of the session
# (conftest.py), so that the counts stay visible when pytest captures output.
SUMMARY = []


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_weights(wl, device="cuda"):
    """Weights of a workload for the GPU path: bf16 (tiny f32 data is rounded
    to bf16) or e4m3 codes + scales."""
    W = make_weights(wl, device=device)
    if wl.dtype == "f32":
        W = {"w1": W["w1"].bfloat16().contiguous(), "w2": W["w2"].bfloat16().contiguous()}
    return W


def path_dtype(wl):
    return wl.dtype if wl.dtype in ("fp8", "fp8b", "mxfp8", "int8", "int4", "int8w") else "bf16"


# One full-size workload's weights at a time: packed on the GPU, row-major
# on the host for the oracle.
_weights_cache = {}


def workload_weights(name):
    if name not in _weights_cache:
        _weights_cache.clear()
        torch.cuda.empty_cache()
        wl = WORKLOADS[name]
        W = device_weights(wl)
        Wc = {k: v.cpu() for k, v in W.items()}
        Wp = __import__("mixture_experts_layer_lds_amd").pack_weights(W, path_dtype(wl))
        del W
        _weights_cache[name] = (Wp, Wc)
    return _weights_cache[name]


def run_gpu(lib, x, ids, w, W, dtype, packed=None):
    """Run routing + forward; W is row-major (packed here) unless `packed` is given."""
    if packed is None:
        packed = lib.pack_weights(W, dtype)
    W = packed
    x = x.cuda().bfloat16().contiguous()
    ids = ids.cuda().contiguous()
    w = w.cuda().float().contiguous()
    out, routing, ws = lib.moe_layer(x, ids, w, W, dtype=dtype)
    torch.cuda.synchronize()
    return out, routing, ws


def oracle_rows(x, ids, w, W, dtype, rows=None, want_quant=False):
    """Oracle output rows (fp64) on the exact bytes the GPU saw."""
    xb = x.detach().cpu().bfloat16().contiguous()
    idc = ids.detach().cpu().contiguous()
    wc = w.detach().cpu().float().contiguous()
    if dtype == "bf16":
        return oracle.forward_bf16(xb, wc, idc, W["w1"].cpu(), W["w2"].cpu(), rows=rows)
    if dtype == "fp8b":
        return oracle.forward_fp8_block(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                                        W["w2_scale"].cpu(), rows=rows, want_quant=want_quant)
    if dtype == "int8w":
        return oracle.forward_w8a16(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                                    W["w2_scale"].cpu(), rows=rows)
    if dtype == "int4":
        return oracle.forward_w4a16(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                                    W["w2_scale"].cpu(), rows=rows)
    if dtype == "int8":
        return oracle.forward_int8(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                                   W["w2_scale"].cpu(), rows=rows, want_quant=want_quant)
    if dtype == "mxfp8":
        return oracle.forward_mxfp8(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                                    W["w2_scale"].cpu(), rows=rows, want_quant=want_quant)
    return oracle.forward_fp8(xb, wc, idc, W["w1"].cpu(), W["w1_scale"].cpu(), W["w2"].cpu(),
                              W["w2_scale"].cpu(), rows=rows, want_quant=want_quant)


def check_tol(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    # bf16 activations (bf16, int4 / int8 weights) or 8-bit activations (fp8, fp8b, mxfp8, int8)
    bound = BF16_REL * scale + BF16_ABS if dtype in ("bf16", "int4", "int8w") else FP8_REL * scale
    cos = float(np.dot(got.ravel(), ref.ravel()) /
                max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300)) if got.size else 1.0
    log(f"  {what} max|err|={err:.3e} max|ref|={scale:.3e} bound={bound:.3e} cos={cos:.6f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= bound, f"{what}: max|err| {err} > bound {bound}"
    return err, bound, cos


def sample_rows(T, n, seed=0):
    if T <= n:
        return list(range(T))
    g = np.random.default_rng(seed)
    mid = sorted(g.choice(np.arange(1, T - 1), size=n - 2, replace=False).tolist())
    return [0] + mid + [T - 1]


def golden(name):
    """A fixture of values printed on the pages (tests/golden/<name>.json, each
    with its citation)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name + ".json")) as f:
        return json.load(f)
