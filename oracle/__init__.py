"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  oracle_init / value tables  -- pinned: every bf16 and e4m3 code against
                                 torch's own decoders.
  e4m3_encode                 -- pinned: torch's float8_e4m3fn cast at every
                                 representable value, midpoint and
                                 midpoint +- 1 ulp; saturation by the format
                                 definition.
  quant_row / quant_rows_bf16 -- pinned: closed-form cases (zero row, exact
                                 448 row, power-of-two rows) and torch's cast.
  route                       -- pinned: brute-force stable sort, invariants,
                                 exhaustive tiny cases.
  quant_groups / forward_fp8_block -- pinned: groups equal the per-row rule
                                 on each group, a dense torch reference on
                                 dequantised block weights and activations.
  w4_dequant / forward_w4a16    -- pinned: nibble order and sign against
                                 torch bit operations, exact cases, a
                                 dense torch reference on dequantised
                                 weights.
  forward_w8a16               -- pinned: a dense torch reference on the
                                 dequantised int8 weights (every code, both
                                 signs, per-row scales), k=1 single expert.
  int8_quant_row / forward_int8 -- pinned: worked cases (integers at amax
                                 127, ties to even, clamping), an independent
                                 torch quantiser, a dense torch reference
                                 (exact integer products).
  mx_quant_rows / forward_mxfp8 -- pinned: OCP worked cases (amax 448, 1,
                                 500, 0, subnormal), torch's e4m3 cast and
                                 frexp on random blocks, dequantisation
                                 bound, dense torch reference of the MX
                                 layer (k=1 single expert, general k).
  router_split / router_scores -- pinned: truncation bracket (W_high <= |W| <
                                 next bf16), torch's RNE cast of the exact
                                 residual, the 2^-15 approximation bound,
                                 exact cases, unit-vector and linearity
                                 laws, fp64 matmul within the bound.
  router_topk                 -- pinned: closed-form weights (logits log 1..4,
                                 equal logits, two-expert sigmoid), brute-force
                                 ranking of every tiny case, softmax of all E
                                 at k = E, ratio and shift laws, torch's
                                 stable sort + softmax on random rows.
  forward_f64/f32/bf16        -- pinned: dense fp64 torch matmul references
                                 (k=1, k=E mean, scattered gate matrix),
                                 structural invariants.
  forward_fp8                 -- pinned: dense torch reference applying
                                 torch's e4m3 cast; exactness of the fp8 dot
                                 products against integer arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math, no contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC", "-Wall", SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_init.restype = None
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [i]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [i]
        L.oracle_e4m3_encode.restype = i
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_quant_row.restype = None
        L.oracle_quant_row.argtypes = [P, i, P, P]
        L.oracle_quant_rows_bf16.restype = None
        L.oracle_quant_rows_bf16.argtypes = [P, i, i, P, P]
        L.oracle_route.restype = i
        L.oracle_route.argtypes = [P, i, i, i, P, P, P, P, i, P, P]
        for name in ("oracle_forward_f64", "oracle_forward_f32", "oracle_forward_bf16"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [P, P, P, P, P, i, i, i, i, i, P, i, P]
        L.oracle_forward_fp8.restype = None
        L.oracle_forward_fp8.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P, P, P, P, P]
        L.oracle_router_topk.restype = None
        L.oracle_router_topk.argtypes = [P, i, i, i, i, i, P, P]
        L.oracle_quant_groups.restype = None
        L.oracle_quant_groups.argtypes = [P, i, P, P]
        L.oracle_forward_fp8_block.restype = None
        L.oracle_forward_fp8_block.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P, P, P, P, P]
        L.oracle_forward_w4a16.restype = None
        L.oracle_forward_w4a16.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P]
        L.oracle_w4_dequant.restype = None
        L.oracle_w4_dequant.argtypes = [P, P, i, i, P]
        L.oracle_forward_w8a16.restype = None
        L.oracle_forward_w8a16.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P]
        L.oracle_int8_quant_row.restype = None
        L.oracle_int8_quant_row.argtypes = [P, i, P, P]
        L.oracle_int8_quant_rows_bf16.restype = None
        L.oracle_int8_quant_rows_bf16.argtypes = [P, i, i, P, P]
        L.oracle_forward_int8.restype = None
        L.oracle_forward_int8.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P, P, P, P, P]
        L.oracle_mx_quant_rows.restype = None
        L.oracle_mx_quant_rows.argtypes = [P, i, i, P, P]
        L.oracle_mx_quant_rows_bf16.restype = None
        L.oracle_mx_quant_rows_bf16.argtypes = [P, i, i, P, P]
        L.oracle_forward_mxfp8.restype = None
        L.oracle_forward_mxfp8.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, P, i, P, P, P, P, P]
        L.oracle_router_split.restype = None
        L.oracle_router_split.argtypes = [P, ctypes.c_long, P, P]
        L.oracle_router_scores.restype = None
        L.oracle_router_scores.argtypes = [P, P, P, i, i, i, P]
        L.oracle_num_threads.restype = i
        L.oracle_init()
        _lib = L
    return _lib


def _np(a, dtype):
    """Contiguous numpy view/copy of a tensor or array with the given dtype."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16)
            elif a.dtype == torch.float8_e4m3fn:
                a = a.view(torch.uint8)
            a = a.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        if dtype in (np.uint16, np.uint8) and a.dtype.itemsize == np.dtype(dtype).itemsize:
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def bf16_value(code: int) -> float:
    return lib().oracle_bf16_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def e4m3_encode_array(v) -> np.ndarray:
    v = _np(v, np.float32).reshape(-1)
    L = lib()
    return np.array([L.oracle_e4m3_encode(float(x)) for x in v], dtype=np.uint8)


def quant_row(v):
    """Per-row e4m3 quantisation of fp32 values -> (codes uint8[n], scale float)."""
    v = _np(v, np.float32).reshape(-1)
    codes = np.zeros(v.size, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    lib().oracle_quant_row(_p(v), v.size, _p(codes), _p(scale))
    return codes, float(scale[0])


def quant_rows_bf16(x):
    """Per-token quantisation of bf16 x [T][H] -> (codes uint8[T][H], scales fp32[T])."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    codes = np.zeros((T, H), dtype=np.uint8)
    scales = np.zeros(T, dtype=np.float32)
    lib().oracle_quant_rows_bf16(_p(xa), T, H, _p(codes), _p(scales))
    return codes, scales


def max_tasks(P: int, E: int, BM: int) -> int:
    return P // BM + min(E, P)


def route(ids, E: int, BM: int):
    """Routing & index build.  Returns a dict of numpy int32 arrays:
    offsets[E+1], sorted[P], pos[P], tasks[num_tasks][4], num_tasks, num_dropped."""
    ida = _np(ids, np.int32).reshape(-1)
    P = ida.size
    mt = max_tasks(P, E, BM)
    offsets = np.zeros(E + 1, dtype=np.int32)
    srt = np.zeros(max(P, 1), dtype=np.int32)
    pos = np.zeros(max(P, 1), dtype=np.int32)
    tasks = np.zeros((max(mt, 1), 4), dtype=np.int32)
    nt = np.zeros(1, dtype=np.int32)
    nd = np.zeros(1, dtype=np.int32)
    rc = lib().oracle_route(_p(ida), P, E, BM, _p(offsets), _p(srt), _p(pos), _p(tasks), mt,
                            _p(nt), _p(nd))
    if rc != 0:
        raise RuntimeError("oracle_route: task list overflow")
    n = int(nt[0])
    return {"offsets": offsets, "sorted": srt[:P], "pos": pos[:P], "tasks": tasks[:n].copy(),
            "num_tasks": n, "num_dropped": int(nd[0])}


def router_topk(logits, k: int, renormalize: bool = True, n_shared: int = 0):
    """Router top-k from fp32 logits [T][E]: (ids int32 [T][k+n_shared],
    weights fp64 [T][k+n_shared]).  Softmax over E, top-k by descending
    score (ties: lower expert id), optional renormalisation over the k
    selected, then n_shared shared-expert columns (ids E.., weight 1)."""
    la = _np(logits, np.float32)
    T, E = la.shape
    if not (1 <= k <= E) or n_shared < 0:
        raise ValueError("need 1 <= k <= E and n_shared >= 0")
    ncol = k + n_shared
    ids = np.zeros((T, ncol), dtype=np.int32)
    w = np.zeros((T, ncol), dtype=np.float64)
    if T:
        lib().oracle_router_topk(_p(la), T, E, k, int(bool(renormalize)), n_shared, _p(ids), _p(w))
    return ids, w


def quant_groups(v):
    """Per-128-group fp8 quantisation of one fp32 row (n % 128 == 0): e4m3
    codes uint8 [n] and fp32 scales [n/128], each group by the per-row rule."""
    va = _np(v, np.float32).reshape(-1)
    codes = np.zeros(va.size, dtype=np.uint8)
    sc = np.zeros(va.size // 128, dtype=np.float32)
    lib().oracle_quant_groups(_p(va), va.size, _p(codes), _p(sc))
    return codes, sc


def forward_fp8_block(x, topk_w, ids, W1, s1, W2, s2, rows=None, want_quant=False):
    """Block-scaled fp8 layer output in fp64: W1/W2 e4m3 codes, s1 fp32
    [E][2I/128][H/128], s2 fp32 [E][H/128][I/128]; x and the intermediate
    quantised per 128-value group of a row."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.uint8)
    W2a = _np(W2, np.uint8)
    s1a = _np(s1, np.float32)
    s2a = _np(s2, np.float32)
    E, I2, _ = W1a.shape
    I = I2 // 2
    assert s1a.shape == (E, I2 // 128, H // 128) and s2a.shape == (E, H // 128, I // 128)
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    xq = sx = hq = sh = None
    if want_quant:
        xq = np.zeros((n, H), dtype=np.uint8)
        sx = np.zeros((n, H // 128), dtype=np.float32)
        hq = np.zeros((n, k, I), dtype=np.uint8)
        sh = np.zeros((n, k, I // 128), dtype=np.float32)
    lib().oracle_forward_fp8_block(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                                   T, k, E, H, I, _p(r) if r is not None else None, n, _p(out),
                                   *(None if a is None else _p(a) for a in (xq, sx, hq, sh)))
    return (out, xq, sx, hq, sh) if want_quant else out


def w4_dequant(codes, scales):
    """fp64 values [R][n] of int4 rows: codes uint8 [R][n/2] (low nibble =
    lower K index, two's complement), fp32 scales [R][n/128]."""
    c = _np(codes, np.uint8)
    sc = _np(scales, np.float32)
    R, nb = c.shape
    n = 2 * nb
    out = np.zeros((R, n), dtype=np.float64)
    lib().oracle_w4_dequant(_p(c), _p(sc), R, n, _p(out))
    return out


def forward_w8a16(x, topk_w, ids, W1, s1, W2, s2, rows=None):
    """int8 w8a16 layer output in fp64: x bf16 [T][H]; W1 int8 [E][2I][H],
    s1 fp32 [E][2I] (one scale per weight row); W2 int8 [E][H][I], s2 fp32
    [E][H]."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.int8)
    W2a = _np(W2, np.int8)
    s1a = _np(s1, np.float32)
    s2a = _np(s2, np.float32)
    E, I2, _ = W1a.shape
    I = I2 // 2
    assert W1a.shape == (E, I2, H) and s1a.shape == (E, I2)
    assert W2a.shape == (E, H, I) and s2a.shape == (E, H)
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    lib().oracle_forward_w8a16(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                               T, k, E, H, I, _p(r) if r is not None else None, n, _p(out))
    return out


def forward_w4a16(x, topk_w, ids, W1, s1, W2, s2, rows=None):
    """int4 w4a16 layer output in fp64: x bf16 [T][H]; W1 uint8 [E][2I][H/2],
    s1 fp32 [E][2I][H/128]; W2 uint8 [E][H][I/2], s2 fp32 [E][H][I/128]."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.uint8)
    W2a = _np(W2, np.uint8)
    s1a = _np(s1, np.float32)
    s2a = _np(s2, np.float32)
    E, I2, _ = W1a.shape
    I = I2 // 2
    assert W1a.shape == (E, I2, H // 2) and s1a.shape == (E, I2, H // 128)
    assert W2a.shape == (E, H, I // 2) and s2a.shape == (E, H, I // 128)
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    lib().oracle_forward_w4a16(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                               T, k, E, H, I, _p(r) if r is not None else None, n, _p(out))
    return out


def int8_quant_row(v):
    """int8 codes (int8 array) and fp32 scale of one fp32 row (symmetric, amax/127)."""
    va = _np(v, np.float32).reshape(-1)
    q = np.zeros(va.size, dtype=np.int8)
    sc = np.zeros(1, dtype=np.float32)
    lib().oracle_int8_quant_row(_p(va), va.size, _p(q), _p(sc))
    return q, float(sc[0])


def int8_quant_rows_bf16(x):
    xa = _np(x, np.uint16)
    T, H = xa.shape
    q = np.zeros((T, H), dtype=np.int8)
    sc = np.zeros(T, dtype=np.float32)
    if T:
        lib().oracle_int8_quant_rows_bf16(_p(xa), T, H, _p(q), _p(sc))
    return q, sc


def forward_int8(x, topk_w, ids, W1, s1, W2, s2, rows=None, want_quant=False):
    """int8 w8a8 (per-channel weight scales) layer output in fp64.  x bf16
    [T][H]; W1/W2 int8 codes (int8 or uint8 tensors of the same bytes);
    s1 fp32 [E][2I], s2 fp32 [E][H]."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.int8)
    W2a = _np(W2, np.int8)
    s1a = _np(s1, np.float32)
    s2a = _np(s2, np.float32)
    E, I2, _ = W1a.shape
    I = I2 // 2
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    xq = sx = hq = sh = None
    if want_quant:
        xq = np.zeros((n, H), dtype=np.int8)
        sx = np.zeros(n, dtype=np.float32)
        hq = np.zeros((n, k, I), dtype=np.int8)
        sh = np.zeros((n, k), dtype=np.float32)
    lib().oracle_forward_int8(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                              T, k, E, H, I, _p(r) if r is not None else None, n, _p(out),
                              *(None if a is None else _p(a) for a in (xq, sx, hq, sh)))
    return (out, xq, sx, hq, sh) if want_quant else out


def mx_quant_rows(v):
    """OCP MXFP8 quantisation of fp32 rows [R][n] (n % 32 == 0): (e4m3 codes
    uint8 [R][n], e8m0 scale codes uint8 [R][n/32])."""
    va = _np(v, np.float32)
    R, n = va.shape
    assert n % 32 == 0
    codes = np.zeros((R, n), dtype=np.uint8)
    scales = np.zeros((R, n // 32), dtype=np.uint8)
    if R:
        lib().oracle_mx_quant_rows(_p(va), R, n, _p(codes), _p(scales))
    return codes, scales


def mx_quant_rows_bf16(x):
    xa = _np(x, np.uint16)
    T, H = xa.shape
    codes = np.zeros((T, H), dtype=np.uint8)
    scales = np.zeros((T, H // 32), dtype=np.uint8)
    if T:
        lib().oracle_mx_quant_rows_bf16(_p(xa), T, H, _p(codes), _p(scales))
    return codes, scales


def mx_values(codes, scales):
    """fp64 values of MX rows (codes [R][n], scale codes [R][n/32])."""
    c = _np(codes, np.uint8)
    s = _np(scales, np.uint8).astype(np.int64)
    vals = np.array([lib().oracle_e4m3_value(i) for i in range(256)])[c]
    return np.ldexp(vals, np.repeat(s, 32, axis=-1) - 127)


def forward_mxfp8(x, topk_w, ids, W1, s1, W2, s2, rows=None, want_quant=False):
    """MXFP8 layer output in fp64.  x bf16 [T][H]; W1/W2 e4m3 codes; s1 e8m0
    codes [E][2I][H/32], s2 [E][H][I/32].  With want_quant also returns
    (xq, sx, hq, sh) of the rows."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.uint8)
    W2a = _np(W2, np.uint8)
    s1a = _np(s1, np.uint8)
    s2a = _np(s2, np.uint8)
    E, I2, _ = W1a.shape
    I = I2 // 2
    assert s1a.shape == (E, 2 * I, H // 32) and s2a.shape == (E, H, I // 32)
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    xq = sx = hq = sh = None
    if want_quant:
        xq = np.zeros((n, H), dtype=np.uint8)
        sx = np.zeros((n, H // 32), dtype=np.uint8)
        hq = np.zeros((n, k, I), dtype=np.uint8)
        sh = np.zeros((n, k, I // 32), dtype=np.uint8)
    lib().oracle_forward_mxfp8(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                               T, k, E, H, I, _p(r) if r is not None else None, n, _p(out),
                               *(None if a is None else _p(a) for a in (xq, sx, hq, sh)))
    return (out, xq, sx, hq, sh) if want_quant else out


def router_split(w):
    """Split fp32 router weights [N][K] into (W_high, W_low) bf16 codes (uint16):
    W_high = truncation of W to bf16, W_low = bf16_rne((W - W_high) * 256)."""
    wa = _np(w, np.float32)
    hi = np.zeros(wa.shape, dtype=np.uint16)
    lo = np.zeros(wa.shape, dtype=np.uint16)
    lib().oracle_router_split(_p(wa), wa.size, _p(hi), _p(lo))
    return hi, lo


def router_scores(x, hi, lo):
    """fp64 scores [T][N] = x . W_high^T + (x . W_low^T) / 256 from bf16 x [T][K]
    (torch bf16 or uint16 codes) and the split weights (uint16 codes [N][K])."""
    xa = _np(x, np.uint16)
    ha = _np(hi, np.uint16)
    la = _np(lo, np.uint16)
    T, K = xa.shape
    N = ha.shape[0]
    assert ha.shape == (N, K) and la.shape == (N, K)
    out = np.zeros((T, N), dtype=np.float64)
    if T and N:
        lib().oracle_router_scores(_p(xa), _p(ha), _p(la), T, N, K, _p(out))
    return out


def _rows_arg(rows, T):
    if rows is None:
        return None, T
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1))
    if r.size and (r.min() < 0 or r.max() >= T):
        raise ValueError("row index out of range")
    return r, r.size


def _forward_plain(fname, x, topk_w, ids, W1, W2, dt, rows):
    xa = _np(x, dt)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1] if ida.ndim == 2 else 1
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, dt)
    W2a = _np(W2, dt)
    E, I2, H1 = W1a.shape
    I = I2 // 2
    assert H1 == H and W2a.shape == (E, H, I)
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    getattr(lib(), fname)(_p(xa), _p(wa), _p(ida), _p(W1a), _p(W2a), T, k, E, H, I,
                          _p(r) if r is not None else None, n, _p(out))
    return out


def forward_f64(x, topk_w, ids, W1, W2, rows=None):
    """Layer output in fp64 from fp64 inputs; rows = token subset (default all)."""
    return _forward_plain("oracle_forward_f64", x, topk_w, ids, W1, W2, np.float64, rows)


def forward_f32(x, topk_w, ids, W1, W2, rows=None):
    return _forward_plain("oracle_forward_f32", x, topk_w, ids, W1, W2, np.float32, rows)


def forward_bf16(x, topk_w, ids, W1, W2, rows=None):
    """Layer output in fp64 from bf16 x/W1/W2 (torch bf16 tensors or uint16 codes)."""
    return _forward_plain("oracle_forward_bf16", x, topk_w, ids, W1, W2, np.uint16, rows)


def forward_fp8(x, topk_w, ids, W1, s1, W2, s2, rows=None, want_quant=False):
    """fp8 w8a8 layer output in fp64.  x bf16 [T][H]; W1/W2 e4m3 codes; s1 [E][2I],
    s2 [E][H] fp32.  With want_quant also returns (xq, sx, hq, sh) of the rows."""
    xa = _np(x, np.uint16)
    T, H = xa.shape
    ida = _np(ids, np.int32)
    k = ida.shape[1]
    wa = _np(topk_w, np.float32)
    W1a = _np(W1, np.uint8)
    W2a = _np(W2, np.uint8)
    s1a = _np(s1, np.float32)
    s2a = _np(s2, np.float32)
    E, I2, _ = W1a.shape
    I = I2 // 2
    r, n = _rows_arg(rows, T)
    out = np.zeros((n, H), dtype=np.float64)
    xq = sx = hq = sh = None
    if want_quant:
        xq = np.zeros((n, H), dtype=np.uint8)
        sx = np.zeros(n, dtype=np.float32)
        hq = np.zeros((n, k, I), dtype=np.uint8)
        sh = np.zeros((n, k), dtype=np.float32)
    lib().oracle_forward_fp8(_p(xa), _p(wa), _p(ida), _p(W1a), _p(s1a), _p(W2a), _p(s2a),
                             T, k, E, H, I, _p(r) if r is not None else None, n, _p(out),
                             _p(xq) if want_quant else None, _p(sx) if want_quant else None,
                             _p(hq) if want_quant else None, _p(sh) if want_quant else None)
    if want_quant:
        return out, (xq, sx, hq, sh)
    return out
