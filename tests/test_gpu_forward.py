"""GPU parity of the forward pass against the oracle.

bf16: max|err| <= 1e-2*max|ref| + 1e-3.  fp8 w8a8: max|err| <= 4e-2*max|ref|
against the oracle applying the same quantisation, and the per-token e4m3
codes and scales of x bit-exact.  Small shapes are compared on every
output (and, on fp8, the x codes and scales bit-exact and the requantised
intermediate within one code step).  The workloads at full size, in the
launch configuration the benchmark times, are compared on every token where
the oracle costs a few seconds, else on a seeded 256-token subset that holds
the first and last token and every token of the most loaded expert's first
two row tiles.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import WORKLOADS, custom_workload, make_tokens, make_weights, random_ids, random_weights_w
from moe_testlib import (SUMMARY, check_tol, device_weights, log, oracle_rows, path_dtype, run_gpu,
                         sample_rows, workload_weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_lds_amd as m
    return m


def out64(out):
    return out.float().cpu().double().numpy()


def e4m3_ordinal(c):
    """Position of e4m3 codes on the number line (+0 and -0 both 0)."""
    c = c.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


_E4M3 = None


def e4m3_values():
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([oracle.e4m3_value(v) for v in range(256)])
    return _E4M3


def e4m3_spacing(v):
    """Distance to the next e4m3 value above |v|: 2^(e-3) for |v| in [2^e, 2^(e+1)),
    2^-9 among the subnormals (below 2^-6)."""
    av = np.abs(v)
    e = np.floor(np.log2(np.maximum(av, 2.0 ** -6)))
    return np.where(av < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))


def check_fp8_quant(lib, T, k, E, H, I, ws, routing, ids, rows, xq, sx, hq, sh, what):
    """fp8 w8a8 workspace against the oracle's quantisation, for the tokens
    `rows` (the oracle's outputs xq, sx, hq, sh are for those tokens).

    x codes and scales: bit-exact (the same rule on the same bf16 inputs).

    The requantised intermediate of every valid pair of those tokens: >= 99%
    of codes equal; every dequantised value within one e4m3 step (at the
    larger of the two magnitudes) plus 2^-11 of its row's amax of the
    oracle's; scales within 1e-3 relative.  The intermediate is not exact on
    this path: the GPU's gate and up sums come from the fp8 MFMA, whose
    128-value unit sums are truncated (the measured summation bound of the
    instruction), and from fp32 adds, against the oracle's exact fp64 sums;
    relative to the row's amax that error is about 1e-5.  So the scale
    amax/448 moves by about that much, a code next to a rounding boundary
    goes one step either way, and among the smallest values, whose e4m3
    steps (2^-9 of the scale) are finer than that error, by a few steps: the
    2^-11 term, far above the error and far below the output tolerance."""
    L = lib.moe_workspace_layout(T, k, E, H, I, "fp8")
    P = T * k
    rsel = torch.tensor(rows, dtype=torch.long, device=ws.device)
    gxq = ws[L["xq"]:L["xq"] + T * H].view(T, H)[rsel].cpu().numpy()
    gsx = ws[L["x_scale"]:L["x_scale"] + 4 * T].view(torch.float32)[rsel].cpu().numpy()
    assert np.array_equal(gxq, xq), f"{what}: x e4m3 codes"
    assert np.array_equal(gsx, sx), f"{what}: x scales"
    idc = ids.cpu().numpy()[rows]
    valid = (idc >= 0) & (idc < E)
    if not valid.any():
        return 1.0
    pos = lib.read_routing(routing, T, k, E, H, I, "fp8")["pos"].numpy().reshape(T, k)[rows]
    psel = torch.from_numpy(pos[valid].astype(np.int64)).to(ws.device)
    ghq = ws[L["h"]:L["h"] + P * I].view(P, I)[psel].cpu().numpy()
    gsh = ws[L["h_scale"]:L["h_scale"] + 4 * P].view(torch.float32)[psel].cpu().numpy()
    rhq, rsh = hq[valid], sh[valid]
    same = float((ghq == rhq).mean())
    step = int(np.abs(e4m3_ordinal(ghq) - e4m3_ordinal(rhq)).max())
    srel = float(np.abs(gsh.astype(np.float64) / rsh - 1.0).max())
    vg, vr = e4m3_values()[ghq], e4m3_values()[rhq]
    ga, ra = vg * gsh[:, None], vr * rsh[:, None]
    amax = 448.0 * rsh.astype(np.float64)[:, None]
    allowed = np.maximum(e4m3_spacing(vg), e4m3_spacing(vr)) * rsh[:, None] * (1 + 1e-6) + 2.0 ** -11 * amax
    dev = np.abs(ga - ra)
    cos = float((ga * ra).sum() / max(np.linalg.norm(ga) * np.linalg.norm(ra), 1e-300))
    log(f"  {what} h codes: {ghq.shape[0]} pair rows, {same:.5f} equal, max code step {step}, "
        f"max |diff|/row amax {float((dev / amax).max()):.2e}, max scale rel diff {srel:.2e}, "
        f"dequantised cosine {cos:.7f}")
    assert same >= 0.99, f"{what}: intermediate codes equal {same}"
    assert np.all(dev <= allowed), f"{what}: intermediate value beyond one step + 2^-11 amax"
    assert srel <= 1e-3, f"{what}: intermediate scales"
    return same


SMALL = [
    # E, H, I, k, T, p_drop
    (8, 128, 64, 2, 4, 0.0),
    (16, 256, 192, 4, 37, 0.1),
    (4, 512, 128, 1, 50, 0.0),
    (64, 256, 320, 8, 129, 0.05),
    (3, 64, 64, 3, 200, 0.0),
    (256, 192, 128, 8, 9, 0.0),
    # many rows per expert: 128-row LDS tiles (ragged last tiles, dropped pairs)
    (8, 256, 192, 2, 700, 0.05),
    (8, 192, 320, 2, 700, 0.0),       # H % 128 != 0; fp8 rows of 192 / 320 bytes
    (16, 512, 256, 4, 1500, 0.02),
    (32, 256, 128, 8, 500, 0.0),      # 128-row tiles about full
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop", SMALL)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_small_shapes_all_outputs(lib, E, H, I, k, T, p_drop, dtype):
    log(f"small {dtype} E={E} H={H} I={I} k={k} T={T}")
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=E + H + I)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 5)
    ids = random_ids(T, k, E, seed=T + 6, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 7)
    out, routing, ws = run_gpu(lib, x, ids, w, W, dtype)
    if dtype == "bf16":
        ref = oracle_rows(x, ids, w, W, dtype)
    else:
        ref, (xq, sx, hq, sh) = oracle_rows(x, ids, w, W, dtype, want_quant=True)
        check_fp8_quant(lib, T, k, E, H, I, ws, routing, ids, list(range(T)), xq, sx, hq, sh, "small")
    check_tol(out64(out), ref, dtype, "out")


# A few dozen to ~80 rows per expert: strips (token rows staged in LDS,
# weights streamed to registers), with split reductions, ragged last tiles,
# dropped pairs and more work items than compute units.
STRIP = [
    # E, H, I, k, T, p_drop, expected tiling (bf16, fp8): 2 strips, 1 LDS tiles,
    # 0 register streaming (fp8 rows too short for any strip stage split)
    (16, 512, 256, 4, 48, 0.05, 2, 2),      # 64-row tiles, three of four row blocks past the rows
    (8, 1024, 512, 2, 128, 0.0, 2, 2),      # 64-row tiles, deep K splits
    (8, 512, 256, 2, 300, 0.02, 2, 2),      # 128-row tiles
    (64, 1024, 640, 8, 256, 0.02, 2, 0),    # 5 strips of 2I, 20-step down reduction
    (64, 2048, 512, 4, 512, 0.0, 2, 2),     # more work items than CUs
    (16, 512, 256, 4, 512, 0.01, 1, 2),     # 128 rows per expert: LDS tiles on bf16, 160-row strips on fp8
    (8, 1024, 512, 2, 500, 0.0, 1, 2),      # 125 rows per expert, 160-row fp8 strips, 2-stage down ring
    (16, 512, 256, 4, 600, 0.0, 1, 2),      # 150 rows per expert: 192-row fp8 strips
    (16, 2048, 2048, 2, 1000, 0.0, 1, 2),   # 160-row fp8 strips, 16 gate-up strips with rotated K loops
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop,til_bf16,til_fp8", STRIP)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_strip_shapes_all_outputs(lib, E, H, I, k, T, p_drop, til_bf16, til_fp8, dtype):
    L = lib.moe_workspace_layout(T, k, E, H, I, dtype)
    log(f"strip {dtype} E={E} H={H} I={I} k={k} T={T} tiling={L['tiling']} "
        f"splits={L['split_k1']},{L['split_k2']}")
    assert L["tiling"] == (til_bf16 if dtype == "bf16" else til_fp8)
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=E + H + I + 1)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 15)
    ids = random_ids(T, k, E, seed=T + 16, p_drop=p_drop)
    w = random_weights_w(T, k, seed=T + 17)
    out, _, _ = run_gpu(lib, x, ids, w, W, dtype)
    ref = oracle_rows(x, ids, w, W, dtype)
    check_tol(out64(out), ref, dtype, "out")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_strip_hot_expert_many_tiles(lib, dtype):
    # expert 0 in every token's first slot: several row tiles of one expert
    # share each weight strip
    E, H, I, k, T = 32, 512, 256, 4, 256
    assert lib.moe_workspace_layout(T, k, E, H, I, dtype)["tiling"] == 2
    log(f"strip hot expert {dtype}")
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=21)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=22)
    ids = random_ids(T, k, E, seed=23)
    ids[:, 0] = 0
    w = random_weights_w(T, k, seed=24)
    out, routing, _ = run_gpu(lib, x, ids, w, W, dtype)
    assert lib.read_routing(routing, T, k, E, H, I, dtype)["num_tasks"] > E
    ref = oracle_rows(x, ids, w, W, dtype)
    check_tol(out64(out), ref, dtype, "out")


# Few rows per expert: register streaming, the reduction split over the
# waves of a workgroup (split chosen from the shape); odd fp8 step counts
# (one-step stages), 32- and 64-row task tiles, many tasks.
STREAM = [
    # E, H, I, k, T, p_drop, hot expert 0 in every token's first slot,
    # 16-row blocks per tile
    (8, 2048, 768, 2, 4, 0.0, False, 1),     # decode-like: few items, deep splits
    (64, 1024, 320, 8, 2, 0.0, False, 1),
    (16, 576, 192, 4, 3, 0.0, False, 1),     # 9 fp8 / 18 bf16 steps
    (8, 320, 192, 2, 48, 0.05, False, 2),    # no strip divides H: 32-row tiles
    (8, 320, 192, 2, 160, 0.02, False, 4),   # 64-row tiles
    (8, 320, 192, 2, 160, 0.02, True, 4),    # hot expert: several 64-row tiles of one expert
    (128, 2048, 768, 8, 8, 0.0, False, 1),   # 64 tasks
]


def _hot_first_slot(ids):
    ids = ids.clone()
    ids[:, 0] = 0
    return ids


@pytest.mark.parametrize("E,H,I,k,T,p_drop,hot,mb", STREAM)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_stream_shapes_all_outputs(lib, E, H, I, k, T, p_drop, hot, mb, dtype):
    L = lib.moe_workspace_layout(T, k, E, H, I, dtype)
    R = lib.moe_routing_layout(T, k, E, H, I, dtype)
    log(f"stream {dtype} E={E} H={H} I={I} k={k} T={T} tiling={L['tiling']} block_m={R['block_m']}")
    assert L["tiling"] == 0 and R["block_m"] == 16 * mb
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=E + H + I + 2)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 25)
    ids = random_ids(T, k, E, seed=T + 26, p_drop=p_drop)
    if hot:
        ids = _hot_first_slot(ids)
    w = random_weights_w(T, k, seed=T + 27)
    out, routing, _ = run_gpu(lib, x, ids, w, W, dtype)
    if hot:
        assert lib.read_routing(routing, T, k, E, H, I, dtype)["num_tasks"] > E
    ref = oracle_rows(x, ids, w, W, dtype)
    check_tol(out64(out), ref, dtype, "out")


# bf16 layers with 9 to 16 rows per expert and H >= 3072: register streaming
# on 32-row tiles with four weight blocks per item (two gate and two up
# blocks, or 64 down columns): ragged second row blocks, dropped pairs, a hot
# expert with several tiles, and the down reduction of I = 640 (one or two
# waves per item).
FOUR_BLOCK = [
    # E, H, I, k, T, p_drop, hot expert 0 in every token's first slot
    (8, 3072, 256, 2, 64, 0.05, False),
    (8, 3072, 256, 2, 64, 0.05, True),
    (16, 3584, 640, 4, 50, 0.02, False),
]


@pytest.mark.parametrize("E,H,I,k,T,p_drop,hot", FOUR_BLOCK)
def test_stream_four_block_bf16_all_outputs(lib, E, H, I, k, T, p_drop, hot):
    L = lib.moe_workspace_layout(T, k, E, H, I, "bf16")
    R = lib.moe_routing_layout(T, k, E, H, I, "bf16")
    log(f"four-block stream bf16 E={E} H={H} I={I} k={k} T={T} hot={hot}")
    assert L["tiling"] == 0 and R["block_m"] == 32
    wl = custom_workload(E, H, I, k, dtype="bf16", seed=E + H + I + 3)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=T + 35)
    ids = random_ids(T, k, E, seed=T + 36, p_drop=p_drop)
    if hot:
        ids = _hot_first_slot(ids)
    w = random_weights_w(T, k, seed=T + 37)
    out, routing, _ = run_gpu(lib, x, ids, w, W, "bf16")
    if hot:
        assert lib.read_routing(routing, T, k, E, H, I, "bf16")["num_tasks"] > E
    check_tol(out64(out), oracle_rows(x, ids, w, W, "bf16"), "bf16", "out")


# One token (decode): k from 1 to 16, odd fp8 step counts, dropped pairs, a
# token whose pairs are all dropped (zero row) and an expert named twice by
# one token.
DECODE = [
    # E, H, I, k
    (8, 256, 192, 1),
    (8, 512, 256, 2),
    (16, 320, 576, 3),      # 9 fp8 steps: one-step stages
    (64, 1024, 640, 8),
    (32, 256, 128, 16),
]


@pytest.mark.parametrize("E,H,I,k", DECODE)
@pytest.mark.parametrize("case", ["plain", "dropped", "all_dropped", "repeated"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_single_token(lib, E, H, I, k, case, dtype):
    log(f"decode {dtype} E={E} H={H} I={I} k={k} {case}")
    assert lib.moe_workspace_layout(1, k, E, H, I, dtype)["tiling"] == 0
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=E + H + I + k)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, 1, seed=k + 40)
    ids = random_ids(1, k, E, seed=k + 41)
    if case == "dropped" and k > 1:
        ids[0, k // 2] = E + 3
    elif case == "all_dropped":
        ids[0, :] = -1
    elif case == "repeated" and k > 1:
        ids[0, 1] = ids[0, 0]
    w = random_weights_w(1, k, seed=k + 42)
    out, _, _ = run_gpu(lib, x, ids, w, W, dtype)
    ref = oracle_rows(x, ids, w, W, dtype)
    if case == "all_dropped":
        assert not out.float().abs().sum().item() and not np.abs(ref).sum()
    else:
        check_tol(out64(out), ref, dtype, "out")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_stream_repeat_forward_same_routing_bitwise(lib, dtype):
    # The same routing buffer serves several forwards; the waves' partial
    # sums are added in a fixed order, so outputs are identical.
    E, H, I, k, T = 8, 2048, 768, 2, 5
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=31)
    W = lib.pack_weights(device_weights(wl), dtype)
    x, _, _ = make_tokens(wl, T, seed=32)
    x = x.cuda()
    ids = _hot_first_slot(random_ids(T, k, E, seed=33)).cuda()
    w = random_weights_w(T, k, seed=34).cuda()
    assert lib.moe_workspace_layout(T, k, E, H, I, dtype)["tiling"] == 0
    routing = lib.alloc_routing(T, k, E, H, I, dtype)
    ws = lib.alloc_workspace(T, k, E, H, I, dtype)
    outs = []
    for rep in range(3):
        out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
        if rep == 0:
            (lib.moe_build_routing_bf16 if dtype == "bf16" else lib.moe_build_routing_fp8)(ids, E, H, I, routing)
        if dtype == "bf16":
            lib.moe_forward_bf16(x, w, routing, W["w1"], W["w2"], ws, out)
        else:
            lib.moe_forward_fp8(x, w, routing, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"], ws, out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    Wc = {kk: v.cpu() for kk, v in device_weights(wl).items()}
    check_tol(out64(outs[0]), oracle_rows(x, ids, w, Wc, dtype), dtype, "out")


def test_tiny_workload(lib):
    wl = WORKLOADS["tiny"]
    W32 = make_weights(wl)                    # fp32 data, drawn on the host
    W = {k: v.bfloat16().cuda().contiguous() for k, v in W32.items()}
    x, ids, w = make_tokens(wl, 4)
    out, _, _ = run_gpu(lib, x, ids, w, W, "bf16")
    ref = oracle_rows(x, ids, w, W, "bf16")
    check_tol(out64(out), ref, "bf16", "tiny vs bf16-rounded oracle")
    # and against the fp32 originals (rounding of x and W to bf16 included)
    ref32 = oracle.forward_f32(x, w, ids, W32["w1"], W32["w2"])
    err = np.max(np.abs(out64(out) - ref32)) / np.max(np.abs(ref32))
    log(f"  tiny vs fp32 oracle rel err {err:.3e}")
    assert err < 3e-2




FULL = [(name, T) for name in ("mixtral", "qwen3", "qwen2", "dsv3", "dsv3b", "dsv3mx", "dsv3i8", "mixtral4", "mixtral8") for T in WORKLOADS[name].Ts]

# Whole-layer oracle cost (multiply-adds, 3*H*I per pair) up to which every
# token of a full-size case is compared: the fp64 oracle runs about 2e10
# multiply-adds a second on 16 host threads, so this is a few seconds.
FULL_COMPARE_MACS = 1.2e11


def full_size_rows(lib, wl, T, routing, dtype):
    """Tokens compared at full size: all of them when the oracle is cheap,
    else a seeded 256-token subset (always t = 0 and t = T-1) plus every token
    of the first two row tiles of the most loaded expert (the hot expert of
    the Qwen2-57B routing, or the fullest tile of a uniform one)."""
    k = wl.k
    if T * k * 3.0 * wl.H * wl.I <= FULL_COMPARE_MACS:
        return list(range(T)), "all tokens"
    rows = set(sample_rows(T, 256, seed=T))
    R = lib.read_routing(routing, T, k, wl.E, wl.H, wl.I, dtype)
    off = R["offsets"].numpy().astype(np.int64)
    counts = off[1:] - off[:-1]
    e = int(np.argmax(counts))
    n = int(min(counts[e], 2 * R["block_m"]))
    hot = (R["sorted"].numpy()[off[e]:off[e] + n] // k).tolist()
    rows |= set(hot)
    return sorted(rows), (f"subset: {len(rows)} of {T} tokens (256 seeded incl. first and last, "
                          f"+ the {n} rows of expert {e}'s first two {R['block_m']}-row tiles)")


@pytest.mark.parametrize("name,T", FULL)
def test_full_size_parity(lib, name, T):
    wl = WORKLOADS[name]
    dtype = path_dtype(wl)
    Wp, Wc = workload_weights(name)
    x, ids, w = make_tokens(wl, T)
    out, routing, ws = run_gpu(lib, x, ids, w, None, dtype, packed=Wp)
    rows, how = full_size_rows(lib, wl, T, routing, dtype)
    log(f"full {name} T={T} {dtype}: {how}")
    if dtype == "fp8":
        ref, (xq, sx, hq, sh) = oracle_rows(x, ids, w, Wc, dtype, rows=rows, want_quant=True)
    else:
        ref = oracle_rows(x, ids, w, Wc, dtype, rows=rows)
    err, bound, cos = check_tol(out64(out)[rows], ref, dtype, f"{name} T={T} rows={len(rows)}")
    assert torch.isfinite(out.float()).all()
    line = (f"{name} T={T} {dtype}: {len(rows)}/{T} tokens, max|err| {err:.3e} = {err / bound:.2f} of the "
            f"bound, cosine {cos:.6f}")
    if dtype == "fp8":
        same = check_fp8_quant(lib, T, wl.k, wl.E, wl.H, wl.I, ws, routing, ids, rows, xq, sx, hq, sh,
                               f"{name} T={T}")
        line += f"; x codes bit-exact, h codes {100 * same:.2f}% equal"
    SUMMARY.append(line)


def test_deterministic_and_permutation_equivariant(lib):
    wl = custom_workload(32, 512, 256, 4, seed=3)
    W = device_weights(wl)
    T = 300
    x, _, _ = make_tokens(wl, T, seed=4)
    ids = random_ids(T, 4, 32, seed=5, p_drop=0.05)
    w = random_weights_w(T, 4, seed=6)
    a, _, _ = run_gpu(lib, x, ids, w, W, "bf16")
    b, _, _ = run_gpu(lib, x, ids, w, W, "bf16")
    assert torch.equal(a, b)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(1))
    c, _, _ = run_gpu(lib, x[perm], ids[perm], w[perm], W, "bf16")
    assert torch.equal(a[perm.cuda()], c)


def test_idle_experts_never_read_and_zero_weight(lib):
    wl = custom_workload(16, 256, 128, 2, seed=7)
    W = device_weights(wl)
    T = 20
    x, _, _ = make_tokens(wl, T, seed=8)
    ids = random_ids(T, 2, 8, seed=9)          # experts 8..15 stay idle
    w = random_weights_w(T, 2, seed=10)
    a, _, _ = run_gpu(lib, x, ids, w, W, "bf16")
    Wn = {"w1": W["w1"].clone(), "w2": W["w2"].clone()}
    Wn["w1"][8:] = float("nan")
    Wn["w2"][8:] = float("nan")
    b, _, _ = run_gpu(lib, x, ids, w, Wn, "bf16")
    assert torch.isfinite(b.float()).all() and torch.equal(a, b)
    # a zero weight removes the pair exactly like a dropped id
    w0 = w.clone()
    w0[3, 1] = 0.0
    ids_d = ids.clone()
    ids_d[3, 1] = -1
    c, _, _ = run_gpu(lib, x, ids, w0, W, "bf16")
    d, _, _ = run_gpu(lib, x, ids_d, w0, W, "bf16")
    assert torch.equal(c, d)


def test_empty_batch_is_a_no_op(lib):
    wl = custom_workload(8, 128, 64, 2, seed=1)
    W = device_weights(wl)
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(0, 2, dtype=torch.int32, device="cuda")
    w = torch.zeros(0, 2, dtype=torch.float32, device="cuda")
    out, _, _ = lib.moe_layer(x, ids, w, lib.pack_weights(W))
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


@pytest.mark.parametrize("E,H,I,k,T,dtype", [
    (16, 256, 192, 4, 33, "bf16"),      # register streaming
    (8, 3072, 256, 2, 64, "bf16"),      # register streaming, 32-row tiles, four weight blocks per item
    (16, 256, 192, 4, 1, "bf16"),       # one token: down with the top-k sum, 16-column items
    (16, 256, 192, 4, 1, "fp8"),        # one token, odd fp8 step count: down + reduction
    (16, 256, 256, 4, 1, "bf16"),       # one token: down with the top-k sum, 8-column items
    (16, 256, 256, 4, 1, "fp8"),
    (32, 512, 256, 4, 256, "bf16"),     # strips
    (32, 512, 256, 4, 256, "fp8"),      # strips, fp8
    (8, 256, 192, 2, 700, "bf16"),      # LDS tiles
    (8, 256, 192, 2, 700, "fp8"),       # LDS tiles, fp8 (in-graph clearing of the row amax slots)
])
def test_graph_capture_replays_match_eager(lib, E, H, I, k, T, dtype):
    log(f"graph {dtype} E={E} H={H} I={I} k={k} T={T} "
        f"tiling={lib.moe_workspace_layout(T, k, E, H, I, dtype)['tiling']}")
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=12)
    Wr = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=13)
    x = x.cuda()
    ids = random_ids(T, k, E, seed=14).cuda()
    w = random_weights_w(T, k, seed=15).cuda()
    routing = lib.alloc_routing(T, k, E, H, I, dtype)
    ws = lib.alloc_workspace(T, k, E, H, I, dtype)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    W = lib.pack_weights(Wr, dtype)

    def chain():
        if dtype == "bf16":
            lib.moe_build_routing_bf16(ids, E, H, I, routing)
            lib.moe_forward_bf16(x, w, routing, W["w1"], W["w2"], ws, out)
        else:
            lib.moe_build_routing_fp8(ids, E, H, I, routing)
            lib.moe_forward_fp8(x, w, routing, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"], ws,
                                out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    # new routing between replays: the captured grids serve any routing
    ids2 = random_ids(T, k, E, seed=16).cuda()
    ids2[:, 0] = 0                      # and a hot expert: several tiles of one expert
    for rep in range(4):
        out.zero_()
        ws.fill_(0x7F)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
    ids.copy_(ids2)
    g.replay()
    torch.cuda.synchronize()
    ref2, _, _ = run_gpu(lib, x, ids2, w, Wr, dtype)
    assert torch.equal(out, ref2)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_strip_all_pairs_dropped(lib, dtype):
    # a strip-sized batch whose ids all fall outside [0, E): no task, zero output
    E, H, I, k, T = 32, 512, 256, 4, 256
    assert lib.moe_workspace_layout(T, k, E, H, I, dtype)["tiling"] == 2
    wl = custom_workload(E, H, I, k, dtype=dtype, seed=31)
    W = device_weights(wl)
    x, _, _ = make_tokens(wl, T, seed=32)
    ids = torch.full((T, k), E, dtype=torch.int32)
    ids[::3, 1] = -5
    w = random_weights_w(T, k, seed=33)
    out, routing, _ = run_gpu(lib, x, ids, w, W, dtype)
    assert lib.read_routing(routing, T, k, E, H, I, dtype)["num_tasks"] == 0
    assert torch.equal(out.float().cpu(), torch.zeros(T, H))


@pytest.mark.parametrize("dtype,E,rows,cols", [("bf16", 3, 32, 64), ("bf16", 2, 48, 160),
                                                ("fp8", 3, 16, 128), ("fp8", 1, 64, 192),
                                                ("int8w", 2, 32, 128), ("int4", 2, 32, 256)])
def test_pack_weights_is_the_documented_permutation(lib, dtype, E, rows, cols):
    g = torch.Generator().manual_seed(rows + cols)
    if dtype == "bf16":
        w = torch.randn(E, rows, cols, generator=g).bfloat16()
        raw = w.view(torch.uint8).view(E, rows, cols * 2)
    elif dtype == "int8w":
        w = torch.randint(-128, 128, (E, rows, cols), generator=g, dtype=torch.int8)
        raw = w.view(torch.uint8)
    elif dtype == "int4":
        w = torch.randint(0, 256, (E, rows, cols // 2), generator=g, dtype=torch.uint8)   # two codes a byte
        raw = w
    else:
        w = torch.randint(0, 256, (E, rows, cols), generator=g, dtype=torch.uint8)
        raw = w
    packed = lib.moe_pack_weights(w.cuda(), dtype).tensor
    torch.cuda.synchronize()
    got = packed.cpu().contiguous().view(torch.uint8).reshape(-1).numpy()
    # reference: chunk (e, row block, 64-byte step) of 1 KiB; piece l = row l%16, bytes 16*(l//16)
    rb = raw.numpy()
    nb = rb.shape[2]
    ref = np.empty(E * rows * nb, dtype=np.uint8)
    o = 0
    for e in range(E):
        for blk in range(rows // 16):
            for step in range(nb // 64):
                for l in range(64):
                    r = blk * 16 + l % 16
                    c0 = step * 64 + 16 * (l // 16)
                    ref[o:o + 16] = rb[e, r, c0:c0 + 16]
                    o += 16
    assert np.array_equal(got, ref)
