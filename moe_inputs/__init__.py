"""Seeded synthetic inputs for the fused MoE layer.

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic (no routing sort, no expert FFN, no activation
quantisation).  Both the CPU oracle's tests and the GPU path read the
tensors it returns, so the two sides always see identical bytes.

The five workloads are layers shaped like the models the SGLang fused-MoE
tuning guide names as tuning targets (Mixtral-8x7B, Qwen2-57B-A14B at TP=4,
DeepSeek-V3; guide section 2.1) plus a Qwen3-30B-A3B-class layer and a tiny
parity case.  The token grid follows the guide's default batch-size grid
(section 2.5).  The guide tunes on captured ``topk_ids`` traces (section 3.1);
those traces are not available, and the routing recipes below stand in for
them: uniform softmax top-k, per-expert-biased (skewed, some experts idle)
and adversarial (a hot expert).

Conventions fixed here (they are inputs, not arithmetic of the method):

* ``W1[e]`` is ``[2I][H]``: rows ``[0, I)`` are the gate projection, rows
  ``[I, 2I)`` the up projection (the guide stacks gate and up into one
  ``2*I`` tensor and halves N after silu_and_mul, section 4.1).
* ``W2[e]`` is ``[H][I]``.  Both are K-contiguous (row-major, last index
  is the reduction index).
* Weights are N(0, std = 1/sqrt(fan_in)), fan_in = H for W1 and I for W2.
* Router logits are N(0, 1) (plus a per-expert N(0, 1.5**2) bias for the
  skewed recipe).  ``topk_ids[t][j]`` lists the chosen experts in
  descending logit order (ties: lower expert id first); ``topk_w`` is the
  softmax over the chosen k logits (renormalised top-k).
* fp8 weights are OCP E4M3 ("e4m3fn") codes with one fp32 scale per output
  channel (per row of W1[e] and W2[e]), made with torch's own cast:
  ``scale = amax(row) / 448`` and ``code = e4m3(W / scale)``.  This is input
  preparation done once, not part of the layer.

Seeds: weights (and the skewed recipe's expert bias) come from generator
seed ``s`` = the workload's index (1..5); token data (x and router logits)
from seed ``1000*s + T``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    E: int
    H: int
    I: int
    k: int
    dtype: str          # "f32" (tiny parity case), "bf16", "fp8", "fp8b" (block-scaled), "mxfp8", "int8",
                        # "int8w" (weight-only int8, bf16 activations) or "int4"
    Ts: tuple
    routing: str        # "softmax", "biased" or "hot0"
    label: str


WORKLOADS = {
    "tiny": Workload("tiny", 1, 8, 128, 64, 2, "f32", (4,), "softmax",
                     "tiny MoE layer, fp32 data, E=8 H=128 I=64 top-2"),
    "mixtral": Workload("mixtral", 2, 8, 4096, 14336, 2, "bf16",
                        (1, 2, 4, 8, 16, 32, 64), "softmax",
                        "Mixtral-8x7B-shaped MoE layer, bf16, E=8 H=4096 I=14336 top-2"),
    "qwen3": Workload("qwen3", 3, 128, 2048, 768, 8, "bf16", (1, 8, 64, 256),
                      "biased",
                      "Qwen3-30B-A3B-shaped MoE layer, bf16, E=128 H=2048 I=768 top-8, skewed routing"),
    "qwen2": Workload("qwen2", 4, 64, 3584, 640, 8, "bf16",
                      (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096),
                      "hot0",
                      "Qwen2-57B-A14B-shaped MoE layer (TP=4 slice), bf16, E=64 H=3584 I=640 top-8, hot expert 0"),
    "dsv3": Workload("dsv3", 5, 256, 7168, 2048, 8, "fp8",
                     (1, 16, 128, 1024, 4096), "softmax",
                     "DeepSeek-V3-shaped MoE layer, fp8 w8a8, E=256 H=7168 I=2048 top-8"),
    "dsv3i8": Workload("dsv3i8", 5, 256, 7168, 2048, 8, "int8",
                       (1, 16, 128, 1024, 4096), "softmax",
                       "DeepSeek-V3-shaped MoE layer, int8 w8a8 per-channel, E=256 H=7168 I=2048 top-8"),
    "mixtral4": Workload("mixtral4", 2, 8, 4096, 14336, 2, "int4",
                         (1, 2, 4, 8, 16, 32, 64), "softmax",
                         "Mixtral-8x7B-shaped MoE layer, int4 w4a16 (group 128), E=8 H=4096 I=14336 top-2"),
    "mixtral8": Workload("mixtral8", 2, 8, 4096, 14336, 2, "int8w",
                         (1, 2, 4, 8, 16, 32, 64), "softmax",
                         "Mixtral-8x7B-shaped MoE layer, int8 w8a16 (per-channel weight scales), E=8 H=4096 I=14336 top-2"),
    "dsv3b": Workload("dsv3b", 5, 256, 7168, 2048, 8, "fp8b",
                      (1, 16, 128, 1024, 4096), "softmax",
                      "DeepSeek-V3-shaped MoE layer, fp8 w8a8 with 128x128 weight blocks and 1x128 token groups, E=256 H=7168 I=2048 top-8"),
    "dsv3mx": Workload("dsv3mx", 5, 256, 7168, 2048, 8, "mxfp8",
                       (1, 16, 128, 1024, 4096), "softmax",
                       "DeepSeek-V3-shaped MoE layer, MXFP8 (OCP MX, 32-element blocks), E=256 H=7168 I=2048 top-8"),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def expert_bias(E: int, seed: int) -> torch.Tensor:
    """Per-expert logit bias b_e ~ N(0, 1.5**2) for the skewed recipe (CPU, fp32)."""
    g = _gen(100 * seed + 7, "cpu")
    return torch.randn(E, generator=g, dtype=torch.float32) * 1.5


def route_from_logits(logits: torch.Tensor, k: int, force_expert0_even: bool = False):
    """Renormalised softmax top-k from fp32 logits [T][E].

    Returns (topk_ids int32 [T][k], topk_w fp32 [T][k]).  Expert order per
    token: descending logit, ties broken by lower expert id (stable sort).
    With ``force_expert0_even`` every even token takes expert 0 first and
    then the top-(k-1) of the remaining experts.
    """
    T, E = logits.shape
    logits = logits.float()
    order = torch.sort(logits, dim=1, descending=True, stable=True).indices
    ids = order[:, :k].clone()
    if force_expert0_even and T > 0:
        others = order[:, :]
        for t in range(0, T, 2):
            rest = others[t][others[t] != 0][: k - 1]
            ids[t, 0] = 0
            ids[t, 1:] = rest
    sel = torch.gather(logits, 1, ids)
    w = torch.softmax(sel, dim=1).float()
    return ids.to(torch.int32).contiguous(), w.contiguous()


def make_router_inputs(wl: Workload, T: int, device="cpu", seed: Optional[int] = None):
    """x [T][H] fp32 and the router logits [T][E] fp32 of a workload's token
    batch (the same draws make_tokens routes from)."""
    s = (1000 * wl.seed + T) if seed is None else seed
    g = _gen(s, device)
    x = torch.randn(T, wl.H, generator=g, device=device, dtype=torch.float32)
    logits = torch.randn(T, wl.E, generator=g, device=device, dtype=torch.float32)
    if wl.routing == "biased":
        logits = logits + expert_bias(wl.E, wl.seed).to(device)
    return x, logits.contiguous()


LOGIT_KINDS = ("normal", "ties", "const", "wide", "nan")


def router_logits(T: int, E: int, seed: int, kind: str = "normal") -> torch.Tensor:
    """Synthetic fp32 router logits [T][E] (CPU) of one of these recipes:
    normal N(0, 1); ties: N(0, 1) rounded to multiples of 1/4 (many equal
    scores per row); const: every score 0.5; wide: N(0, 1) * 1e30; nan:
    N(0, 1) with about 5% of the scores NaN."""
    g = _gen(seed, "cpu")
    l = torch.randn(T, E, generator=g, dtype=torch.float32)
    if kind == "ties":
        l = torch.round(l * 4) / 4
    elif kind == "const":
        l = torch.full((T, E), 0.5, dtype=torch.float32)
    elif kind == "wide":
        l = l * 1e30
    elif kind == "nan":
        l = torch.where(torch.rand(T, E, generator=g) < 0.05, torch.full_like(l, float("nan")), l)
    elif kind != "normal":
        raise ValueError(kind)
    return l.contiguous()


def router_weight(N: int, K: int, seed: int, std: float = 0.02) -> torch.Tensor:
    """fp32 router weights [N][K] ~ N(0, std^2) (a typical router init), CPU."""
    g = _gen(seed, "cpu")
    return (torch.randn(N, K, generator=g, dtype=torch.float32) * std).contiguous()


def router_hidden(T: int, K: int, seed: int) -> torch.Tensor:
    """bf16 hidden states [T][K] for the router: N(0, 1) per channel, with eight
    outlier channels scaled by 30-60 (LLM residual streams carry a few such
    channels; they are what makes the low mantissa bits of the router weights
    matter).  CPU."""
    g = _gen(seed, "cpu")
    scale = torch.ones(K)
    idx = torch.randperm(K, generator=g)[: min(8, K)]
    scale[idx] = 30.0 + 30.0 * torch.rand(idx.numel(), generator=g)
    return (torch.randn(T, K, generator=g) * scale).bfloat16().contiguous()


def make_tokens(wl: Workload, T: int, device="cpu", seed: Optional[int] = None):
    """x [T][H] (fp32 for the tiny case, else bf16), topk_ids, topk_w."""
    x, logits = make_router_inputs(wl, T, device, seed)
    ids, w = route_from_logits(logits.cpu(), wl.k, force_expert0_even=(wl.routing == "hot0"))
    if wl.dtype != "f32":
        x = x.to(torch.bfloat16)
    return x.contiguous(), ids.to(device), w.to(device)


def _randn_experts(E, rows, cols, std, g, device, out_dtype, chunk_elems=1 << 27):
    out = torch.empty(E, rows, cols, dtype=out_dtype, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32)
        out[e0:e1] = (blk * std).to(out_dtype)
    return out


def quantize_weight_rows(w: torch.Tensor):
    """Per-output-channel e4m3 codes of fp32 weights [.., rows, cols].

    scale = amax(row)/448 (fp32; 1 for an all-zero row) and codes = torch's
    RNE cast of w/scale.  Returns (uint8 codes, fp32 scales [.., rows]).
    """
    amax = w.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()
    q = (w / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).contiguous(), scale.contiguous()


def _fp8_experts(E, rows, cols, std, g, device, chunk_elems=1 << 27):
    codes = torch.empty(E, rows, cols, dtype=torch.uint8, device=device)
    scales = torch.empty(E, rows, dtype=torch.float32, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32) * std
        q, s = quantize_weight_rows(blk)
        codes[e0:e1] = q
        scales[e0:e1] = s
    return codes, scales


def quantize_weight_block_fp8(w: torch.Tensor, block: int = 128):
    """e4m3 codes of fp32 weights [.., rows, cols] (both multiples of `block`)
    with one fp32 scale per block x block tile: scale = amax(tile) / 448 (1 for
    an all-zero tile), codes = torch's RNE e4m3 cast of w / scale.  Returns
    (uint8 codes [.., rows, cols], fp32 scales [.., rows/block, cols/block])."""
    *lead, rows, cols = w.shape
    t = w.reshape(*lead, rows // block, block, cols // block, block)
    amax = t.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()
    q = (t / scale.unsqueeze(-1).unsqueeze(-3)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(*lead, rows, cols).contiguous(), scale.contiguous()


def _block_fp8_experts(E, rows, cols, std, g, device, chunk_elems=1 << 27):
    codes = torch.empty(E, rows, cols, dtype=torch.uint8, device=device)
    scales = torch.empty(E, rows // 128, cols // 128, dtype=torch.float32, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32) * std
        q, sc = quantize_weight_block_fp8(blk)
        codes[e0:e1] = q
        scales[e0:e1] = sc
    return codes, scales


def quantize_weight_int4(w: torch.Tensor, group: int = 128):
    """Symmetric int4 codes of fp32 weights [.., rows, cols] (cols % group
    == 0) with one fp32 scale per `group` consecutive values of a row:
    scale = amax / 7 (1 for an all-zero group), q = torch's half-to-even
    rounding of w / scale clamped to [-8, 7], two codes per byte (the lower
    column in the low nibble, two's complement).  Returns (uint8 [.., rows,
    cols/2], fp32 scales [.., rows, cols/group])."""
    *lead, cols = w.shape
    g = w.reshape(*lead, cols // group, group)
    amax = g.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax)).float()
    q = torch.round(g / scale.unsqueeze(-1)).clamp(-8, 7).to(torch.int16).reshape(*lead, cols)
    n = (q & 0xF).to(torch.uint8)
    packed = n[..., 0::2] | (n[..., 1::2] << 4)
    return packed.contiguous(), scale.contiguous()


def _int4_experts(E, rows, cols, std, g, device, chunk_elems=1 << 27):
    codes = torch.empty(E, rows, cols // 2, dtype=torch.uint8, device=device)
    scales = torch.empty(E, rows, cols // 128, dtype=torch.float32, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32) * std
        q, sc = quantize_weight_int4(blk)
        codes[e0:e1] = q
        scales[e0:e1] = sc
    return codes, scales


def quantize_weight_int8(w: torch.Tensor):
    """Per-output-channel symmetric int8 codes of fp32 weights [.., rows, cols]:
    scale = amax(row) / 127 (1 for an all-zero row), codes = torch's
    half-to-even rounding of w / scale, clamped to [-127, 127].
    Returns (int8 codes, fp32 scales [.., rows])."""
    amax = w.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax)).float()
    q = torch.round(w / scale.unsqueeze(-1)).clamp(-127, 127).to(torch.int8)
    return q.contiguous(), scale.contiguous()


def _int8_experts(E, rows, cols, std, g, device, chunk_elems=1 << 27):
    codes = torch.empty(E, rows, cols, dtype=torch.int8, device=device)
    scales = torch.empty(E, rows, dtype=torch.float32, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32) * std
        q, sc = quantize_weight_int8(blk)
        codes[e0:e1] = q
        scales[e0:e1] = sc
    return codes, scales


def quantize_weight_mx(w: torch.Tensor):
    """OCP MXFP8 codes of fp32 weights [.., rows, cols] (cols % 32 == 0), one
    e8m0 scale per 32 consecutive values of a row: shared exponent
    s = floor(log2(amax)) - 8 clamped to [-127, 127] (-127 for a zero
    block), codes = torch's RNE e4m3 cast of w / 2^s clamped to +-448.
    Returns (uint8 codes [.., rows, cols], uint8 scale codes [.., rows, cols/32])."""
    *lead, cols = w.shape
    blk = w.reshape(*lead, cols // 32, 32)
    amax = blk.abs().amax(dim=-1)
    _, e = torch.frexp(amax)
    s = torch.where(amax > 0, e - 1 - 8, torch.full_like(e, -127)).clamp(-127, 127)
    v = blk * torch.exp2(-s.float()).unsqueeze(-1)
    q = v.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(*lead, cols).contiguous(), (s + 127).to(torch.uint8).contiguous()


def _mx_experts(E, rows, cols, std, g, device, chunk_elems=1 << 27):
    codes = torch.empty(E, rows, cols, dtype=torch.uint8, device=device)
    scales = torch.empty(E, rows, cols // 32, dtype=torch.uint8, device=device)
    per = max(1, chunk_elems // (rows * cols))
    for e0 in range(0, E, per):
        e1 = min(E, e0 + per)
        blk = torch.randn(e1 - e0, rows, cols, generator=g, device=device, dtype=torch.float32) * std
        q, sc = quantize_weight_mx(blk)
        codes[e0:e1] = q
        scales[e0:e1] = sc
    return codes, scales


def make_weights(wl: Workload, device="cpu", seed: Optional[int] = None, E: Optional[int] = None):
    """Expert weights of a workload.

    bf16 / f32 workloads: {"w1": [E][2I][H], "w2": [E][H][I]} in bf16 (f32 for
    the tiny case).  fp8 workloads: {"w1": uint8 codes, "w1_scale": [E][2I],
    "w2": uint8 codes, "w2_scale": [E][H]}.
    """
    s = wl.seed if seed is None else seed
    E = wl.E if E is None else E
    g = _gen(s, device)
    H, I = wl.H, wl.I
    if wl.dtype == "fp8":
        w1, s1 = _fp8_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device)
        w2, s2 = _fp8_experts(E, H, I, 1.0 / math.sqrt(I), g, device)
        return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}
    if wl.dtype == "fp8b":
        w1, s1 = _block_fp8_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device)
        w2, s2 = _block_fp8_experts(E, H, I, 1.0 / math.sqrt(I), g, device)
        return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}
    if wl.dtype == "int4":
        w1, s1 = _int4_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device)
        w2, s2 = _int4_experts(E, H, I, 1.0 / math.sqrt(I), g, device)
        return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}
    if wl.dtype in ("int8", "int8w"):   # the same per-channel weights; int8w keeps bf16 activations
        w1, s1 = _int8_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device)
        w2, s2 = _int8_experts(E, H, I, 1.0 / math.sqrt(I), g, device)
        return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}
    if wl.dtype == "mxfp8":
        w1, s1 = _mx_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device)
        w2, s2 = _mx_experts(E, H, I, 1.0 / math.sqrt(I), g, device)
        return {"w1": w1, "w1_scale": s1, "w2": w2, "w2_scale": s2}
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    w1 = _randn_experts(E, 2 * I, H, 1.0 / math.sqrt(H), g, device, dt)
    w2 = _randn_experts(E, H, I, 1.0 / math.sqrt(I), g, device, dt)
    return {"w1": w1, "w2": w2}


def custom_workload(E, H, I, k, dtype="bf16", routing="softmax", seed=11, name="custom"):
    """A workload of arbitrary shape (used for parity cases off the five named layers)."""
    return Workload(name, seed, E, H, I, k, dtype, (), routing, f"{name} E={E} H={H} I={I} top-{k} {dtype}")


def random_ids(T: int, k: int, E: int, seed: int, p_drop: float = 0.0, lo: int = 0,
               hi: Optional[int] = None) -> torch.Tensor:
    """Uniform random expert ids in [lo, hi) (int32 [T][k]); with probability
    p_drop an id is replaced by an out-of-range value (-1 or E + something),
    which the layer treats as a dropped pair."""
    g = _gen(seed, "cpu")
    hi = E if hi is None else hi
    ids = torch.randint(lo, hi, (T, k), generator=g, dtype=torch.int64)
    if p_drop > 0:
        m = torch.rand(T, k, generator=g) < p_drop
        bad = torch.where(torch.rand(T, k, generator=g) < 0.5,
                          torch.full((T, k), -1, dtype=torch.int64),
                          E + torch.randint(0, 5, (T, k), generator=g))
        ids = torch.where(m, bad, ids)
    return ids.to(torch.int32).contiguous()


def random_weights_w(T: int, k: int, seed: int) -> torch.Tensor:
    """Positive fp32 routing weights [T][k] summing to 1 per token."""
    g = _gen(seed, "cpu")
    w = torch.rand(T, k, generator=g, dtype=torch.float32) + 0.05
    return (w / w.sum(dim=1, keepdim=True)).float().contiguous()
