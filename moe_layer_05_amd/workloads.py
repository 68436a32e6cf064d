"""Seeded synthetic workloads for the fused MoE layer.

This module only draws inputs.  It holds none of the layer's arithmetic and is
shared, unchanged, by the tests (which hand the same tensors to the CPU oracle
and to the HIP library) and by the benchmark.

The pages name no dataset or model; their workloads are thin decode batches
(one token per sequence, M = 1 or M < 64), top-k = 8 routing and FP8
per-tensor-quantised experts, and a tensor-parallel share of 8 ways
(toolboxkart.tech page, results table and "Swap-AB"; aib.vote page, second and
third paragraphs).  The shapes below stand in for them:

    name               T                H     I      E    K  weights
    tiny               4                128   64     8    2  float32, N(0, 1/sqrt(fan_in))
    bf16_decode        1, 8, 16, 64     4096  14336  8    2  bfloat16, N(0, 0.02)
    fp8_decode         1, 8, 32, 64     7168  2048   256  8  E4M3 + fp32 scale per expert tensor
    fp8_tp8_slice      1, 16, 64, 256   4096  192    128  8  E4M3 (one GPU's 1/8 slice of I=1536)
    fp8_prefill_zipf   4096             7168  2048   256  8  E4M3; routing skewed by Zipf(1.2)

Activations x ~ N(0, 1) rounded to bfloat16; router logits ~ N(0, 1) in
float32, plus log(p_e) with p_e proportional to (e + 1)^-1.2 for the skewed
case (expert 0 is the hottest).  Weights are drawn in float32; the E4M3 ones are
then stored as codes with the scale amax|w_e| / 448 of each expert tensor,
using torch's float8_e4m3fn cast (round to nearest even).

Weights and tokens come from separate ``torch.Generator`` streams seeded from
(seed, role, T), so the weights of a configuration do not depend on T.  The
values depend on the device the generator runs on (CPU and GPU streams
differ); every consumer receives the same tensors, so this does not matter.
"""

from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class MoEConfig:
    name: str
    H: int
    I: int
    E: int
    K: int
    wdtype: str                  # "float32" | "bf16" | "fp8"
    Ts: tuple
    weight_std: object           # float, or "fan_in" for 1/sqrt(fan_in)
    routing: str = "normal"      # "normal" | "zipf"
    zipf_s: float = 1.2
    notes: str = field(default="", compare=False)


CONFIGS = {
    "tiny": MoEConfig("tiny", H=128, I=64, E=8, K=2, wdtype="float32",
                      Ts=(4,), weight_std="fan_in"),
    "bf16_decode": MoEConfig("bf16_decode", H=4096, I=14336, E=8, K=2,
                             wdtype="bf16", Ts=(1, 8, 16, 64),
                             weight_std=0.02),
    "fp8_decode": MoEConfig("fp8_decode", H=7168, I=2048, E=256, K=8,
                            wdtype="fp8", Ts=(1, 8, 32, 64), weight_std=0.02),
    "fp8_tp8_slice": MoEConfig("fp8_tp8_slice", H=4096, I=192, E=128, K=8,
                               wdtype="fp8", Ts=(1, 16, 64, 256),
                               weight_std=0.02),
    "fp8_prefill_zipf": MoEConfig("fp8_prefill_zipf", H=7168, I=2048, E=256,
                                  K=8, wdtype="fp8", Ts=(4096,),
                                  weight_std=0.02, routing="zipf",
                                  zipf_s=1.2),
}

FP8_MAX = 448.0
E5M2_MAX = 57344.0
_FP8_TYPES = {"e4m3": (torch.float8_e4m3fn, FP8_MAX), "e5m2": (torch.float8_e5m2, E5M2_MAX)}
_ROLE_WEIGHTS = 1
_ROLE_TOKENS = 2


def _gen(device, seed, role, T=0):
    g = torch.Generator(device=device)
    g.manual_seed(((seed & 0xFFFF) << 40) | ((role & 0xFF) << 32) | (T & 0xFFFFFFFF))
    return g


def _std(cfg, fan_in):
    if cfg.weight_std == "fan_in":
        return 1.0 / math.sqrt(fan_in)
    return float(cfg.weight_std)


def fp8_codes_per_expert(w, fmt="e4m3"):
    """(uint8 codes, float32 scales) of float32 weights [E, R, C]; one scale per
    expert tensor, amax / max, via torch's float8 cast (e4m3fn or e5m2)."""
    dt, vmax = _FP8_TYPES[fmt]
    E = w.shape[0]
    amax = w.abs().reshape(E, -1).amax(dim=1).to(torch.float32)
    scale = torch.where(amax > 0, amax / vmax, torch.ones_like(amax))
    q = (w / scale.view(E, 1, 1)).clamp_(-vmax, vmax)
    return q.to(dt).view(torch.uint8), scale


def fp8_codes_per_row(w, fmt="e4m3"):
    """(uint8 codes, float32 scales [E, R]) of float32 weights [E, R, C]; one
    scale per expert row (output channel), amax / max, via torch's float8
    cast."""
    dt, vmax = _FP8_TYPES[fmt]
    amax = w.abs().amax(dim=2).to(torch.float32)
    scale = torch.where(amax > 0, amax / vmax, torch.ones_like(amax))
    q = (w / scale.unsqueeze(2)).clamp_(-vmax, vmax)
    return q.to(dt).view(torch.uint8), scale


def make_weights(cfg, seed=0, device="cpu", wdtype=None, chunk=8, scales="tensor",
                 fp8_format="e4m3"):
    """Expert weights of ``cfg``.

    Returns a dict with w13 [E, 2I, H] and w2 [E, H, I] (float32, bfloat16 or
    uint8 E4M3 codes) and, for E4M3, w13_scale and w2_scale: [E] float32, or
    with ``scales="row"`` one per output row, [E, 2I] and [E, H]; the codes
    are E4M3, or E5M2 with ``fp8_format="e5m2"`` (scale amax / 57344).
    ``wdtype`` overrides the configuration's storage type (the tiny float32
    case is also run as bfloat16 and as E4M3).  Experts are drawn ``chunk`` at a
    time to bound the float32 staging memory; the stream order is w13 of the
    chunk, then w2 of the chunk.
    """
    wdtype = wdtype or cfg.wdtype
    H, I, E = cfg.H, cfg.I, cfg.E
    g = _gen(device, seed, _ROLE_WEIGHTS)
    s13, s2 = _std(cfg, H), _std(cfg, I)
    store = {"float32": torch.float32, "bf16": torch.bfloat16,
             "fp8": torch.uint8}[wdtype]
    w13 = torch.empty(E, 2 * I, H, dtype=store, device=device)
    w2 = torch.empty(E, H, I, dtype=store, device=device)
    rows = scales == "row"
    sc13 = torch.empty((E, 2 * I) if rows else (E,), dtype=torch.float32, device=device)
    sc2 = torch.empty((E, H) if rows else (E,), dtype=torch.float32, device=device)
    quant = fp8_codes_per_row if rows else fp8_codes_per_expert
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        a = torch.randn(e1 - e0, 2 * I, H, generator=g, device=device) * s13
        b = torch.randn(e1 - e0, H, I, generator=g, device=device) * s2
        if wdtype == "fp8":
            w13[e0:e1], sc13[e0:e1] = quant(a, fp8_format)
            w2[e0:e1], sc2[e0:e1] = quant(b, fp8_format)
        else:
            w13[e0:e1] = a.to(store)
            w2[e0:e1] = b.to(store)
        del a, b
    out = {"w13": w13, "w2": w2, "wdtype": wdtype}
    if wdtype == "fp8":
        out["w13_scale"] = sc13
        out["w2_scale"] = sc2
        out["fp8_format"] = fp8_format
    return out


def zipf_bias(E, s):
    """log p_e with p_e proportional to (e + 1)^-s, normalised over E."""
    r = torch.arange(1, E + 1, dtype=torch.float64)
    p = r.pow(-s)
    p = p / p.sum()
    return p.log().to(torch.float32)


def make_tokens(cfg, T, seed=0, device="cpu"):
    """x [T, H] bfloat16 and router logits [T, E] float32 of ``cfg``."""
    g = _gen(device, seed, _ROLE_TOKENS, T)
    logits = torch.randn(T, cfg.E, generator=g, device=device)
    if cfg.routing == "zipf":
        logits = logits + zipf_bias(cfg.E, cfg.zipf_s).to(device)
    x = torch.randn(T, cfg.H, generator=g, device=device).to(torch.bfloat16)
    return {"x": x, "logits": logits.to(torch.float32).contiguous()}


def tie_heavy_logits(T, E, seed=0, device="cpu", levels=4):
    """Logits drawn from a few integer levels, so most rows hold ties."""
    g = _gen(device, seed, 3, T)
    v = torch.randint(0, levels, (T, E), generator=g, device=device)
    return v.to(torch.float32)


# ---------------------------------------------------------------------------
# The attention-side kernel the pages name next to the MoE layer: inverse
# rotary embedding of attention heads followed by per-head FP8 quantisation,
# called with a token count that changes from call to call (toolboxkart.tech
# page, section 3; aib.vote page, fourth paragraph).  The pages give no model;
# the shapes stand in for one GPU's share at 8-way tensor parallelism of a
# 128-head attention with 128-feature heads (16 heads per GPU), fully rotary
# (half layout), and a partly rotary variant (64 of 192 features, interleaved
# pairs).  Positions: a decode batch draws them at random below max_pos; a
# prefill batch is one sequence, positions 0..T-1.

@dataclass(frozen=True)
class RopeConfig:
    name: str
    NH: int                      # heads per token
    D: int                       # features per head
    R: int                       # rotated features (the rest pass through)
    interleaved: bool            # pairs (2i, 2i+1) instead of (i, i + R/2)
    max_pos: int
    base: float
    Ts: tuple


ROPE_CONFIGS = {
    "inv_rope_tp8": RopeConfig("inv_rope_tp8", NH=16, D=128, R=128, interleaved=False,
                               max_pos=32768, base=10000.0, Ts=(1, 16, 64, 4096)),
    "inv_rope_partial": RopeConfig("inv_rope_partial", NH=16, D=192, R=64, interleaved=True,
                                   max_pos=32768, base=10000.0, Ts=(1, 16, 64, 4096)),
}

_ROLE_HEADS = 4


def rope_table(max_pos, R, base=10000.0):
    """[max_pos, R] float32 table: cos of the R/2 angles p * base^(-2i/R) of
    position p, then their sin (computed in float64, rounded once)."""
    i = torch.arange(R // 2, dtype=torch.float64)
    inv_freq = base ** (-2.0 * i / R)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv_freq[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32).contiguous()


def make_heads(cfg, T, seed=0, device="cpu", prefill=None):
    """x [T, NH, D] bfloat16 ~ N(0, 1) and positions [T] int64 of ``cfg``:
    one sequence 0..T-1 when ``prefill`` (default: T > 64), else random
    positions below max_pos (a decode batch of independent sequences)."""
    g = _gen(device, seed, _ROLE_HEADS, T)
    x = torch.randn(T, cfg.NH, cfg.D, generator=g, device=device).to(torch.bfloat16)
    if prefill is None:
        prefill = T > 64
    if prefill:
        pos = torch.arange(T, dtype=torch.int64, device=device)
    else:
        pos = torch.randint(0, cfg.max_pos, (T,), generator=g, device=device, dtype=torch.int64)
    return {"x": x, "positions": pos}
