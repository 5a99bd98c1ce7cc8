"""Seeded synthetic workloads for the MoE FFN layer.

This module only draws random inputs and stores them in the storage formats
the layer consumes (float32, bfloat16, OCP FP8 E4M3 with per-128x128-block
float32 scales).  It holds none of the layer's arithmetic, so both the GPU
path and the CPU oracle can take their inputs from it.

Everything is drawn on the CPU with torch generators seeded per
(workload, tensor, expert), so any single expert can be regenerated on its own
and the values do not depend on the device they end up on.

Workloads (shapes from the models the pages describe: Mixtral 8x7B with 8
experts top-2, DeepSeek-V3 with 256 routed experts top-8 plus one shared
expert):

  0 tiny-fp32          T=64   d=128  N=8   k=2 d_ff=256   fp32, softmax
  1 mixtral-decode     T=16   d=4096 N=8   k=2 d_ff=14336 bf16, softmax
  2 mixtral-prefill    T=8192 d=4096 N=8   k=2 d_ff=14336 bf16, softmax
  3 dsv3-prefill       T=4096 d=7168 N=256 k=8 d_ff=2048  bf16, sigmoid+bias,
                       1 shared expert
  4 dsv3-decode-fp8    T=256  d=7168 N=256 k=8 d_ff=2048  fp8 weights, sigmoid
                       + bias, 1 shared expert, Zipf-skewed router offsets
  5, 6 the Mixtral decode and prefill shapes with MXFP4 expert weights (E2M1
                       codes, one E8M0 scale per 32 inputs)

Distributions: x ~ N(0, 1); router W ~ N(0, 1/d) in float32; W_gate, W_up ~
N(0, 1/d) and W_down ~ N(0, 1/d_ff) (fan-in scaling); selection bias ~
U(-0.1, 0.1); bfloat16 by round-to-nearest-even.  FP8 weights: per 128x128
block, scale = amax / 448 and the codes are the round-to-nearest E4M3 of
w / scale.

Skewed routing: the router gets a per-expert additive offset
-c * ln(rank_e) with rank a seeded permutation of 1..N (a Zipf-rank shape);
c = 0.25 puts the most loaded expert at about 8x the mean load.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, Optional

import torch

# tensor ids used in the seed formula
TID_X, TID_ROUTER, TID_BIAS, TID_ZIPF, TID_GATE, TID_UP, TID_DOWN = range(7)

FP8_BLOCK = 128
FP8_MAX = 448.0


@dataclass(frozen=True)
class MoEConfig:
    index: int
    name: str
    T: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    route: str           # "softmax" | "sigmoid"
    n_shared: int        # 0 or 1
    act_dtype: str       # "f32" | "bf16"  (x and out)
    w_dtype: str         # "f32" | "bf16" | "fp8" | "mxfp4"
    select_bias: bool    # U(-0.1, 0.1) selection-only bias (sigmoid router)
    zipf_c: Optional[float] = None  # router offset -c*ln(rank)

    def with_tokens(self, T: int) -> "MoEConfig":
        return replace(self, T=T)


CONFIGS = [
    MoEConfig(0, "tiny-fp32", 64, 128, 8, 2, 256, "softmax", 0, "f32", "f32", False),
    MoEConfig(1, "mixtral-decode", 16, 4096, 8, 2, 14336, "softmax", 0, "bf16", "bf16", False),
    MoEConfig(2, "mixtral-prefill", 8192, 4096, 8, 2, 14336, "softmax", 0, "bf16", "bf16", False),
    MoEConfig(3, "dsv3-prefill", 4096, 7168, 256, 8, 2048, "sigmoid", 1, "bf16", "bf16", True),
    MoEConfig(4, "dsv3-decode-fp8", 256, 7168, 256, 8, 2048, "sigmoid", 1, "bf16", "fp8", True, 0.25),
    # the Mixtral decode and prefill shapes with their experts in MXFP4
    MoEConfig(5, "mixtral-decode-mxfp4", 16, 4096, 8, 2, 14336, "softmax", 0, "bf16", "mxfp4",
              False),
    MoEConfig(6, "mixtral-prefill-mxfp4", 8192, 4096, 8, 2, 14336, "softmax", 0, "bf16", "mxfp4",
              False),
]


def seed_for(cfg: MoEConfig, tensor_id: int, e: int = 0) -> int:
    """Seed of one tensor: workload * 10^6 + tensor * 10^3 + expert."""
    return cfg.index * 1_000_000 + tensor_id * 1_000 + e


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def _to_storage(w: torch.Tensor, dtype: str):
    if dtype == "f32":
        return w.contiguous()
    if dtype == "bf16":
        return w.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def quantize_fp8_block(w: torch.Tensor):
    """float32 [R][C] -> (E4M3 codes uint8 [R][C], float32 scales
    [ceil(R/128)][ceil(C/128)]).  Data preparation only."""
    R, C = w.shape
    bR, bC = -(-R // FP8_BLOCK), -(-C // FP8_BLOCK)
    pad = torch.zeros(bR * FP8_BLOCK, bC * FP8_BLOCK, dtype=torch.float32)
    pad[:R, :C] = w
    blocks = pad.view(bR, FP8_BLOCK, bC, FP8_BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    q = q.view(bR * FP8_BLOCK, bC * FP8_BLOCK)[:R, :C].to(torch.float8_e4m3fn)
    return q.view(torch.uint8).contiguous(), scale.float().contiguous()


MX_BLOCK = 32
# midpoints between consecutive E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
_FP4_MID = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def quantize_mxfp4(w: torch.Tensor):
    """float32 [R][C] (C % 32 == 0) -> (packed E2M1 codes uint8 [R][C/2],
    element 2j in the low nibble; E8M0 scales uint8 [R][C/32]).  Data
    preparation only: per 32-element block the shared exponent is
    floor(log2(amax)) - 2 (the largest E2M1 magnitude is 1.5 * 2^2), values
    are divided by 2^exponent and rounded to the nearest E2M1 value (ties to
    the even code), saturating at 6."""
    R, C = w.shape
    b = w.float().reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = b.abs().amax(dim=2)
    ex = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
    ex = ex.clamp(-127, 127)
    v = (b / torch.exp2(ex)[..., None]).clamp(-6.0, 6.0)
    a = v.abs()
    mag = torch.bucketize(a, _FP4_MID)  # midpoints below |v| (a tie counts as above)
    tie = (mag < 7) & (a == _FP4_MID[mag.clamp(max=6)]) & (mag % 2 == 1)
    mag = (mag + tie.to(mag.dtype)).to(torch.uint8)  # a tie goes to the even code
    codes = (mag | torch.where(v < 0, 8, 0).to(torch.uint8)).reshape(R, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    return packed, (ex + 127).to(torch.uint8).contiguous()


def make_x(cfg: MoEConfig) -> torch.Tensor:
    """Token hidden states [T][d] in the activation storage type."""
    x = torch.randn(cfg.T, cfg.d_model, generator=_gen(seed_for(cfg, TID_X)))
    return _to_storage(x, cfg.act_dtype)


def make_router(cfg: MoEConfig) -> Dict[str, Optional[torch.Tensor]]:
    """Router weight [d][N] float32, optional selection bias [N] and optional
    logit offset [N] (float32)."""
    d, N = cfg.d_model, cfg.n_experts
    w = torch.randn(d, N, generator=_gen(seed_for(cfg, TID_ROUTER))) / math.sqrt(d)
    bias = None
    if cfg.select_bias:
        bias = torch.rand(N, generator=_gen(seed_for(cfg, TID_BIAS))) * 0.2 - 0.1
    offset = None
    if cfg.zipf_c is not None:
        rank = torch.randperm(N, generator=_gen(seed_for(cfg, TID_ZIPF))) + 1
        offset = (-cfg.zipf_c * torch.log(rank.double())).float()
    return {"w_router": w.float().contiguous(), "select_bias": bias,
            "logit_offset": offset}


def make_expert(cfg: MoEConfig, e: int) -> Dict[str, torch.Tensor]:
    """Expert e's weights in storage format, [out][in] row-major.

    e in [0, N) is a routed expert, e == N the shared expert.  Keys: gate
    [d_ff][d], up [d_ff][d], down [d][d_ff]; for fp8 also gate_scale,
    up_scale, down_scale (float32 per 128x128 block); for mxfp4 the matrices
    are packed codes [out][in/2] and the scales E8M0 bytes [out][in/32].
    """
    d, f = cfg.d_model, cfg.d_ff
    out = {}
    for key, tid, shape, fan_in in (("gate", TID_GATE, (f, d), d),
                                    ("up", TID_UP, (f, d), d),
                                    ("down", TID_DOWN, (d, f), f)):
        w = torch.randn(*shape, generator=_gen(seed_for(cfg, tid, e)))
        w.mul_(1.0 / math.sqrt(fan_in))
        if cfg.w_dtype == "fp8":
            q, s = quantize_fp8_block(w)
            out[key], out[key + "_scale"] = q, s
        elif cfg.w_dtype == "mxfp4":
            q, s = quantize_mxfp4(w)
            out[key], out[key + "_scale"] = q, s
        else:
            out[key] = _to_storage(w, cfg.w_dtype)
    return out


def for_each_expert(cfg: MoEConfig, fn, experts=None, threads: int = 16):
    """Generate experts in a thread pool and hand each to ``fn(e, weights)``
    in expert order (so the caller can copy it out and drop it)."""
    ids = list(range(cfg.n_experts + cfg.n_shared)) if experts is None else list(experts)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        futs = {}
        nxt = 0
        # keep a bounded window of experts in flight
        window = 2 * max(1, threads)
        for pos, e in enumerate(ids):
            while nxt < len(ids) and nxt < pos + window:
                futs[nxt] = ex.submit(make_expert, cfg, ids[nxt])
                nxt += 1
            fn(e, futs.pop(pos).result())


def storage_bytes_per_expert(cfg: MoEConfig) -> int:
    """Bytes of one expert's three matrices (plus FP8 scales)."""
    n = 3 * cfg.d_ff * cfg.d_model
    if cfg.w_dtype == "mxfp4":
        return n // 2 + n // MX_BLOCK
    if cfg.w_dtype == "fp8":
        nb = 3 * (-(-cfg.d_ff // FP8_BLOCK)) * (-(-cfg.d_model // FP8_BLOCK))
        return n + 4 * nb
    return n * (4 if cfg.w_dtype == "f32" else 2)
