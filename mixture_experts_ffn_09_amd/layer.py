"""Device-side setup of one MoE layer: upload a seeded workload's weights,
pack them with the library's pack entry point, own the workspace, and call
``moe_layer_forward``.  Glue only; all arithmetic is in the HIP library.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import torch

from . import moe
from .workloads import MoEConfig, for_each_expert, make_router, make_x


@dataclass
class DeviceLayer:
    cfg: MoEConfig
    shape: moe.Shape
    tensors: Dict[str, torch.Tensor] = field(default_factory=dict)
    weights: Optional[moe.Weights] = None

    def routing_buffers(self, T: Optional[int] = None) -> Dict[str, torch.Tensor]:
        T = self.cfg.T if T is None else T
        dev, k, N = "cuda", self.cfg.top_k, self.cfg.n_experts
        i32 = dict(dtype=torch.int32, device=dev)
        return {"topk_idx": torch.empty(T, k, **i32),
                "topk_w": torch.empty(T, k, dtype=torch.float32, device=dev),
                "counts": torch.empty(N, **i32), "offsets": torch.empty(N + 1, **i32),
                "perm_token": torch.empty(T * k, **i32), "inv_perm": torch.empty(T, k, **i32)}

    def shape_for(self, T: int) -> moe.Shape:
        s = moe.Shape.from_buffer_copy(self.shape)
        s.n_tokens = T
        return s

    def workspace(self, T: Optional[int] = None) -> torch.Tensor:
        n = moe.moe_workspace_bytes(self.shape_for(self.cfg.T if T is None else T))
        return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")

    def forward(self, x: torch.Tensor, ws: Optional[torch.Tensor] = None,
                routing: Optional[Dict[str, torch.Tensor]] = None) -> torch.Tensor:
        T = x.shape[0]
        out = torch.empty_like(x)
        ws = self.workspace(T) if ws is None else ws
        r = moe.make_routing(**routing) if routing is not None else None
        moe.moe_layer_forward(self.shape_for(T), self.weights, x, out, ws, r)
        return out


def _act_torch(cfg: MoEConfig):
    return torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16


def build_device_layer(cfg: MoEConfig, threads: int = 16,
                       edit: Optional[Callable[[int, dict], dict]] = None) -> DeviceLayer:
    """Generate cfg's weights expert by expert, upload and pack them.

    ``edit(e, weights)``, when given, may change expert e's generated
    weights (storage format, the keys of ``make_expert``) before upload."""
    shape = moe.make_shape(cfg.T, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff, cfg.n_shared,
                           cfg.route, cfg.act_dtype, cfg.w_dtype)
    dev = "cuda"
    L = DeviceLayer(cfg, shape)
    r = make_router(cfg)
    t = L.tensors
    t["w_router"] = r["w_router"].to(dev)
    if r["logit_offset"] is not None:
        t["logit_offset"] = r["logit_offset"].to(dev)
    if r["select_bias"] is not None:
        t["select_bias"] = r["select_bias"].to(dev)

    one = moe.Shape.from_buffer_copy(shape)
    b13 = moe.moe_packed_weight_bytes(one, 0, 1)
    b2 = moe.moe_packed_weight_bytes(one, 1, 1)
    N = cfg.n_experts
    t["w13"] = torch.empty(N * b13, dtype=torch.uint8, device=dev)
    t["w2"] = torch.empty(N * b2, dtype=torch.uint8, device=dev)
    fp8 = cfg.w_dtype == "fp8"
    scaled = cfg.w_dtype in ("fp8", "mxfp4")
    if fp8:   # float32 per 128x128 block
        sr13 = 2 * (cfg.d_ff // 128) * (cfg.d_model // 128)
        sr2 = (cfg.d_model // 128) * (cfg.d_ff // 128)
        sdt = torch.float32
    else:     # MXFP4: E8M0 bytes, repacked by the library (which = 2, 3)
        sr13 = moe.moe_packed_weight_bytes(one, 2, 1)
        sr2 = moe.moe_packed_weight_bytes(one, 3, 1)
        sdt = torch.uint8
    if scaled:
        t["w13_scale"] = torch.empty(N * sr13, dtype=sdt, device=dev)
        t["w2_scale"] = torch.empty(N * sr2, dtype=sdt, device=dev)
    if cfg.n_shared:
        t["w13_shared"] = torch.empty(b13, dtype=torch.uint8, device=dev)
        t["w2_shared"] = torch.empty(b2, dtype=torch.uint8, device=dev)
        if scaled:
            t["w13_shared_scale"] = torch.empty(sr13, dtype=sdt, device=dev)
            t["w2_shared_scale"] = torch.empty(sr2, dtype=sdt, device=dev)

    def upload(e, w):
        if edit is not None:
            w = edit(e, w)
        shared = e == N
        g = w["gate"].to(dev, non_blocking=False)
        u = w["up"].to(dev)
        dn = w["down"].to(dev)
        dst13 = t["w13_shared"] if shared else t["w13"][e * b13:(e + 1) * b13]
        dst2 = t["w2_shared"] if shared else t["w2"][e * b2:(e + 1) * b2]
        moe.moe_pack_weights(one, 0, 1, g, u, dst13)
        moe.moe_pack_weights(one, 1, 1, dn, None, dst2)
        if scaled:
            s13 = torch.cat([w["gate_scale"].reshape(-1), w["up_scale"].reshape(-1)]).to(dev)
            s2 = w["down_scale"].reshape(-1).to(dev)
            d13 = t["w13_shared_scale"] if shared else t["w13_scale"][e * sr13:(e + 1) * sr13]
            d2 = t["w2_shared_scale"] if shared else t["w2_scale"][e * sr2:(e + 1) * sr2]
            if fp8:   # natural layout
                d13.copy_(s13)
                d2.copy_(s2)
            else:     # natural [2][d_ff][d/32] and [d][d_ff/32] bytes -> packed
                moe.moe_pack_weights(one, 2, 1, s13, None, d13)
                moe.moe_pack_weights(one, 3, 1, s2, None, d2)
        torch.cuda.current_stream().synchronize()  # sources may be freed next

    for_each_expert(cfg, upload, threads=threads)
    L.weights = moe.make_weights(**t)
    return L


def device_x(cfg: MoEConfig) -> torch.Tensor:
    return make_x(cfg).to("cuda")
