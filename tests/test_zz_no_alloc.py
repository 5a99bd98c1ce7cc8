"""moe_layer_forward_noalloc (static device scratch, no allocation) against
moe_layer_forward (caller workspace): the same kernels, so outputs and
routing must agree bit for bit, on consecutive calls whose second batch is
smaller (the shared scratch keeps the previous call's contents)."""

import ctypes as C
import sys

import pytest
import torch

from mixture_experts_ffn_09_amd import moe, workloads as W
from mixture_experts_ffn_09_amd.layer import build_device_layer
from tests import _harness as H

CW = W.CONFIGS


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_oversized_shape_is_rejected_on_the_host():
    """A shape whose workspace passes the static scratch is refused before
    any HIP call (no GPU needed)."""
    c = CW[2]  # Mixtral prefill, T = 8192: about 580 MiB of scratch
    s = moe.make_shape(c.T, c.d_model, c.n_experts, c.top_k, c.d_ff)
    assert moe.moe_workspace_bytes(s) > (64 << 20)
    fake = C.c_void_p(0x1000)
    w = moe.Weights(w_router=0x1000, w13=0x1000, w2=0x1000)
    st = moe.lib().moe_layer_forward_noalloc(C.byref(s), C.byref(w), fake, C.c_void_p(0x2000),
                                             None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    assert b"scratch" in moe.lib().moe_last_error()


CASES = [
    # the DeepSeek-V3-shaped fp8 decode workload at full size (58 MiB of
    # scratch), then 37 of its tokens
    (CW[4], (256, 37)),
    # the Mixtral-shaped decode workload (16 tokens), then 5
    (CW[1], (16, 5)),
    # a reduced prefill-shaped layer through the tiled GEMM (routed + shared),
    # then a batch small enough for the streaming kernel
    (H.small_config(CW[3], 170, T=640, d_model=256, d_ff=128, n_experts=32, zipf_c=1.5),
     (640, 24)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_noalloc_matches_layer_forward(ci):
    cfg, sizes = CASES[ci]
    _log(f"[case] noalloc {cfg.name} idx={cfg.index} T={sizes}")
    L = build_device_layer(cfg)
    x_all = W.make_x(cfg).to("cuda")
    for T in sizes:
        x = x_all[:T].contiguous()
        s = L.shape_for(T)
        assert moe.moe_workspace_bytes(s) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        ref = torch.empty_like(x)
        rref = L.routing_buffers(T)
        moe.moe_layer_forward(s, L.weights, x, ref, L.workspace(T), moe.make_routing(**rref))
        got = torch.full_like(x, float("nan"))
        rgot = {k: torch.full_like(v, -5) for k, v in L.routing_buffers(T).items()}
        moe.moe_layer_forward_noalloc(s, L.weights, x, got, moe.make_routing(**rgot))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), T
        for k in rref:
            assert torch.equal(rgot[k], rref[k]), (T, k)
        _log(f"  T={T}: bit-exact")
