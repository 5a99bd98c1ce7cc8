"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case, the full-size workloads included, compares every token's output
(and, at full size, every expert row) with the oracle.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_ffn_09_amd import moe, workloads as W
from mixture_experts_ffn_09_amd.layer import build_device_layer
from tests import _harness as H

pytestmark = pytest.mark.gpu

C = W.CONFIGS
SMALL = {
    "c1_tiny_f32": C[0],
    "c1_ragged_T37": H.small_config(C[0], 100, T=37),
    "c2_mixtral_decode": C[1],
    "c3_structure_T300": H.small_config(C[2], 101, T=300, d_model=512, d_ff=1024),
    "c4_structure_T37": H.small_config(C[3], 102, T=37, d_model=256, d_ff=128),
    "c5_structure_T64": H.small_config(C[4], 103, T=64, d_model=256, d_ff=256),
    "k_equals_n": H.small_config(C[2], 104, T=40, d_model=64, n_experts=4, top_k=4, d_ff=96),
    "single_token_sigmoid": H.small_config(C[3], 105, T=1, d_model=256, d_ff=128),
    "hot_expert_skew": H.small_config(C[4], 106, T=48, d_model=256, d_ff=128, w_dtype="bf16",
                                      zipf_c=6.0),
    "fp8_rows_over_64": H.small_config(C[4], 107, T=200, d_model=256, d_ff=256, n_experts=8,
                                       top_k=2),
    # tiled-GEMM path: 256-row tiles with a ragged last tile
    "gemm_bm256_ragged": H.small_config(C[2], 108, T=600, d_model=256, d_ff=256, n_experts=4),
    # routed and shared experts in one GEMM launch (128-row tiles)
    "gemm_routed_plus_shared": H.small_config(C[3], 109, T=160, d_model=256, d_ff=128,
                                              n_experts=16),
    # both row-tile classes in one layer: experts of 0..128 rows on 128-row
    # tiles, larger ones (up to 640 rows, three ragged 256-row tiles) and the
    # 640-row shared expert on 256-row tiles
    "gemm_row_classes": H.small_config(C[3], 114, T=640, d_model=256, d_ff=128, n_experts=32,
                                       zipf_c=1.5),
    # router logits through the LDS-ring kernel (T >= 1024, N % 128 == 0):
    # a ragged last token tile and an odd number of 32-K stages; then five
    # K splits, the last one a single stage
    "router_ring_T1100_d288": H.small_config(C[3], 115, T=1100, d_model=288, n_experts=128,
                                             d_ff=128),
    "router_ring_splits": H.small_config(C[3], 116, T=1024, d_model=1056, n_experts=128,
                                         d_ff=128),
    # the shape limits: 512 experts (eight per lane in the top-k wave) with
    # k = 16, and k = 64 (every lane of the wave holds a slot)
    "wide_router_N512_k16": H.small_config(C[3], 117, T=70, d_model=256, n_experts=512,
                                           top_k=16, d_ff=128),
    "many_slots_k64": H.small_config(C[2], 118, T=20, d_model=128, n_experts=100, top_k=64,
                                     d_ff=64),
    # the LDS-ring router at the widest N with a multi-block permute; and the
    # first batch past the fused small-batch router (T = 65, N = 8), which
    # takes the split-K logits and the separate top-k kernel
    "ring_N512_k16_T1024": H.small_config(C[3], 119, T=1024, d_model=256, n_experts=512,
                                          top_k=16, d_ff=128),
    "router_split_path_T65": H.small_config(C[1], 120, T=65, d_model=512, d_ff=256),
    # a last round of few tiles per XCD: its tiles (256, 128 and 64 rows) are
    # cut into 2 or 4 parts of the weight rows; routed only, and routed +
    # shared in one launch, both passes
    "gemm_split_tail": H.small_config(C[2], 121, T=512, d_model=2048, n_experts=4, d_ff=1024),
    "gemm_split_shared": H.small_config(C[3], 122, T=300, d_model=1024, n_experts=4, top_k=2,
                                        d_ff=1024),
    # groups of 257..512 rows (two row tiles each, the second 64, 128 or 256
    # rows tall): whole tiles, and last rounds cut into 2 or 4 parts, on both
    # passes
    "gemm_tall_parts": H.small_config(C[2], 125, T=1500, d_model=512, d_ff=1024, n_experts=8,
                                      zipf_c=0.3),
    "gemm_tall_whole": H.small_config(C[2], 128, T=1500, d_model=2048, d_ff=2048, n_experts=8,
                                      zipf_c=0.3),
    "gemm_tall_mixed": H.small_config(C[2], 129, T=1500, d_model=1280, d_ff=1536, n_experts=8,
                                      zipf_c=0.3),
    # FP8 weights through the GEMM path (routed + shared)
    "gemm_fp8": H.small_config(C[4], 110, T=256, d_model=256, d_ff=256, n_experts=8, top_k=4),
    # decode-sized batches: ragged T, odd N, sigmoid + selection bias + logit
    # offsets with a shared expert, fp32 x
    "decode_T5_N6": H.small_config(C[1], 111, T=5, d_model=288, n_experts=6, top_k=3,
                                   d_ff=96),
    "decode_sigmoid_T16": H.small_config(C[4], 112, T=16, d_model=128, n_experts=8, top_k=3,
                                         d_ff=128, w_dtype="bf16"),
    "decode_f32_N7": H.small_config(C[0], 113, T=11, d_model=96, n_experts=7, top_k=2),
    # MXFP4 expert weights (E2M1 codes, E8M0 scale per 32 inputs): decode,
    # 256 experts + shared with the sigmoid router, and many rows per expert
    # (streaming passes of 64 rows)
    "mxfp4_decode": H.small_config(C[1], 150, T=16, d_model=512, d_ff=1024, w_dtype="mxfp4"),
    "mxfp4_sigmoid_shared": H.small_config(C[3], 151, T=40, d_model=256, d_ff=256,
                                           w_dtype="mxfp4"),
    "mxfp4_many_rows": H.small_config(C[2], 152, T=300, d_model=256, d_ff=256, n_experts=4,
                                      w_dtype="mxfp4"),
    # MXFP4 weights through the four-wave GEMM (E2M1 codes and E8M0 scales
    # in LDS, decoded to bf16 on the way to the MFMAs): 256-row tiles with a
    # ragged last tile and last rounds cut into 2 or 4 parts; routed + shared
    # in one launch with the sigmoid router; whole tiles on the gate/up pass;
    # K = 768 and 384 (the last 512-input scale chunk partly used)
    "mxfp4_gemm_routed": H.small_config(C[6], 190, T=1200, d_model=512, d_ff=1024,
                                        n_experts=4),
    "mxfp4_gemm_shared": H.small_config(C[3], 191, T=800, d_model=512, d_ff=512, n_experts=16,
                                        top_k=2, w_dtype="mxfp4"),
    "mxfp4_gemm_parts": H.small_config(C[6], 192, T=512, d_model=2048, n_experts=4, d_ff=1024),
    "mxfp4_gemm_whole": H.small_config(C[6], 194, T=2048, d_model=1024, d_ff=2048,
                                       n_experts=4),
    "mxfp4_gemm_k768": H.small_config(C[6], 193, T=600, d_model=768, d_ff=384, n_experts=4),
    # skewed routing: MXFP4 groups of every row class, full-height tiles
    # (1 x 4 waves of 256 x 64) cut short by a group's end, on both passes
    "mxfp4_gemm_skew": H.small_config(C[6], 195, T=1500, d_model=512, d_ff=1024, n_experts=8,
                                      zipf_c=0.3),
    # odd K-step counts (3 on gate/up, 5 on down: a ring depth of 1) with a
    # hot expert of more than 32 rows in a 16-row launch (its 64-row passes)
    "stream_odd_ksteps_hot": H.small_config(C[1], 123, T=64, d_model=96, d_ff=160,
                                            zipf_c=3.0),
    # float32 activations with more than 8 experts: the tiled fp32 router
    "router_tiled_f32_N16": H.small_config(C[0], 124, T=100, n_experts=16, top_k=4),
}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_gpu(cfg):
    _log(f"[case] {cfg.name} idx={cfg.index} T={cfg.T} d={cfg.d_model} N={cfg.n_experts} "
         f"k={cfg.top_k} d_ff={cfg.d_ff} w={cfg.w_dtype}")
    L = build_device_layer(cfg)
    x = W.make_x(cfg)
    xd = x.to("cuda")
    rb = L.routing_buffers()
    out = L.forward(xd, routing=rb)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in rb.items()}
    return L, x, xd, out, g


def _check_case(cfg, x, out, g):
    xo = H.x_f64(cfg, x)
    w_r, off, bias = H.oracle_router(cfg)
    R = O.route_tokens(xo, w_r, cfg.top_k, cfg.route, off, bias)
    ref_idx, ties = H.resolve_routing(R, g["topk_idx"], cfg.top_k)
    ref_g = O.gate_weights(R.logits, ref_idx, cfg.route)
    H.check_gates(g["topk_idx"], g["topk_w"], ref_idx, ref_g)
    H.check_permutation(g, ref_idx, cfg.n_experts)
    shared = H.oracle_expert(cfg, cfg.n_experts) if cfg.n_shared else None
    ref, _, _, _ = O.moe_forward_with_routing(xo, ref_idx, ref_g,
                                              lambda e: H.oracle_expert(cfg, e),
                                              cfg.n_experts, shared)
    got = H.to_np(out)
    err = H.assert_close(got, ref, H.TOL[cfg.w_dtype])
    if cfg.w_dtype == "f32":
        H.assert_close(got, ref, H.TOL_F32_INTERNAL, "out (f32 internal bar)")
    _log(f"  ok: max abs err {err[0]:.3e}, max rel {err[1]:.3e}, ties {len(ties)}")
    return ref_idx, ties


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    cfg = SMALL[name]
    L, x, xd, out, g = _run_gpu(cfg)
    _check_case(cfg, x, out, g)


def _worst(got, ref, tol):
    """Largest |got - ref| / (tol (1 + |ref|)) (1.0 = at the bar)."""
    return float((np.abs(got - ref) / (tol * (1.0 + np.abs(ref)))).max())


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5, 6])
def test_layer_full_size(ci):
    """Each full-size workload on every token: routing, gates and the
    permutation against the oracle, the layer output of every token, and the
    expert rows y_perm / y_shared of a staged run (router, permute, grouped
    FFN, combine through their own entry points) row by row.  The oracle
    streams the experts (generated and decoded in parallel)."""
    cfg = C[ci]
    L, x, xd, out, g = _run_gpu(cfg)
    s, ws = L.shape_for(cfg.T), L.workspace()
    rb = L.routing_buffers()
    moe.moe_router_topk(s, xd, L.weights, rb["topk_idx"], rb["topk_w"], ws)
    moe.moe_permute(s, rb["topk_idx"], None, moe.make_routing(**rb), ws)
    y = torch.empty(cfg.T * cfg.top_k, cfg.d_model, dtype=xd.dtype, device="cuda")
    ys = torch.empty(cfg.T, cfg.d_model, dtype=xd.dtype, device="cuda") if cfg.n_shared else None
    moe.moe_grouped_ffn(s, xd, None, rb["perm_token"], rb["offsets"], L.weights, y, ys, ws)
    out2 = torch.empty_like(xd)
    moe.moe_combine(s, y, ys, rb["inv_perm"], rb["topk_w"], out2)
    torch.cuda.synchronize()
    for key, v in g.items():
        assert np.array_equal(v, rb[key].cpu().numpy()), key
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    got_out, got_y = H.to_np(out), H.to_np(y)
    got_ys = H.to_np(ys) if ys is not None else None
    del L, ws, y, ys, out2, rb
    torch.cuda.empty_cache()

    xo = H.x_f64(cfg, x)
    w_r, off, bias = H.oracle_router(cfg)
    R = O.route_tokens(xo, w_r, cfg.top_k, cfg.route, off, bias)
    ref_idx, ties = H.resolve_routing(R, g["topk_idx"], cfg.top_k)
    ref_g = O.gate_weights(R.logits, ref_idx, cfg.route)
    H.check_gates(g["topk_idx"], g["topk_w"], ref_idx, ref_g)
    H.check_permutation(g, ref_idx, cfg.n_experts)
    _log(f"  routing ok on all {cfg.T} tokens (near-ties {len(ties)}); oracle layer ...")
    ref, P, yref, ysref = H.oracle_layer(cfg, xo, ref_idx, ref_g)
    tol = H.TOL[cfg.w_dtype]
    err = H.assert_close(got_out, ref, tol)
    H.assert_close(got_y, yref, tol, "y_perm")
    worst = {"out": _worst(got_out, ref, tol), "y_perm": _worst(got_y, yref, tol)}
    if cfg.n_shared:
        H.assert_close(got_ys, ysref, tol, "y_shared")
        worst["y_shared"] = _worst(got_ys, ysref, tol)
    _log(f"  ok: {cfg.T} tokens, {cfg.T * cfg.top_k} expert rows; max abs err {err[0]:.3e}; "
         "worst err / bound " + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()))


@pytest.mark.parametrize("name", ["c4_structure_T37", "decode_sigmoid_T16"])
def test_stages_through_abi_match_layer_forward(name):
    """router -> permute (with x_perm) -> grouped_ffn -> combine, each
    through its own entry point, reproduces moe_layer_forward bit for bit,
    and the permuted gather is exactly x[perm_token]."""
    cfg = SMALL[name]
    L, x, xd, out, g = _run_gpu(cfg)
    s = L.shape_for(cfg.T)
    ws = L.workspace()
    rb = L.routing_buffers()
    moe.moe_router_topk(s, xd, L.weights, rb["topk_idx"], rb["topk_w"], ws)
    x_perm = torch.empty(cfg.T * cfg.top_k, cfg.d_model, dtype=xd.dtype, device="cuda")
    moe.moe_permute(s, rb["topk_idx"], xd, moe.make_routing(**rb), ws, x_perm)
    y = torch.empty(cfg.T * cfg.top_k, cfg.d_model, dtype=xd.dtype, device="cuda")
    ys = torch.empty(cfg.T, cfg.d_model, dtype=xd.dtype, device="cuda")
    moe.moe_grouped_ffn(s, xd, x_perm, None, rb["offsets"], L.weights, y, ys, ws)
    out2 = torch.empty_like(xd)
    moe.moe_combine(s, y, ys, rb["inv_perm"], rb["topk_w"], out2)
    # the other input path: x plus perm_token instead of x_perm
    y3 = torch.empty_like(y)
    ys3 = torch.empty_like(ys)
    moe.moe_grouped_ffn(s, xd, None, rb["perm_token"], rb["offsets"], L.weights, y3, ys3, ws)
    # and the two per-row entry points
    h4 = torch.empty(cfg.T * cfg.top_k, cfg.d_ff, dtype=xd.dtype, device="cuda")
    hs4 = torch.empty(cfg.T, cfg.d_ff, dtype=xd.dtype, device="cuda")
    y4 = torch.empty_like(y)
    ys4 = torch.empty_like(ys)
    moe.moe_expert_gate_up(s, xd, None, rb["perm_token"], rb["offsets"], L.weights, h4, hs4, ws)
    moe.moe_expert_down(s, h4, hs4, rb["offsets"], L.weights, y4, ys4, ws)
    torch.cuda.synchronize()
    for key, v in g.items():  # routing from the staged calls = from the single call
        assert np.array_equal(v, rb[key].cpu().numpy()), key
    assert torch.equal(y.view(torch.int16), y4.view(torch.int16))
    assert torch.equal(ys.view(torch.int16), ys4.view(torch.int16))
    assert torch.equal(x_perm, xd[rb["perm_token"].long()])
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(y.view(torch.int16), y3.view(torch.int16))
    assert torch.equal(ys.view(torch.int16), ys3.view(torch.int16))
    # per-row expert outputs against the oracle
    xo = H.x_f64(cfg, x)
    idx = rb["topk_idx"].cpu().numpy()
    P = O.permute_assignments(idx, cfg.n_experts)
    yref = np.zeros((cfg.T * cfg.top_k, cfg.d_model))
    for e in range(cfg.n_experts):
        lo, hi = P.offsets[e], P.offsets[e + 1]
        if hi > lo:
            yref[lo:hi] = O.swiglu_expert(xo[P.perm_token[lo:hi]], *H.oracle_expert(cfg, e))
    H.assert_close(H.to_np(y), yref, H.TOL["bf16"], "y_perm")
    H.assert_close(H.to_np(ys), O.swiglu_expert(xo, *H.oracle_expert(cfg, cfg.n_experts)),
                   H.TOL["bf16"], "y_shared")


@pytest.mark.parametrize("name", ["c5_structure_T64", "gemm_split_shared", "ring_N512_k16_T1024"])
def test_deterministic_and_workspace_independent(name):
    """Bitwise-equal outputs across calls and whatever the workspace held
    (streaming path; GEMM with last-round tiles cut into parts; LDS-ring
    router logits)."""
    cfg = SMALL[name]
    L, x, xd, out, g = _run_gpu(cfg)
    ws = L.workspace()
    ws.fill_(0xFF)
    out2 = L.forward(xd, ws=ws)
    ws.fill_(0)
    out3 = L.forward(xd, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out3.view(torch.int16))


def test_token_independence_on_gpu():
    """Permuting token rows permutes output rows (tokens are independent)."""
    cfg = SMALL["c3_structure_T300"]
    L, x, xd, out, g = _run_gpu(cfg)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(cfg.T)).cuda()
    out_p = L.forward(xd[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out[perm].view(torch.int16))


def test_zero_tokens_is_a_noop():
    cfg = SMALL["c4_structure_T37"]
    L = build_device_layer(cfg)
    s = L.shape_for(0)
    x = torch.empty(0, cfg.d_model, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    moe.moe_layer_forward(s, L.weights, x, out, ws)
    assert moe.moe_workspace_bytes(s) == 0


@pytest.mark.parametrize("T,N,k", [(1000, 300, 5), (16, 8, 2), (256, 512, 8), (4096, 256, 8)])
def test_permute_direct_against_sorted(T, N, k):
    """moe_permute on given ids (several 256-token blocks, a ragged tail,
    N above 256): counts, offsets and rows equal a Python sort of the valid
    (expert, token, slot) keys; out-of-range ids are not counted and map to
    -1; a token listing an expert twice gets consecutive rows."""
    rng = np.random.default_rng(T + N + k)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32)
    if T > 20:
        idx[3, 0] = -1
        idx[7, k - 1] = N + 3
        idx[11, 1] = idx[11, 0]  # duplicate within a token
    s = moe.make_shape(T, 64, N, k, 64)
    dev = "cuda"
    r = {"counts": torch.empty(N, dtype=torch.int32, device=dev),
         "offsets": torch.empty(N + 1, dtype=torch.int32, device=dev),
         "perm_token": torch.full((T * k,), -7, dtype=torch.int32, device=dev),
         "inv_perm": torch.empty(T, k, dtype=torch.int32, device=dev)}
    ws = torch.empty(moe.moe_workspace_bytes(s), dtype=torch.uint8, device=dev)
    moe.moe_permute(s, torch.from_numpy(idx).to(dev), None, moe.make_routing(**r), ws)
    torch.cuda.synchronize()
    g = {kk: v.cpu().numpy() for kk, v in r.items()}
    keys = sorted((int(idx[t, i]), t, i) for t in range(T) for i in range(k) if 0 <= idx[t, i] < N)
    nvalid = len(keys)
    cnt = np.zeros(N, dtype=np.int64)
    for e, _, _ in keys:
        cnt[e] += 1
    assert np.array_equal(g["counts"], cnt)
    assert np.array_equal(g["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
    assert list(g["perm_token"][:nvalid]) == [t for _, t, _ in keys]
    want_inv = np.full((T, k), -1)
    for row, (e, t, i) in enumerate(keys):
        want_inv[t, i] = row
    assert np.array_equal(g["inv_perm"], want_inv)


def test_eight_wave_gemm_past_32bit_offsets():
    """A batch whose H buffer (T k d_ff bf16) passes 2^31 bytes takes the
    eight-wave GEMM (128-row tiles, 64-bit operand addresses) instead of the
    four-wave one; every token against the oracle."""
    cfg = H.small_config(C[2], 160, T=70000, d_model=256, n_experts=16, top_k=8, d_ff=2048)
    assert cfg.T * cfg.top_k * cfg.d_ff * 2 > 0x7FFFFFFF
    L, x, xd, out, g = _run_gpu(cfg)
    del L
    torch.cuda.empty_cache()
    _check_case(cfg, x, out, g)


@pytest.mark.parametrize("T,N,k,nan_experts,bf16_x", [(20, 8, 2, (1, 4), True),
                                                      (20, 8, 7, (1, 4), True),
                                                      (100, 16, 4, (0, 5, 6), True),
                                                      (100, 16, 15, (0, 5, 6), False)])
def test_nan_scores_rank_last(T, N, k, nan_experts, bf16_x):
    """Experts whose logit offset is NaN rank below every other expert (lower
    index first among them), on the fused small-batch router and on the
    separate top-k kernel: ids equal the oracle's and stay in [0, N); gates
    equal the oracle's, NaN exactly where a NaN expert had to be taken."""
    base = C[1] if bf16_x else C[0]
    cfg = H.small_config(base, 161, T=T, d_model=128, n_experts=N, top_k=k, d_ff=64)
    _log(f"[case] nan scores T={T} N={N} k={k} nan={nan_experts} bf16_x={bf16_x}")
    L = build_device_layer(cfg)
    off = torch.zeros(N)
    off[list(nan_experts)] = float("nan")
    t = dict(L.tensors)
    t["logit_offset"] = off.cuda()
    w = moe.make_weights(**t)
    x = W.make_x(cfg)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_router_topk(L.shape_for(T), x.cuda(), w, idx, gw, L.workspace())
    torch.cuda.synchronize()
    gi, gg = idx.cpu().numpy(), gw.cpu().numpy()
    w_r, _, bias = H.oracle_router(cfg)
    R = O.route_tokens(H.x_f64(cfg, x), w_r, k, cfg.route, off.double().numpy(), bias)
    assert ((gi >= 0) & (gi < N)).all()
    ref_idx, _ = H.resolve_routing(R, gi, k)
    assert np.array_equal(gi, ref_idx)
    ref_g = O.gate_weights(R.logits, ref_idx, cfg.route)
    assert np.array_equal(np.isnan(gg), np.isnan(ref_g))
    ok = ~np.isnan(ref_g)
    assert np.all(np.abs(gg[ok] - ref_g[ok]) <= 1e-5)
    assert np.isnan(ref_g).any() == (k > N - len(nan_experts))


def _plant_scale_codes(cfg, seed):
    """An ``edit`` for the expert weights: in every expert, some 32-element
    blocks of each matrix get the E8M0 scale codes 0, 1 and 2 (2^-127,
    2^-126, 2^-125: the first a denormal float32), and each routed expert's
    down matrix gets code 255 (NaN) in one block of one row."""
    def edit(e, w):
        w = dict(w)
        rng = np.random.default_rng(seed * 1000 + e)
        for key in ("gate", "up", "down"):
            s = w[key + "_scale"].clone()
            R, B = s.shape
            for code in (0, 1, 2):
                for _ in range(3):
                    s[int(rng.integers(R)), int(rng.integers(B))] = code
            if key == "down" and e < cfg.n_experts:
                s[(7 * e + 3) % R, int(rng.integers(B))] = 255
            w[key + "_scale"] = s
        return w
    return edit


@pytest.mark.parametrize("name,cfg", [
    ("stream", H.small_config(C[1], 170, T=16, d_model=512, d_ff=1024, w_dtype="mxfp4")),
    ("stream_shared", H.small_config(C[3], 171, T=40, d_model=256, d_ff=256, w_dtype="mxfp4")),
    ("gemm", H.small_config(C[6], 172, T=1200, d_model=512, d_ff=1024)),
])
def test_mxfp4_extreme_scale_codes(name, cfg):
    """MXFP4 weights whose E8M0 scales take the extreme codes: 0..2 decode
    to 2^-127..2^-125 and 255 to NaN.  The layer's output is NaN exactly
    where the oracle's is (the down rows carrying a NaN scale, for the tokens
    routed to that expert) and equals it everywhere else."""
    assert cfg.w_dtype == "mxfp4"
    edit = _plant_scale_codes(cfg, cfg.index)
    _log(f"[case] mxfp4 scale codes {name} T={cfg.T} d={cfg.d_model} N={cfg.n_experts} "
         f"k={cfg.top_k} d_ff={cfg.d_ff}")
    L = build_device_layer(cfg, edit=edit)
    x = W.make_x(cfg)
    rb = L.routing_buffers()
    out = L.forward(x.to("cuda"), routing=rb)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in rb.items()}
    xo = H.x_f64(cfg, x)
    w_r, off, bias = H.oracle_router(cfg)
    R = O.route_tokens(xo, w_r, cfg.top_k, cfg.route, off, bias)
    ref_idx, _ = H.resolve_routing(R, g["topk_idx"], cfg.top_k)
    ref_g = O.gate_weights(R.logits, ref_idx, cfg.route)
    shared = H.oracle_expert(cfg, cfg.n_experts, edit) if cfg.n_shared else None
    ref, _, _, _ = O.moe_forward_with_routing(xo, ref_idx, ref_g,
                                              lambda e: H.oracle_expert(cfg, e, edit),
                                              cfg.n_experts, shared)
    got = H.to_np(out)
    nan = np.isnan(ref)
    assert nan.any() and not nan.all()
    assert np.array_equal(np.isnan(got), nan)
    err = H.assert_close(got[~nan], ref[~nan], H.TOL[cfg.w_dtype])
    _log(f"  ok: {int(nan.sum())} NaN outputs where the oracle's are, max abs err {err[0]:.3e}")
