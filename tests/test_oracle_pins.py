"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function checks one part of the oracle against what the pages
print, a closed form, a library routine, or brute force; the test functions
call them, and ``test_planted_mistakes_are_caught`` plants plausible mistakes
in the oracle (on the CPU) and checks that some pin fails for each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from tests import _brute as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close_at(printed, value, decimals):
    """``value`` rounds to ``printed`` at the page's printed precision."""
    return abs(value - printed) <= 0.5 * 10 ** (-decimals) + 1e-12


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_router_worked_example_skillsuites():
    g = _golden("router_worked_example_skillsuites.json")
    logits = np.array([g["logits"]])
    scores = O.selection_scores(logits, "softmax")
    idx = O.top_k_select(scores, g["top_k"])
    assert [int(e) + 1 for e in idx[0]] == g["selected_1based"]
    gates = O.gate_weights(logits, idx, "softmax")[0]
    for p, v in zip(g["gates"], gates):
        assert _close_at(p, v, g["gates_decimals"]), (p, v)
    assert abs(gates.sum() - 1.0) < 1e-12
    # the exponentials the page prints
    for p, e in zip(g["exp_selected"], idx[0]):
        assert _close_at(p, math.exp(g["logits"][e]), g["exp_decimals"])
    # softmax over all eight (the contrast the page draws)
    full = np.exp(logits[0] - logits[0].max())
    full /= full.sum()
    sel = full[idx[0]]
    for p, v in zip(g["full_softmax_selected"], sel):
        assert _close_at(p, v, g["full_softmax_decimals"]), (p, v)
    assert _close_at(g["full_softmax_sum"], sel.sum(), g["full_softmax_decimals"])


def _page12_logits(g):
    total = g["exp_total"]
    p3, p6 = g["probabilities"]
    l = np.full(8, math.log((total - total * p3 - total * p6) / 6.0))
    l[2] = math.log(p3 * total)
    l[5] = math.log(p6 * total)
    return l


def pin_router_worked_example_ai_infra():
    g = _golden("router_worked_example_ai_infra_part12.json")
    logits = _page12_logits(g)[None, :]
    assert _close_at(g["exp_total"], np.exp(logits).sum(), g["exp_total_decimals"])
    idx = O.top_k_select(O.selection_scores(logits, "softmax"), g["top_k"])
    assert [int(e) + 1 for e in idx[0]] == g["selected_1based"]
    p = np.exp(logits[0]) / np.exp(logits[0]).sum()
    for pr, v in zip(g["probabilities"], p[idx[0]]):
        assert _close_at(pr, v, g["probabilities_decimals"])
    assert _close_at(g["probability_sum"], p[idx[0]].sum(), g["probabilities_decimals"])
    gates = O.gate_weights(logits, idx, "softmax")[0]
    for pr, v in zip(g["mixing_weights"], gates):
        assert _close_at(pr, v, g["mixing_weights_decimals"]), (pr, v)
    # combine: the layer output is the gate-weighted sum of the two expert
    # vectors; with the printed 2-decimal weights the result may differ by at
    # most 0.005 * (|a| + |b|) per element.
    e3 = np.array(g["expert_outputs"]["E3"])
    e6 = np.array(g["expert_outputs"]["E6"])
    y = np.stack([e3, e6])                     # rows in slot order
    out = O.combine(y, gates[None, :], np.array([[0, 1]]))[0]
    printed = g["mixing_weights"][0] * e3 + g["mixing_weights"][1] * e6
    assert np.all(np.abs(out - printed) <= 0.005 * (np.abs(e3) + np.abs(e6)) + 1e-12)


def pin_softmax_placement_equivalence(seed=0):
    """Softmax over the selected logits == softmax over all, keep top-k,
    renormalise (Chapter 19, 19.3.2)."""
    rng = np.random.default_rng(seed)
    for N, k in ((8, 2), (16, 4), (256, 8)):
        logits = rng.normal(0, 2, size=(64, N))
        idx = O.top_k_select(O.selection_scores(logits, "softmax"), k)
        g = O.gate_weights(logits, idx, "softmax")
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ps = np.take_along_axis(p, idx, axis=1)
        ref = ps / ps.sum(axis=1, keepdims=True)
        assert np.max(np.abs(g - ref) / ref) <= 1e-12
        # selected probabilities are the k largest
        kth = np.sort(p, axis=1)[:, -k]
        assert np.all(ps.min(axis=1) >= kth - 1e-15)


def pin_brute_force_routing(seed=1):
    rng = np.random.default_rng(seed)
    for route in ("softmax", "sigmoid"):
        for N, k in ((4, 2), (6, 3), (8, 2), (5, 5), (7, 1)):
            logits = rng.normal(0, 1.5, size=(12, N))
            logits[0, :] = 0.25                       # exact ties
            logits[1, 1] = logits[1, 3]               # a pair tie
            bias = rng.uniform(-0.1, 0.1, size=N) if route == "sigmoid" else None
            sc = O.selection_scores(logits, route, bias)
            idx = O.top_k_select(sc, k)
            g = O.gate_weights(logits, idx, route)
            for t in range(logits.shape[0]):
                row = [float(v) for v in logits[t]]
                if route == "softmax":
                    sel, gb = B.route_softmax_all_renorm(row, k)
                else:
                    sel, gb = B.route_sigmoid_bias(row, k, [float(b) for b in bias])
                assert list(idx[t]) == sel, (route, N, k, t, idx[t], sel)
                assert np.allclose(g[t], gb, rtol=1e-12, atol=1e-15)


def pin_sigmoid_invariants(seed=2):
    rng = np.random.default_rng(seed)
    T, N, k = 32, 16, 4
    logits = rng.normal(0, 1, size=(T, N))
    # (1) gates sum to one
    bias = rng.uniform(-0.1, 0.1, N)
    idx = O.top_k_select(O.selection_scores(logits, "sigmoid", bias), k)
    g = O.gate_weights(logits, idx, "sigmoid")
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
    # (2) the bias moves selection, never the weights: a bias that keeps the
    # selection keeps the gates bit for bit
    idx0 = O.top_k_select(O.selection_scores(logits, "sigmoid", None), k)
    tiny = np.full(N, 1e-30)
    idx1 = O.top_k_select(O.selection_scores(logits, "sigmoid", tiny), k)
    assert np.array_equal(idx0, idx1)
    g0 = O.gate_weights(logits, idx0, "sigmoid")
    g1 = O.gate_weights(logits, idx1, "sigmoid")
    assert np.array_equal(g0, g1)
    # a big bias on expert 0 forces it in; its weight is its unbiased affinity
    big = np.zeros(N)
    big[0] = 10.0
    idx2 = O.top_k_select(O.selection_scores(logits, "sigmoid", big), k)
    assert np.all(idx2[:, 0] == 0)
    g2 = O.gate_weights(logits, idx2, "sigmoid")
    a = 1.0 / (1.0 + np.exp(-logits))
    asel = np.take_along_axis(a, idx2, axis=1)
    assert np.allclose(g2, asel / asel.sum(axis=1, keepdims=True), rtol=1e-13)
    # (3) equal logits, zero bias -> uniform 1/k on the k lowest indices
    eq = np.zeros((3, N))
    idx3 = O.top_k_select(O.selection_scores(eq, "sigmoid", None), k)
    assert np.array_equal(idx3, np.tile(np.arange(k), (3, 1)))
    assert np.allclose(O.gate_weights(eq, idx3, "sigmoid"), 1.0 / k, atol=1e-15)
    # (4) k = N, zero bias -> sigmoid / sum of sigmoids
    idx4 = O.top_k_select(O.selection_scores(logits, "sigmoid", None), N)
    g4 = O.gate_weights(logits, idx4, "sigmoid")
    full = a / a.sum(axis=1, keepdims=True)
    assert np.allclose(g4, np.take_along_axis(full, idx4, axis=1), rtol=1e-13)


def pin_sigmoid_function():
    z = np.array([-800.0, -30.0, -1.0, 0.0, 1.0, 30.0, 800.0])
    s = O.sigmoid(z)
    ref = [B.sig(float(v)) for v in z]
    assert np.allclose(s, ref, rtol=1e-15, atol=0)
    assert s[3] == 0.5 and np.all(np.isfinite(s))


def pin_router_logits_brute(seed=3):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(5, 7))
    w = rng.normal(size=(7, 4))
    off = rng.normal(size=4)
    got = O.router_logits(x, w, off)
    ref = B.matvec_rows(x.tolist(), w.tolist())
    ref = [[v + off[e] for e, v in enumerate(row)] for row in ref]
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)


def pin_permutation(seed=4):
    rng = np.random.default_rng(seed)
    for T, N, k in ((1, 4, 2), (37, 8, 2), (64, 16, 4), (100, 256, 8), (5, 5, 5)):
        idx = np.stack([rng.permutation(N)[:k] for _ in range(T)])
        p = O.permute_assignments(idx, N)
        assert p.counts.sum() == T * k
        assert np.array_equal(p.counts, [sum(int(v == e) for v in idx.reshape(-1)) for e in range(N)])
        assert p.offsets[0] == 0 and p.offsets[-1] == T * k
        assert np.all(np.diff(p.offsets) == p.counts)
        # bijection
        assert np.array_equal(np.sort(p.inv_perm.reshape(-1)), np.arange(T * k))
        # brute force: Python sorted() of (expert, token, slot)
        keys = sorted((int(idx[t, i]), t, i) for t in range(T) for i in range(k))
        assert [t for _, t, _ in keys] == list(p.perm_token)
        assert [i for _, _, i in keys] == list(p.perm_slot)
        for r, (e, t, i) in enumerate(keys):
            assert p.inv_perm[t, i] == r
            assert p.offsets[e] <= r < p.offsets[e + 1]
    # empty experts are allowed
    idx = np.zeros((10, 1), dtype=np.int64)
    p = O.permute_assignments(idx, 3)
    assert list(p.counts) == [10, 0, 0] and list(p.offsets) == [0, 10, 10, 10]


def _tiny_layer(rng, T=4, d=8, N=4, k=2, d_ff=6, shared=False):
    x = rng.normal(size=(T, d))
    w_r = rng.normal(size=(d, N)) / math.sqrt(d)
    experts = [(rng.normal(size=(d_ff, d)) / math.sqrt(d), rng.normal(size=(d_ff, d)) / math.sqrt(d),
                rng.normal(size=(d, d_ff)) / math.sqrt(d_ff)) for _ in range(N)]
    sh = None
    if shared:
        sh = (rng.normal(size=(d_ff, d)), rng.normal(size=(d_ff, d)), rng.normal(size=(d, d_ff)))
    return x, w_r, experts, sh


def pin_layer_brute_force(seed=5):
    rng = np.random.default_rng(seed)
    for route, shared in (("softmax", False), ("sigmoid", True), ("sigmoid", False)):
        x, w_r, experts, sh = _tiny_layer(rng, shared=shared)
        bias = rng.uniform(-0.1, 0.1, size=4) if route == "sigmoid" else None
        off = rng.normal(size=4) * 0.3
        out, _, _ = O.moe_forward(x, w_r, experts, 2, route, logit_offset=off,
                                  select_bias=bias, shared=sh)
        tolist = lambda m: np.asarray(m).tolist()
        ref = B.moe_layer(tolist(x), tolist(w_r),
                          [tuple(tolist(m) for m in ex) for ex in experts], 2, route,
                          None if bias is None else tolist(bias),
                          None if sh is None else tuple(tolist(m) for m in sh),
                          offset=tolist(off))
        assert np.allclose(out, ref, rtol=1e-10, atol=1e-12), (route, shared)


def _dense_swiglu_torch(x, wg, wu, wd):
    X = torch.from_numpy(np.asarray(x, dtype=np.float64))
    g = X @ torch.from_numpy(wg).T
    u = X @ torch.from_numpy(wu).T
    return (torch.nn.functional.silu(g) * u @ torch.from_numpy(wd).T).numpy()


def pin_identical_experts_equal_dense(seed=6):
    """With every expert identical and gates summing to 1, the layer is the
    dense FFN ("same scale a dense FFN would have produced"); checked against
    torch's float64 silu + matmul at k = N and k < N, with a shared expert."""
    rng = np.random.default_rng(seed)
    T, d, d_ff = 24, 32, 48
    x = rng.normal(size=(T, d))
    W = (rng.normal(size=(d_ff, d)) / math.sqrt(d), rng.normal(size=(d_ff, d)) / math.sqrt(d),
         rng.normal(size=(d, d_ff)) / math.sqrt(d_ff))
    S = (rng.normal(size=(d_ff, d)) / math.sqrt(d), rng.normal(size=(d_ff, d)) / math.sqrt(d),
         rng.normal(size=(d, d_ff)) / math.sqrt(d_ff))
    dense = _dense_swiglu_torch(x, *W)
    dense_s = _dense_swiglu_torch(x, *S)
    for route in ("softmax", "sigmoid"):
        for N, k in ((8, 8), (8, 2), (16, 5)):
            w_r = rng.normal(size=(d, N))
            bias = rng.uniform(-0.1, 0.1, N) if route == "sigmoid" else None
            out, _, _ = O.moe_forward(x, w_r, [W] * N, k, route, select_bias=bias)
            assert np.allclose(out, dense, rtol=1e-12, atol=1e-12)
            out2, _, _ = O.moe_forward(x, w_r, [W] * N, k, route, select_bias=bias, shared=S)
            assert np.allclose(out2, dense + dense_s, rtol=1e-12, atol=1e-12)


def pin_distinct_experts_k_equals_n(seed=7):
    """k = N with distinct experts: out = sum_e softmax(s)_e * FFN_e(x) over
    all experts (no selection left), against torch float64."""
    rng = np.random.default_rng(seed)
    T, d, d_ff, N = 10, 16, 24, 4
    x, w_r, experts, _ = _tiny_layer(rng, T, d, N, N, d_ff)
    out, _, _ = O.moe_forward(x, w_r, experts, N, "softmax")
    s = torch.from_numpy(x @ w_r)
    p = torch.softmax(s, dim=1).numpy()
    ref = sum(p[:, e:e + 1] * _dense_swiglu_torch(x, *experts[e]) for e in range(N))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def pin_token_independence_and_relabel(seed=8):
    rng = np.random.default_rng(seed)
    x, w_r, experts, sh = _tiny_layer(rng, T=16, d=12, N=6, k=3, d_ff=10, shared=True)
    out, _, _ = O.moe_forward(x, w_r, experts, 3, "softmax", shared=sh)
    pr = rng.permutation(16)
    out_p, _, _ = O.moe_forward(x[pr], w_r, experts, 3, "softmax", shared=sh)
    assert np.allclose(out_p, out[pr], rtol=1e-13, atol=1e-13)
    pe = rng.permutation(6)
    out_e, _, _ = O.moe_forward(x, w_r[:, pe], [experts[e] for e in pe], 3, "softmax", shared=sh)
    assert np.allclose(out_e, out, rtol=1e-13, atol=1e-13)


def pin_bf16_decoder():
    codes = np.arange(65536, dtype=np.uint16)
    got = O.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def pin_e4m3_decoder():
    codes = np.arange(256, dtype=np.uint8)
    got = O.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert np.nanmax(got) == 448.0 and int(np.isnan(got).sum()) == 2


def pin_fp8_block_dequant(seed=9):
    rng = np.random.default_rng(seed)
    R, C = 130, 260                              # ragged last blocks
    q = rng.integers(0, 256, size=(R, C), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    sc = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    w = O.dequant_fp8_block(q, sc)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()
    for r in (0, 1, 127, 128, 129):
        for c in (0, 127, 128, 255, 256, 259):
            assert w[r, c] == dec[r, c] * float(sc[r // 128, c // 128])
    assert w[5, 5] == dec[5, 5] * float(sc[0, 0])
    # code 0x38 is exactly 1.0
    q1 = np.full((128, 128), 0x38, dtype=np.uint8)
    assert np.all(O.dequant_fp8_block(q1, np.array([[3.0]], dtype=np.float32)) == 3.0)


def pin_experts_touched():
    g = _golden("experts_touched.json")
    t = g["table_8_top2"]
    for B_, read, pct in t["rows"]:
        v = O.expected_experts_touched(t["n_experts"], t["top_k"], B_)
        assert _close_at(read, v, t["decimals"]), (B_, read, v)
        assert abs(100 * v / t["n_experts"] - pct) <= 0.5 + 1e-9 or pct == 100
    f = g["fine_grained_256_top8_b64"]
    v = O.expected_experts_touched(f["n_experts"], f["top_k"], f["batch"])
    assert abs(v - f["approx"]) <= f["rel_tol"] * f["approx"]
    s = g["share_woken_1_in_32"]
    for B_, pct in s["rows_percent"]:
        v = O.expected_experts_touched(s["n_experts"], s["top_k"], B_)
        assert abs(100 * v / s["n_experts"] - pct) <= 0.5 + 1e-9, (B_, pct, v)


def pin_touched_statistics(seed=10):
    """Uniform random routing: the mean distinct-expert count over trials is
    within 4 standard errors of the closed form."""
    rng = np.random.default_rng(seed)
    for N, k, Bt in ((8, 2, 4), (8, 2, 16), (256, 8, 64)):
        trials = 4000
        vals = np.empty(trials)
        for i in range(trials):
            idx = np.stack([rng.permutation(N)[:k] for _ in range(Bt)])
            vals[i] = np.count_nonzero(O.expert_counts(idx, N))
        mu = O.expected_experts_touched(N, k, Bt)
        assert abs(vals.mean() - mu) <= 4 * vals.std() / math.sqrt(trials) + 1e-9



# ---------------------------------------------------------------------------
# load statistics and the selection-bias controller
# ---------------------------------------------------------------------------

def pin_router_probabilities():
    """Softmax mode is the library softmax; sigmoid mode equals the softmax
    of log-sigmoid (a different route to sigmoid / sum); rows sum to 1; the
    most probable expert is the softmax-mode top-1."""
    rng = np.random.default_rng(21)
    s = rng.normal(0, 2, (37, 11))
    p = O.router_probabilities(s, "softmax")
    ref = torch.softmax(torch.tensor(s, dtype=torch.float64), dim=1).numpy()
    assert np.allclose(p, ref, rtol=1e-13, atol=1e-15)
    q = O.router_probabilities(s, "sigmoid")
    refq = torch.softmax(torch.nn.functional.logsigmoid(torch.tensor(s, dtype=torch.float64)), dim=1).numpy()
    assert np.allclose(q, refq, rtol=1e-12, atol=1e-15)
    assert np.allclose(q.sum(axis=1), 1.0) and np.allclose(p.sum(axis=1), 1.0)
    top1 = O.top_k_select(O.selection_scores(s, "softmax"), 1)[:, 0]
    assert np.array_equal(np.argmax(p, axis=1), top1)


def pin_load_statistics_closed_forms():
    """[CH19] 19.3.3: L_aux = alpha * N * sum f_i P_i.  With P uniform the
    sum is 1/N whatever f is, so L_aux = alpha; likewise with f uniform; when
    every token goes to one expert with probability -> 1, L_aux -> alpha * N."""
    rng = np.random.default_rng(22)
    T, N, k, alpha = 40, 8, 2, 0.01
    counts = rng.multinomial(T * k, rng.dirichlet(np.ones(N)))
    flat = O.router_probabilities(np.zeros((T, N)), "softmax")
    f, P, aux = O.load_statistics(counts, flat, k, alpha)
    assert abs(aux - alpha) < 1e-15 and abs(f.sum() - 1) < 1e-15 and abs(P.sum() - 1) < 1e-12
    probs = O.router_probabilities(rng.normal(0, 1, (T, N)), "softmax")
    _, _, aux2 = O.load_statistics(np.full(N, T * k // N), probs, k, alpha)
    assert abs(aux2 - alpha) < 1e-14
    s = np.full((T, N), -60.0)
    s[:, 0] = 60.0
    one = np.zeros(N, dtype=np.int64)
    one[0] = T
    _, P3, aux3 = O.load_statistics(one, O.router_probabilities(s, "softmax"), 1, alpha)
    assert abs(aux3 - alpha * N) < 1e-12 and abs(P3[0] - 1) < 1e-12


def pin_load_statistics_brute():
    rng = np.random.default_rng(23)
    T, N, k, alpha = 6, 5, 2, 0.01
    s = rng.normal(0, 1, (T, N))
    counts = [2, 0, 5, 3, 2]
    f, P, aux = O.load_statistics(counts, O.router_probabilities(s, "softmax"), k, alpha)
    bf, bP, baux = B.load_stats(s.tolist(), counts, k, alpha)
    assert np.allclose(f, bf, rtol=0, atol=1e-15) and np.allclose(P, bP, rtol=1e-13)
    assert abs(aux - baux) < 1e-14


def pin_bias_controller_rule():
    """[AIS-12] "How are experts kept evenly busy?": overloaded experts' biases
    drop by 0.001, underloaded ones rise by 0.001; exactly at the mean the
    bias stays.  Mean 2 (T*k = 8 over N = 4) and mean 2.5 (10 over 4)."""
    d = np.float32(0.001)
    b = O.bias_controller_step(np.zeros(4, np.float32), [5, 1, 2, 0], 2)
    assert b.dtype == np.float32 and np.array_equal(b, np.array([-d, d, 0, d], np.float32))
    b0 = np.array([0.5, -0.25, 0.1, 0.0], np.float32)
    b = O.bias_controller_step(b0, [3, 2, 3, 2], 1)
    want = np.array([b0[0] - d, b0[1] + d, b0[2] - d, b0[3] + d], dtype=np.float32)
    assert np.array_equal(b, want)


def pin_bias_controller_balances():
    """[MoE-LLM] "DeepSeek-style bias controller": applied batch after batch,
    the biases settle where traffic spreads evenly.  A skewed sigmoid router
    (per-expert logit offsets) routes fresh random batches; the controller
    (step 0.01 to converge quickly) lowers the max/mean load."""
    rng = np.random.default_rng(24)
    N, d, k, T = 16, 8, 2, 256
    w = rng.normal(0, 1 / math.sqrt(d), (d, N))
    off = -1.0 * np.log(np.arange(1, N + 1))
    bias = np.zeros(N, np.float32)
    imb = []
    for it in range(60):
        x = rng.normal(0, 1, (T, d))
        r = O.route_tokens(x, w, k, "sigmoid", off, bias.astype(np.float64))
        c = O.expert_counts(r.idx, N)
        imb.append(c.max() / c.mean())
        bias = O.bias_controller_step(bias, c, k, step=0.01)
    assert np.mean(imb[-10:]) < 0.6 * np.mean(imb[:3]), imb


# ---------------------------------------------------------------------------
# capacity-limited dispatch
# ---------------------------------------------------------------------------

def pin_capacity_limit():
    """[CH19] 19.6.1: C = ceil(c * T * K / N).  T*K/N = 100 and c = 1.1 give
    110 (the float product 1.1 * 100 is 110.00000000000001, and the binary
    value of 1.1 also exceeds 11/10); T*K/N = 10: c = 1.1 gives 11, c = 1.25
    gives 13 (12.5 up), c = 1.0 gives 10; T*K/N = 2.5 with c = 1.0 gives 3."""
    assert O.capacity_limit(1.1, 20, 2, 4) == 11
    assert O.capacity_limit(1.1, 100, 1, 1) == 110
    assert O.capacity_limit(1.1, 400, 2, 8) == 110
    assert O.capacity_limit(1.25, 20, 2, 4) == 13
    assert O.capacity_limit(1.0, 20, 2, 4) == 10
    assert O.capacity_limit(1.0, 5, 2, 4) == 3
    assert O.capacity_limit(2.0, 64, 1, 8) == 16


def pin_capacity_dispatch_brute():
    rng = np.random.default_rng(31)
    T, N, k = 40, 6, 2
    scores = rng.normal(0, 1, (T, N)) + np.array([1.5, 1.0, 0, 0, 0, 0])  # two hot experts
    idx = O.top_k_select(scores, k)
    for cap in (0, 3, 9, 40):
        P, keep = O.capacity_dispatch(idx, N, cap)
        bk = B.capacity_keep(idx.tolist(), N, cap)
        assert keep.tolist() == bk
        assert np.array_equal(P.counts, np.minimum(np.bincount(idx.ravel(), minlength=N), cap))
        kept = [(int(idx[t, i]), t, i) for t in range(T) for i in range(k) if bk[t][i]]
        assert [(int(idx[t, i]), t, i) for t, i in zip(P.perm_token, P.perm_slot)] == sorted(kept)
        for t in range(T):
            for i in range(k):
                r = P.inv_perm[t, i]
                assert (r >= 0) == bk[t][i] and (r < 0 or (P.perm_token[r], P.perm_slot[r]) == (t, i))


def pin_capacity_layer():
    """C >= max load is the dropless layer; C = 0 leaves only the shared
    expert; with a cap, a dropped branch contributes nothing and the kept
    gate keeps its value (no renormalisation)."""
    rng = np.random.default_rng(32)
    T, d, N, k, f = 24, 8, 4, 2, 6
    x = rng.normal(0, 1, (T, d))
    w = rng.normal(0, 1, (d, N)) + np.array([0.8, 0, 0, 0])
    ex = [tuple(rng.normal(0, 0.3, s) for s in ((f, d), (f, d), (d, f))) for _ in range(N + 1)]
    full, r, _ = O.moe_forward(x, w, ex[:N], k, "softmax", shared=ex[N])
    same, _, keep = O.moe_forward_capacity(x, w, ex[:N], k, T * k, "softmax", shared=ex[N])
    assert keep.all() and np.allclose(same, full, rtol=0, atol=1e-15)
    zero, _, _ = O.moe_forward_capacity(x, w, ex[:N], k, 0, "softmax", shared=ex[N])
    assert np.allclose(zero, O.swiglu_expert(x, *ex[N]), rtol=0, atol=1e-15)
    cap = 5
    out, r, keep = O.moe_forward_capacity(x, w, ex[:N], k, cap, "softmax")
    assert not keep.all()
    for t in range(T):
        want = sum(r.gates[t, i] * O.swiglu_expert(x[t:t + 1], *ex[r.idx[t, i]])[0]
                   for i in range(k) if keep[t, i]) if keep[t].any() else np.zeros(d)
        assert np.allclose(out[t], want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# group-limited selection
# ---------------------------------------------------------------------------

def pin_group_limited_selection():
    rng = np.random.default_rng(41)
    T, N, k = 60, 24, 4
    sc = rng.normal(0, 1, (T, N))
    sc[5, :] = 0.25  # all tied: groups and experts fall to the lowest indices
    # every group allowed: plain top-k
    assert np.array_equal(O.group_limited_top_k(sc, k, 6, 6), O.top_k_select(sc, k))
    # one group: the group of the best expert
    one = O.group_limited_top_k(sc, k, 4, 1)
    best = np.argmax(sc.astype(np.float32), axis=1)
    assert np.array_equal(one // 6, np.repeat((best // 6)[:, None], k, axis=1))
    for G, M in ((6, 2), (4, 3), (8, 3), (12, 4)):
        got = O.group_limited_top_k(sc, k, G, M)
        gs = N // G
        assert all(len(set((got[t] // gs).tolist())) <= M for t in range(T))
        bf = B.group_limited(sc.tolist(), k, G, M)
        assert got.tolist() == bf, (G, M)


def pin_nan_scores_rank_last():
    """A NaN selection score ranks below every other score, -inf included
    (NaN among themselves by index): k experts are always chosen.  Brute
    force with Python's sort on an explicit key; a group's best score skips
    NaN (NaN only when the whole group is NaN) and ranks the same way."""
    nan, inf = float("nan"), float("inf")
    rows = [[nan, 0.5, -inf, nan, 0.1, nan, 2.0, -1.0],
            [nan] * 8,
            [-inf, nan, -inf, nan, -inf, nan, -inf, nan],
            [nan, nan, 1.0, nan, nan, nan, nan, 3.0]]
    sc = np.array(rows)

    def key(v, e):
        return (1, 0.0, e) if v != v else (0, -v, e)

    for k in (1, 3, 6, 8):
        want = [sorted(range(8), key=lambda e: key(r[e], e))[:k] for r in rows]
        assert O.top_k_select(sc, k).tolist() == want, k
    for G, M, k in ((4, 2, 3), (2, 1, 2), (8, 3, 3)):
        gs = 8 // G
        want = []
        for r in rows:
            def gbest(g):
                vals = [r[e] for e in range(g * gs, (g + 1) * gs) if r[e] == r[e]]
                return max(vals) if vals else nan
            kept = sorted(range(G), key=lambda g: key(gbest(g), g))[:M]
            allowed = [e for g in kept for e in range(g * gs, (g + 1) * gs)]
            want.append(sorted(allowed, key=lambda e: key(r[e], e))[:k])
        assert O.group_limited_top_k(sc, k, G, M).tolist() == want, (G, M)


# ---------------------------------------------------------------------------
# MXFP4 weights
# ---------------------------------------------------------------------------

def pin_e8m0_decoder():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = O.e8m0_bits_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def pin_e2m1_decoder():
    """Every E2M1 value is an E4M3 value: sign kept, exponent field rebiased
    (bias 1 -> 7; the subnormal 0.5 is E4M3 exponent field 6), the mantissa
    bit moved to the top of the 3-bit field.  Decoded through the E4M3 table
    (itself pinned against torch) the 16 codes must agree."""
    got = O.e2m1_bits_to_f64(np.arange(16))
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            e4 = 0
        elif e == 0:
            e4 = (s << 7) | (6 << 3)
        else:
            e4 = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        ref = float(O.e4m3_bits_to_f64(np.array([e4], np.uint8))[0])
        assert got[c] == ref or (c == 8 and got[c] == 0.0), (c, got[c], ref)
    assert sorted(set(abs(v) for v in got)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def pin_mxfp4_dequant():
    rng = np.random.default_rng(51)
    out, inn = 3, 96
    packed = rng.integers(0, 256, (out, inn // 2), dtype=np.uint8)
    scales = rng.integers(115, 135, (out, inn // 32), dtype=np.uint8)
    got = O.dequant_mxfp4(packed, scales)
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for r in range(out):
        for c in range(inn):
            byte = int(packed[r, c // 2])
            code = byte & 0xF if c % 2 == 0 else byte >> 4
            v = (-1 if code & 8 else 1) * mags[code & 7] * 2.0 ** (int(scales[r, c // 32]) - 127)
            assert got[r, c] == v, (r, c)

ALL_PINS = [
    pin_router_worked_example_skillsuites, pin_router_worked_example_ai_infra,
    pin_softmax_placement_equivalence, pin_brute_force_routing,
    pin_sigmoid_invariants, pin_sigmoid_function, pin_router_logits_brute,
    pin_permutation, pin_layer_brute_force, pin_identical_experts_equal_dense,
    pin_distinct_experts_k_equals_n, pin_token_independence_and_relabel,
    pin_bf16_decoder, pin_e4m3_decoder, pin_fp8_block_dequant,
    pin_experts_touched, pin_router_probabilities, pin_load_statistics_closed_forms,
    pin_load_statistics_brute, pin_bias_controller_rule, pin_bias_controller_balances,
    pin_capacity_limit, pin_capacity_dispatch_brute, pin_capacity_layer,
    pin_group_limited_selection, pin_nan_scores_rank_last, pin_e8m0_decoder, pin_e2m1_decoder, pin_mxfp4_dequant,
]


@pytest.mark.parametrize("pin", ALL_PINS + [pin_touched_statistics], ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _m_full_softmax_no_renorm(logits, idx, route):
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, idx, axis=1)


def _m_gates_from_biased(orig):
    def f(logits, idx, route):
        if route == "sigmoid":
            a = O.sigmoid(np.take_along_axis(logits, idx, axis=1)) + 0.05 * (idx == 0)
            return a / a.sum(axis=1, keepdims=True)
        return orig(logits, idx, route)
    return f


def _m_topk_smallest(scores, k):
    return np.argsort(np.asarray(scores, dtype=np.float32), axis=1, kind="stable")[:, :k]


def _m_topk_ties_high(scores, k):
    s = np.asarray(scores, dtype=np.float32)
    N = s.shape[1]
    order = np.argsort(-s[:, ::-1], axis=1, kind="stable")
    return (N - 1 - order)[:, :k]


def _m_silu_on_up(X, wg, wu, wd):
    g = X @ wg.T
    u = X @ wu.T
    return (g * O.sigmoid(u) * u) @ wd.T


def _m_down_transposed(X, wg, wu, wd):
    h = O.silu(X @ wg.T) * (X @ wu.T)
    return h @ wd.reshape(wd.shape[1], wd.shape[0])


def _m_combine_drop_shared(y, g, inv, ys=None):
    return _orig_combine(y, g, inv, None)


def _m_combine_slot_swap(y, g, inv, ys=None):
    return _orig_combine(y, g[:, ::-1], inv, ys)


def _m_perm_unstable(idx, n):
    p = _orig_perm(idx, n)
    T, k = np.asarray(idx).shape
    # reverse token order inside each expert
    for e in range(n):
        lo, hi = p.offsets[e], p.offsets[e + 1]
        p.perm_token[lo:hi] = p.perm_token[lo:hi][::-1].copy()
    return p


def _m_bf16_truncate_sign(bits):
    return np.abs(_orig_bf16(bits))


def _m_e4m3_bias8(bits):
    return _orig_e4m3(bits) / 2.0


def _m_touched_linear(N, k, b):
    return min(N, k * b)


def _m_logits_no_offset(x, w, off=None):
    return _orig_logits(x, w, None)


def _m_aux_without_n(counts, probs, k, alpha=0.01):
    f, P, aux = _orig_load_stats(counts, probs, k, alpha)
    return f, P, aux / len(f)


def _m_probs_before_normalise(logits, route):
    s = np.asarray(logits, dtype=np.float64)
    return np.exp(s - s.max(axis=1, keepdims=True)) if route == "softmax" else O.sigmoid(s)


def _m_bias_sign_flipped(bias, counts, k, step=1e-3):
    return _orig_bias_step(bias, counts, k, -step)


def _m_bias_moves_at_mean(bias, counts, k, step=1e-3):
    c = np.asarray(counts)
    sign = np.where(c * len(c) > c.sum(), -1.0, 1.0).astype(np.float32)
    return (np.asarray(bias, np.float32) + np.float32(step) * sign).astype(np.float32)


_orig_load_stats = O.load_statistics
_orig_bias_step = O.bias_controller_step


def _m_capacity_float_ceil(factor, T, k, n):
    return int(math.ceil(factor * T * k / n))


def _m_capacity_keeps_last(idx, n_experts, capacity):
    rev = np.asarray(idx)[::-1]
    P, keep = _orig_cap_dispatch(rev, n_experts, capacity)
    return P, keep[::-1]


def _m_capacity_renormalise(x, w_router, experts, k, capacity, route="softmax", offset=None,
                            select_bias=None, shared=None):
    x = np.asarray(x, dtype=np.float64)
    r = O.route_tokens(x, w_router, k, route, offset, select_bias)
    _, keep = O.capacity_dispatch(r.idx, w_router.shape[1], capacity)
    g = np.where(keep, r.gates, 0.0)
    s = g.sum(axis=1, keepdims=True)
    g = np.where(s > 0, g / np.where(s > 0, s, 1), 0)
    out, _, _, _ = O.moe_forward_with_routing(x, r.idx, g, experts, w_router.shape[1], shared)
    return out, r, keep


_orig_cap_dispatch = O.capacity_dispatch


def _m_group_score_sum(scores, k, n_groups, max_groups):
    s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)
    T, N = s32.shape
    gs = N // n_groups
    gscore = s32.reshape(T, n_groups, gs).sum(axis=2)
    keep_g = np.argsort(-gscore, axis=1, kind="stable")[:, :max_groups]
    allowed = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(allowed, keep_g, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), s32, np.float32(-np.inf))
    return np.argsort(-masked, axis=1, kind="stable")[:, :k].astype(np.int64)


def _m_group_strided(scores, k, n_groups, max_groups):
    s = np.asarray(scores)
    T, N = s.shape
    perm = np.arange(N).reshape(N // n_groups, n_groups).T.reshape(-1)  # strided groups
    got = _orig_group_topk(s[:, perm], k, n_groups, max_groups)
    return perm[got]


_orig_group_topk = O.group_limited_top_k


def _m_e2m1_bias0(codes):
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    return s * np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e))


def _m_mxfp4_high_nibble_first(packed, scales, block=32):
    p = np.asarray(packed).astype(np.uint8)
    swapped = ((p & 0xF) << 4) | (p >> 4)
    return _orig_mxfp4(swapped, scales, block)


def _m_e8m0_bias128(bits):
    return _orig_e8m0(bits) / 2.0


_orig_mxfp4 = O.dequant_mxfp4
_orig_e8m0 = O.e8m0_bits_to_f64


_orig_perm = O.permute_assignments
_orig_bf16 = O.bf16_bits_to_f64
_orig_e4m3 = O.e4m3_bits_to_f64
_orig_logits = O.router_logits
_orig_combine = O.combine

MUTATIONS = {
    "gates_softmax_all_no_renormalise": ("gate_weights", lambda: _m_full_softmax_no_renorm),
    "gates_from_biased_scores": ("gate_weights", lambda: _m_gates_from_biased(O.gate_weights)),
    "topk_picks_smallest": ("top_k_select", lambda: _m_topk_smallest),
    "topk_ties_to_higher_index": ("top_k_select", lambda: _m_topk_ties_high),
    "silu_on_up_branch": ("swiglu_expert", lambda: _m_silu_on_up),
    "down_projection_transposed": ("swiglu_expert", lambda: _m_down_transposed),
    "combine_drops_shared": ("combine", lambda: _m_combine_drop_shared),
    "combine_swaps_slots": ("combine", lambda: _m_combine_slot_swap),
    "permutation_not_token_ordered": ("permute_assignments", lambda: _m_perm_unstable),
    "bf16_decoder_loses_sign": ("bf16_bits_to_f64", lambda: _m_bf16_truncate_sign),
    "e4m3_decoder_wrong_bias": ("e4m3_bits_to_f64", lambda: _m_e4m3_bias8),
    "experts_touched_linear": ("expected_experts_touched", lambda: _m_touched_linear),
    "router_drops_offset": ("router_logits", lambda: _m_logits_no_offset),
    "aux_loss_without_n": ("load_statistics", lambda: _m_aux_without_n),
    "probabilities_not_normalised": ("router_probabilities", lambda: _m_probs_before_normalise),
    "bias_controller_sign_flipped": ("bias_controller_step", lambda: _m_bias_sign_flipped),
    "bias_controller_moves_at_mean": ("bias_controller_step", lambda: _m_bias_moves_at_mean),
    "capacity_float_ceiling": ("capacity_limit", lambda: _m_capacity_float_ceil),
    "capacity_keeps_last_arrivals": ("capacity_dispatch", lambda: _m_capacity_keeps_last),
    "capacity_renormalises_gates": ("moe_forward_capacity", lambda: _m_capacity_renormalise),
    "group_score_is_sum": ("group_limited_top_k", lambda: _m_group_score_sum),
    "groups_strided_not_contiguous": ("group_limited_top_k", lambda: _m_group_strided),
    "e2m1_wrong_bias": ("e2m1_bits_to_f64", lambda: _m_e2m1_bias0),
    "mxfp4_high_nibble_first": ("dequant_mxfp4", lambda: _m_mxfp4_high_nibble_first),
    "e8m0_wrong_bias": ("e8m0_bits_to_f64", lambda: _m_e8m0_bias128),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(O, attr, make())
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
