"""Plain float64 CPU oracle of the token-choice sparse MoE FFN forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke entry point and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Sources (the pages are cited by title and section):
  [MoE-LLM]   "Mixture of Experts for LLM Inference" (talalahmed.dev), sections
              "The MoE change is surprisingly local", "Opening the router",
              "Shared experts: stop relearning the basics",
              "DeepSeek-style bias controller".
  [AIS-12]    "AI Infrastructure series - Part 12 of 24" (drpranayjha.com),
              sections "How does the router decide? A worked example",
              "What is a shared expert?",
              "What happens when many users share the GPU?".
  [CH19]      "Chapter 19: Mixture-of-Experts Models", 19.3.2 "A concrete
              router computation", 19.3.3, 19.3.4, 19.6.1 "Expert capacity".
  [MoE-EXP]   "Mixture of Experts Explained" (skillsuites.com), sections
              "The router, with real numbers", "The slot it replaces, and what
              an expert is", "Why batching erodes the advantage".

The method is exact (no approximation), so every function here is the plain
definition written out, with NumPy matmul / sort / bincount as the only library
steps.  Readings where the pages are silent (each also listed in the design
notes):
  * Expert form: SwiGLU, y = W_down (silu(W_gate x) * (W_up x)), silu on the
    gate branch, no biases.  The pages only say an expert is a complete FFN of
    "3 matrices" ([MoE-EXP] "The slot it replaces").
  * Selection is decided on float32-rounded scores (the kernel's precision),
    exact ties to the lower expert index; slot order = descending score.
  * The selection score is the logit in softmax mode (softmax is monotone) and
    sigmoid(logit) + bias in sigmoid mode.
  * The shared expert is added with coefficient 1, outside the router.
  * No residual add and no normalisation: the layer fills the FFN slot only.

Parity status: every function has a pin in ``tests/test_oracle_pins.py``
against values the pages print, closed forms, library routines or brute force;
see ``PARITY_PINS``.  None is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "e4m3_bits_to_f64", "dequant_fp8_block",
    "e2m1_bits_to_f64", "e8m0_bits_to_f64", "dequant_mxfp4",
    "router_logits", "sigmoid", "selection_scores", "top_k_select",
    "gate_weights", "Routing", "route_tokens",
    "expert_counts", "expert_offsets", "Permutation", "permute_assignments",
    "gather_rows", "silu", "swiglu_expert", "combine",
    "moe_forward", "moe_forward_with_routing", "expected_experts_touched",
    "router_probabilities", "load_statistics", "bias_controller_step",
    "capacity_limit", "capacity_dispatch", "moe_forward_capacity",
    "group_limited_top_k", "PARITY_PINS",
]

# Which test pins each function (documentation for readers of the oracle).
PARITY_PINS = {
    "bf16_bits_to_f64": "exhaustive 65536 codes vs torch bfloat16 -> float",
    "e4m3_bits_to_f64": "exhaustive 256 codes vs torch float8_e4m3fn -> float",
    "dequant_fp8_block": "hand-built blocks with known scales; brute force",
    "e8m0_bits_to_f64": "exhaustive 256 codes vs torch float8_e8m0fnu",
    "e2m1_bits_to_f64": "all 16 codes re-encoded bit by bit as E4M3 and read "
        "with the (torch-pinned) E4M3 decoder; the format's magnitude list",
    "dequant_mxfp4": "pure-Python nibble loop; hand-built blocks",
    "router_logits": "pure-Python triple loop on tiny inputs",
    "top_k_select / gate_weights (softmax)": "page worked examples "
        "([MoE-EXP] router with real numbers; [AIS-12] worked example); "
        "equivalence softmax-all->top-k->renormalise ([CH19] 19.3.2); "
        "brute-force subset enumeration",
    "top_k_select / gate_weights (sigmoid)": "invariants: gates sum to 1, "
        "bias moves selection never weights, equal logits -> 1/k, k=N -> "
        "sigmoid/sum; brute force",
    "expert_counts / permute_assignments": "invariants + brute force with "
        "Python sorted()",
    "swiglu_expert / combine / moe_forward": "identical experts == dense "
        "SwiGLU (torch fp64 library) at k=N and k<N; pure-Python brute "
        "force; [AIS-12] combine arithmetic; token independence",
    "expected_experts_touched": "[MoE-EXP] batching table, [AIS-12] 3/64/98%",
    "router_probabilities": "rows sum to 1; softmax mode vs torch.softmax "
        "(library); sigmoid mode reduces to softmax of log-sigmoid; top-1 of "
        "the probabilities equals the selection in softmax mode",
    "load_statistics": "closed forms: L_aux = alpha when P (or f) is uniform, "
        "alpha*N at full collapse; sum f = sum P = 1; pure-Python brute force",
    "bias_controller_step": "[AIS-12] +-0.001 rule on hand-built counts "
        "(over, under, exactly at the mean); float32 exactness",
    "capacity_limit": "[CH19] 19.6.1 formula on exact cases, including "
        "factors whose float product overshoots an integer",
    "group_limited_top_k": "all groups allowed == top_k_select; one group "
        "== the best expert's group; pure-Python enumeration of group subsets; "
        "selections span <= max_groups groups.  The group-ranking rule itself "
        "(best expert score) is a reading the pages do not fix",
    "capacity_dispatch / moe_forward_capacity": "pure-Python first-come "
        "brute force; C >= max load equals dropless; C = 0 leaves only the "
        "shared expert; dropped branches contribute 0, gates not renormalised",
}


# ---------------------------------------------------------------------------
# Number formats (inputs arrive as raw bit patterns)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    bfloat16 is the top half of an IEEE binary32 word, so the value is the
    binary32 whose high 16 bits are ``bits`` and whose low 16 bits are zero.
    """
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN payloads stay NaN
        return u.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    """All 256 OCP FP8 E4M3 values, from the format's definition.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field
    0 is subnormal (m/8 * 2^-6).  S.1111.111 is NaN; there is no infinity, so
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if (code >> 7) & 1 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = math.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3 = _e4m3_table()


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 bit patterns (uint8) -> float64 (table from the format)."""
    return _E4M3[np.asarray(bits).astype(np.uint8)]


def e2m1_bits_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (0..15) -> float64, from the format's definition: 1 sign
    bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 is
    subnormal (m/2).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN.
    The MX element format of expert weights in MXFP4 ([AIS-12] "Quantize the
    experts first": gpt-oss ships its experts in MXFP4; the format itself is
    the OCP microscaling one)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return s * mag


def e8m0_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """E8M0 shared scales (uint8) -> float64: 2^(e - 127), e = 255 is NaN."""
    e = np.asarray(bits).astype(np.int64)
    with np.errstate(invalid="ignore"):
        return np.where(e == 255, math.nan, np.exp2(e - 127.0))


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """MXFP4 weight [out][in] -> float64: packed holds two E2M1 codes per byte
    ([out][in/2], element 2j in the low nibble), scales one E8M0 per 32
    consecutive elements of a row ([out][in/32]); w = e2m1 * 2^(e - 127)."""
    p = np.asarray(packed).astype(np.uint8)
    out, half = p.shape
    codes = np.empty((out, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    sc = e8m0_bits_to_f64(scales)
    return e2m1_bits_to_f64(codes) * np.repeat(sc, block, axis=1)


def dequant_fp8_block(q_bits: np.ndarray, scales: np.ndarray,
                      block: int = 128) -> np.ndarray:
    """Block-scaled FP8 weight -> float64.

    ``q_bits`` is an [rows][cols] uint8 matrix of E4M3 codes and ``scales`` an
    [ceil(rows/block)][ceil(cols/block)] float32 matrix; element (r, c) is
    ``e4m3(q[r, c]) * scales[r // block, c // block]``.  This is the
    8-bit expert-weight storage the pages speak of ([CH19] 19.4, [MoE-LLM]
    "Memory and expert parallelism") with one scale per 128x128 tile.
    """
    w = e4m3_bits_to_f64(q_bits)
    rows, cols = w.shape
    sc = np.asarray(scales, dtype=np.float64)
    assert sc.shape == (-(-rows // block), -(-cols // block)), sc.shape
    full = np.repeat(np.repeat(sc, block, axis=0), block, axis=1)[:rows, :cols]
    return w * full


# ---------------------------------------------------------------------------
# a1: router logits
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_offset: Optional[np.ndarray] = None) -> np.ndarray:
    """One raw score per expert: ``s = x @ W_router`` (+ per-expert offset).

    [MoE-LLM] "Opening the router": a small learned linear layer maps the
    token's hidden vector to N scores.  [CH19] 19.3.2: ``gate_logits =
    hidden_state @ W_router``; [MoE-EXP]: the router is one d_model x
    n_experts matrix.  ``x`` is [T][d], ``w_router`` is [d][N]; float64.
    ``logit_offset`` is an optional per-expert additive term (a router with a
    bias term), used by the skewed decode workload.
    """
    s = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64)
    if logit_offset is not None:
        s = s + np.asarray(logit_offset, dtype=np.float64)[None, :]
    return s


# ---------------------------------------------------------------------------
# a2: score, select, gate
# ---------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def selection_scores(logits: np.ndarray, route: str,
                     select_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """The quantity top-k ranks, in float64.

    softmax mode: the logit itself.  Softmax is monotone, so ranking logits
    ranks probabilities ([CH19] 19.3.2 takes top-k of the logits).
    sigmoid mode: sigmoid affinity plus the per-expert bias, the bias serving
    selection only ([MoE-LLM] "DeepSeek-style bias controller"; [CH19] 19.3.4;
    [AIS-12] worked example, DeepSeek-V3 paragraph).
    """
    if route == "softmax":
        return np.asarray(logits, dtype=np.float64)
    if route == "sigmoid":
        a = sigmoid(logits)
        if select_bias is not None:
            a = a + np.asarray(select_bias, dtype=np.float64)[None, :]
        return a
    raise ValueError(f"unknown route {route!r}")


def top_k_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best experts per token, best first.

    Ranking is done on float32-rounded scores (the precision the GPU decides
    in); exact ties go to the lower expert index.  A NaN score ranks below
    every other score, -inf included (NaN among themselves by index), so k
    experts are always chosen.  Returns int64 [T][k].
    """
    s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)
    T, N = s32.shape
    if not 1 <= k <= N:
        raise ValueError("need 1 <= k <= N")
    # Stable sort by descending score keeps lower indices first among ties.
    order = np.argsort(-s32, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def group_limited_top_k(scores: np.ndarray, k: int, n_groups: int,
                        max_groups: int) -> np.ndarray:
    """Top-k restricted to at most max_groups groups of experts ([MoE-LLM]
    "Three tricks that tame the all-to-alls": DeepSeek-V3 ranges experts into
    groups, one per node, and caps how many nodes a token may visit; [AIS-12]
    "How much traffic is that? A worked example": at most 4 servers).

    Groups are contiguous runs of N / n_groups experts.  Reading (the pages
    give no ranking rule for groups): a group's score is the best selection
    score among its experts; the max_groups best groups are kept (exact ties
    to the lower group index), then the usual top-k runs over the experts of
    the kept groups.  Decisions on float32-rounded scores, as top_k_select."""
    s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)
    T, N = s32.shape
    if N % n_groups or not 1 <= max_groups <= n_groups:
        raise ValueError("need n_groups | N and 1 <= max_groups <= n_groups")
    gs = N // n_groups
    if k > max_groups * gs:
        raise ValueError("k exceeds the experts of the allowed groups")
    # a NaN score ranks below every other one (as in top_k_select): a group's
    # best score skips NaN and is NaN only when all of its scores are
    with np.errstate(invalid="ignore"):
        gscore = np.fmax.reduce(s32.reshape(T, n_groups, gs), axis=2)
    keep_g = np.argsort(-gscore, axis=1, kind="stable")[:, :max_groups]
    allowed = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(allowed, keep_g, True, axis=1)
    # experts of the kept groups first, each part by (score desc, NaN last),
    # exact ties to the lower index (lexsort is stable; its last key is primary)
    outside = ~np.repeat(allowed, gs, axis=1)
    order = np.lexsort((-s32, outside), axis=1)
    return order[:, :k].astype(np.int64)


def gate_weights(logits: np.ndarray, idx: np.ndarray, route: str) -> np.ndarray:
    """Mixing weights of the selected experts; each row sums to 1.

    softmax mode: softmax over the k selected logits ([CH19] 19.3.2;
    [MoE-EXP] "The router, with real numbers"), which equals softmax over all
    N, keep top-k, renormalise ([MoE-LLM] "Opening the router").
    sigmoid mode: the selected *unbiased* sigmoid affinities divided by their
    sum ([AIS-12] DeepSeek-V3 paragraph; [CH19] 19.3.4: mixing weights come
    from the original affinities, not the biased ones).
    """
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx, axis=1)
    if route == "softmax":
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    if route == "sigmoid":
        a = sigmoid(sel)
        return a / a.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown route {route!r}")


@dataclass
class Routing:
    logits: np.ndarray   # [T][N] float64
    scores: np.ndarray   # [T][N] float64 selection scores
    idx: np.ndarray      # [T][k] int64 expert ids, best first
    gates: np.ndarray    # [T][k] float64, rows sum to 1


def route_tokens(x, w_router, k: int, route: str = "softmax",
                 logit_offset=None, select_bias=None, groups=None) -> Routing:
    """Score, select, renormalise ([MoE-LLM] "Opening the router": the
    skeleton is the same for softmax and sigmoid routers).  groups =
    (n_groups, max_groups) limits the groups a token may use."""
    if select_bias is not None and route != "sigmoid":
        raise ValueError("a selection bias belongs to the sigmoid router")
    logits = router_logits(x, w_router, logit_offset)
    scores = selection_scores(logits, route, select_bias)
    if groups is None:
        idx = top_k_select(scores, k)
    else:
        idx = group_limited_top_k(scores, k, *groups)
    gates = gate_weights(logits, idx, route)
    return Routing(logits, scores, idx, gates)


# ---------------------------------------------------------------------------
# a3 / a4: counts, offsets, expert-contiguous permutation ("route and pack")
# ---------------------------------------------------------------------------

def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    """Number of (token, slot) assignments per expert ([CH19] 19.7.3 lists
    per-expert token counts as the evidence to collect)."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n_experts).astype(np.int64)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum with the total appended: [N + 1]."""
    out = np.zeros(len(counts) + 1, dtype=np.int64)
    out[1:] = np.cumsum(counts)
    return out


@dataclass
class Permutation:
    counts: np.ndarray      # [N]
    offsets: np.ndarray     # [N + 1]
    perm_token: np.ndarray  # [T*k] token of each expert-contiguous row
    perm_slot: np.ndarray   # [T*k] slot (0..k-1) of each row
    inv_perm: np.ndarray    # [T][k] row of each (token, slot)


def permute_assignments(idx: np.ndarray, n_experts: int) -> Permutation:
    """Pack assignments expert by expert ([CH19] 19.6.3 "Route and pack").

    Rows are ordered by (expert ascending, token ascending).  A token picks
    an expert at most once, so this key is unique and the order is fixed.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1)                       # position f = t * k + i
    order = np.argsort(flat, kind="stable")      # stable: token order kept
    counts = expert_counts(idx, n_experts)
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return Permutation(counts, expert_offsets(counts), order // k, order % k,
                       inv.reshape(T, k))


def gather_rows(x: np.ndarray, perm_token: np.ndarray) -> np.ndarray:
    """Expert-contiguous copy of the token rows: row r = x[perm_token[r]]."""
    return np.asarray(x)[np.asarray(perm_token)]


# ---------------------------------------------------------------------------
# a5 / a6: the expert FFN
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z)."""
    return np.asarray(z, dtype=np.float64) * sigmoid(z)


def swiglu_expert(X: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down: np.ndarray) -> np.ndarray:
    """One expert on its rows: ``(silu(X Wg^T) * (X Wu^T)) Wd^T``.

    Weights are stored [out][in]: ``w_gate``, ``w_up`` are [d_ff][d] and
    ``w_down`` is [d][d_ff].  An expert is a complete FFN with its own
    parameters ([MoE-LLM] "The MoE change is surprisingly local"; [CH19]
    19.3.1), built of three matrices ([MoE-EXP] "The slot it replaces").
    """
    X = np.asarray(X, dtype=np.float64)
    g = X @ np.asarray(w_gate, dtype=np.float64).T
    u = X @ np.asarray(w_up, dtype=np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down, dtype=np.float64).T


# ---------------------------------------------------------------------------
# a7: weighted combine (+ shared expert)
# ---------------------------------------------------------------------------

def combine(y_perm: np.ndarray, gates: np.ndarray, inv_perm: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    """``out[t] = sum_i gates[t, i] * Y[inv_perm[t, i]] (+ Y_shared[t])``.

    The weighted sum of the selected experts' outputs ([MoE-LLM] "The MoE
    change is surprisingly local"; [CH19] 19.3.2), plus the always-on shared
    expert with coefficient 1 ([MoE-LLM] "Shared experts"; [AIS-12] "What is
    a shared expert?").
    """
    y_perm = np.asarray(y_perm, dtype=np.float64)
    T, k = np.asarray(inv_perm).shape
    out = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for i in range(k):
        out += np.asarray(gates, dtype=np.float64)[:, i:i + 1] * y_perm[np.asarray(inv_perm)[:, i]]
    if y_shared is not None:
        out += np.asarray(y_shared, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------

ExpertWeights = Tuple[np.ndarray, np.ndarray, np.ndarray]


def moe_forward_with_routing(x: np.ndarray, idx: np.ndarray, gates: np.ndarray,
                             experts: Sequence[ExpertWeights] | Callable[[int], ExpertWeights],
                             n_experts: int,
                             shared: Optional[ExpertWeights] = None):
    """Experts and combine for a given routing (steps a3..a7).

    ``experts`` is a sequence (or callable) giving expert e's (w_gate, w_up,
    w_down) as float64 arrays; only experts that received rows are fetched,
    mirroring that unselected experts' bytes are never read ([MoE-EXP]
    "Why heads cannot be sparsified the same way").  Dropless: every
    assignment is processed ([MoE-EXP] capacity paragraph: inference runs
    without a capacity factor).  Returns (out [T][d], Permutation, Y [T*k][d],
    Y_shared or None).
    """
    get = experts if callable(experts) else experts.__getitem__
    x = np.asarray(x, dtype=np.float64)
    perm = permute_assignments(idx, n_experts)
    y = np.zeros((x.shape[0] * np.asarray(idx).shape[1], x.shape[1]), dtype=np.float64)
    for e in range(n_experts):
        lo, hi = int(perm.offsets[e]), int(perm.offsets[e + 1])
        if hi == lo:
            continue
        wg, wu, wd = get(e)
        y[lo:hi] = swiglu_expert(gather_rows(x, perm.perm_token[lo:hi]), wg, wu, wd)
    y_shared = swiglu_expert(x, *shared) if shared is not None else None
    out = combine(y, gates, perm.inv_perm, y_shared)
    return out, perm, y, y_shared


def moe_forward(x, w_router, experts, k: int, route: str = "softmax",
                logit_offset=None, select_bias=None, shared=None):
    """The MoE FFN layer forward: route, run the chosen experts and the
    shared expert, return the gate-weighted sum.  Returns (out, Routing,
    Permutation)."""
    n_experts = np.asarray(w_router).shape[1]
    r = route_tokens(x, w_router, k, route, logit_offset, select_bias)
    out, perm, _, _ = moe_forward_with_routing(x, r.idx, r.gates, experts,
                                               n_experts, shared)
    return out, r, perm


# ---------------------------------------------------------------------------
# Decode-bytes accounting
# ---------------------------------------------------------------------------

def expected_experts_touched(n_experts: int, k: int, batch: int) -> float:
    """Expected number of distinct experts B independently routed tokens
    wake: N * (1 - (1 - k/N)^B) ([AIS-12] "What happens when many users share
    the GPU?"; [MoE-EXP] "Why batching erodes the advantage")."""
    return n_experts * (1.0 - (1.0 - k / n_experts) ** batch)


# ---------------------------------------------------------------------------
# Load statistics and the selection-bias controller
# ---------------------------------------------------------------------------

def router_probabilities(logits: np.ndarray, route: str) -> np.ndarray:
    """Each token's routing probability over all N experts, [T][N].

    Softmax mode: the softmax of the N logits, the distribution the Switch
    balancing term averages ([CH19] 19.3.3: P_i is the batch's average routing
    probability of expert i).  Sigmoid mode (reading: the pages define no
    probability for it): the affinities sigmoid(s) divided by their sum over
    all N experts.  The selection bias never enters ([CH19] 19.3.4)."""
    s = np.asarray(logits, dtype=np.float64)
    if route == "softmax":
        z = np.exp(s - s.max(axis=1, keepdims=True))
    elif route == "sigmoid":
        z = sigmoid(s)
    else:
        raise ValueError(route)
    return z / z.sum(axis=1, keepdims=True)


def load_statistics(counts: np.ndarray, probs: np.ndarray, k: int,
                    alpha: float = 0.01):
    """Assignment shares f, mean probabilities P and the Switch balancing term
    L_aux = alpha * N * sum_i f_i P_i ([CH19] 19.3.3; weight 0.01 as Switch
    set it, [MoE-LLM] "Classic fix: auxiliary loss").

    f_i is expert i's share of the batch's T*k assignments (for top-1, the
    fraction of tokens routed to i, as the pages define it).  Returns
    (f [N], P [N], L_aux)."""
    counts = np.asarray(counts, dtype=np.float64)
    p = np.asarray(probs, dtype=np.float64)
    T, N = p.shape
    f = counts / (T * k)
    P = p.mean(axis=0)
    return f, P, alpha * N * float(np.dot(f, P))


def bias_controller_step(bias: np.ndarray, counts: np.ndarray, k: int,
                         step: float = 1e-3) -> np.ndarray:
    """One step of the selection-bias controller ([MoE-LLM] "DeepSeek-style
    bias controller"; [AIS-12] "How are experts kept evenly busy?": after a
    batch, an overloaded expert's bias drops by 0.001 and an underloaded
    one's rises by 0.001; [CH19] 19.3.4).

    Load is compared with the mean T*k/N in exact integer arithmetic
    (c_i * N against T*k); an expert exactly at the mean keeps its bias
    (reading: the pages name only the two other cases).  The bias is a float32
    parameter and the step is added in float32.  The result is the bias the
    next batch selects with: the controller reads only past batches."""
    c = np.asarray(counts, dtype=np.int64)
    N = c.shape[0]
    total = int(c.sum())
    if total % k:
        raise ValueError("counts must sum to T*k")
    sign = np.sign(total - c * N).astype(np.float32)  # +1 under-, -1 overloaded
    b = np.asarray(bias, dtype=np.float32)
    return (b + np.float32(step) * sign).astype(np.float32)


# ---------------------------------------------------------------------------
# Capacity-limited dispatch
# ---------------------------------------------------------------------------

def capacity_limit(factor, T: int, k: int, n_experts: int) -> int:
    """Per-expert capacity C = ceil(c * T * k / N) ([CH19] 19.6.1), computed
    exactly in rational arithmetic with the factor taken as the decimal number
    it is written as (a float's shortest decimal form), so that c = 1.1 with
    T*k/N = 100 gives 110, not the 111 a float product would give."""
    from fractions import Fraction
    c = Fraction(repr(float(factor))) if isinstance(factor, float) else Fraction(factor)
    q = c * T * k / n_experts
    return int(math.ceil(q))


def capacity_dispatch(idx: np.ndarray, n_experts: int, capacity: int):
    """Dispatch with a per-expert cap ([CH19] 19.6.1 "Capacity-limited";
    [AIS-12] "How are experts kept evenly busy?"; [MoE-EXP] capacity
    paragraph): each expert keeps its first `capacity` assignments in token
    order (then slot order) and drops the rest.

    Returns (Permutation of the kept assignments in the same (expert, token,
    slot) order, keep mask [T][k]).  Dropped assignments have inv_perm -1."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    full = permute_assignments(idx, n_experts)
    keep = np.zeros((T, k), dtype=bool)
    counts = np.minimum(full.counts, capacity)
    offsets = expert_offsets(counts)
    perm = np.zeros(int(offsets[-1]), dtype=np.int64)
    slot = np.zeros(int(offsets[-1]), dtype=np.int64)
    inv = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for i in range(k):
            e = int(idx[t, i])
            rank = int(full.inv_perm[t, i]) - int(full.offsets[e])
            if rank < capacity:
                keep[t, i] = True
                r = int(offsets[e]) + rank
                perm[r], slot[r] = t, i
                inv[t, i] = r
    return Permutation(counts=counts, offsets=offsets, perm_token=perm, perm_slot=slot,
                       inv_perm=inv), keep


def moe_forward_capacity(x, w_router, experts, k: int, capacity: int, route: str = "softmax",
                         offset=None, select_bias=None, shared=None):
    """The layer with capacity-limited dispatch: a dropped assignment's
    branch contributes nothing and the remaining gates are not renormalised
    (reading: the pages say only that the dropped branch skips its expert,
    [MoE-EXP] capacity paragraph; [CH19] 19.6.1)."""
    x = np.asarray(x, dtype=np.float64)
    r = route_tokens(x, w_router, k, route, offset, select_bias)
    _, keep = capacity_dispatch(r.idx, w_router.shape[1], capacity)
    gates = np.where(keep, r.gates, 0.0)
    out, _, _, _ = moe_forward_with_routing(x, r.idx, gates, experts, w_router.shape[1], shared)
    return out, r, keep
