"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes as C
import os
import re
import subprocess
import sys

import pytest

from mixture_experts_ffn_09_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")

FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_ffn.so is not built (python -m mixture_experts_ffn_09_amd.build)")
    return moe.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_router_topk", "moe_permute", "moe_grouped_ffn", "moe_combine",
              "moe_layer_forward"):
        assert n in names
    assert set(names) == set(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for n in _declared():
        assert hasattr(L, n), n


def shape(**kw):
    base = dict(T=16, d_model=4096, n_experts=8, top_k=2, d_ff=14336)
    base.update({k: v for k, v in kw.items() if k in base})
    rest = {k: v for k, v in kw.items() if k not in base}
    return moe.make_shape(base["T"], base["d_model"], base["n_experts"], base["top_k"],
                          base["d_ff"], **rest)


def _status(fn, *args):
    return getattr(_lib(), fn)(*args)


def test_status_strings():
    L = _lib()
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(3) == b"workspace too small"


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=600, top_k=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=100, top_k=65), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_model=4016), moe.MOE_ERR_UNSUPPORTED),                  # bf16 needs % 32
    (dict(w_dtype="fp8", d_ff=14336 + 64), moe.MOE_ERR_UNSUPPORTED),  # fp8 needs % 128
    (dict(act_dtype="f32", w_dtype="bf16"), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype="bf16", w_dtype="f32"), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_shared=2), moe.MOE_ERR_INVALID_ARG),
])
def test_bad_shapes_are_rejected(kw, code):
    s = shape(**kw)
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value)
    st = _status("moe_layer_forward", C.byref(s), C.byref(w), FAKE, C.c_void_p(0x2000), None,
                 FAKE, C.c_size_t(1 << 40), None)
    assert st == code, (kw, st, _lib().moe_last_error())
    assert _lib().moe_workspace_bytes(C.byref(s)) == C.c_size_t(-1).value


def test_null_shape_and_pointers():
    assert _status("moe_layer_forward", None, None, None, None, None, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARG
    s = shape()
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value)
    ws = C.c_size_t(moe.moe_workspace_bytes(s))
    # null x
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), None, FAKE, None, FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    # null router weight
    w2 = moe.Weights(w13=FAKE.value, w2=FAKE.value)
    assert _status("moe_layer_forward", C.byref(s), C.byref(w2), FAKE, C.c_void_p(0x2000), None,
                   FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    # x == out
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), FAKE, FAKE, None, FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    # selection bias with the softmax router
    w3 = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value, select_bias=FAKE.value)
    assert _status("moe_router_topk", C.byref(s), FAKE, C.byref(w3), FAKE, FAKE, FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    # shared expert without its weights
    s_sh = shape(n_shared=1, route="sigmoid")
    assert _status("moe_grouped_ffn", C.byref(s_sh), FAKE, None, FAKE, FAKE, C.byref(w), FAKE,
                   FAKE, FAKE, C.c_size_t(1 << 40), None) == moe.MOE_ERR_INVALID_ARG
    # fp8 without scales
    s8 = shape(w_dtype="fp8")
    assert _status("moe_grouped_ffn", C.byref(s8), FAKE, None, FAKE, FAKE, C.byref(w), FAKE,
                   None, FAKE, C.c_size_t(1 << 40), None) == moe.MOE_ERR_INVALID_ARG
    # permute without outputs
    r = moe.Routing()
    assert _status("moe_permute", C.byref(s), FAKE, None, C.byref(r), None, FAKE, ws, None) == \
        moe.MOE_ERR_INVALID_ARG
    # pack: src_b must be given exactly for the gate/up weight
    assert _status("moe_pack_weights", C.byref(s), 0, 1, FAKE, None, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert _status("moe_pack_weights", C.byref(s), 1, 1, FAKE, FAKE, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert _status("moe_pack_weights", C.byref(s), 5, 1, FAKE, None, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    # which = 2, 3 (scale packing) exists for MXFP4 weights only
    assert _status("moe_pack_weights", C.byref(s), 2, 1, FAKE, None, FAKE, None) == \
        moe.MOE_ERR_UNSUPPORTED


def test_misaligned_buffers_are_rejected():
    """Buffers moved with 16-byte vector accesses must be 16-byte aligned."""
    MIS = C.c_void_p(0x1008)
    s = shape()
    ws_n = C.c_size_t(moe.moe_workspace_bytes(s))
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value)
    err = moe.MOE_ERR_INVALID_ARG
    # misaligned x, out, workspace
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), MIS, C.c_void_p(0x4000), None,
                   FAKE, ws_n, None) == err
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), FAKE, MIS, None,
                   C.c_void_p(0x4000), ws_n, None) == err
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), FAKE, C.c_void_p(0x4000), None,
                   MIS, ws_n, None) == err
    # misaligned expert weight
    wm = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=MIS.value)
    assert _status("moe_layer_forward", C.byref(s), C.byref(wm), FAKE, C.c_void_p(0x4000), None,
                   C.c_void_p(0x8000), ws_n, None) == err
    # combine output, pack destination
    assert _status("moe_combine", C.byref(s), FAKE, None, FAKE, FAKE, MIS, None) == err
    assert _status("moe_pack_weights", C.byref(s), 1, 1, FAKE, None, MIS, None) == err


def test_workspace_too_small():
    s = shape()
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value)
    need = moe.moe_workspace_bytes(s)
    st = _status("moe_layer_forward", C.byref(s), C.byref(w), FAKE, C.c_void_p(0x2000), None,
                 FAKE, C.c_size_t(need - 1), None)
    assert st == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert b"needed" in _lib().moe_last_error()


def _router_splits(T, N, d, bf16=True):
    """Number of K-splits of the router logits (restated from the library's
    sizing rule: ~1024 workgroups, at least 256 of K per split)."""
    cdiv = lambda a, b: -(-a // b)
    if bf16 and (N > 8 or T >= 1024):   # the MFMA form: 64 x 64 tiles
        tiles = cdiv(T, 64) * cdiv(N, 64)
    elif N <= 8:
        tiles = cdiv(T, 256)
    else:
        tiles = cdiv(T, 32) * cdiv(N, 64)
    S = max(1, 1024 // tiles)
    S = min(S, cdiv(d, 256))
    KC = cdiv(cdiv(d, S), 64) * 64
    return cdiv(d, KC)


@pytest.mark.parametrize("T,N,k,d,f,sh", [(100, 256, 8, 7168, 2048, 1), (16, 8, 2, 4096, 14336, 0),
                                          (8192, 8, 2, 4096, 14336, 0)])
def test_workspace_size_formula(T, N, k, d, f, sh):
    s = shape(T=T, n_experts=N, top_k=k, d_model=d, d_ff=f, n_shared=sh,
              route="sigmoid" if sh else "softmax")
    a = lambda v: (v + 255) // 256 * 256
    S = _router_splits(T, N, d)
    # router scratch: partial logits, then (bf16 x, N > 8 or T >= 1024) the
    # three weight planes
    mfma = N > 8 or T >= 1024
    planes = a(S * T * N * 4) + (-(-d // 32)) * (-(-N // 16)) * 3 * 1024 if mfma else S * T * N * 4
    want = (a(planes) + 2 * a(T * k * 4) + a(N * 4) + a((N + 1) * 4) + 2 * a(T * k * 4)
            + a(-(-T // 256) * N * 4) + a(-(-T // 16) * N * 4)
            + a(N * 4) + a((N + 1) * 4) + 2 * a(T * k * 4) + a(2048 * 4) + a(T * k * f * 2)
            + a(sh * T * f * 2) + a(T * k * d * 2)
            + a(sh * T * d * 2))
    assert moe.moe_workspace_bytes(s) == want


def test_packed_sizes():
    s = shape(T=100, n_experts=256, top_k=8, d_model=7168, d_ff=2048, n_shared=1, route="sigmoid")
    d, f = 7168, 2048
    assert moe.moe_packed_weight_bytes(s, 0, 3) == 3 * 2 * d * f * 2
    assert moe.moe_packed_weight_bytes(s, 1, 1) == d * f * 2
    s8 = shape(w_dtype="fp8")
    assert moe.moe_packed_weight_bytes(s8, 1, 2) == 2 * 4096 * 14336
    # scale packing exists for MXFP4 only
    assert moe.moe_packed_weight_bytes(s, 2, 1) == 0
    assert moe.moe_packed_weight_bytes(s8, 3, 1) == 0
    assert moe.moe_packed_weight_bytes(s, 4, 1) == 0


def test_packed_mxfp4_scale_sizes():
    # rows x ceil(cols / 512) chunks of 16 bytes (one byte per 32 inputs,
    # padded to a whole group of four 128-wide K steps)
    s4 = shape(w_dtype="mxfp4")      # d 4096, d_ff 14336: no padding
    assert moe.moe_packed_weight_bytes(s4, 2, 3) == 3 * 2 * 14336 * (4096 // 32)
    assert moe.moe_packed_weight_bytes(s4, 3, 1) == 4096 * (14336 // 32)
    s4p = shape(w_dtype="mxfp4", d_model=384, d_ff=640)
    assert moe.moe_packed_weight_bytes(s4p, 2, 1) == 2 * 640 * 16
    assert moe.moe_packed_weight_bytes(s4p, 3, 2) == 2 * 384 * 32
    assert moe.moe_packed_weight_bytes(s4p, 0, 1) == 2 * 384 * 640 // 2


def test_pack_scale_argument_checks():
    call = lambda *a: _status("moe_pack_weights", *a)
    s = shape()
    assert call(C.byref(s), 2, 1, FAKE, None, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    s4 = shape(w_dtype="mxfp4")
    assert call(C.byref(s4), 2, 1, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call(C.byref(s4), 3, 1, None, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call(C.byref(s4), 4, 1, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call(C.byref(s4), 2, 0, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def test_zero_tokens_needs_no_device():
    s = shape(T=0)
    assert moe.moe_workspace_bytes(s) == 0
    w = moe.Weights()
    assert _status("moe_layer_forward", C.byref(s), C.byref(w), None, None, None, None, 0,
                   None) == moe.MOE_OK
    assert _status("moe_combine", C.byref(s), None, None, None, None, None, None) == moe.MOE_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()


def test_load_stats_argument_checks():
    s = shape()
    w = moe.Weights(w_router=FAKE.value)
    ws = C.c_size_t(moe.moe_workspace_bytes(s))
    f = C.c_float
    call = lambda *a: _status("moe_load_stats", *a)
    # x or counts missing
    assert call(C.byref(s), None, C.byref(w), FAKE, f(0.01), f(1e-3), None, None, None, None,
                FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    assert call(C.byref(s), FAKE, C.byref(w), None, f(0.01), f(1e-3), None, None, None, None,
                FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    # the bias belongs to the sigmoid router
    assert call(C.byref(s), FAKE, C.byref(w), FAKE, f(0.01), f(1e-3), None, None, None, FAKE,
                FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    # NaN step, small workspace, no router weight
    assert call(C.byref(s), FAKE, C.byref(w), FAKE, f(0.01), f(float("nan")), None, None, None,
                None, FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    assert call(C.byref(s), FAKE, C.byref(w), FAKE, f(0.01), f(1e-3), None, None, None, None,
                FAKE, C.c_size_t(ws.value - 1), None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call(C.byref(s), FAKE, C.byref(moe.Weights()), FAKE, f(0.01), f(1e-3), None, None, None,
                None, FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG
    # zero tokens: a no-op that touches nothing
    s0 = shape(T=0)
    assert call(C.byref(s0), None, None, None, f(0.01), f(1e-3), None, None, None, None, None,
                C.c_size_t(0), None) == moe.MOE_OK


def test_capacity_argument_checks():
    s = shape()
    ws = C.c_size_t(moe.moe_workspace_bytes(s))
    r = moe.Routing(counts=FAKE.value, offsets=FAKE.value, perm_token=FAKE.value,
                    inv_perm=FAKE.value)
    assert _status("moe_permute_capacity", C.byref(s), FAKE, -1, C.byref(r), FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    assert _status("moe_permute_capacity", C.byref(s), None, 4, C.byref(r), FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    assert _status("moe_permute_capacity", C.byref(s), FAKE, 4, C.byref(moe.Routing()), FAKE, ws,
                   None) == moe.MOE_ERR_INVALID_ARG
    assert _status("moe_permute_capacity", C.byref(s), FAKE, 4, C.byref(r), FAKE,
                   C.c_size_t(ws.value - 1), None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value)
    assert _status("moe_layer_forward_capacity", C.byref(s), C.byref(w), FAKE,
                   C.c_void_p(0x2000), -3, None, FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG


def test_grouped_argument_checks():
    s = shape(T=16, n_experts=256, top_k=8, d_model=7168, d_ff=2048, n_shared=1, route="sigmoid")
    ws = C.c_size_t(moe.moe_workspace_bytes(s))
    w = moe.Weights(w_router=FAKE.value, w13=FAKE.value, w2=FAKE.value, w13_shared=FAKE.value,
                    w2_shared=FAKE.value)
    call = lambda G, M: _status("moe_router_topk_grouped", C.byref(s), FAKE, C.byref(w), G, M,
                                FAKE, FAKE, FAKE, ws, None)
    assert call(0, 1) == moe.MOE_ERR_INVALID_ARG      # no groups
    assert call(7, 2) == moe.MOE_ERR_INVALID_ARG      # 7 does not divide 256
    assert call(128, 4) == moe.MOE_ERR_UNSUPPORTED    # more than 64 groups
    assert call(8, 0) == moe.MOE_ERR_INVALID_ARG      # max_groups < 1
    assert call(8, 9) == moe.MOE_ERR_INVALID_ARG      # max_groups > n_groups
    assert call(64, 1) == moe.MOE_ERR_INVALID_ARG     # 4 experts per group < top_k = 8
    assert _status("moe_layer_forward_grouped", C.byref(s), C.byref(w), FAKE, C.c_void_p(0x2000),
                   7, 2, None, FAKE, ws, None) == moe.MOE_ERR_INVALID_ARG


def test_validation_layer_under_host_sanitizers():
    """The host code of the C ABI (argument checks, workspace sizing and
    carving in abi.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer runs every other test of this file without a
    report (a report aborts the run)."""
    if os.environ.get("MOE_FFN_LIB"):
        pytest.skip("already running against another build of the library")
    from mixture_experts_ffn_09_amd import build as B
    lib = B.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "not instrumented"
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), MOE_FFN_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.abspath(__file__), "-q", "-x",
                        "-p", "no:cacheprovider", "-k", "not host_sanitizers"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
